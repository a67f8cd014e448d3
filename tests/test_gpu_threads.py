"""Concurrent use of the C ABI from several host threads.

Every entry point is documented as thread-safe: the per-device tables of a
seed are built once under a lock, and calls on different streams share no
state.  Here four threads, each on its own stream and with its own sketch
seed (so the first calls build the tables concurrently), encode keys with
all three encoders, decode and score, three times over; every result must
equal, bit for bit, the same calls made afterwards one at a time on the
default stream, and the first thread's sign bits must equal the oracle's.
"""

import threading

import numpy as np
import pytest

import oracle

from .gpu_util import dev_f32, dev_u16, host_u32, say

pytestmark = pytest.mark.gpu

D, M, N, HKV, G = 128, 256, 4096, 2, 4
THREADS, ROUNDS = 4, 3


def _inputs(i):
    rng = np.random.default_rng(9100 + i)
    keys = oracle.float64_to_bf16_bits(rng.standard_normal((1, HKV, N, D)))
    vals = oracle.float64_to_bf16_bits(rng.standard_normal((1, HKV, N, D)))
    q = rng.standard_normal((1, HKV * G, D)).astype(np.float32)
    return keys, vals, q


def _run_all(qjl, seed, keys, vals, q, stream):
    """Every entry point once on `stream`; returns the results as int32 bit
    patterns (device tensors)."""
    import torch
    with torch.cuda.stream(stream):
        signs = torch.zeros((1, HKV, N, M // 32), dtype=torch.int32, device="cuda")
        norms = torch.zeros((1, HKV, N), dtype=torch.float32, device="cuda")
        qjl.encode_keys(keys, signs, norms, 0, seed, M, stream=stream)
        out = qjl.decode_attention(q, signs, norms, vals, N, seed, M, stream=stream)
        codes = torch.zeros((1, HKV, N, D * 2 // 32), dtype=torch.int32, device="cuda")
        bits = torch.zeros((1, HKV, N, D // 32), dtype=torch.int32, device="cuda")
        tnorms = torch.zeros((1, HKV, N), dtype=torch.float32, device="cuda")
        gammas = torch.zeros((1, HKV, N), dtype=torch.float32, device="cuda")
        qjl.tq_encode_keys(keys, codes, bits, tnorms, gammas, 0, seed, 2, stream=stream)
        scores = qjl.tq_scores(q, codes, bits, tnorms, gammas, N, seed, 2, stream=stream)
        pcodes = torch.zeros((1, HKV, N, 12), dtype=torch.int32, device="cuda")
        radii = torch.zeros((1, HKV, N), dtype=torch.float32, device="cuda")
        qjl.pq_encode_keys(keys, pcodes, radii, 0, seed, stream=stream)
    res = {"signs": signs, "norms": norms, "out": out, "codes": codes, "bits": bits,
           "tnorms": tnorms, "gammas": gammas, "scores": scores, "pcodes": pcodes, "radii": radii}
    return {k: v.view(torch.int32) for k, v in res.items()}


def test_threads_match_sequential(gpu_lib):
    import torch
    qjl = gpu_lib
    host = [_inputs(i) for i in range(THREADS)]
    dev = [(dev_u16(k), dev_u16(v), dev_f32(q)) for k, v, q in host]
    seeds = [7301 + 17 * i for i in range(THREADS)]   # used by no other test
    torch.cuda.synchronize()

    say("threads: 4 host threads x 3 rounds, every entry point, own streams and seeds")
    results = [[None] * ROUNDS for _ in range(THREADS)]
    errors = []
    start = threading.Barrier(THREADS)

    def worker(i):
        try:
            stream = torch.cuda.Stream()
            start.wait()
            for r in range(ROUNDS):
                results[i][r] = _run_all(qjl, seeds[i], *dev[i], stream)
            stream.synchronize()
        except BaseException as exc:   # reported by the main thread
            errors.append((i, exc))

    ts = [threading.Thread(target=worker, args=(i,)) for i in range(THREADS)]
    for t in ts:
        t.start()
    for t in ts:
        t.join(timeout=300)
    assert not any(t.is_alive() for t in ts), "a worker thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()

    say("threads: the same calls one at a time on the default stream")
    for i in range(THREADS):
        ref = _run_all(qjl, seeds[i], *dev[i], torch.cuda.current_stream())
        torch.cuda.synchronize()
        for r in range(ROUNDS):
            for name, t in ref.items():
                assert torch.equal(results[i][r][name], t), (i, r, name)

    # the first thread's sign words and norms against the oracle
    keys0 = host[0][0].reshape(-1, D)
    words, nrm = oracle.encode(keys0, oracle.sketch(seeds[0], D, M))
    got = host_u32(results[0][0]["signs"]).reshape(-1, M // 32)
    np.testing.assert_array_equal(got, words)
    gn = results[0][0]["norms"].view(torch.float32).cpu().numpy().reshape(-1)
    np.testing.assert_allclose(gn, nrm, rtol=1e-5)

#!/usr/bin/env python3
"""QJL KV-cache benchmark on one MI355X: decode HBM GB/s and encode keys/s.

A step is one pass of the whole hot path over one batch of synthetic input:
encode the workload's cached keys (sign bits + norms), then one decode step
over them (S^T q, bit-estimated scores, online softmax, weighted sum of bf16
values).  The headline workload is ``gqa32k``: Llama-3.1-8B-shaped GQA
decode, 32 query / 8 kv heads, d = 128, m = 256, batch 1, 32768 cached
tokens.

Headline ``value``: the decode step's effective HBM bandwidth, algorithmic
bytes (sign words + norms + bf16 values + q + out) over the decode kernel's
duration, timed with HIP events on the launch stream around K decode
launches issued back to back (a spin kernel ahead of the first event holds
the GPU until the host has queued all K, so the events time the kernels, not
the host's launch rate).  The encode is timed the same way.

Every timed loop cycles through a ring of buffer sets whose bytes touched by
the timed kernels (read and written) add up to more than 600 MiB, more than
twice the 256 MB last-level cache, so no launch finds its inputs left in that
cache by an earlier one.

With no ``--workload`` the line also carries ``configs``, one entry per
other workload, each measured the same way in the same run:

* ``small``    - 1 kv / 8 q heads, 4096 tokens: encode and decode latency;
* ``prefill``  - 16 x 8192 tokens x 8 kv heads: encode keys/s, fraction of
                 the bf16 matrix-core peak and of HBM bandwidth;
* ``long64k``  - m = 512, 65536 cached tokens, then 64 consecutive decode
                 steps that each append one token (encode of one key per kv
                 head, then the decode over all tokens): per-step median,
                 total and HBM fraction;
* ``mha16k``   - 40 heads, batch 8, 16384 tokens: decode time and HBM
                 fraction (and the encode of its 5.2 M keys);
* ``rotq``     - TurboQuant_prod and PolarQuant encodes of the 32K workload's
                 keys and TurboQuant scores over them.

The headline also times the fused decode step (one launch that appends a
token and decodes) and the uncompressed bf16-KV baseline at equal context.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, 8 TB/s
FP64_PEAK_TFLOPS = 78.6         # MI355X fp64 (vector and matrix)
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
SEED = 42
RING_BYTES = 600 * 2 ** 20      # > 2 x 256 MB last-level cache, per timed loop
MAX_SETS = 512
METRIC = "decode attention effective HBM GB/s (% peak) + encode keys/sec, 32K ctx"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def sha256_of(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def kernel_sources(kind):
    csrc = os.path.join(ROOT, "jl_rotated_bit_amd", "csrc")
    return [os.path.join(csrc, f"{kind}.hip"), os.path.join(csrc, "internal.h"),
            os.path.join(csrc, "exact_sign.h")]


def measured_traffic(kind, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary,
    or None when there is none or the kernel source changed since."""
    path = os.path.join(ROOT, "profiles", f"{kind}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256") != sha256_of(kernel_sources(kind)):
        return None
    return rec.get("hbm_bytes_per_launch")


DESCRIPTIONS = {
    "gqa32k": "gqa32k: Llama-3.1-8B-shaped GQA decode, 32 q / 8 kv heads, d=128, m=256, batch 1, "
              "32768 cached tokens; encode of those 262144 keys + one decode step",
    "small": "small: 1 kv / 8 q heads, d=128, m=256, 4096 tokens",
    "tp8": "tp8: one GPU's share of gqa32k under 8-way tensor parallelism: 1 kv / 4 q heads, d=128, "
           "m=256, batch 1, 32768 tokens",
    "prefill": "prefill: encode of 16 x 8192 tokens x 8 kv heads (1048576 keys), d=128, m=256",
    "long64k": "long64k: 8 kv / 32 q heads, d=128, m=512, 65536 cached tokens, then 64 decode steps "
               "that each append one token",
    "mha16k": "mha16k: LLaMA-2-13B-shaped MHA decode, 40 heads, d=128, m=256, batch 8, 16384 tokens",
}


def decode_bytes(B, Hq, Hkv, N, d, m):
    """Algorithmic bytes of one decode call: per (token, kv head) m/8 bytes of
    sign words, a 4-byte norm and 2d bytes of bf16 values; q and out."""
    return B * Hkv * N * (m // 8 + 4 + 2 * d) + B * Hq * d * 4 * 2


def baseline_bytes(B, Hq, Hkv, N, d):
    """Algorithmic bytes of the uncompressed baseline: bf16 keys and values."""
    return B * Hkv * N * 4 * d + B * Hq * d * 4 * 2


def encode_bytes_per_key(d, m):
    """Per key: the bf16 key read, m/8 bytes of sign words and a norm written."""
    return 2 * d + m // 8 + 4


def ring_sets(touched_bytes):
    return int(min(MAX_SETS, max(1, -(-RING_BYTES // max(1, touched_bytes)))))


def roofline(achieved_gbs, traffic, kernel, alg_bytes):
    return {"bound": "hbm", "achieved": round(achieved_gbs, 2), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
            "kernel": kernel, "algorithmic_bytes_per_launch": int(alg_bytes)}


# GPU clock cycles of hold per queued call (~250 us at 2.4 GHz)
HOLD_CYCLES_PER_CALL = 600_000


class Timer:
    """HIP events on the launch stream (torch's current stream, which is
    the stream every call below is issued on)."""

    def __init__(self):
        import torch
        self.torch = torch
        self.stream = torch.cuda.current_stream()

    def b2b(self, fn, reps):
        """fn(i) for i < reps issued back to back between two events; ms per call.

        A spin kernel queued ahead of the first event holds the GPU while the
        host issues the reps calls (Python and ctypes take ~10-30 us a call),
        so the events time the kernels back to back, not the launch rate; the
        host's issue time is compared with the hold and a shortfall logged.
        """
        import time
        torch = self.torch
        torch.cuda.synchronize()
        h0 = torch.cuda.Event(enable_timing=True)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        h0.record(self.stream)
        torch.cuda._sleep(int(reps * HOLD_CYCLES_PER_CALL))
        e0.record(self.stream)
        t0 = time.perf_counter()
        for i in range(reps):
            fn(i)
        host_ms = (time.perf_counter() - t0) * 1e3
        e1.record(self.stream)
        torch.cuda.synchronize()
        hold_ms = h0.elapsed_time(e0)
        if host_ms > hold_ms:
            log(f"[bench] note: host issue {host_ms:.2f} ms outlasted the {hold_ms:.2f} ms hold "
                f"(the timing below is partly launch-bound)")
        return e0.elapsed_time(e1) / reps

    def each(self, fn, reps):
        """fn(i) back to back with an event between consecutive calls (the
        GPU held as in b2b while the host queues them); returns the per-call
        durations (ms) and the total (ms)."""
        torch = self.torch
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        torch.cuda._sleep(int(reps * HOLD_CYCLES_PER_CALL))
        ev[0].record(self.stream)
        for i in range(reps):
            fn(i)
            ev[i + 1].record(self.stream)
        torch.cuda.synchronize()
        per = [ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]
        return per, ev[0].elapsed_time(ev[reps])


def dev(a):
    import numpy as np
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def caches(B, Hkv, cap, m):
    import torch
    return (torch.zeros((B, Hkv, cap, m // 32), dtype=torch.int32, device="cuda"),
            torch.zeros((B, Hkv, cap), dtype=torch.float32, device="cuda"))


# ----------------------------------------------------------------------------
# headline: gqa32k (encode of the cached keys + one decode step)
# ----------------------------------------------------------------------------

def bench_gqa32k(qjl, w, args, T):
    import numpy as np
    import torch
    B, Hq, Hkv, N, cap, d, m = w.B, w.H_q, w.H_kv, w.N, w.cap, w.d, w.m
    n_keys = B * Hkv * N
    dbytes = decode_bytes(B, Hq, Hkv, N, d, m)
    ebytes = n_keys * encode_bytes_per_key(d, m)
    n_sets = ring_sets(min(dbytes, ebytes))
    log(f"[bench] gqa32k: {n_sets} buffer sets (decode touches {dbytes / 2**20:.1f} MiB, "
        f"encode {ebytes / 2**20:.1f} MiB per call)")
    keys_h, vals_h = w.keys[:, :, :N], w.values
    sets = []
    for _ in range(n_sets):
        signs, norms = caches(B, Hkv, cap, m)
        sets.append(dict(keys=dev(keys_h), values=dev(vals_h), signs=signs, norms=norms,
                         q=dev(w.q), out=torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")))
    ws = torch.zeros(qjl.decode_workspace_bytes(B, Hq, Hkv, N, d, m), dtype=torch.uint8, device="cuda")
    stream = T.stream

    def enc(i):
        s = sets[i % n_sets]
        qjl.encode_keys(s["keys"], s["signs"], s["norms"], 0, SEED, m)

    def dec(i):
        s = sets[i % n_sets]
        qjl.decode_attention(s["q"], s["signs"], s["norms"], s["values"], N, SEED, m,
                             out=s["out"], workspace=ws)

    def step(i, ev=None):
        if ev is not None:
            ev[0].record(stream)
        enc(i)
        if ev is not None:
            ev[1].record(stream)
        dec(i)
        if ev is not None:
            ev[2].record(stream)

    log(f"[bench] gqa32k warmup {args.warmup}")
    for i in range(max(args.warmup, n_sets)):
        step(i)
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    log(f"[bench] gqa32k timing {args.steps} steps")
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
    stop.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    enc_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    dec_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])

    # Kernel durations for the rooflines: each kernel launched back to back
    # over the ring (events around single launches inside a step also hold
    # the ~2-3 us of dispatch that a kernel following other work does not pay).
    b2b_dec_ms = T.b2b(dec, args.steps)
    b2b_enc_ms = T.b2b(enc, args.steps)
    log(f"[bench] gqa32k back to back: decode {b2b_dec_ms * 1e3:.2f} us, encode {b2b_enc_ms * 1e3:.2f} us")

    # A decode step that first appends one token: the newest key of every
    # (batch, kv head) is encoded into row N - 1, then the decode runs over
    # all N tokens.  (Writing the new value row is the caller's copy.)
    new_keys = [s["keys"][:, :, N - 1:N].contiguous() for s in sets]

    def append_step(i):
        s = sets[i % n_sets]
        qjl.encode_keys(new_keys[i % n_sets], s["signs"], s["norms"], N - 1, SEED, m)
        dec(i)
    append_ms = T.b2b(append_step, args.steps)
    log(f"[bench] gqa32k append step (encode of {B * Hkv} keys + decode): {append_ms * 1e3:.2f} us")

    # The same step in one launch (qjl_decode_step): the append of token
    # N - 1 (its key encoded, its value row copied) happens inside the decode.
    new_vals = [s["values"][:, :, N - 1].contiguous() for s in sets]
    new_keys1 = [k.reshape(B, Hkv, d) for k in new_keys]

    def fused_step(i):
        s = sets[i % n_sets]
        qjl.decode_step(s["q"], new_keys1[i % n_sets], new_vals[i % n_sets], s["signs"], s["norms"],
                        s["values"], N - 1, SEED, m, out=s["out"], workspace=ws)
    fused_ms = T.b2b(fused_step, args.steps)
    log(f"[bench] gqa32k fused step (append inside the decode launch): {fused_ms * 1e3:.2f} us")

    # The uncompressed baseline at the same context: exact attention over the
    # bf16 keys and values (2 x 256 bytes per token and kv head), same ring.
    bbytes = baseline_bytes(B, Hq, Hkv, N, d)
    nb = ring_sets(bbytes)

    def base(i):
        s = sets[i % min(nb, n_sets)]
        qjl.baseline_decode_attention_bf16(s["q"], s["keys"], s["values"], N, out=s["out"], workspace=ws)
    base(0)
    base_ms = T.b2b(base, args.steps)
    log(f"[bench] gqa32k bf16-KV baseline decode: {base_ms * 1e3:.2f} us")

    if args.copy_calibration:
        a = torch.empty(256 * 2 ** 20, dtype=torch.uint8, device="cuda").fill_(1)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        log("[bench] copy calibration: 3 x 256 MiB device copies done")

    dec_s, enc_s = b2b_dec_ms / 1e3, b2b_enc_ms / 1e3
    dec_gbs = dbytes / dec_s / 1e9
    enc_gbs = ebytes / enc_s / 1e9
    enc_tflops = 2.0 * n_keys * d * m / enc_s / 1e12
    res = {
        "ms_per_step": round(total_ms / args.steps, 5),
        "value": round(dec_gbs, 2),
        "decode_frac_of_hbm_peak": round(dec_gbs / HBM_PEAK_GBS, 4),
        "decode_us": round(dec_s * 1e6, 3),
        "decode_us_in_step": round(float(dec_ms.mean()) * 1e3, 3),
        "decode_us_in_step_p10_p90": [round(float(np.percentile(dec_ms, 10)) * 1e3, 3),
                                      round(float(np.percentile(dec_ms, 90)) * 1e3, 3)],
        "append_step_us": round(append_ms * 1e3, 3),
        "append_step_frac_of_hbm_peak": round(dbytes / (append_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
        "fused_step_us": round(fused_ms * 1e3, 3),
        "baseline_bf16_decode_us": round(base_ms * 1e3, 3),
        "baseline_bf16_frac_of_hbm_peak": round(bbytes / (base_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
        "speedup_vs_bf16_kv": round(base_ms / b2b_dec_ms, 3),
        "fused_step_frac_of_hbm_peak": round(dbytes / (fused_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
        "encode_keys_per_s": round(n_keys / enc_s, 1),
        "encode_us": round(enc_s * 1e6, 3),
        "encode_us_in_step": round(float(enc_ms.mean()) * 1e3, 3),
        "ring_sets": n_sets,
        "roofline": roofline(dec_gbs, measured_traffic("decode", "gqa32k"), "decode_kernel", dbytes),
        "roofline_encode": dict(roofline(enc_gbs, measured_traffic("encode", "gqa32k"), "encode_kernel", ebytes),
                                mfma_tflops=round(enc_tflops, 2),
                                mfma_frac_of_bf16_peak=round(enc_tflops / BF16_MFMA_PEAK_TFLOPS, 4)),
    }
    del sets, ws
    torch.cuda.empty_cache()
    return res


# ----------------------------------------------------------------------------
# other workloads
# ----------------------------------------------------------------------------

def bench_small(qjl, w, args, T, name="small", note="latency-bound (1.2 MB per decode call)"):
    import torch
    B, Hq, Hkv, N, d, m = w.B, w.H_q, w.H_kv, w.N, w.d, w.m
    dbytes = decode_bytes(B, Hq, Hkv, N, d, m)
    ebytes = B * Hkv * N * encode_bytes_per_key(d, m)
    n_sets = ring_sets(min(dbytes, ebytes))
    sets = []
    keys_d, vals_d, q_d = dev(w.keys), dev(w.values), dev(w.q)
    for _ in range(n_sets):
        signs, norms = caches(B, Hkv, N, m)
        sets.append(dict(keys=keys_d.clone(), values=vals_d.clone(), signs=signs, norms=norms, q=q_d.clone(),
                         out=torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")))
    ws = torch.zeros(qjl.decode_workspace_bytes(B, Hq, Hkv, N, d, m), dtype=torch.uint8, device="cuda")

    def enc(i):
        s = sets[i % n_sets]
        qjl.encode_keys(s["keys"], s["signs"], s["norms"], 0, SEED, m)

    def dec(i):
        s = sets[i % n_sets]
        qjl.decode_attention(s["q"], s["signs"], s["norms"], s["values"], N, SEED, m, out=s["out"], workspace=ws)
    reps = max(args.steps, n_sets)
    for i in range(n_sets):
        enc(i)
        dec(i)
    enc_ms = T.b2b(enc, reps)
    dec_ms = T.b2b(dec, reps)
    log(f"[bench] {name}: encode {enc_ms * 1e3:.2f} us, decode {dec_ms * 1e3:.2f} us")
    del sets
    torch.cuda.empty_cache()
    gbs = dbytes / (dec_ms / 1e3) / 1e9
    return {"workload": DESCRIPTIONS[name], "encode_us": round(enc_ms * 1e3, 3),
            "encode_keys_per_s": round(B * Hkv * N / (enc_ms / 1e3), 1),
            "decode_us": round(dec_ms * 1e3, 3), "decode_gbs": round(gbs, 2),
            "roofline": roofline(gbs, measured_traffic("decode", name), "decode_kernel", dbytes), "ring_sets": n_sets,
            "note": note}


def bench_tp8(qjl, w, args, T):
    return bench_small(qjl, w, args, T, name="tp8",
                       note="one GPU's share at 8-way tensor parallelism (9.6 MB per decode call)")


def bench_prefill(qjl, w, args, T):
    import torch
    B, Hkv, n, d, m = w.B, w.H_kv, w.N, w.d, w.m
    n_keys = B * Hkv * n
    ebytes = n_keys * encode_bytes_per_key(d, m)
    n_sets = ring_sets(ebytes)
    sets = []
    for _ in range(n_sets):
        signs, norms = caches(B, Hkv, n, m)
        sets.append((dev(w.keys), signs, norms))

    def enc(i):
        k, s, nm = sets[i % n_sets]
        qjl.encode_keys(k, s, nm, 0, SEED, m)
    for i in range(max(args.warmup, n_sets)):
        enc(i)
    ms = T.b2b(enc, args.steps)
    sec = ms / 1e3
    gbs = ebytes / sec / 1e9
    tflops = 2.0 * n_keys * d * m / sec / 1e12
    log(f"[bench] prefill: encode {ms * 1e3:.2f} us ({n_keys / sec / 1e9:.2f} G keys/s, "
        f"{tflops:.0f} TFLOP/s)")
    del sets
    torch.cuda.empty_cache()
    r = roofline(gbs, measured_traffic("encode", "prefill"), "encode_kernel", ebytes)
    return {"workload": DESCRIPTIONS["prefill"], "encode_us": round(sec * 1e6, 3),
            "encode_keys_per_s": round(n_keys / sec, 1),
            "mfma_tflops": round(tflops, 2),
            "mfma_frac_of_bf16_peak": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "roofline": r,
            "roofline_mfma": {"bound": "mfma", "achieved": round(tflops, 2),
                              "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                              "frac": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4),
                              "flops_per_launch": 2 * n_keys * d * m},
            "ring_sets": n_sets}


def bench_long64k(qjl, w, args, T):
    import numpy as np
    import torch
    B, Hq, Hkv, N0, cap, d, m = w.B, w.H_q, w.H_kv, w.N, w.cap, w.d, w.m
    steps = len(w.steps)
    dbytes_last = decode_bytes(B, Hq, Hkv, N0 + steps, d, m)
    n_sets = ring_sets(decode_bytes(B, Hq, Hkv, N0 + 1, d, m))
    sets = []
    keys_d = dev(w.keys)
    new_keys = [keys_d[:, :, N0 + s:N0 + s + 1].contiguous() for s in range(steps)]
    qs = [dev(q) for q in w.steps]
    ws = torch.zeros(qjl.decode_workspace_bytes(B, Hq, Hkv, cap, d, m), dtype=torch.uint8, device="cuda")
    for _ in range(n_sets):
        signs, norms = caches(B, Hkv, cap, m)
        # every set holds the whole encoded cache (the prefill, and the rows
        # the steps append, which they re-encode identically)
        qjl.encode_keys(keys_d, signs, norms, 0, SEED, m)
        sets.append(dict(values=dev(w.values), signs=signs, norms=norms,
                         out=torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")))
    del keys_d

    new_keys1 = [k.reshape(B, Hkv, d) for k in new_keys]
    new_vals = [dev(w.values[:, :, N0 + s].copy()) for s in range(steps)]

    def step(s):       # one launch: qjl_decode_step appends token N0 + s, then attends
        st = sets[s % n_sets]
        qjl.decode_step(qs[s], new_keys1[s], new_vals[s], st["signs"], st["norms"], st["values"],
                        N0 + s, SEED, m, out=st["out"], workspace=ws)

    def step2(s):      # two calls: encode of the new keys, then the decode
        st = sets[s % n_sets]
        qjl.encode_keys(new_keys[s], st["signs"], st["norms"], N0 + s, SEED, m)
        qjl.decode_attention(qs[s], st["signs"], st["norms"], st["values"], N0 + s + 1, SEED, m,
                             out=st["out"], workspace=ws)
    T.each(step, steps)                           # warmup: the 64 steps once
    per, _ = T.each(step, steps)                  # per-step times (events between the steps)
    per2, _ = T.each(step2, steps)
    # totals: the 64 steps back to back, no events between them
    total = T.b2b(step, steps) * steps
    total2 = T.b2b(step2, steps) * steps
    per = np.array(per)
    med = float(np.median(per))
    alg = np.array([decode_bytes(B, Hq, Hkv, N0 + s + 1, d, m) for s in range(steps)], dtype=np.float64)
    gbs_med = float(np.median(alg / (per / 1e3) / 1e9))
    # the decode kernel alone, back to back, at the last step's context
    dec_ms = T.b2b(lambda i: qjl.decode_attention(qs[-1], sets[i % n_sets]["signs"], sets[i % n_sets]["norms"],
                                                  sets[i % n_sets]["values"], N0 + steps, SEED, m,
                                                  out=sets[i % n_sets]["out"], workspace=ws), args.steps)
    dec_gbs = dbytes_last / (dec_ms / 1e3) / 1e9
    log(f"[bench] long64k: fused step median {med * 1e3:.2f} us, total {total:.3f} ms for {steps} steps; "
        f"two calls {float(np.median(per2)) * 1e3:.2f} us; decode alone {dec_ms * 1e3:.2f} us")
    del sets, ws
    torch.cuda.empty_cache()
    return {"workload": DESCRIPTIONS["long64k"], "steps": steps,
            "step_us_median": round(med * 1e3, 3),
            "step_us_p10_p90": [round(float(np.percentile(per, 10)) * 1e3, 3),
                                round(float(np.percentile(per, 90)) * 1e3, 3)],
            "total_ms": round(total, 4),
            "two_call_step_us_median": round(float(np.median(per2)) * 1e3, 3),
            "two_call_total_ms": round(total2, 4),
            "step_frac_of_hbm_peak": round(gbs_med / HBM_PEAK_GBS, 4),
            "decode_us": round(dec_ms * 1e3, 3),
            "roofline": roofline(dec_gbs, measured_traffic("decode", "long64k"), "decode_kernel", dbytes_last),
            "ring_sets": n_sets,
            "note": "a step = qjl_decode_step: the append of one token per kv head (key encoded, value "
                    "row copied) and the decode over all tokens, in one launch; two_call_* = "
                    "qjl_encode_keys of the new keys then qjl_decode_attention; step fraction = the "
                    "step's decode bytes / the step's time; per-step times carry an event between "
                    "steps, the totals none"}


def bench_mha16k(qjl, w, args, T):
    import torch
    B, Hq, Hkv, N, d, m = w.B, w.H_q, w.H_kv, w.N, w.d, w.m
    n_keys = B * Hkv * N
    dbytes = decode_bytes(B, Hq, Hkv, N, d, m)
    ebytes = n_keys * encode_bytes_per_key(d, m)
    n_sets = ring_sets(dbytes)       # one set of 1.5 GB already exceeds the ring size (n_sets = 1)
    keys_d = dev(w.keys)
    signs, norms = caches(B, Hkv, N, m)
    enc_reps = max(2, min(args.steps, 5))
    for _ in range(2):
        qjl.encode_keys(keys_d, signs, norms, 0, SEED, m)
    enc_ms = T.b2b(lambda i: qjl.encode_keys(keys_d, signs, norms, 0, SEED, m), enc_reps)
    sets = [dict(values=dev(w.values), signs=signs if k == 0 else signs.clone(),
                 norms=norms if k == 0 else norms.clone(), q=dev(w.q),
                 out=torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")) for k in range(n_sets)]
    ws = torch.zeros(qjl.decode_workspace_bytes(B, Hq, Hkv, N, d, m), dtype=torch.uint8, device="cuda")

    def dec(i):
        s = sets[i % n_sets]
        qjl.decode_attention(s["q"], s["signs"], s["norms"], s["values"], N, SEED, m, out=s["out"], workspace=ws)
    for i in range(max(2, args.warmup)):
        dec(i)
    dec_ms = T.b2b(dec, args.steps)
    gbs = dbytes / (dec_ms / 1e3) / 1e9
    # the uncompressed baseline over the same bf16 keys and values (2.7 GB)
    bbytes = baseline_bytes(B, Hq, Hkv, N, d)
    s0 = sets[0]
    base = lambda i: qjl.baseline_decode_attention_bf16(s0["q"], keys_d, s0["values"], N, out=s0["out"],
                                                        workspace=ws)
    base(0)
    base_ms = T.b2b(base, max(2, args.steps // 2))
    log(f"[bench] mha16k: decode {dec_ms * 1e3:.2f} us ({gbs:.0f} GB/s), encode {enc_ms * 1e3:.2f} us, "
        f"bf16-KV baseline {base_ms * 1e3:.2f} us")
    del sets, ws, signs, norms, keys_d
    torch.cuda.empty_cache()
    return {"workload": DESCRIPTIONS["mha16k"], "decode_us": round(dec_ms * 1e3, 3),
            "decode_gbs": round(gbs, 2), "decode_frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "roofline": roofline(gbs, measured_traffic("decode", "mha16k"), "decode_kernel", dbytes),
            "encode_us": round(enc_ms * 1e3, 3), "encode_keys_per_s": round(n_keys / (enc_ms / 1e3), 1),
            "encode_hbm_frac": round(ebytes / (enc_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
            "baseline_bf16_decode_us": round(base_ms * 1e3, 3),
            "baseline_bf16_frac_of_hbm_peak": round(bbytes / (base_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
            "speedup_vs_bf16_kv": round(base_ms / dec_ms, 3),
            "ring_sets": n_sets}


def bench_rotq(qjl, w, args, T):
    """TurboQuant_prod (k = 2: 3 bits per coordinate) and PolarQuant encodes of
    the 32K GQA workload's keys, and TurboQuant scores of its 32 query heads
    over them.  The encodes run their rotation (and TurboQuant's residual
    sketch) in fp64, so they are priced against the fp64 peak; the scores
    kernels read 56 bytes per (token, kv head) and write 4 bytes per (token,
    query head), priced against HBM, at batch 1 and (random cache contents)
    at batch 8."""
    import torch
    B, Hq, Hkv, N, d = w.B, w.H_q, w.H_kv, w.N, w.d
    k = 2
    R = B * Hkv * N
    tq_bytes = R * (2 * d + d * k // 8 + d // 8 + 8)
    n_sets = ring_sets(tq_bytes)
    sets = []
    for _ in range(n_sets):
        sets.append(dict(
            keys=dev(w.keys[:, :, :N]),
            codes=torch.zeros((B, Hkv, N, d * k // 32), dtype=torch.int32, device="cuda"),
            bits=torch.zeros((B, Hkv, N, d // 32), dtype=torch.int32, device="cuda"),
            norms=torch.zeros((B, Hkv, N), dtype=torch.float32, device="cuda"),
            gammas=torch.zeros((B, Hkv, N), dtype=torch.float32, device="cuda"),
            pq=torch.zeros((B, Hkv, N, 12), dtype=torch.int32, device="cuda"),
            radii=torch.zeros((B, Hkv, N), dtype=torch.float32, device="cuda"),
            q=dev(w.q), scores=torch.empty((B, Hq, N), dtype=torch.float32, device="cuda")))

    def tq(i):
        s = sets[i % n_sets]
        qjl.tq_encode_keys(s["keys"], s["codes"], s["bits"], s["norms"], s["gammas"], 0, SEED, k)

    def pq(i):
        s = sets[i % n_sets]
        qjl.pq_encode_keys(s["keys"], s["pq"], s["radii"], 0, SEED)

    def sc(i):
        s = sets[i % n_sets]
        qjl.tq_scores(s["q"], s["codes"], s["bits"], s["norms"], s["gammas"], N, SEED, k, out=s["scores"])
    for i in range(n_sets):
        tq(i)
        pq(i)
        sc(i)
    reps = max(4, args.steps // 2)
    tq_ms = T.b2b(tq, reps)
    pq_ms = T.b2b(pq, reps)
    sc_ms = T.b2b(sc, reps)
    log(f"[bench] rotq (32K GQA keys): TurboQuant encode {tq_ms * 1e3:.1f} us, PolarQuant encode "
        f"{pq_ms * 1e3:.1f} us, TurboQuant scores {sc_ms * 1e3:.1f} us")
    del sets
    torch.cuda.empty_cache()
    # The scores at batch 8 of the same shape, where the launch and latency
    # costs are spread over 8x the bytes.  Cache contents are seeded random
    # bit patterns (every pattern is a valid cache), norms in [0.5, 4),
    # residual norms in [0, 1).
    B8 = 8
    b8_bytes = B8 * Hkv * N * (d * k // 8 + d // 8 + 8) + B8 * Hq * N * 4
    n8 = ring_sets(b8_bytes)
    g = torch.Generator(device="cuda")
    g.manual_seed(2024)
    sets8 = []
    for _ in range(n8):
        sets8.append(dict(
            codes=torch.randint(-2 ** 31, 2 ** 31, (B8, Hkv, N, d * k // 32), dtype=torch.int32, device="cuda",
                                generator=g),
            bits=torch.randint(-2 ** 31, 2 ** 31, (B8, Hkv, N, d // 32), dtype=torch.int32, device="cuda", generator=g),
            norms=torch.rand((B8, Hkv, N), device="cuda", generator=g) * 3.5 + 0.5,
            gammas=torch.rand((B8, Hkv, N), device="cuda", generator=g),
            q=torch.randn((B8, Hq, d), device="cuda", generator=g),
            scores=torch.empty((B8, Hq, N), dtype=torch.float32, device="cuda")))

    def sc8(i):
        s = sets8[i % n8]
        qjl.tq_scores(s["q"], s["codes"], s["bits"], s["norms"], s["gammas"], N, SEED, k, out=s["scores"])
    for i in range(n8):
        sc8(i)
    sc8_ms = T.b2b(sc8, reps)
    log(f"[bench] rotq: TurboQuant scores at batch 8 {sc8_ms * 1e3:.1f} us")
    del sets8
    torch.cuda.empty_cache()
    tq_flops = R * 2.0 * (2 * d * d)            # rotation + residual sketch (m = d)
    pq_flops = R * 2.0 * d * d                  # rotation
    sc_bytes = R * (d * k // 8 + d // 8 + 8) + B * Hq * N * 4
    fp64 = lambda fl, ms, tr: {"bound": "mfma", "dtype": "f64", "achieved": round(fl / (ms / 1e3) / 1e12, 2),
                               "peak": FP64_PEAK_TFLOPS, "unit": "TFLOP/s",
                               "frac": round(fl / (ms / 1e3) / 1e12 / FP64_PEAK_TFLOPS, 4),
                               "traffic": tr, "flops_per_launch": int(fl)}
    return {"workload": "the 262144 keys and 32 query heads of the 32K GQA workload; TurboQuant_prod at "
                        "3 bits per coordinate (2-bit codes + 1-bit QJL of the residual), PolarQuant "
                        "4/2-bit levels",
            "tq_encode_us": round(tq_ms * 1e3, 3), "tq_encode_keys_per_s": round(R / (tq_ms / 1e3), 1),
            "tq_encode_roofline": fp64(tq_flops, tq_ms, measured_traffic("rotq", "tq_encode")),
            "pq_encode_us": round(pq_ms * 1e3, 3), "pq_encode_keys_per_s": round(R / (pq_ms / 1e3), 1),
            "pq_encode_roofline": fp64(pq_flops, pq_ms, measured_traffic("rotq", "pq_encode")),
            "tq_scores_us": round(sc_ms * 1e3, 3),
            "tq_scores_roofline": roofline(sc_bytes / (sc_ms / 1e3) / 1e9, measured_traffic("rotq", "tq_scores_b1"),
                                           "tq_query_kernel + tq_scores_mfma_kernel", sc_bytes),
            "tq_scores_batch8_us": round(sc8_ms * 1e3, 3),
            "tq_scores_batch8_roofline": roofline(b8_bytes / (sc8_ms / 1e3) / 1e9, measured_traffic("rotq", "tq_scores_b8"),
                                                  "tq_query_kernel + tq_scores_mfma_kernel", b8_bytes),
            "ring_sets": n_sets}


# ----------------------------------------------------------------------------
# the oracle on the host (cpu_baseline)
# ----------------------------------------------------------------------------

def cpu_baseline(w, min_decode_s=8.0, min_encode_s=4.0):
    """The oracle, as it stands, on this host: decode steps of the same
    workload (repeated until ~8 s) and an encode of a bounded key sample."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        threads = max(i.get("num_threads", 1) for i in info) if info else 1
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    d, m = w.d, w.m
    S = oracle.sketch(SEED, d, m)
    sample_keys = w.keys.reshape(-1, d)[: min(65536, w.B * w.H_kv * w.N)]
    t0 = time.perf_counter()
    enc_reps = 0
    while True:
        oracle.encode(sample_keys, S)
        enc_reps += 1
        if time.perf_counter() - t0 >= min_encode_s:
            break
    enc_time = time.perf_counter() - t0
    words, norms = oracle.encode(w.keys.reshape(-1, d), S)
    words = words.reshape(w.B, w.H_kv, w.cap, m // 32)
    norms = norms.reshape(w.B, w.H_kv, w.cap)
    t0 = time.perf_counter()
    reps = 0
    while True:
        oracle.decode(w.q, words, norms, w.values, w.N, S)
        reps += 1
        if time.perf_counter() - t0 >= min_decode_s:
            break
    dec_time = time.perf_counter() - t0
    dbytes = decode_bytes(w.B, w.H_q, w.H_kv, w.N, d, m)
    return {
        "value": dbytes * reps / dec_time / 1e9,
        "unit": "GB/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"{reps} full decode step(s) of the same workload (fp64 numpy, "
                   f"{dec_time:.1f} s); encode: {enc_reps} x {sample_keys.shape[0]} keys "
                   f"({enc_time:.1f} s)"),
        "encode_keys_per_s": enc_reps * sample_keys.shape[0] / enc_time,
        "host_cpus": os.cpu_count(),
        "affinity_cpus": len(os.sched_getaffinity(0)),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="all", choices=["all", "rotq", *sorted(DESCRIPTIONS)],
                    help="all (default): the gqa32k headline plus every other workload in `configs`; "
                         "a name: that workload alone (for profiling)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (counter calibration runs)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the QJL path runs on one GPU (no sharding or collectives).", file=sys.stderr)
        sys.exit(2)

    import torch
    from jl_rotated_bit_amd import qjl
    from jl_rotated_bit_amd import workloads as wl

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    torch.cuda.set_device(0)
    qjl.load()
    T = Timer()

    runners = {"small": bench_small, "tp8": bench_tp8, "prefill": bench_prefill, "long64k": bench_long64k,
               "mha16k": bench_mha16k, "rotq": bench_rotq}
    if args.workload not in ("all", "gqa32k"):
        name = args.workload
        log(f"[bench] generating workload {name}")
        res = runners[name](qjl, wl.WORKLOADS[{"rotq": "gqa32k"}.get(name, name)](), args, T)
        if args.copy_calibration:
            a = torch.empty(256 * 2 ** 20, dtype=torch.uint8, device="cuda").fill_(1)
            b = torch.empty_like(a)
            for _ in range(3):
                b.copy_(a)
            torch.cuda.synchronize()
        print(json.dumps({"workload_only": name, **res}), flush=True)
        return

    log("[bench] generating workload gqa32k")
    w = wl.gqa32k()
    head = bench_gqa32k(qjl, w, args, T)
    configs = {}
    if args.workload == "all":
        for name in ("small", "tp8", "prefill", "long64k", "mha16k"):
            log(f"[bench] generating workload {name}")
            t0 = time.perf_counter()
            wk = wl.WORKLOADS[name]()
            log(f"[bench] {name} generated in {time.perf_counter() - t0:.1f} s")
            configs[name] = runners[name](qjl, wk, args, T)
            del wk
        configs["rotq"] = bench_rotq(qjl, w, args, T)
    line = {
        "metric": METRIC,
        "value": head.pop("value"),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head.pop("ms_per_step"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": DESCRIPTIONS["gqa32k"], "batch": w.B, "q_heads": w.H_q,
                   "kv_heads": w.H_kv, "context": w.N, "head_dim": w.d, "sketch_m": w.m,
                   "sketch_seed": SEED},
        **head,
        "configs": configs,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle (cpu_baseline)")
        line["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

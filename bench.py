#!/usr/bin/env python3
"""QJL KV-cache benchmark on one MI355X: decode HBM GB/s and encode keys/s.

A step is one pass of the whole hot path over one batch of synthetic input:
encode the workload's cached keys (sign bits + norms), then one decode step
over them (S^T q, bit-estimated scores, online softmax, weighted sum of bf16
values).  The default workload is ``gqa32k``: Llama-3.1-8B-shaped GQA decode,
32 query / 8 kv heads, d = 128, m = 256, batch 1, 32768 cached tokens.

Reported ``value`` is the decode step's effective HBM bandwidth: algorithmic
bytes (sign words + norms + bf16 values + q + out) over the decode kernel's
duration, timed with HIP events around K decode launches issued back to back
(each on the next buffer set).  ``encode_keys_per_s`` is timed the same way.
The event times of each kernel inside the K timed steps are reported too
(``*_in_step``); they include the dispatch gap after the preceding event.  Inputs live in HBM before timing starts; every step uses the
next of several buffer sets whose total exceeds 512 MB, so the 256 MB
last-level cache cannot serve a step from an earlier one.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload gqa32k]
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

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
SEED = 42
RING_BYTES = 600 * 2 ** 20      # > 2 x 256 MB last-level cache


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
    return [os.path.join(csrc, f"{kind}.hip"), os.path.join(csrc, "internal.h")]


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


def make_workload(name):
    from jl_rotated_bit_amd import workloads as wl
    if name == "gqa32k":
        return wl.gqa32k()
    if name == "mha16k":
        return wl.mha16k()
    if name == "small":
        return wl.small()
    if name == "long64k":
        w = wl.long64k(steps=1)
        w.N = w.cap
        return w
    raise SystemExit(f"unknown workload {name}")


DESCRIPTIONS = {
    "gqa32k": "gqa32k: Llama-3.1-8B-shaped GQA decode, 32 q / 8 kv heads, d=128, m=256, batch 1, "
              "32768 cached tokens; encode of those 262144 keys + one decode step",
    "mha16k": "mha16k: LLaMA-2-13B-shaped MHA decode, 40 heads, d=128, m=256, batch 8, 16384 tokens",
    "small": "small: 1 kv / 8 q heads, d=128, m=256, 4096 tokens",
    "long64k": "long64k: 8 kv / 32 q heads, d=128, m=512, 65537 tokens",
}


def cpu_baseline(w, min_decode_s=8.0, min_encode_s=4.0):
    """The oracle, as it stands, on this host: decode steps of the same
    workload (repeated until ~8 s) and an encode of a bounded key sample."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max(i.get("num_threads", 1) for i in threadpool_info()) if threadpool_info() else 1
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    d, m = w.d, w.m
    S = oracle.sketch(SEED, d, m)
    sample_keys = w.keys.reshape(-1, d)[: min(65536, w.B * w.H_kv * w.N)]
    t0 = time.perf_counter()
    enc_reps = 0
    while True:
        words_s, _ = oracle.encode(sample_keys, S)
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
    dec_bytes = decode_bytes(w)
    return {
        "value": dec_bytes * reps / dec_time / 1e9,
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


def decode_bytes(w):
    per_token = w.m // 8 + 4 + 2 * w.d
    return w.B * w.H_kv * w.N * per_token + w.B * w.H_q * w.d * 4 * 2


def encode_bytes_per_key(w):
    return 2 * w.d + w.m // 8 + 4


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gqa32k", choices=sorted(DESCRIPTIONS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (counter calibration runs)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the QJL path runs on one GPU (no sharding or collectives).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from jl_rotated_bit_amd import qjl

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    torch.cuda.set_device(0)
    qjl.load()

    log(f"[bench] generating workload {args.workload}")
    w = make_workload(args.workload)
    B, Hq, Hkv, N, cap, d, m = w.B, w.H_q, w.H_kv, w.N, w.cap, w.d, w.m
    n_keys = B * Hkv * N

    set_bytes = (w.keys.nbytes + w.values.nbytes + B * Hkv * cap * (m // 8 + 4))
    n_sets = max(2, -(-RING_BYTES // set_bytes))
    log(f"[bench] {n_sets} buffer sets of {set_bytes / 2**20:.0f} MiB")
    keys_h = torch.from_numpy(w.keys[:, :, :N].copy().view(np.int16))
    vals_h = torch.from_numpy(w.values.view(np.int16))
    sets = []
    for _ in range(n_sets):
        sets.append(dict(
            keys=keys_h.cuda(), values=vals_h.cuda(),
            signs=torch.zeros((B, Hkv, cap, m // 32), dtype=torch.int32, device="cuda"),
            norms=torch.zeros((B, Hkv, cap), dtype=torch.float32, device="cuda"),
            q=torch.from_numpy(w.q).cuda(),
            out=torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")))
    ws = torch.zeros(qjl.decode_workspace_bytes(B, Hq, Hkv, N, d, m), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        s = sets[i % n_sets]
        if ev is not None:
            ev[0].record(stream)
        qjl.encode_keys(s["keys"], s["signs"], s["norms"], 0, SEED, m)
        if ev is not None:
            ev[1].record(stream)
        qjl.decode_attention(s["q"], s["signs"], s["norms"], s["values"], N, SEED, m,
                             out=s["out"], workspace=ws)
        if ev is not None:
            ev[2].record(stream)

    log(f"[bench] warmup {args.warmup}")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
    stop.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    total_ms = start.elapsed_time(stop)
    enc_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    dec_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])
    log(f"[bench] done: {total_ms:.3f} ms total, wall {t_wall * 1e3:.1f} ms")

    # Per-kernel durations for the rooflines: each kernel launched back to back
    # over the same buffer sets (a different set per launch), two events
    # around the whole run.  Events around single launches inside the step
    # (enc_ms / dec_ms above) also hold the ~2-3 us of dispatch that a kernel
    # following other work in a stream does not pay.
    def back_to_back(kind, reps):
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(reps):
            s = sets[i % n_sets]
            if kind == "encode":
                qjl.encode_keys(s["keys"], s["signs"], s["norms"], 0, SEED, m)
            else:
                qjl.decode_attention(s["q"], s["signs"], s["norms"], s["values"], N, SEED, m,
                                     out=s["out"], workspace=ws)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps
    b2b_dec_ms = back_to_back("decode", args.steps)
    b2b_enc_ms = back_to_back("encode", args.steps)
    log(f"[bench] back to back: decode {b2b_dec_ms * 1e3:.2f} us, encode {b2b_enc_ms * 1e3:.2f} us")

    # A decode step that first appends one token: the newest key of every
    # (batch, kv head) is encoded into row N - 1 of the caches, then the
    # decode runs over all N tokens.  (Writing the new value row is the
    # caller's copy and is not timed.)
    new_keys = [s["keys"][:, :, N - 1:N].contiguous() for s in sets]
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        s = sets[i % n_sets]
        qjl.encode_keys(new_keys[i % n_sets], s["signs"], s["norms"], N - 1, SEED, m)
        qjl.decode_attention(s["q"], s["signs"], s["norms"], s["values"], N, SEED, m,
                             out=s["out"], workspace=ws)
    e1.record(stream)
    torch.cuda.synchronize()
    append_ms = e0.elapsed_time(e1) / args.steps
    log(f"[bench] append step (encode of {B * Hkv} keys + decode): {append_ms * 1e3:.2f} us")

    if args.copy_calibration:
        a = torch.empty(256 * 2 ** 20, dtype=torch.uint8, device="cuda").fill_(1)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        log("[bench] copy calibration: 3 x 256 MiB device copies done")

    dbytes = decode_bytes(w)
    dec_s = b2b_dec_ms / 1e3
    enc_s = b2b_enc_ms / 1e3
    dec_gbs = dbytes / dec_s / 1e9
    ebytes = n_keys * encode_bytes_per_key(w)
    enc_gbs = ebytes / enc_s / 1e9
    enc_tflops = 2.0 * n_keys * d * m / enc_s / 1e12
    trf_dec = measured_traffic("decode", args.workload)
    trf_enc = measured_traffic("encode", args.workload)

    line = {
        "metric": "decode attention effective HBM GB/s (% peak) + encode keys/sec, 32K ctx",
        "value": round(dec_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": DESCRIPTIONS[args.workload], "batch": B, "q_heads": Hq,
                   "kv_heads": Hkv, "context": N, "head_dim": d, "sketch_m": m,
                   "sketch_seed": SEED},
        "decode_frac_of_hbm_peak": round(dec_gbs / HBM_PEAK_GBS, 4),
        "decode_us": round(dec_s * 1e6, 3),
        "decode_us_in_step": round(float(dec_ms.mean()) * 1e3, 3),
        "decode_us_in_step_p10_p90": [round(float(np.percentile(dec_ms, 10)) * 1e3, 3),
                                      round(float(np.percentile(dec_ms, 90)) * 1e3, 3)],
        "append_step_us": round(append_ms * 1e3, 3),
        "append_step_frac_of_hbm_peak": round(dbytes / (append_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
        "encode_keys_per_s": round(n_keys / enc_s, 1),
        "encode_us": round(enc_s * 1e6, 3),
        "encode_us_in_step": round(float(enc_ms.mean()) * 1e3, 3),
        "roofline": {"bound": "hbm", "achieved": round(dec_gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
                     "traffic": trf_dec, "kernel": "decode_kernel",
                     "algorithmic_bytes_per_launch": dbytes},
        "roofline_encode": {"bound": "hbm", "achieved": round(enc_gbs, 2), "peak": HBM_PEAK_GBS,
                            "unit": "GB/s", "frac": round(enc_gbs / HBM_PEAK_GBS, 4),
                            "traffic": trf_enc, "kernel": "encode_kernel",
                            "algorithmic_bytes_per_launch": ebytes,
                            "mfma_tflops": round(enc_tflops, 2),
                            "mfma_frac_of_bf16_peak": round(enc_tflops / BF16_MFMA_PEAK_TFLOPS, 4)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle (cpu_baseline)")
        line["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

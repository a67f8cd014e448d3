"""Helpers for the GPU parity tests: host <-> device marshalling and metrics."""

import sys

import numpy as np

SENTINEL = 0x5A5A5A5A


def say(*args):
    """Names the case about to run on the GPU (flushed, so it survives a crash)."""
    print("[gpu]", *args, flush=True, file=sys.stderr)


def dev_u16(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def dev_f32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def dev_u32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint32).view(np.int32)).cuda()


def host_u32(t):
    return t.cpu().numpy().view(np.uint32)


def gpu_encode(qjl, keys_u16, m, seed, cap=None, pos=0, signs=None, norms=None):
    """keys_u16: [B][H][n][d].  Returns device (signs int32, norms fp32) caches."""
    import torch
    B, H, n, d = keys_u16.shape
    cap = n + pos if cap is None else cap
    if signs is None:
        signs = torch.full((B, H, cap, m // 32), SENTINEL, dtype=torch.int32, device="cuda")
    if norms is None:
        norms = torch.full((B, H, cap), float("nan"), dtype=torch.float32, device="cuda")
    qjl.encode_keys(dev_u16(keys_u16), signs, norms, pos, seed, m)
    torch.cuda.synchronize()
    return signs, norms


def row_rel_l2(got, ref):
    """max over rows of ||got - ref|| / ||ref|| (rows = all but the last axis)."""
    g = np.asarray(got, dtype=np.float64).reshape(-1, got.shape[-1])
    r = np.asarray(ref, dtype=np.float64).reshape(-1, ref.shape[-1])
    num = np.linalg.norm(g - r, axis=1)
    den = np.maximum(np.linalg.norm(r, axis=1), 1e-300)
    return float((num / den).max())


def oracle_encode(keys_flat, S, chunk=16384):
    """oracle.encode over [R][d] keys, in chunks spread over host threads.

    The oracle itself is unchanged: each chunk is one oracle.encode call, and
    the chunks are joined in order.  numpy releases the interpreter lock in
    its array loops, so threads run the chunks in parallel (one BLAS thread
    each, so the threads do not oversubscribe the cores).
    """
    import os
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    from threadpoolctl import threadpool_limits

    keys_flat = np.ascontiguousarray(keys_flat)
    R = keys_flat.shape[0]
    if R <= chunk:
        return oracle.encode(keys_flat, S)
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    starts = list(range(0, R, chunk))
    with threadpool_limits(1), ThreadPoolExecutor(workers) as ex:
        parts = list(ex.map(lambda c: oracle.encode(keys_flat[c:c + chunk], S), starts))
    return (np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts]))


_WL_CACHE = {}


def cached_workload(name):
    """The named workload, drawn once per test session (several GPU tests
    share the large ones), with the oracle's encode of its keys."""
    import oracle
    from jl_rotated_bit_amd import workloads as wl

    if name not in _WL_CACHE:
        _WL_CACHE.clear()
        w = wl.WORKLOADS[name]()
        d = w.keys.shape[-1]
        words, norms = oracle_encode(w.keys.reshape(-1, d), oracle.sketch(w.seed, d, w.m))
        B, H, n = w.keys.shape[:3]
        _WL_CACHE[name] = (w, words.reshape(B, H, n, w.m // 32), norms.reshape(B, H, n))
    return _WL_CACHE[name]

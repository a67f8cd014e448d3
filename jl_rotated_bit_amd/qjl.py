"""Python binding of libqjl.so (ctypes).  Argument marshalling only.

The functions below take torch tensors for device memory and the current
torch stream, and call the C ABI declared in include/qjl.h.  All computation
happens in the HIP kernels; there is no fallback: if the library is missing
or a call fails, an exception is raised.

Names and semantics follow the C entry points:

* ``sketch_host(seed, d, m)``                 -> qjl_sketch_host
* ``encode_keys(keys, signs, norms, pos, seed, m)``        -> qjl_encode_keys
* ``decode_attention(q, signs, norms, values, N, seed, m, scale)`` -> qjl_decode_attention
* ``decode_step(q, new_keys, new_values, signs, norms, values, pos, seed, m)`` -> qjl_decode_step
* ``decode_attention_noalloc(q, signs, norms, values, N, seed, m, out)``  -> qjl_decode_attention_noalloc
* ``baseline_decode_attention_bf16(q, keys, values, N)`` -> qjl_baseline_decode_attention_bf16
* ``tq_encode_keys`` / ``tq_scores`` / ``pq_encode_keys`` -> qjl_tq_encode_keys / qjl_tq_scores /
  qjl_pq_encode_keys; ``rotation_host`` / ``tq_codebook_host`` / ``pq_codebook_host``
* ``decode_workspace_bytes`` / ``decode_num_splits`` / ``release_cache``
* ``testing_set_encode_small_max`` -> qjl_testing_set_encode_small_max (a
  per-thread test hook, not part of the public header)
"""

from __future__ import annotations

import ctypes
import os
import threading

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libqjl.so")
ABI_VERSION = 3

STATUS = {0: "QJL_OK", 1: "QJL_EINVAL", 2: "QJL_EUNSUPPORTED", 3: "QJL_EWORKSPACE",
          4: "QJL_EHIP", 5: "QJL_ENOMEM"}

_lib = None
_lock = threading.Lock()
_workspaces: dict = {}


class QJLError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


def load(path: str | None = None) -> ctypes.CDLL:
    """Loads libqjl.so (built by jl_rotated_bit_amd.build); raises if absent."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise RuntimeError(f"{p} not found: build it with `python -m jl_rotated_bit_amd.build`")
        lib = ctypes.CDLL(p)
        c_int, c_u64, c_vp, c_sz = ctypes.c_int32, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_size_t
        lib.qjl_abi_version.restype = c_int
        lib.qjl_abi_version.argtypes = []
        lib.qjl_last_error.restype = ctypes.c_char_p
        lib.qjl_last_error.argtypes = []
        lib.qjl_sketch_host.restype = c_int
        lib.qjl_sketch_host.argtypes = [c_u64, c_int, c_int, c_vp]
        lib.qjl_rotation_host.restype = c_int
        lib.qjl_rotation_host.argtypes = [c_u64, c_int, c_vp]
        lib.qjl_tq_codebook_host.restype = c_int
        lib.qjl_tq_codebook_host.argtypes = [c_int, c_int, c_vp]
        lib.qjl_pq_codebook_host.restype = c_int
        lib.qjl_pq_codebook_host.argtypes = [c_int, c_int, c_vp, c_vp]
        lib.qjl_encode_keys.restype = c_int
        lib.qjl_encode_keys.argtypes = [c_vp, c_int, c_int, c_int, c_int, c_int, c_u64, c_vp, c_vp,
                                        c_int, c_int, c_vp]
        lib.qjl_decode_num_splits.restype = c_int
        lib.qjl_decode_num_splits.argtypes = [c_int] * 6
        lib.qjl_decode_workspace_bytes.restype = c_sz
        lib.qjl_decode_workspace_bytes.argtypes = [c_int] * 6
        lib.qjl_decode_attention.restype = c_int
        lib.qjl_decode_attention.argtypes = [c_vp, c_vp, c_vp, c_vp, c_int, c_int, c_int, c_int,
                                             c_int, c_int, c_int, c_u64, ctypes.c_float, c_vp,
                                             c_vp, c_sz, c_vp]
        lib.qjl_decode_attention_noalloc.restype = c_int
        lib.qjl_decode_attention_noalloc.argtypes = [c_vp, c_vp, c_vp, c_vp, c_int, c_int, c_int,
                                                     c_int, c_int, c_int, c_int, c_u64,
                                                     ctypes.c_float, c_vp, c_vp]
        lib.qjl_decode_step.restype = c_int
        lib.qjl_decode_step.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_int, c_int, c_int,
                                        c_int, c_int, c_int, c_int, c_u64, ctypes.c_float, c_vp,
                                        c_vp, c_sz, c_vp]
        lib.qjl_baseline_decode_attention_bf16.restype = c_int
        lib.qjl_baseline_decode_attention_bf16.argtypes = [c_vp, c_vp, c_vp, c_int, c_int, c_int, c_int,
                                                           c_int, c_int, ctypes.c_float, c_vp, c_vp,
                                                           c_sz, c_vp]
        lib.qjl_tq_encode_keys.restype = c_int
        lib.qjl_tq_encode_keys.argtypes = [c_vp, c_int, c_int, c_int, c_int, c_int, c_u64, c_vp, c_vp,
                                           c_vp, c_vp, c_int, c_int, c_vp]
        lib.qjl_pq_encode_keys.restype = c_int
        lib.qjl_pq_encode_keys.argtypes = [c_vp, c_int, c_int, c_int, c_int, c_u64, c_vp, c_vp, c_int,
                                           c_int, c_vp]
        lib.qjl_tq_scores.restype = c_int
        lib.qjl_tq_scores.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_int, c_int, c_int, c_int, c_int,
                                      c_int, c_int, c_u64, c_vp, c_vp, c_sz, c_vp]
        lib.qjl_tq_scores_workspace_bytes.restype = c_sz
        lib.qjl_tq_scores_workspace_bytes.argtypes = [c_int, c_int, c_int]
        lib.qjl_testing_set_rotq_margin.restype = c_int
        lib.qjl_testing_set_rotq_margin.argtypes = [c_int]
        lib.qjl_release_cache.restype = c_int
        lib.qjl_release_cache.argtypes = []
        lib.qjl_testing_set_encode_small_max.restype = c_int
        lib.qjl_testing_set_encode_small_max.argtypes = [c_int]
        v = lib.qjl_abi_version()
        if v != ABI_VERSION:
            raise RuntimeError(f"libqjl ABI version {v}, binding expects {ABI_VERSION}")
        _lib = lib
        return lib


def _check(status: int):
    if status != 0:
        raise QJLError(status, load().qjl_last_error().decode(errors="replace"))


def last_error() -> str:
    return load().qjl_last_error().decode(errors="replace")


def sketch_host(seed: int, d: int, m: int) -> np.ndarray:
    """bf16 bit patterns of S, [d][m] uint16 (host only)."""
    out = np.empty((d, m), dtype=np.uint16)
    _check(load().qjl_sketch_host(seed & (2 ** 64 - 1), d, m, out.ctypes.data))
    return out


def rotation_host(seed: int, d: int) -> np.ndarray:
    """The seeded rotation Pi, fp32 [d][d] (host only)."""
    out = np.empty((d, d), dtype=np.float32)
    _check(load().qjl_rotation_host(seed & (2 ** 64 - 1), d, out.ctypes.data))
    return out


def tq_codebook_host(d: int, k: int) -> np.ndarray:
    """TurboQuant's 2^k Lloyd-Max centroids for dimension d (host only)."""
    out = np.empty(2 ** k, dtype=np.float32)
    _check(load().qjl_tq_codebook_host(d, k, out.ctypes.data))
    return out


def pq_codebook_host(level: int, bits: int):
    """PolarQuant's (centroids, thresholds) of one level (host only)."""
    cents = np.empty(2 ** bits, dtype=np.float32)
    nt = 2 ** bits // 4 - 1 if level == 1 else 2 ** bits - 1
    thr = np.empty(max(1, nt), dtype=np.float32)
    _check(load().qjl_pq_codebook_host(level, bits, cents.ctypes.data, thr.ctypes.data))
    return cents, thr[:nt]


def _resolve_stream(stream):
    import torch
    return torch.cuda.current_stream() if stream is None else stream


def _stream_handle(stream):
    return _resolve_stream(stream).cuda_stream


def _ptr(t):
    return t.data_ptr() if t is not None else None


def encode_keys(keys, signs, norms, pos: int, seed: int, m: int, stream=None):
    """Encodes keys [B][H_kv][n][d] (bf16 or int16 bits, CUDA) into the caches.

    signs: int32 [B][H_kv][cap][m/32] (uint32 bit patterns); norms: fp32
    [B][H_kv][cap].  Rows [pos, pos + n) are written.
    """
    B, H, n, d = keys.shape
    cap = signs.shape[2]
    if not keys.is_contiguous() or not signs.is_contiguous() or not norms.is_contiguous():
        raise ValueError("keys, signs and norms must be contiguous")
    if tuple(signs.shape) != (B, H, cap, m // 32) or tuple(norms.shape) != (B, H, cap):
        raise ValueError("signs must be [B][H_kv][cap][m/32] and norms [B][H_kv][cap]")
    if keys.element_size() != 2 or signs.element_size() != 4 or norms.element_size() != 4:
        raise ValueError("keys must be 16-bit (bf16 bits), signs 32-bit, norms fp32")
    _check(load().qjl_encode_keys(_ptr(keys), B, H, n, d, m, seed & (2 ** 64 - 1), _ptr(signs),
                                  _ptr(norms), cap, pos, _stream_handle(stream)))


def decode_num_splits(B, H_q, H_kv, N, d, m) -> int:
    return load().qjl_decode_num_splits(B, H_q, H_kv, N, d, m)


def decode_workspace_bytes(B, H_q, H_kv, N, d, m) -> int:
    return load().qjl_decode_workspace_bytes(B, H_q, H_kv, N, d, m)


def workspace_for(nbytes: int, device, stream=None, tag: str = "decode"):
    """A zero-filled workspace of at least nbytes, cached per (device, stream).

    It is allocated and zero-filled on ``stream`` (default: the current
    stream), so it is ready for the kernels queued there, and the caching
    allocator keeps its memory for that stream.  Calls on one stream share
    it (each call returns its counters to zero); calls on other streams get
    their own.  ``tag`` keeps workspaces of different entry points apart.
    """
    import torch
    s = _resolve_stream(stream)
    key = (str(device), s.cuda_stream, tag)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        with torch.cuda.stream(s):
            ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def decode_attention(q, signs, norms, values, N: int, seed: int, m: int, scale: float | None = None,
                     out=None, workspace=None, stream=None):
    """One QJL decode step; returns out fp32 [B][H_q][d].

    Runs on ``stream`` (default: the current stream).  The inputs must be
    ready on that stream (the caller orders other streams' writes before
    it); ``out`` and the cached workspace, when this function makes them,
    are allocated on that stream.
    """
    import torch
    B, H_q, d = q.shape
    _, H_kv, cap, _ = values.shape
    if q.dtype != torch.float32 or not q.is_contiguous():
        raise ValueError("q must be contiguous fp32 [B][H_q][d]")
    if values.element_size() != 2 or not values.is_contiguous():
        raise ValueError("values must be contiguous 16-bit (bf16 bits) [B][H_kv][cap][d]")
    if tuple(signs.shape) != (B, H_kv, cap, m // 32) or tuple(norms.shape) != (B, H_kv, cap):
        raise ValueError("signs/norms shapes do not match values")
    s = _resolve_stream(stream)
    if out is None:
        with torch.cuda.stream(s):
            out = torch.empty((B, H_q, d), dtype=torch.float32, device=q.device)
    need = decode_workspace_bytes(B, H_q, H_kv, N, d, m)
    if workspace is None:
        workspace = workspace_for(need, q.device, s)
    _check(load().qjl_decode_attention(
        _ptr(q), _ptr(signs), _ptr(norms), _ptr(values), B, H_q, H_kv, N, cap, d, m,
        seed & (2 ** 64 - 1), 0.0 if scale is None else float(scale), _ptr(out),
        _ptr(workspace), workspace.numel() * workspace.element_size(), s.cuda_stream))
    return out


def decode_step(q, new_keys, new_values, signs, norms, values, pos: int, seed: int, m: int,
                scale: float | None = None, out=None, workspace=None, stream=None):
    """qjl_decode_step: appends token ``pos`` (new_keys / new_values, bf16
    [B][H_kv][d]) to the caches (sign bits + norm, value row) and decodes
    over tokens [0, pos] in one launch; returns out fp32 [B][H_q][d]."""
    import torch
    B, H_q, d = q.shape
    _, H_kv, cap, _ = values.shape
    if q.dtype != torch.float32 or not q.is_contiguous():
        raise ValueError("q must be contiguous fp32 [B][H_q][d]")
    for name, t in (("new_keys", new_keys), ("new_values", new_values)):
        if tuple(t.shape) != (B, H_kv, d) or t.element_size() != 2 or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous 16-bit (bf16 bits) [B][H_kv][d]")
    if values.element_size() != 2 or not values.is_contiguous():
        raise ValueError("values must be contiguous 16-bit (bf16 bits) [B][H_kv][cap][d]")
    if tuple(signs.shape) != (B, H_kv, cap, m // 32) or tuple(norms.shape) != (B, H_kv, cap):
        raise ValueError("signs/norms shapes do not match values")
    if not signs.is_contiguous() or not norms.is_contiguous():
        raise ValueError("signs and norms must be contiguous")
    s = _resolve_stream(stream)
    if out is None:
        with torch.cuda.stream(s):
            out = torch.empty((B, H_q, d), dtype=torch.float32, device=q.device)
    need = decode_workspace_bytes(B, H_q, H_kv, pos + 1, d, m)
    if workspace is None:
        workspace = workspace_for(need, q.device, s)
    _check(load().qjl_decode_step(
        _ptr(q), _ptr(new_keys), _ptr(new_values), _ptr(signs), _ptr(norms), _ptr(values),
        B, H_q, H_kv, pos, cap, d, m, seed & (2 ** 64 - 1), 0.0 if scale is None else float(scale),
        _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(), s.cuda_stream))
    return out


def baseline_decode_attention_bf16(q, keys, values, N: int, scale: float | None = None, out=None,
                                   workspace=None, stream=None):
    """qjl_baseline_decode_attention_bf16: exact softmax attention over bf16
    keys and values (the uncompressed baseline); returns out fp32 [B][H_q][d]."""
    import torch
    B, H_q, d = q.shape
    _, H_kv, cap, _ = values.shape
    if q.dtype != torch.float32 or not q.is_contiguous():
        raise ValueError("q must be contiguous fp32 [B][H_q][d]")
    for name, t in (("keys", keys), ("values", values)):
        if tuple(t.shape) != (B, H_kv, cap, d) or t.element_size() != 2 or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous 16-bit (bf16 bits) [B][H_kv][cap][d]")
    s = _resolve_stream(stream)
    if out is None:
        with torch.cuda.stream(s):
            out = torch.empty((B, H_q, d), dtype=torch.float32, device=q.device)
    need = decode_workspace_bytes(B, H_q, H_kv, N, d, 256)
    if workspace is None:
        workspace = workspace_for(need, q.device, s)
    _check(load().qjl_baseline_decode_attention_bf16(
        _ptr(q), _ptr(keys), _ptr(values), B, H_q, H_kv, N, cap, d,
        0.0 if scale is None else float(scale), _ptr(out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), s.cuda_stream))
    return out


def tq_encode_keys(keys, codes, bits, norms, gammas, pos: int, seed: int, k: int, stream=None):
    """qjl_tq_encode_keys: keys [B][H_kv][n][d] bf16 bits -> rows [pos, pos + n)
    of codes int32 [B][H_kv][cap][d k/32], bits int32 [B][H_kv][cap][d/32],
    norms and gammas fp32 [B][H_kv][cap]."""
    B, H, n, d = keys.shape
    cap = norms.shape[2]
    for t in (keys, codes, bits, norms, gammas):
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    if tuple(codes.shape) != (B, H, cap, d * k // 32) or tuple(bits.shape) != (B, H, cap, d // 32) \
            or tuple(gammas.shape) != (B, H, cap):
        raise ValueError("cache shapes do not match")
    _check(load().qjl_tq_encode_keys(_ptr(keys), B, H, n, d, k, seed & (2 ** 64 - 1), _ptr(codes),
                                     _ptr(bits), _ptr(norms), _ptr(gammas), cap, pos,
                                     _stream_handle(stream)))


def tq_scores_workspace_bytes(B: int, H_q: int, d: int) -> int:
    """qjl_tq_scores_workspace_bytes."""
    return load().qjl_tq_scores_workspace_bytes(B, H_q, d)


def tq_scores(q, codes, bits, norms, gammas, N: int, seed: int, k: int, out=None, workspace=None,
              stream=None):
    """qjl_tq_scores: estimated <q, k_t> -> fp32 [B][H_q][N].

    The workspace (prepared queries, overwritten by every call) is cached per
    (device, stream) apart from the decode workspace, whose counters must stay
    zero between calls.
    """
    import torch
    B, H_q, d = q.shape
    _, H_kv, cap = norms.shape
    if q.dtype != torch.float32 or not q.is_contiguous():
        raise ValueError("q must be contiguous fp32 [B][H_q][d]")
    s = _resolve_stream(stream)
    if out is None:
        with torch.cuda.stream(s):
            out = torch.empty((B, H_q, N), dtype=torch.float32, device=q.device)
    need = tq_scores_workspace_bytes(B, H_q, d)
    if workspace is None:
        workspace = workspace_for(need, q.device, s, tag="tq_scores")
    _check(load().qjl_tq_scores(_ptr(q), _ptr(codes), _ptr(bits), _ptr(norms), _ptr(gammas), B, H_q,
                                H_kv, N, cap, d, k, seed & (2 ** 64 - 1), _ptr(out), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), s.cuda_stream))
    return out


def pq_encode_keys(keys, codes, radii, pos: int, seed: int, stream=None):
    """qjl_pq_encode_keys: keys [B][H_kv][n][d] -> rows [pos, pos + n) of codes
    int32 [B][H_kv][cap][12] and radii fp32 [B][H_kv][cap]."""
    B, H, n, d = keys.shape
    cap = radii.shape[2]
    if tuple(codes.shape) != (B, H, cap, 12):
        raise ValueError("codes must be [B][H_kv][cap][12]")
    _check(load().qjl_pq_encode_keys(_ptr(keys), B, H, n, d, seed & (2 ** 64 - 1), _ptr(codes),
                                     _ptr(radii), cap, pos, _stream_handle(stream)))


def testing_set_rotq_margin(log2_factor: int) -> int:
    """Test hook (csrc/qjl_testing.h): widen the rotate-then-quantize
    certificates of the calling thread by 2^log2_factor; returns the previous value."""
    return load().qjl_testing_set_rotq_margin(log2_factor)


def decode_attention_noalloc(q, signs, norms, values, N: int, seed: int, m: int, out,
                             scale: float | None = None, stream=None):
    """qjl_decode_attention_noalloc: one QJL decode step into ``out`` (fp32
    [B][H_q][d], caller-provided) using the library's static per-GPU scratch;
    nothing is allocated, here or in the library.  Calls that may overlap on
    one GPU race (they share the scratch)."""
    import torch
    B, H_q, d = q.shape
    _, H_kv, cap, _ = values.shape
    if q.dtype != torch.float32 or not q.is_contiguous():
        raise ValueError("q must be contiguous fp32 [B][H_q][d]")
    if values.element_size() != 2 or not values.is_contiguous():
        raise ValueError("values must be contiguous 16-bit (bf16 bits) [B][H_kv][cap][d]")
    if tuple(signs.shape) != (B, H_kv, cap, m // 32) or tuple(norms.shape) != (B, H_kv, cap):
        raise ValueError("signs/norms shapes do not match values")
    if out is None or tuple(out.shape) != (B, H_q, d) or out.dtype != torch.float32 \
            or not out.is_contiguous():
        raise ValueError("out must be a contiguous fp32 [B][H_q][d] tensor")
    _check(load().qjl_decode_attention_noalloc(
        _ptr(q), _ptr(signs), _ptr(norms), _ptr(values), B, H_q, H_kv, N, cap, d, m,
        seed & (2 ** 64 - 1), 0.0 if scale is None else float(scale), _ptr(out),
        _stream_handle(stream)))
    return out


NOALLOC_SCRATCH_BYTES = 4096 + (4 << 20)   # QJL_NOALLOC_SCRATCH_BYTES in include/qjl.h


def testing_set_encode_small_max(keys: int) -> int:
    """Test hook (csrc/qjl_testing.h): the largest encode call, in keys, that
    the calling thread sends to the small-set kernel; returns the thread's
    previous limit (a negative ``keys`` only queries it)."""
    return load().qjl_testing_set_encode_small_max(keys)


def release_cache():
    """qjl_release_cache: frees the device tables of every seed; call it only
    while no other thread is inside the library."""
    _check(load().qjl_release_cache())

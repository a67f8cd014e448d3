"""Python binding of libqjl.so (ctypes).  Argument marshalling only.

The functions below take torch tensors for device memory and the current
torch stream, and call the C ABI declared in include/qjl.h.  All computation
happens in the HIP kernels; there is no fallback: if the library is missing
or a call fails, an exception is raised.

Names and semantics follow the C entry points:

* ``sketch_host(seed, d, m)``                 -> qjl_sketch_host
* ``encode_keys(keys, signs, norms, pos, seed, m)``        -> qjl_encode_keys
* ``decode_attention(q, signs, norms, values, N, seed, m, scale)`` -> qjl_decode_attention
* ``decode_workspace_bytes`` / ``decode_num_splits`` / ``release_cache`` /
  ``set_encode_small_max``
"""

from __future__ import annotations

import ctypes
import os
import threading

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libqjl.so")
ABI_VERSION = 1

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
        lib.qjl_release_cache.restype = c_int
        lib.qjl_release_cache.argtypes = []
        lib.qjl_set_encode_small_max.restype = c_int
        lib.qjl_set_encode_small_max.argtypes = [c_int]
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


def _stream_handle(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


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


def workspace_for(nbytes: int, device):
    """A zero-filled workspace of at least nbytes, cached per device.

    Calls on one stream may share it (each call returns its counters to zero);
    callers running decode on several streams at once pass their own.
    """
    import torch
    key = (str(device),)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def decode_attention(q, signs, norms, values, N: int, seed: int, m: int, scale: float | None = None,
                     out=None, workspace=None, stream=None):
    """One QJL decode step; returns out fp32 [B][H_q][d]."""
    import torch
    B, H_q, d = q.shape
    _, H_kv, cap, _ = values.shape
    if q.dtype != torch.float32 or not q.is_contiguous():
        raise ValueError("q must be contiguous fp32 [B][H_q][d]")
    if values.element_size() != 2 or not values.is_contiguous():
        raise ValueError("values must be contiguous 16-bit (bf16 bits) [B][H_kv][cap][d]")
    if tuple(signs.shape) != (B, H_kv, cap, m // 32) or tuple(norms.shape) != (B, H_kv, cap):
        raise ValueError("signs/norms shapes do not match values")
    if out is None:
        out = torch.empty((B, H_q, d), dtype=torch.float32, device=q.device)
    need = decode_workspace_bytes(B, H_q, H_kv, N, d, m)
    if workspace is None:
        workspace = workspace_for(need, q.device)
    _check(load().qjl_decode_attention(
        _ptr(q), _ptr(signs), _ptr(norms), _ptr(values), B, H_q, H_kv, N, cap, d, m,
        seed & (2 ** 64 - 1), 0.0 if scale is None else float(scale), _ptr(out),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream_handle(stream)))
    return out


def set_encode_small_max(keys: int) -> int:
    """Largest encode call (in keys) that runs the small-set kernel; returns
    the previous limit (a negative ``keys`` only queries it)."""
    return load().qjl_set_encode_small_max(keys)


def release_cache():
    _check(load().qjl_release_cache())

"""Thin Python binding of the C ABI in include/tq.h (argument marshalling only).

torch supplies device memory and the current HIP stream; every step of the
path runs in the library's HIP kernels.  If libtq.so has not been built the
binding raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libtq.so")

TQ_OK, TQ_ERR_INVALID_ARG, TQ_ERR_UNSUPPORTED, TQ_ERR_ALIGNMENT, TQ_ERR_WORKSPACE, TQ_ERR_HIP = range(6)
TQ_ROT_HAAR, TQ_ROT_HADAMARD = 0, 1
TQ_F32, TQ_F16 = 0, 1
TQ_KEYS, TQ_VALUES = 0, 1
TQ_LAW_GAUSSIAN, TQ_LAW_BETA = 0, 1
TQ_LAYER_BETA_CODEBOOK = 1
TQ_LAYER_DITHER = 2
TQ_LAYER_VALUE_QJL = 4

EXPORTS = ["tq_abi_version", "tq_status_string", "tq_last_error", "tq_layer_blob_bytes",
           "tq_cache_bytes", "tq_make_rotation", "tq_make_layer", "tq_host_tables", "tq_get_codebook",
           "tq_get_codebook_law",
           "tq_quantize_kv", "tq_decode_workspace_bytes", "tq_attn_decode", "tq_attn_decode_static",
           "tq_dequantize", "tq_dequantize_prod"]
DECODE_STATIC_SCRATCH_BYTES = 16 << 20


class tq_layer(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("rot", ctypes.c_int32), ("k_bits", ctypes.c_int32),
                ("k_qjl", ctypes.c_int32), ("v_bits", ctypes.c_int32),
                ("flags", ctypes.c_int32), ("seed", ctypes.c_uint64),
                ("blob", ctypes.c_void_p), ("blob_bytes", ctypes.c_size_t)]


class tq_cache(ctypes.Structure):
    _fields_ = [("idx", ctypes.c_void_p), ("sign", ctypes.c_void_p), ("norm", ctypes.c_void_p),
                ("rnorm", ctypes.c_void_p), ("seqs", ctypes.c_int64), ("cap", ctypes.c_int64)]


class TQError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"tq status {status}: {message}")
        self.status = status


_lib = None


def load(path: Optional[str] = None):
    """Load libtq.so (built in-tree by build.py); raise if it is missing."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"{p} is not built; run python -m compressed_attention_turboquant_amd.build")
    lib = ctypes.CDLL(p)
    i32, i64, u64, sz, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_size_t, ctypes.c_void_p
    L, C = ctypes.POINTER(tq_layer), ctypes.POINTER(tq_cache)
    sig = {
        "tq_abi_version": (i32, []),
        "tq_status_string": (ctypes.c_char_p, [i32]),
        "tq_last_error": (ctypes.c_char_p, []),
        "tq_layer_blob_bytes": (sz, [i32]),
        "tq_cache_bytes": (i32, [L, i32, i64, i64, ctypes.POINTER(sz)]),
        "tq_make_rotation": (i32, [L, i32, i32, u64, i32, i32, i32, vp, sz, vp]),
        "tq_make_layer": (i32, [L, i32, i32, u64, i32, i32, i32, i32, vp, sz, vp]),
        "tq_host_tables": (i32, [i32, i32, u64, vp, vp]),
        "tq_get_codebook": (i32, [i32, i32, vp, vp]),
        "tq_get_codebook_law": (i32, [i32, i32, i32, vp, vp]),
        "tq_quantize_kv": (i32, [L, i32, vp, i32, i64, i64, i64, C, vp]),
        "tq_decode_workspace_bytes": (sz, [L, i32, i32, i32, i32, i64]),
        "tq_attn_decode": (i32, [L, vp, i32, i32, i32, i32, i32, i64, i32, C, C, vp, vp, vp, sz, vp]),
        "tq_attn_decode_static": (i32, [L, vp, i32, i32, i32, i32, i32, i64, i32, C, C, vp, vp, vp]),
        "tq_dequantize": (i32, [L, i32, C, i64, vp, i32, vp]),
        "tq_dequantize_prod": (i32, [L, i32, C, i64, vp, i32, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def check(status: int):
    if status != TQ_OK:
        raise TQError(status, load().tq_last_error().decode())


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float16:
        return TQ_F16
    if t.dtype == torch.float32:
        return TQ_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


# ---------------------------------------------------------------- host-only --

def get_codebook(d: int, bits: int, law: int = TQ_LAW_GAUSSIAN):
    import numpy as np
    c = np.zeros(1 << bits, np.float32)
    b = np.zeros((1 << bits) - 1, np.float32)
    check(load().tq_get_codebook_law(d, bits, law, c.ctypes.data, b.ctypes.data))
    return c, b


def host_tables(d: int, rot: int, seed: int):
    import numpy as np
    R = np.zeros((d, d), np.float64)
    S = np.zeros((d, d), np.float64)
    check(load().tq_host_tables(d, rot, seed, R.ctypes.data, S.ctypes.data))
    return R, S


# ------------------------------------------------------------------ device --

class Layer:
    """A layer's codec tables on the device (owns the blob tensor)."""

    def __init__(self, d, rot, seed, k_bits, k_qjl, v_bits, device="cuda", stream=None, flags=0):
        import torch
        lib = load()
        self.blob = torch.empty(lib.tq_layer_blob_bytes(d), dtype=torch.uint8, device=device)
        self.c = tq_layer()
        check(lib.tq_make_layer(ctypes.byref(self.c), d, rot, seed, k_bits, k_qjl, v_bits, flags,
                                self.blob.data_ptr(), self.blob.numel(), _stream(stream)))

    @property
    def d(self):
        return self.c.d


def make_rotation(d, rot, seed, k_bits, k_qjl, v_bits, device="cuda", stream=None, flags=0) -> Layer:
    """tq_make_layer (tq_make_rotation when flags == 0)."""
    return Layer(d, rot, seed, k_bits, k_qjl, v_bits, device, stream, flags)


class Cache:
    """A compressed K or V cache (owns its device arrays)."""

    def __init__(self, layer: Layer, which: int, seqs: int, cap: int, device="cuda", arrays=None):
        import torch
        sizes = (ctypes.c_size_t * 4)()
        check(load().tq_cache_bytes(ctypes.byref(layer.c), which, seqs, cap, sizes))
        if arrays is None:
            arrays = {
                "idx": torch.zeros(sizes[0], dtype=torch.uint8, device=device),
                "sign": torch.zeros(sizes[1], dtype=torch.uint8, device=device) if sizes[1] else None,
                "norm": torch.zeros(sizes[2] // 4, dtype=torch.float32, device=device),
                "rnorm": torch.zeros(sizes[3] // 4, dtype=torch.float32, device=device) if sizes[3] else None,
            }
        self.arrays = arrays
        self.which = which
        self.c = tq_cache(_ptr(arrays["idx"]), _ptr(arrays.get("sign")), _ptr(arrays["norm"]),
                          _ptr(arrays.get("rnorm")), seqs, cap)

    def __getitem__(self, k):
        return self.arrays[k]


def quantize_kv(layer: Layer, which: int, x, cache: Cache, t0: int = 0, stream=None):
    """x: [seqs, n, d] float16/float32 device tensor (contiguous)."""
    assert x.is_contiguous() and x.dim() == 3 and x.shape[2] == layer.d
    check(load().tq_quantize_kv(ctypes.byref(layer.c), which, x.data_ptr(), _dtype_code(x),
                                x.shape[0], x.shape[1], t0, ctypes.byref(cache.c), _stream(stream)))


def decode_workspace_bytes(layer: Layer, B, Hq, Hkv, Tq, N) -> int:
    return load().tq_decode_workspace_bytes(ctypes.byref(layer.c), B, Hq, Hkv, Tq, N)


def attn_decode(layer: Layer, q, K: Cache, V: Cache, N: int, Hkv: int, causal: int = 0,
                want_scores: bool = False, out=None, scores=None, workspace=None, stream=None):
    """q: [B, Hq, Tq, d] device tensor.  Returns (out float32, scores or None)."""
    import torch
    assert q.is_contiguous() and q.dim() == 4 and q.shape[3] == layer.d
    B, Hq, Tq, d = q.shape
    if out is None:
        out = torch.empty((B, Hq, Tq, d), dtype=torch.float32, device=q.device)
    if want_scores and scores is None:
        scores = torch.empty((B, Hq, Tq, N), dtype=torch.float32, device=q.device)
    if workspace is None:
        nbytes = decode_workspace_bytes(layer, B, Hq, Hkv, Tq, N)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    check(load().tq_attn_decode(ctypes.byref(layer.c), q.data_ptr(), _dtype_code(q), B, Hq, Hkv, Tq,
                                N, causal, ctypes.byref(K.c), ctypes.byref(V.c), out.data_ptr(),
                                _ptr(scores), workspace.data_ptr(), workspace.numel(), _stream(stream)))
    return out, scores


def attn_decode_static(layer: Layer, q, K: Cache, V: Cache, N: int, Hkv: int, causal: int = 0,
                       want_scores: bool = False, out=None, scores=None, stream=None):
    """tq_attn_decode_static: as attn_decode, with the library's fixed device
    scratch instead of a workspace (out and scores are allocated here when not
    given; the call itself allocates nothing)."""
    import torch
    assert q.is_contiguous() and q.dim() == 4 and q.shape[3] == layer.d
    B, Hq, Tq, d = q.shape
    if out is None:
        out = torch.empty((B, Hq, Tq, d), dtype=torch.float32, device=q.device)
    if want_scores and scores is None:
        scores = torch.empty((B, Hq, Tq, N), dtype=torch.float32, device=q.device)
    check(load().tq_attn_decode_static(ctypes.byref(layer.c), q.data_ptr(), _dtype_code(q), B, Hq, Hkv, Tq,
                                       N, causal, ctypes.byref(K.c), ctypes.byref(V.c), out.data_ptr(),
                                       _ptr(scores), _stream(stream)))
    return out, scores


def dequantize(layer: Layer, which: int, cache: Cache, n: int, out_dtype=None, stream=None, out=None,
               prod: bool = False):
    """tq_dequantize (tq_dequantize_prod with prod=True) into out ([seqs][n][d],
    float32 or float16; allocated when not given, of out_dtype, default float32)."""
    import torch
    if out is None:
        out = torch.empty((cache.c.seqs, n, layer.d), dtype=out_dtype or torch.float32, device=cache["idx"].device)
    elif tuple(out.shape) != (cache.c.seqs, n, layer.d) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [seqs][n][d] tensor")
    fn = load().tq_dequantize_prod if prod else load().tq_dequantize
    check(fn(ctypes.byref(layer.c), which, ctypes.byref(cache.c), n, out.data_ptr(), _dtype_code(out),
             _stream(stream)))
    return out

"""CPU tests of the HIP library: it loads, exports the declared C ABI, builds
the same layer tables as the oracle, and rejects bad arguments before touching
the GPU (validation runs on the host ahead of any HIP call)."""
import ctypes
import os
import re

import numpy as np
import pytest

from compressed_attention_turboquant_amd import binding as B
from oracle import codebook, transforms

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = []
    for fname in os.listdir(os.path.join(ROOT, "include")):
        if fname.endswith(".h"):
            with open(os.path.join(ROOT, "include", fname)) as f:
                text = f.read()
            names += re.findall(r"^[A-Za-z_][\w\s\*]*?\b(tq_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_library_loads_and_exports_every_declared_symbol(lib):
    declared = _declared_functions()
    assert len(declared) >= 12
    for name in declared:
        assert hasattr(lib, name), name
    assert set(B.EXPORTS) <= set(declared)
    assert lib.tq_abi_version() == 2


@pytest.mark.parametrize("law", ["gaussian", "beta"])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_codebooks_bit_equal_to_oracle(d, law):
    for bits in (1, 2, 3, 4):
        c, b = B.get_codebook(d, bits, B.TQ_LAW_BETA if law == "beta" else B.TQ_LAW_GAUSSIAN)
        oc, ob = codebook.codebook(bits, d, law)
        assert np.array_equal(c, oc) and np.array_equal(b, ob), (d, bits, law)


@pytest.mark.parametrize("law", ["gaussian", "beta"])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_codebooks_fit_the_quantizer_bin_table(d, law):
    """The Hadamard quantizer takes 3- and 4-bit codes from a table of 64 bins
    of width 1/8 on the codebook's N(0, 1) scale (b * sqrt(d)), covering
    [-4, 4): every boundary must lie inside that range and any two must be
    more than a bin apart, so that a bin holds at most one."""
    for bits in (3, 4):
        _, b = B.get_codebook(d, bits, B.TQ_LAW_BETA if law == "beta" else B.TQ_LAW_GAUSSIAN)
        z = b.astype(np.float64) * np.sqrt(d)
        assert np.abs(z).max() < 4.0 - 0.125, (d, bits, law)
        assert np.diff(z).min() > 0.125 * 1.5, (d, bits, law, np.diff(z).min())


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("rot", ["haar", "hadamard"])
def test_rotation_and_projection_match_oracle(d, rot):
    code = B.TQ_ROT_HAAR if rot == "haar" else B.TQ_ROT_HADAMARD
    R, S = B.host_tables(d, code, 12345)
    assert np.abs(R - transforms.rotation(d, rot, 12345)).max() < 1e-13
    assert np.abs(S - transforms.gaussian_projection(d, 12345)).max() < 1e-14
    assert np.abs(R @ R.T - np.eye(d)).max() < 1e-13


def _layer(d=128, kb=2, qjl=1, vb=2):
    L = B.tq_layer()
    L.d, L.rot, L.k_bits, L.k_qjl, L.v_bits = d, 0, kb, qjl, vb
    L.blob = 4096
    L.blob_bytes = B.load().tq_layer_blob_bytes(d)
    return L


def _cache(seqs=2, cap=16, qjl=True):
    return B.tq_cache(1 << 20, (2 << 20) if qjl else None, 3 << 20, (4 << 20) if qjl else None, seqs, cap)


def _err(lib):
    return lib.tq_last_error().decode()


def test_make_rotation_rejects_bad_arguments(lib):
    L = B.tq_layer()
    nb = lib.tq_layer_blob_bytes(128)
    assert lib.tq_layer_blob_bytes(96) == 0
    assert lib.tq_make_rotation(ctypes.byref(L), 96, 0, 0, 2, 1, 2, 4096, nb, None) == B.TQ_ERR_UNSUPPORTED
    assert lib.tq_make_rotation(ctypes.byref(L), 128, 5, 0, 2, 1, 2, 4096, nb, None) == B.TQ_ERR_INVALID_ARG
    assert lib.tq_make_rotation(ctypes.byref(L), 128, 0, 0, 5, 1, 2, 4096, nb, None) == B.TQ_ERR_INVALID_ARG
    assert lib.tq_make_rotation(ctypes.byref(L), 128, 0, 0, 2, 2, 2, 4096, nb, None) == B.TQ_ERR_INVALID_ARG
    assert lib.tq_make_rotation(ctypes.byref(L), 128, 0, 0, 2, 1, 2, None, nb, None) == B.TQ_ERR_INVALID_ARG
    assert lib.tq_make_rotation(ctypes.byref(L), 128, 0, 0, 2, 1, 2, 4100, nb, None) == B.TQ_ERR_ALIGNMENT
    assert lib.tq_make_rotation(ctypes.byref(L), 128, 0, 0, 2, 1, 2, 4096, nb - 1, None) == B.TQ_ERR_INVALID_ARG
    assert "blob_bytes" in _err(lib)
    assert lib.tq_make_rotation(None, 128, 0, 0, 2, 1, 2, 4096, nb, None) == B.TQ_ERR_INVALID_ARG
    assert L.d == 0  # nothing was written on failure


def test_layer_flags_and_codebook_law_are_checked(lib):
    L = B.tq_layer()
    nb = lib.tq_layer_blob_bytes(128)
    assert lib.tq_make_layer(ctypes.byref(L), 128, 0, 0, 2, 1, 2, 8, 4096, nb, None) == B.TQ_ERR_INVALID_ARG
    assert "flags" in _err(lib)
    c = (ctypes.c_float * 4)()
    b = (ctypes.c_float * 3)()
    assert lib.tq_get_codebook_law(128, 2, 2, c, b) == B.TQ_ERR_INVALID_ARG
    Lf = _layer()
    Lf.flags = 8
    K = _cache()
    assert lib.tq_quantize_kv(ctypes.byref(Lf), 0, 4096, 1, 2, 8, 0, ctypes.byref(K), None) == B.TQ_ERR_INVALID_ARG
    assert "flags" in _err(lib)


def test_dither_needs_hadamard_without_qjl(lib):
    """The dithered variant is defined on the randomized Hadamard rotation, for
    MSE-only keys; other layers asking for it are refused before any GPU call."""
    L = B.tq_layer()
    nb = lib.tq_layer_blob_bytes(128)
    D = B.TQ_LAYER_DITHER
    # Haar rotation
    assert lib.tq_make_layer(ctypes.byref(L), 128, B.TQ_ROT_HAAR, 0, 2, 0, 2, D, 4096, nb, None) == B.TQ_ERR_INVALID_ARG
    assert "Hadamard" in _err(lib)
    # keys with QJL
    assert lib.tq_make_layer(ctypes.byref(L), 128, B.TQ_ROT_HADAMARD, 0, 2, 1, 2, D, 4096, nb, None) == \
        B.TQ_ERR_INVALID_ARG
    assert L.d == 0
    for rot, qjl in ((0, 0), (1, 1)):
        Lf = _layer(qjl=qjl)
        Lf.rot, Lf.flags = rot, D
        K = _cache(qjl=bool(qjl))
        assert lib.tq_quantize_kv(ctypes.byref(Lf), 0, 4096, 1, 2, 8, 0, ctypes.byref(K), None) == \
            B.TQ_ERR_INVALID_ARG
        assert "DITHER" in _err(lib)


def test_dither_excludes_values_with_qjl(lib):
    L = B.tq_layer()
    nb = lib.tq_layer_blob_bytes(128)
    flags = B.TQ_LAYER_DITHER | B.TQ_LAYER_VALUE_QJL
    assert lib.tq_make_layer(ctypes.byref(L), 128, B.TQ_ROT_HADAMARD, 0, 2, 0, 2, flags, 4096, nb, None) == \
        B.TQ_ERR_INVALID_ARG
    assert L.d == 0


def test_values_with_qjl_carry_signs_and_residual_norms(lib):
    """TQ_LAYER_VALUE_QJL gives value rows the same sign and residual-norm
    arrays as keys with QJL; quantize, decode and dequantize_prod check them."""
    L = _layer(d=128, kb=3, qjl=0, vb=2)
    L.flags = B.TQ_LAYER_VALUE_QJL
    out = (ctypes.c_size_t * 4)()
    assert lib.tq_cache_bytes(ctypes.byref(L), B.TQ_VALUES, 4, 64, out) == B.TQ_OK
    assert list(out) == [4 * 64 * 32, 4 * 64 * 16, 4 * 64 * 4, 4 * 64 * 4]
    assert lib.tq_cache_bytes(ctypes.byref(L), B.TQ_KEYS, 4, 64, out) == B.TQ_OK
    assert list(out) == [4 * 64 * 48, 0, 4 * 64 * 4, 0]
    # value caches without sign or rnorm are refused
    assert lib.tq_quantize_kv(ctypes.byref(L), B.TQ_VALUES, 4096, 1, 2, 8, 0, ctypes.byref(_cache(qjl=False)),
                              None) == B.TQ_ERR_INVALID_ARG
    assert "rnorm" in _err(lib)
    call = lambda which, cache: lib.tq_dequantize_prod(ctypes.byref(L), which, ctypes.byref(cache), 8, 4096, 0,
                                                       None)
    assert call(B.TQ_VALUES, _cache(qjl=False)) == B.TQ_ERR_INVALID_ARG
    assert call(B.TQ_KEYS, _cache(qjl=False)) == B.TQ_ERR_INVALID_ARG      # these keys carry no QJL

    def decode(Hq, Hkv, Tq, V):
        ws = lib.tq_decode_workspace_bytes(ctypes.byref(L), 1, Hq, Hkv, Tq, 16)
        return lib.tq_attn_decode(ctypes.byref(L), 4096, 1, 1, Hq, Hkv, Tq, 16, 0,
                                  ctypes.byref(_cache(seqs=Hkv, qjl=False)), ctypes.byref(V), 8192, None,
                                  1 << 16, max(ws, 1), None)
    assert decode(4, 2, 1, _cache(seqs=2, qjl=False)) == B.TQ_ERR_INVALID_ARG
    # the split kernel keeps both value sums of every query row of a KV head
    # on chip: 128 rows of d = 128 are beyond it (64 are not)
    assert decode(128, 1, 1, _cache(seqs=1)) == B.TQ_ERR_UNSUPPORTED
    assert lib.tq_decode_workspace_bytes(ctypes.byref(L), 1, 64, 1, 1, 16) > 0


def test_cache_bytes(lib):
    L = _layer(d=128, kb=3, qjl=1, vb=2)
    out = (ctypes.c_size_t * 4)()
    assert lib.tq_cache_bytes(ctypes.byref(L), B.TQ_KEYS, 4, 64, out) == B.TQ_OK
    assert list(out) == [4 * 64 * 48, 4 * 64 * 16, 4 * 64 * 4, 4 * 64 * 4]
    assert lib.tq_cache_bytes(ctypes.byref(L), B.TQ_VALUES, 4, 64, out) == B.TQ_OK
    assert list(out) == [4 * 64 * 32, 0, 4 * 64 * 4, 0]
    assert lib.tq_cache_bytes(ctypes.byref(L), B.TQ_VALUES, 4, 60, out) == B.TQ_ERR_INVALID_ARG


def test_quantize_rejects_bad_arguments(lib):
    L = _layer()
    K = _cache()
    bad = lambda **kw: lib.tq_quantize_kv(ctypes.byref(kw.get("L", L)), kw.get("which", 0), kw.get("x", 4096),
                                          kw.get("dt", 1), kw.get("seqs", 2), kw.get("n", 8),
                                          kw.get("t0", 0), ctypes.byref(kw.get("K", K)), None)
    assert bad(which=2) == B.TQ_ERR_INVALID_ARG
    assert bad(dt=7) == B.TQ_ERR_INVALID_ARG
    assert bad(n=-1) == B.TQ_ERR_INVALID_ARG
    assert bad(t0=10) == B.TQ_ERR_INVALID_ARG                    # t0 + n > cap
    assert bad(seqs=3) == B.TQ_ERR_INVALID_ARG                   # more than the cache holds
    assert bad(x=0) == B.TQ_ERR_INVALID_ARG
    assert bad(x=4100) == B.TQ_ERR_ALIGNMENT
    assert bad(K=_cache(cap=12)) == B.TQ_ERR_INVALID_ARG
    assert bad(K=_cache(qjl=False)) == B.TQ_ERR_INVALID_ARG      # keys with QJL need sign/rnorm
    assert bad(K=B.tq_cache(1 << 20 | 4, 2 << 20, 3 << 20, 4 << 20, 2, 16)) == B.TQ_ERR_ALIGNMENT
    L2 = _layer(d=96)
    assert bad(L=L2) == B.TQ_ERR_UNSUPPORTED
    L3 = _layer()
    L3.blob_bytes = 10
    assert bad(L=L3) == B.TQ_ERR_INVALID_ARG


def test_decode_rejects_bad_arguments(lib):
    L = _layer()
    K, V = _cache(seqs=2), _cache(seqs=2, qjl=False)
    ws = lib.tq_decode_workspace_bytes(ctypes.byref(L), 1, 4, 2, 1, 16)
    assert ws > 0

    def call(**kw):
        a = dict(q=4096, qdt=1, B=1, Hq=4, Hkv=2, Tq=1, N=16, causal=0, K=K, V=V, out=8192,
                 scores=None, ws=1 << 16, wsb=ws)
        a.update(kw)
        return lib.tq_attn_decode(ctypes.byref(L), a["q"], a["qdt"], a["B"], a["Hq"], a["Hkv"], a["Tq"],
                                  a["N"], a["causal"], ctypes.byref(a["K"]), ctypes.byref(a["V"]),
                                  a["out"], a["scores"], a["ws"], a["wsb"], None)
    assert call(Hq=3) == B.TQ_ERR_INVALID_ARG
    assert call(N=0) == B.TQ_ERR_INVALID_ARG
    assert call(N=17) == B.TQ_ERR_INVALID_ARG                    # beyond capacity
    assert call(Tq=20, N=16, causal=1) == B.TQ_ERR_INVALID_ARG   # causal needs Tq <= N
    assert call(B=2) == B.TQ_ERR_INVALID_ARG                     # caches hold B*Hkv sequences
    assert call(qdt=3) == B.TQ_ERR_INVALID_ARG
    assert call(q=0) == B.TQ_ERR_INVALID_ARG
    assert call(out=8196) == B.TQ_ERR_ALIGNMENT
    assert call(ws=None) == B.TQ_ERR_WORKSPACE
    assert call(wsb=ws - 1) == B.TQ_ERR_WORKSPACE
    assert call(ws=(1 << 16) + 16) == B.TQ_ERR_ALIGNMENT
    assert call(V=_cache(seqs=2, cap=24, qjl=False)) == B.TQ_ERR_INVALID_ARG


def test_dequantize_rejects_bad_arguments(lib):
    L = _layer()
    K = _cache()
    call = lambda **kw: lib.tq_dequantize(ctypes.byref(L), kw.get("which", 0), ctypes.byref(kw.get("K", K)),
                                          kw.get("n", 8), kw.get("out", 4096), kw.get("dt", 0), None)
    assert call(n=17) == B.TQ_ERR_INVALID_ARG
    assert call(dt=2) == B.TQ_ERR_INVALID_ARG
    assert call(out=0) == B.TQ_ERR_INVALID_ARG
    assert call(out=4098) == B.TQ_ERR_ALIGNMENT
    assert call(which=3) == B.TQ_ERR_INVALID_ARG


def test_dequantize_prod_needs_keys_with_qjl(lib):
    """The two-stage reconstruction is defined for rows that carry QJL signs:
    values of a layer without TQ_LAYER_VALUE_QJL, and keys of a layer without
    QJL, are rejected before any GPU call."""
    K = _cache()
    call = lambda L, which, cache: lib.tq_dequantize_prod(ctypes.byref(L), which, ctypes.byref(cache), 8, 4096, 0, None)
    assert call(_layer(qjl=1), B.TQ_VALUES, _cache(qjl=False)) == B.TQ_ERR_INVALID_ARG
    assert call(_layer(qjl=0), B.TQ_KEYS, _cache(qjl=False)) == B.TQ_ERR_INVALID_ARG
    assert "k_qjl" in _err(lib)
    assert call(_layer(qjl=1), B.TQ_KEYS, _cache(qjl=False)) == B.TQ_ERR_INVALID_ARG
    assert call(_layer(qjl=1), B.TQ_KEYS, B.tq_cache(1 << 20, (2 << 20) + 4, 3 << 20, 4 << 20, 2, 16)) == \
        B.TQ_ERR_ALIGNMENT


def test_status_strings(lib):
    for s in range(6):
        assert lib.tq_status_string(s)
    assert lib.tq_status_string(B.TQ_ERR_WORKSPACE) == b"workspace too small"


def test_product_code_does_not_touch_the_oracle():
    """The library and its binding share no code with oracle/ and never import it."""
    pkg = os.path.join(ROOT, "compressed_attention_turboquant_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                with open(os.path.join(dirpath, f)) as fh:
                    text = fh.read()
                assert not re.search(r"^\s*(from|import)\s+oracle", text, flags=re.M), f
                assert "oracle/" not in text, f
    for f in os.listdir(os.path.join(ROOT, "oracle")):
        if f.endswith(".py"):
            with open(os.path.join(ROOT, "oracle", f)) as fh:
                assert "compressed_attention_turboquant_amd" not in fh.read(), f


def test_cache_size_limit_is_rejected_before_any_gpu_call(lib):
    """Each cache array of one sequence is addressed with 32-bit offsets, so
    cap * d * bits / 8 must stay below 2^31 - 2^20 bytes: at d = 256 with
    4-bit codes, cap = 2^24 - 2^13 is the largest accepted capacity."""
    L = _layer(d=256, kb=4, qjl=0, vb=4)
    out = (ctypes.c_size_t * 4)()
    ok_cap, bad_cap = (1 << 24) - (1 << 13), 1 << 24
    assert lib.tq_cache_bytes(ctypes.byref(L), B.TQ_KEYS, 1, ok_cap, out) == B.TQ_OK
    assert out[0] == ok_cap * 128
    assert lib.tq_cache_bytes(ctypes.byref(L), B.TQ_KEYS, 1, bad_cap, out) == B.TQ_ERR_UNSUPPORTED
    assert lib.tq_cache_bytes(ctypes.byref(L), B.TQ_VALUES, 1, bad_cap, out) == B.TQ_ERR_UNSUPPORTED
    big_k = B.tq_cache(1 << 20, None, 3 << 20, None, 1, bad_cap)
    big_v = B.tq_cache(5 << 20, None, 6 << 20, None, 1, bad_cap)
    ws = 1 << 16
    st = lib.tq_attn_decode(ctypes.byref(L), 4096, 1, 1, 4, 1, 1, 16, 0, ctypes.byref(big_k),
                            ctypes.byref(big_v), 8192, None, ws, 1 << 30, None)
    assert st == B.TQ_ERR_UNSUPPORTED and "2^31" in _err(lib)
    assert lib.tq_quantize_kv(ctypes.byref(L), B.TQ_KEYS, 4096, 1, 1, 8, 0, ctypes.byref(big_k),
                              None) == B.TQ_ERR_UNSUPPORTED
    assert lib.tq_dequantize(ctypes.byref(L), B.TQ_VALUES, ctypes.byref(big_v), 8, 4096, 0,
                             None) == B.TQ_ERR_UNSUPPORTED
    # d = 128, 3-bit keys: 48 bytes per token allow caps up to 44,717,568.
    L3 = _layer(d=128, kb=3, qjl=1, vb=3)
    limit = ((1 << 31) - (1 << 20)) // 48
    assert lib.tq_cache_bytes(ctypes.byref(L3), B.TQ_KEYS, 1, limit // 8 * 8, out) == B.TQ_OK
    assert lib.tq_cache_bytes(ctypes.byref(L3), B.TQ_KEYS, 1, limit // 8 * 8 + 8, out) == B.TQ_ERR_UNSUPPORTED


def test_static_scratch_decode_rejects_shapes_beyond_its_scratch(lib):
    """tq_attn_decode_static checks the shape's scratch need against its fixed
    16 MiB before any GPU call: 32768 query rows of d = 128 need 17.3 MB."""
    L = _layer(d=128, kb=2, qjl=1, vb=2)
    Bn, Hq, Hkv, N = 1024, 32, 8, 32
    need = lib.tq_decode_workspace_bytes(ctypes.byref(L), Bn, Hq, Hkv, 1, N)
    assert need > B.DECODE_STATIC_SCRATCH_BYTES
    K = _cache(seqs=Bn * Hkv, cap=32, qjl=True)
    V = _cache(seqs=Bn * Hkv, cap=32, qjl=False)
    st = lib.tq_attn_decode_static(ctypes.byref(L), 4096, 1, Bn, Hq, Hkv, 1, N, 0, ctypes.byref(K),
                                   ctypes.byref(V), 8192, None, None)
    assert st == B.TQ_ERR_WORKSPACE
    assert str(need) in _err(lib) and "tq_attn_decode with a workspace" in _err(lib)
    # argument errors come first, as for tq_attn_decode
    assert lib.tq_attn_decode_static(ctypes.byref(L), 4096, 1, Bn, 3, Hkv, 1, N, 0, ctypes.byref(K),
                                     ctypes.byref(V), 8192, None, None) == B.TQ_ERR_INVALID_ARG

"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Sizes here are the five layer configurations cut down (fewer batches and
tokens, ragged token counts that end inside a tile) so the oracle finishes in
seconds; tests/test_gpu_fullsize.py covers the full sizes on sampled outputs.
"""
import math

import numpy as np
import pytest
import torch

import workloads
from compressed_attention_turboquant_amd import binding as B
from oracle import attention, codec
from tests import harness as H

pytestmark = pytest.mark.gpu

REDUCED = {
    "C1": workloads.CONFIGS["C1"],
    "C2": workloads.CONFIGS["C2"].with_(N=1003),
    "C3": workloads.CONFIGS["C3"].with_(B=1, N=777),
    "C4": workloads.CONFIGS["C4"].with_(B=2, N=600),
    "C5": workloads.CONFIGS["C5"].with_(B=1, N=515),
}


def _kv(cfg, which, seed=0):
    x = workloads.kv_numpy(cfg, seed, which)
    return x.reshape(cfg.B * cfg.Hkv, cfg.N, cfg.d)


def _rows(S, cap, n):
    return np.array([s * cap + t for s in range(S) for t in range(n)], dtype=np.int64)


@pytest.mark.parametrize("name", list(REDUCED))
def test_quantize_keys_parity(name):
    cfg = REDUCED[name]
    H.log(f"[quantize K] {name} {cfg}")
    x = _kv(cfg, "K")
    S, n, d = x.shape
    layer, ol, cache, enc, cap = H.run_quantize_both(cfg, x, B.TQ_KEYS)
    rows = _rows(S, cap, n)
    gidx = H.gpu_codes_key(cache, S, cap, d, cfg.k_bits, rows)
    gnorm = cache["norm"].cpu().numpy()[rows]
    if cfg.k_qjl:
        gsign = H.gpu_signs(cache, S, cap, d, rows)
        _, st = H.check_keys(gidx, gnorm, enc, ol, f"{name} K", gsign, cache["rnorm"].cpu().numpy()[rows])
    else:
        _, st = H.check_keys(gidx, gnorm, enc, ol, f"{name} K")
    assert st["code_rows"] < 0.01 * len(rows)
    # packed bytes are identical for every row without a band difference
    flipped = (gidx != enc["idx"]).any(axis=1)
    rb = d * cfg.k_bits // 8
    gbytes = cache["idx"].cpu().numpy().reshape(S * cap, rb)[rows]
    obytes = codec.pack_key_codes(enc["idx"], cfg.k_bits)
    assert np.array_equal(gbytes[~flipped], obytes[~flipped])
    H.log(f"  rows={len(rows)} band-flipped code rows={st['code_rows']} sign rows={st['sign_rows']}")


@pytest.mark.parametrize("name", list(REDUCED))
def test_quantize_values_parity(name):
    cfg = REDUCED[name]
    H.log(f"[quantize V] {name}")
    x = _kv(cfg, "V")
    S, n, d = x.shape
    layer, ol, cache, enc, cap = H.run_quantize_both(cfg, x, B.TQ_VALUES)
    rows = _rows(S, cap, n)
    gidx = H.gpu_codes_value(cache, S, cap, d, cfg.v_bits)[rows]
    _, flips = H.check_values(gidx, cache["norm"].cpu().numpy()[rows], enc, ol, f"{name} V")
    assert flips < 0.01 * len(rows)


def _decode_both(cfg, packed, q_np, N, want_scores=True):
    S = cfg.B * cfg.Hkv
    cap = (N + 7) // 8 * 8
    layer = H.gpu_layer(cfg)
    ol = H.OracleLayer(cfg)
    K, V = H.upload_packed(layer, cfg, packed, S, cap)
    q = torch.from_numpy(q_np).cuda()
    out, scores = B.attn_decode(layer, q, K, V, N, cfg.Hkv, cfg.causal, want_scores=want_scores)
    torch.cuda.synchronize()
    cache = attention.unpack_cache(packed, cfg.B, cfg.Hkv, cap, cfg.d, cfg.k_bits, cfg.v_bits, cfg.k_qjl,
                                   cfg.v_qjl)
    ref_out, ref_scores = attention.decode(q_np, ol.R, ol.S, ol.ck, ol.cv, cache, N, cfg.causal)
    return out.cpu().numpy(), (scores.cpu().numpy() if scores is not None else None), \
        ref_out, ref_scores, cache, ol


@pytest.mark.parametrize("name", list(REDUCED))
def test_decode_on_random_cache(name):
    """Decode alone: any byte pattern is a valid packed cache, so both sides read
    the same seeded random cache and must agree on every score and output."""
    cfg = REDUCED[name]
    N = cfg.N
    cap = (N + 7) // 8 * 8
    H.log(f"[decode random cache] {name} N={N}")
    packed = workloads.random_packed_numpy(cfg, cfg.B * cfg.Hkv, cap, seed=1)
    q = workloads.q_numpy(cfg, seed=1)
    out, scores, ref_out, ref_scores, cache, ol = _decode_both(cfg, packed, q, N)
    scale = H.score_scale(q, ol.R, ol.S, ol.ck, cache, N, cfg.G, cfg.k_qjl)
    rel = H.compare_scores(scores, ref_scores, scale, name)
    err = H.compare_out(out, ref_out, name)
    H.log(f"  score rel err {rel:.2e}  out abs err {err:.2e}")


# Query rows per KV head (G * Tq) around the decode kernel's row groups of 4
# and 8: one partial group, exactly one group, a full group plus a partial one,
# several groups; causal chunks take Tq > 1.
ROW_GROUP_CASES = {
    "5 rows (G=5)": workloads.CONFIGS["C2"].with_(Hq=5, Hkv=1, N=300),
    "8 rows (G=8)": workloads.CONFIGS["C2"].with_(Hq=16, Hkv=2, N=300),
    "12 rows (G=4, Tq=3, causal)": workloads.CONFIGS["C4"].with_(B=1, Hq=8, Hkv=2, Tq=3, N=300),
    "20 rows (G=4, Tq=5, causal, d=256)": workloads.CONFIGS["C5"].with_(B=1, Hq=8, Hkv=2, Tq=5, N=300,
                                                                      causal=1, k_qjl=1, k_bits=2,
                                                                      v_bits=3),
    # 2048 query rows in all: the combine merges 4 rows per block.
    "16 rows x 128 heads (G=4, Tq=4, causal)": workloads.CONFIGS["C3"].with_(B=16, Tq=4, N=203, causal=1,
                                                                             dist="normal"),
    # 64 and more rows per KV head at d = 128 take the wide kernel (4 waves x 32
    # rows per workgroup): half a row group, two groups with a partial second
    # one and MSE-only keys, fp32 queries.
    "64 rows (G=8, Tq=8, causal): wide kernel, half a group": workloads.CONFIGS["C4"].with_(B=1, Tq=8, N=300),
    "200 rows (G=8, Tq=25, causal, K3 V4 MSE-only): wide kernel, 2 groups":
        workloads.CONFIGS["C4"].with_(B=1, Hq=8, Hkv=1, Tq=25, N=333, k_bits=3, v_bits=4, k_qjl=0),
    "128 rows fp32 (G=16, Tq=8): wide kernel": workloads.CONFIGS["C1"].with_(Hq=16, Hkv=1, Tq=8, N=300),
}


@pytest.mark.parametrize("name", list(ROW_GROUP_CASES))
def test_decode_row_groups(name):
    """Decode of heads whose query rows fill the kernel's row groups partly,
    exactly and over several groups: every score and output against the oracle."""
    cfg = ROW_GROUP_CASES[name]
    N = cfg.N
    cap = (N + 7) // 8 * 8
    H.log(f"[decode row groups] {name}")
    packed = workloads.random_packed_numpy(cfg, cfg.B * cfg.Hkv, cap, seed=7)
    q = workloads.q_numpy(cfg, seed=7)
    out, scores, ref_out, ref_scores, cache, ol = _decode_both(cfg, packed, q, N)
    scale = H.score_scale(q, ol.R, ol.S, ol.ck, cache, N, cfg.G, cfg.k_qjl)
    rel = H.compare_scores(scores, ref_scores, scale, name)
    err = H.compare_out(out, ref_out, name)
    H.log(f"  score rel err {rel:.2e}  out abs err {err:.2e}")


# Grids of exactly two 4-wave workgroups per CU on a 256-CU part (128 row
# groups x 4 key splits of more than 64 blocks), where the splits dispatched
# first get more key blocks than the others; N = 8500 leaves a ragged last block.
SPLIT_CASES = {
    "128 heads x 4 unequal splits, 8500 keys": workloads.CONFIGS["C3"].with_(B=16, N=8500, dist="normal"),
}


@pytest.mark.parametrize("name", list(SPLIT_CASES))
def test_decode_unequal_splits(name):
    cfg = SPLIT_CASES[name]
    N = cfg.N
    cap = (N + 7) // 8 * 8
    H.log(f"[decode unequal splits] {name}")
    packed = workloads.random_packed_numpy(cfg, cfg.B * cfg.Hkv, cap, seed=9)
    q = workloads.q_numpy(cfg, seed=9)
    out, scores, ref_out, ref_scores, cache, ol = _decode_both(cfg, packed, q, N)
    scale = H.score_scale(q, ol.R, ol.S, ol.ck, cache, N, cfg.G, cfg.k_qjl)
    rel = H.compare_scores(scores, ref_scores, scale, name)
    err = H.compare_out(out, ref_out, name)
    H.log(f"  score rel err {rel:.2e}  out abs err {err:.2e}")


def test_decode_eight_wave_workgroups():
    """8 heads x 32768 keys: the 4-wave plan fills the chip with short key
    loops, so the call runs one 8-wave workgroup per CU (64 splits of 512 keys
    become 32 of 1024).  The score-free call (8-wave kernel) is compared with
    the oracle and with the call that also writes the scores (4-wave kernel on
    the same grid)."""
    cfg = workloads.CONFIGS["C2"]
    N = cfg.N
    cap = (N + 7) // 8 * 8
    H.log("[decode 8-wave workgroups] C2 shape")
    packed = workloads.random_packed_numpy(cfg, cfg.B * cfg.Hkv, cap, seed=11)
    q = workloads.q_numpy(cfg, seed=11)
    out, scores, ref_out, ref_scores, cache, ol = _decode_both(cfg, packed, q, N)
    scale = H.score_scale(q, ol.R, ol.S, ol.ck, cache, N, cfg.G, cfg.k_qjl)
    H.compare_scores(scores, ref_scores, scale, "C2 scores")
    H.compare_out(out, ref_out, "C2 with scores")
    layer = H.gpu_layer(cfg)
    K, V = H.upload_packed(layer, cfg, packed, cfg.B * cfg.Hkv, cap)
    out8, _ = B.attn_decode(layer, torch.from_numpy(q).cuda(), K, V, N, cfg.Hkv, cfg.causal)
    torch.cuda.synchronize()
    err = H.compare_out(out8.cpu().numpy(), ref_out, "C2 without scores")
    assert np.abs(out8.cpu().numpy() - out).max() <= 2e-3
    H.log(f"  out abs err {err:.2e}")


def _end_to_end(cfg, what, seed=2, out_scale=1.0):
    """Quantize K and V and decode on the GPU; the oracle encodes the same raw
    inputs itself, validates every GPU field and decodes the cache the GPU
    wrote (its codes and signs, the oracle's norms and gammas); every score
    and output is compared."""
    xk, xv = _kv(cfg, "K", seed=seed), _kv(cfg, "V", seed=seed)
    return _decode_check(cfg, xk, xv, workloads.q_numpy(cfg, seed=seed), what, out_scale)


def _decode_check(cfg, xk, xv, q_np, what, out_scale=1.0):
    N = xk.shape[1]
    layer, ol, K, V, cache, st = H.quantize_and_check(cfg, xk, xv, what=what)
    out, scores = B.attn_decode(layer, torch.from_numpy(q_np).cuda(), K, V, N, cfg.Hkv, cfg.causal,
                                want_scores=True)
    torch.cuda.synchronize()
    ref_out, ref_scores = attention.decode(q_np, ol.R, ol.S, ol.ck, ol.cv, cache, N, cfg.causal)
    scale = H.score_scale(q_np, ol.R, ol.S, ol.ck, cache, N, cfg.G, cfg.k_qjl)
    rel = H.compare_scores(scores.cpu().numpy(), ref_scores, np.maximum(scale, 1e-30), what)
    err = H.compare_out(out.cpu().numpy(), ref_out, what, out_scale)
    H.log(f"  band rows: codes K {st['code_rows']} V {st['value_rows']}, signs {st['sign_rows']}; "
          f"score rel {rel:.2e}  out abs {err:.2e}")
    return rel, err


@pytest.mark.parametrize("name", list(REDUCED))
def test_end_to_end_from_raw_inputs(name):
    cfg = REDUCED[name]
    H.log(f"[end to end] {name}")
    _end_to_end(cfg, name)


# Every key width through the matrix-core quantize and decode kernels at
# d = 128 (Haar, fp16), with and without QJL (MSE-only keys), value widths
# chosen so that every value width occurs too.
@pytest.mark.parametrize("qjl", [0, 1])
@pytest.mark.parametrize("kb", [1, 2, 3, 4])
def test_key_widths_d128(kb, qjl):
    cfg = workloads.CONFIGS["C2"].with_(Hq=8, Hkv=2, N=301, k_bits=kb, k_qjl=qjl, v_bits=5 - kb)
    H.log(f"[key widths d128] k_bits={kb} k_qjl={qjl} v_bits={5 - kb}")
    _end_to_end(cfg, f"d128 K{kb}{'+QJL' if qjl else ''} V{5 - kb}", seed=8)


# Layers whose codebooks are the Lloyd-Max quantizers of the exact coordinate
# law (1 - t^2)^((d-3)/2) ([Mobilint], "Coordinates Become Predictable After
# Rotation"): every kernel family reads its codebook from the layer tables.
BETA_CASES = {
    "haar d128 fp16 K3+QJL V2 (matrix-core quantize and decode)":
        workloads.CONFIGS["C2"].with_(Hq=8, Hkv=2, N=301, k_bits=3, v_bits=2, codebook="beta"),
    "hadamard d256 fp16 K4 V4 (transform quantize)":
        workloads.CONFIGS["C5"].with_(B=1, Hq=8, Hkv=2, N=301, codebook="beta"),
    "haar d64 fp32 K2+QJL V3 (scalar kernels)":
        workloads.CONFIGS["C1"].with_(d=64, Hq=4, Hkv=2, N=301, k_bits=2, v_bits=3, codebook="beta"),
}


@pytest.mark.parametrize("name", list(BETA_CASES))
def test_beta_codebook_end_to_end(name):
    cfg = BETA_CASES[name]
    H.log(f"[exact-law codebook] {name}")
    _end_to_end(cfg, name, seed=15)
    # dequantize reconstructs with the same codebook
    _check_dequantize(cfg, B.TQ_VALUES)


# The dithered randomized Hadamard variant (thelatestinai.com paper page
# 2606.10458, third abstract): one seeded offset per token is subtracted from
# its rotated coordinates before quantizing and added back in every
# reconstruction.  d = 64 decodes on the scalar kernels, d = 128 and 256 on the
# matrix-core split kernel with 4- and 8-row groups; 128 query rows per KV head
# would take the many-rows kernel for other layers.  Zero key rows, causal
# chunks and ragged lengths included.
DITHER_CASES = {
    "d128 fp16 K3 V2, 4 rows per KV head": workloads.CONFIGS["C2"].with_(
        Hq=8, Hkv=2, N=301, k_bits=3, k_qjl=0, v_bits=2, rot="hadamard", dither=1),
    "d128 fp16 K2 V3, 8 heads x 4 causal tokens": workloads.CONFIGS["C4"].with_(
        B=1, N=203, Tq=4, k_qjl=0, v_bits=3, rot="hadamard", dither=1),
    "d128 fp16 K1 V4, 128 rows per KV head": workloads.CONFIGS["C4"].with_(
        B=1, N=150, k_bits=1, k_qjl=0, v_bits=4, rot="hadamard", dither=1),
    "d256 fp16 K4 V4": workloads.CONFIGS["C5"].with_(B=1, Hq=8, Hkv=2, N=301, dither=1),
    "d256 fp16 K2 V1, exact-law codebook": workloads.CONFIGS["C5"].with_(
        B=1, Hq=8, Hkv=2, N=97, k_bits=2, v_bits=1, codebook="beta", dither=1),
    "d64 fp32 K1 V4": workloads.CONFIGS["C1"].with_(
        d=64, Hq=4, Hkv=2, N=133, k_bits=1, k_qjl=0, v_bits=4, rot="hadamard", dither=1),
}


@pytest.mark.parametrize("name", list(DITHER_CASES))
def test_dithered_hadamard_end_to_end(name):
    cfg = DITHER_CASES[name]
    H.log(f"[dithered hadamard] {name}")
    xk, xv = _kv(cfg, "K", seed=19), _kv(cfg, "V", seed=19)
    xk[:, 5] = 0  # zero key rows: codes of -delta
    _decode_check(cfg, xk, xv, workloads.q_numpy(cfg, seed=19), name)
    for which in (B.TQ_KEYS, B.TQ_VALUES):
        err = _check_dequantize(cfg, which)
        H.log(f"  dequantize which={which}: max error / norm {err:.2e}")


# Values with QJL (TurboQuant_prod on V; [Mobilint] "Two-Stage Approach",
# final reconstruction): each value row is n (R^T c[idx] + sqrt(pi/2)/d gamma
# S^T sigma).  Decode keeps the sum of the softmax-weighted QJL terms beside
# the MSE sum and back-projects it once per query row.  Haar and Hadamard,
# d = 64, 128 and 256, keys with and without QJL, causal chunks, up to 64
# query rows per KV head; a zero value row; ragged lengths.
VALUE_QJL_CASES = {
    "haar d128 fp16 K2+QJL V2+QJL, 4 rows per KV head": workloads.CONFIGS["C2"].with_(
        Hq=8, Hkv=2, N=301, k_bits=2, v_bits=2, v_qjl=1),
    "haar d128 fp16 K3 V3+QJL, 8 heads x 4 causal tokens": workloads.CONFIGS["C4"].with_(
        B=1, N=203, Tq=4, k_bits=3, k_qjl=0, v_bits=3, rot="haar", v_qjl=1),
    "haar d128 fp16 K2+QJL V1+QJL, 64 rows per KV head": workloads.CONFIGS["C2"].with_(
        Hq=16, Hkv=1, Tq=4, causal=1, N=150, v_bits=1, v_qjl=1),
    "hadamard d256 fp16 K4 V4+QJL": workloads.CONFIGS["C5"].with_(B=1, Hq=8, Hkv=2, N=155, v_qjl=1),
    "haar d64 fp32 K1+QJL V4+QJL": workloads.CONFIGS["C1"].with_(
        d=64, Hq=4, Hkv=2, N=133, k_bits=1, v_bits=4, v_qjl=1),
}


@pytest.mark.parametrize("name", list(VALUE_QJL_CASES))
def test_values_with_qjl_end_to_end(name):
    cfg = VALUE_QJL_CASES[name]
    H.log(f"[values with QJL] {name}")
    xk, xv = _kv(cfg, "K", seed=23), _kv(cfg, "V", seed=23)
    xv[:, 3] = 0  # a zero value row: zero norm, no QJL term
    _decode_check(cfg, xk, xv, workloads.q_numpy(cfg, seed=23), name)


@pytest.mark.parametrize("name", list(VALUE_QJL_CASES)[:2])
def test_values_with_qjl_on_random_cache(name):
    """Decode alone: seeded random codes, value signs and residual norms."""
    cfg = VALUE_QJL_CASES[name]
    cap = (cfg.N + 7) // 8 * 8
    packed = workloads.random_packed_numpy(cfg, cfg.B * cfg.Hkv, cap, seed=29)
    q = workloads.q_numpy(cfg, seed=29)
    out, scores, ref_out, ref_scores, cache, ol = _decode_both(cfg, packed, q, cfg.N)
    scale = H.score_scale(q, ol.R, ol.S, ol.ck, cache, cfg.N, cfg.G, cfg.k_qjl)
    H.compare_scores(scores, ref_scores, scale, name)
    err = H.compare_out(out, ref_out, name)
    # the values' QJL term is really there: the oracle without it differs
    mse = {k: v for k, v in cache.items() if k not in ("v_sign", "v_rnorm")}
    ref_mse, _ = attention.decode(q, ol.R, ol.S, ol.ck, ol.cv, mse, cfg.N, cfg.causal)
    assert np.abs(ref_mse - ref_out).max() > 50 * max(err, 1e-6)
    H.log(f"  out abs err {err:.2e}, QJL term up to {np.abs(ref_mse - ref_out).max():.2e}")


@pytest.mark.parametrize("qjl", [0, 1])
@pytest.mark.parametrize("d,rows", [(128, 4), (256, 4), (128, 64)])
def test_decode_all_width_pairs(d, rows, qjl):
    """Decode alone on seeded random caches for all 16 (key bits, value bits)
    pairs of the matrix-core kernels, with and without QJL keys; 64 query rows
    per KV head (8 heads x 8 causal tokens) take the wide kernel."""
    worst = 0.0
    for kb in (1, 2, 3, 4):
        for vb in (1, 2, 3, 4):
            cfg = workloads.CONFIGS["C2"].with_(d=d, Hq=8, Hkv=2, N=211, k_bits=kb, v_bits=vb, k_qjl=qjl)
            if rows == 64:
                cfg = cfg.with_(Hq=16, Tq=8, causal=1)
            cap = (cfg.N + 7) // 8 * 8
            packed = workloads.random_packed_numpy(cfg, cfg.B * cfg.Hkv, cap, seed=20 + kb * 4 + vb)
            q = workloads.q_numpy(cfg, seed=20 + kb * 4 + vb)
            out, scores, ref_out, ref_scores, cache, ol = _decode_both(cfg, packed, q, cfg.N)
            scale = H.score_scale(q, ol.R, ol.S, ol.ck, cache, cfg.N, cfg.G, cfg.k_qjl)
            what = f"d={d} rows={rows} qjl={qjl} K{kb} V{vb}"
            worst = max(worst, H.compare_scores(scores, ref_scores, scale, what))
            H.compare_out(out, ref_out, what)
    H.log(f"[decode width pairs] d={d} rows={rows} qjl={qjl}: worst score rel {worst:.2e}")


# Rows with norms far above the fp16 range of the P.V operand: fp32 inputs
# (reference quantize kernel) and fp16 inputs (matrix-core kernel), keys and
# values of norm > 1e5.  The outputs are of order max ||v|| / sqrt(d), so the
# 2e-3 output bound is applied relative to that scale.
LARGE_NORM_CASES = {
    "fp32 d128 QJL, |k| ~ 3.4e5, |v| ~ 2.3e5": (workloads.CONFIGS["C1"].with_(N=300, Hq=4, Hkv=2), 3e4, 2e4),
    "fp16 d128 QJL, |k| ~ 1.1e5, |v| ~ 1.1e5": (workloads.CONFIGS["C2"].with_(Hq=8, Hkv=2, N=300), 1e4, 1e4),
    "fp16 d256 Hadamard, |v| ~ 1.6e5": (workloads.CONFIGS["C5"].with_(B=1, Hq=8, Hkv=2, N=300, dist="normal"),
                                        1.0, 1e4),
}


@pytest.mark.parametrize("name", list(LARGE_NORM_CASES))
def test_large_norms(name):
    cfg, ks, vs = LARGE_NORM_CASES[name]
    H.log(f"[large norms] {name}")
    dt = np.float16 if cfg.dtype == "f16" else np.float32
    xk = (_kv(cfg, "K", seed=12).astype(np.float64) * ks).astype(dt)
    xv = (_kv(cfg, "V", seed=12).astype(np.float64) * vs).astype(dt)
    assert np.isfinite(xk).all() and np.isfinite(xv).all()
    vmax = float(np.linalg.norm(xv.astype(np.float64), axis=-1).max())
    assert vmax > 1e5
    _decode_check(cfg, xk, xv, workloads.q_numpy(cfg, seed=12), name, out_scale=vmax / math.sqrt(cfg.d))


def test_decode_random_cache_huge_value_norms():
    """Value norms from 1 to 1e7 in one sequence (the decode's value scale is
    lowered as larger norms arrive, mid-loop)."""
    cfg = workloads.CONFIGS["C3"].with_(B=2, N=1500, dist="normal")
    cap = (cfg.N + 7) // 8 * 8
    packed = workloads.random_packed_numpy(cfg, cfg.B * cfg.Hkv, cap, seed=13)
    ramp = np.logspace(0, 7, cap, dtype=np.float64)
    packed["v_norm"] = (packed["v_norm"].reshape(-1, cap) * ramp[None, :]).astype(np.float32).reshape(-1)
    q = workloads.q_numpy(cfg, seed=13)
    out, scores, ref_out, ref_scores, cache, ol = _decode_both(cfg, packed, q, cfg.N)
    scale = H.score_scale(q, ol.R, ol.S, ol.ck, cache, cfg.N, cfg.G, cfg.k_qjl)
    H.compare_scores(scores, ref_scores, scale, "huge value norms")
    vmax = float(packed["v_norm"].max())
    err = H.compare_out(out, ref_out, "huge value norms", vmax / math.sqrt(cfg.d))
    H.log(f"[huge value norms] out abs err {err:.2e} (scale {vmax / math.sqrt(cfg.d):.2e})")


# Append one token per step into a preallocated cache and decode after every
# step ([tq-kv] page: single-key compression appended to a growing compressed
# cache; [cuTile] listing: decode with one query token over the cache).  The
# cache starts with a bulk-quantized prefix; the appended tokens cross 8-token
# value tiles; the capacity exceeds the last length.
APPEND_LOOP_CASES = {
    "haar d128 K2+QJL V3": workloads.CONFIGS["C2"].with_(B=2, Hq=8, Hkv=2, N=37),
    "haar d128 MSE-only K4 V2": workloads.CONFIGS["C2"].with_(B=2, Hq=8, Hkv=2, N=37, k_bits=4, k_qjl=0,
                                                               v_bits=2),
    "hadamard d256 K4 V4": workloads.CONFIGS["C5"].with_(B=1, Hq=8, Hkv=2, N=37),
}


@pytest.mark.parametrize("name", list(APPEND_LOOP_CASES))
def test_append_decode_loop(name):
    cfg = APPEND_LOOP_CASES[name]
    steps, cap = 14, 64
    H.log(f"[append + decode loop] {name}: prefix {cfg.N}, {steps} single-token steps, capacity {cap}")
    S, d = cfg.B * cfg.Hkv, cfg.d
    total = cfg.N + steps
    xk = _kv(cfg.with_(N=total), "K", seed=14)
    xv = _kv(cfg.with_(N=total), "V", seed=14)
    q_all = workloads.q_numpy(cfg.with_(Tq=steps), seed=14)       # query of step i: token i
    layer = H.gpu_layer(cfg)
    ol = H.OracleLayer(cfg)
    K = B.Cache(layer, B.TQ_KEYS, S, cap)
    V = B.Cache(layer, B.TQ_VALUES, S, cap)
    dk, dv = torch.from_numpy(xk).cuda(), torch.from_numpy(xv).cuda()
    B.quantize_kv(layer, B.TQ_KEYS, dk[:, :cfg.N].contiguous(), K)
    B.quantize_kv(layer, B.TQ_VALUES, dv[:, :cfg.N].contiguous(), V)
    Sk = ol.S if cfg.k_qjl else None
    ek = codec.encode_rows(xk.reshape(-1, d), ol.R, ol.ck, ol.bk, Sk)
    ev = codec.encode_rows(xv.reshape(-1, d), ol.R, ol.cv, ol.bv)
    wsb = max(B.decode_workspace_bytes(layer, cfg.B, cfg.Hq, cfg.Hkv, 1, n) for n in range(cfg.N + 1, total + 1))
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    worst_rel, worst_out = 0.0, 0.0
    for i in range(steps):
        t = cfg.N + i
        B.quantize_kv(layer, B.TQ_KEYS, dk[:, t:t + 1].contiguous(), K, t0=t)
        B.quantize_kv(layer, B.TQ_VALUES, dv[:, t:t + 1].contiguous(), V, t0=t)
        q_np = np.ascontiguousarray(q_all[:, :, i:i + 1])
        out, scores = B.attn_decode(layer, torch.from_numpy(q_np).cuda(), K, V, t + 1, cfg.Hkv,
                                    want_scores=True, workspace=ws)
        torch.cuda.synchronize()
        n = t + 1
        rows = _rows(S, cap, n)
        orow = np.array([s * total + u for s in range(S) for u in range(n)], dtype=np.int64)
        sub = lambda e: {k: v[orow] for k, v in e.items()}
        ekn, evn = sub(ek), sub(ev)
        if cfg.k_qjl:
            kf, _ = H.check_keys(H.gpu_codes_key(K, S, cap, d, cfg.k_bits, rows), K["norm"].cpu().numpy()[rows],
                                 ekn, ol, f"step {i} K", H.gpu_signs(K, S, cap, d, rows),
                                 K["rnorm"].cpu().numpy()[rows])
        else:
            kf, _ = H.check_keys(H.gpu_codes_key(K, S, cap, d, cfg.k_bits, rows), K["norm"].cpu().numpy()[rows],
                                 ekn, ol, f"step {i} K")
        vf, _ = H.check_values(H.gpu_codes_value(V, S, cap, d, cfg.v_bits)[rows], V["norm"].cpu().numpy()[rows],
                               evn, ol, f"step {i} V")
        cache = H.oracle_cache(kf, vf, cfg.B, cfg.Hkv, n, d)
        ref_out, ref_scores = attention.decode(q_np, ol.R, ol.S, ol.ck, ol.cv, cache, n, False)
        scale = H.score_scale(q_np, ol.R, ol.S, ol.ck, cache, n, cfg.G, cfg.k_qjl)
        worst_rel = max(worst_rel, H.compare_scores(scores.cpu().numpy(), ref_scores, scale, f"step {i}"))
        worst_out = max(worst_out, H.compare_out(out.cpu().numpy(), ref_out, f"step {i}"))
    # tokens past the last one were never written
    assert float(K["norm"].view(S, cap)[:, total:].abs().max()) == 0.0
    H.log(f"  worst score rel {worst_rel:.2e}, worst out abs {worst_out:.2e}")


def _check_dequantize(cfg, which, n_out=None):
    """Quantize cfg's rows, dequantize the first n_out tokens of each sequence
    and compare with the oracle's reconstruction n * R^T c[idx]."""
    x = _kv(cfg, "K" if which == B.TQ_KEYS else "V", seed=3)
    S, n, d = x.shape
    n_out = n if n_out is None else n_out
    layer, ol, cache, enc, cap = H.run_quantize_both(cfg, x, which)
    got = B.dequantize(layer, which, cache, n_out).cpu().numpy().reshape(-1, d)
    c, bnd = (ol.ck, ol.bk) if which == B.TQ_KEYS else (ol.cv, ol.bv)
    keep = np.array([s * n + t for s in range(S) for t in range(n_out)], dtype=np.int64)
    dith = enc["dither"][keep] if "dither" in enc else None
    ref = codec.reconstruct_mse(enc["idx"][keep], enc["norm"][keep], ol.R, c, dither=dith)
    rows = np.array([s * cap + t for s in range(S) for t in range(n)])
    bits = cfg.k_bits if which == B.TQ_KEYS else cfg.v_bits
    gidx = (H.gpu_codes_key(cache, S, cap, d, bits, rows) if which == B.TQ_KEYS
            else H.gpu_codes_value(cache, S, cap, d, bits)[rows])
    flipped = H.compare_codes(gidx, enc, bnd, "codes")[keep]
    scale = enc["norm"][keep][:, None]
    err = np.abs(got - ref) / np.maximum(scale, 1e-30)
    assert err[~flipped].max() < 2e-6
    half = B.dequantize(layer, which, cache, n_out, out_dtype=torch.float16).cpu().numpy().reshape(-1, d)
    np.testing.assert_allclose(half[~flipped], got[~flipped], rtol=2e-3, atol=1e-3)
    # fp16 rows against the oracle: half an ulp of the output (2^-11 relative,
    # 2^-25 absolute below the normal range) plus what the arithmetic may add
    # before that rounding -- at most 1.1e-4 of the norm (fp16 copies of the
    # scaled centroids within 1e-4 relative, R^T split hi + lo) -- since
    # sum_k |R_jk c_k| <= ||R_j|| ||c|| <= 1 for a unit reconstruction.
    half64 = half.astype(np.float64)
    tol = 2.0 ** -11 * np.abs(ref) + 1.1e-4 * scale + 2.0 ** -25
    over = (np.abs(half64 - ref) - tol)[~flipped]
    assert over.max() <= 0, f"fp16 rows: error above the bound by {over.max():.2e}"
    return err[~flipped].max()


@pytest.mark.parametrize("name", ["C1", "C3", "C5"])
@pytest.mark.parametrize("which", [B.TQ_KEYS, B.TQ_VALUES])
def test_dequantize_parity(name, which):
    H.log(f"[dequantize] {name} which={which}")
    _check_dequantize(REDUCED[name], which)


# Head dimensions, widths and token counts the workloads above leave out:
# d = 64, 1-bit codes, fewer tokens than one 8-token value tile, an exact
# multiple of the kernel's 64-token step, and a prefix of the stored tokens.
DEQUANT_SHAPES = {
    "hadamard d64 K1 V2, 70 tokens": (workloads.CONFIGS["C5"].with_(B=1, Hq=2, Hkv=2, N=70, d=64, dtype="f32",
                                                                     k_bits=1, v_bits=2), None),
    "haar d128 K4 V1, 5 tokens": (workloads.CONFIGS["C2"].with_(Hq=4, Hkv=2, N=5, k_bits=4, v_bits=1), None),
    "haar d128 K2 V3, 128 tokens": (workloads.CONFIGS["C2"].with_(Hq=4, Hkv=2, N=128), None),
    "hadamard d256 K3 V2, first 67 of 200": (workloads.CONFIGS["C5"].with_(B=1, Hq=4, Hkv=2, N=200, k_bits=3,
                                                                            v_bits=2), 67),
    # fp16 rows of the Haar kernel at the other head dimensions (its output
    # tile is staged in LDS and written as whole rows): several 64-token
    # steps and a ragged last one.
    "haar d64 fp16 K2 V3, 150 tokens": (workloads.CONFIGS["C2"].with_(Hq=4, Hkv=2, N=150, d=64), None),
    "haar d256 fp16 K3 V4, 131 tokens": (workloads.CONFIGS["C2"].with_(Hq=4, Hkv=2, N=131, d=256, k_bits=3,
                                                                        v_bits=4), None),
}


@pytest.mark.parametrize("name", list(DEQUANT_SHAPES))
@pytest.mark.parametrize("which", [B.TQ_KEYS, B.TQ_VALUES])
def test_dequantize_shapes(name, which):
    cfg, n_out = DEQUANT_SHAPES[name]
    H.log(f"[dequantize] {name} which={which}")
    err = _check_dequantize(cfg, which, n_out)
    H.log(f"  max error / norm {err:.2e}")


# Two-stage reconstruction of rows with QJL ([Mobilint] "Two-Stage Approach",
# final reconstruction): keys with QJL and values of layers with QJL on
# values, every head dimension and both output dtypes, a prefix of the stored
# tokens, ragged lengths.
PROD_CASES = {
    "haar d128 fp16 K2+QJL": (workloads.CONFIGS["C2"].with_(Hq=4, Hkv=2, N=203, k_bits=2), None, B.TQ_KEYS),
    "haar d128 fp16 K3+QJL, first 100 of 130": (workloads.CONFIGS["C3"].with_(B=1, N=130), 100, B.TQ_KEYS),
    "haar d128 fp32 K1+QJL": (workloads.CONFIGS["C1"].with_(N=150, k_bits=1), None, B.TQ_KEYS),
    "haar d128 fp32 K4+QJL, first 129 of 200": (workloads.CONFIGS["C1"].with_(N=200, k_bits=4), 129, B.TQ_KEYS),
    "hadamard d256 fp16 K3+QJL": (workloads.CONFIGS["C5"].with_(B=1, Hq=4, Hkv=2, N=77, k_qjl=1, k_bits=3), None,
                                  B.TQ_KEYS),
    "haar d64 fp32 K1+QJL": (workloads.CONFIGS["C1"].with_(d=64, Hq=2, Hkv=2, N=70, k_bits=1), None, B.TQ_KEYS),
    "haar d64 fp16 K3+QJL, first 140 of 150": (workloads.CONFIGS["C2"].with_(d=64, Hq=4, Hkv=2, N=150, k_bits=3,
                                                                              k_qjl=1), 140, B.TQ_KEYS),
    "haar d128 fp16 V3+QJL, first 90 of 203": (workloads.CONFIGS["C2"].with_(Hq=4, Hkv=2, N=203, v_qjl=1), 90,
                                               B.TQ_VALUES),
    "hadamard d256 fp16 V4+QJL": (workloads.CONFIGS["C5"].with_(B=1, Hq=4, Hkv=2, N=77, v_qjl=1), None,
                                  B.TQ_VALUES),
    "hadamard d64 fp32 V2+QJL": (workloads.CONFIGS["C5"].with_(B=1, Hq=2, Hkv=2, N=70, d=64, dtype="f32",
                                                               v_bits=2, v_qjl=1), None, B.TQ_VALUES),
}


@pytest.mark.parametrize("name", list(PROD_CASES))
def test_dequantize_prod(name):
    cfg, n_out, which = PROD_CASES[name]
    H.log(f"[dequantize prod] {name}")
    values = which == B.TQ_VALUES
    x = _kv(cfg, "V" if values else "K", seed=17)
    S, n, d = x.shape
    n_out = n if n_out is None else n_out
    layer, ol, cache, enc, cap = H.run_quantize_both(cfg, x, which)
    rows = _rows(S, cap, n)
    bits = cfg.v_bits if values else cfg.k_bits
    gidx = (H.gpu_codes_value(cache, S, cap, d, bits)[rows] if values
            else H.gpu_codes_key(cache, S, cap, d, bits, rows))
    kf, st = H.check_keys(gidx, cache["norm"].cpu().numpy()[rows], enc, ol, name,
                          H.gpu_signs(cache, S, cap, d, rows), cache["rnorm"].cpu().numpy()[rows], values=values)
    keep = np.array([s * n + t for s in range(S) for t in range(n_out)], dtype=np.int64)
    ref = codec.reconstruct_prod(kf["idx"][keep], kf["norm"][keep], kf["sign"][keep], kf["rnorm"][keep],
                                 ol.R, ol.cv if values else ol.ck, ol.S)
    got = B.dequantize(layer, which, cache, n_out, prod=True).cpu().numpy().reshape(-1, d)
    err = np.abs(got - ref) / np.maximum(kf["norm"][keep][:, None], 1e-30)
    assert err.max() < 2e-6, f"{name}: error {err.max():.2e} of the norm"
    # the QJL term is really there: the MSE-only rows differ from these
    mse = B.dequantize(layer, which, cache, n_out).cpu().numpy().reshape(-1, d)
    assert (np.abs(mse - got) / kf["norm"][keep][:, None]).max() > 1e-2
    half = B.dequantize(layer, which, cache, n_out, out_dtype=torch.float16, prod=True).cpu().numpy()
    np.testing.assert_allclose(half.reshape(-1, d), got, rtol=2e-3, atol=2e-3)
    # fp16 rows: the output's rounding (2^-11 of each coordinate) plus 2e-4 of
    # the norm for the single fp16 copies of the centroids and of S^T
    herr = np.abs(half.reshape(-1, d).astype(np.float64) - ref) - 2.0 ** -11 * np.abs(ref)
    hmax = (herr / np.maximum(kf["norm"][keep][:, None], 1e-30)).max()
    assert hmax < 2e-4, f"{name}: fp16 rows off by {hmax:.2e} of the norm beyond their rounding"
    H.log(f"  max error / norm {err.max():.2e}, fp16 rows {hmax:.2e} beyond rounding "
          f"(band rows: codes {st['code_rows']}, signs {st['sign_rows']})")


PROD_EDGE_CASES = {
    "haar d128 fp16 K3+QJL (one pass)": workloads.CONFIGS["C3"].with_(B=1, Hkv=2, Hq=4, N=70),
    "haar d64 fp32 K2+QJL (one pass)": workloads.CONFIGS["C1"].with_(d=64, N=70),
    "hadamard d256 fp16 K3+QJL (two passes)": workloads.CONFIGS["C5"].with_(B=1, Hq=4, Hkv=2, N=70, k_qjl=1,
                                                                            k_bits=3),
}


@pytest.mark.parametrize("name", list(PROD_EDGE_CASES))
def test_dequantize_prod_edges(name):
    """n = 0 writes nothing and succeeds; token 0 of every sequence is a zero
    input row (norm 0), which comes back as exact zeros in both output dtypes;
    a two-token prefix matches the oracle on token 1."""
    cfg = PROD_EDGE_CASES[name]
    H.log(f"[dequantize prod edges] {name}")
    x = _kv(cfg, "K", seed=23)
    x[:, 0] = 0
    S, n, d = x.shape
    layer, ol, cache, enc, cap = H.run_quantize_both(cfg, x, B.TQ_KEYS)
    rows = _rows(S, cap, n)
    kf, _ = H.check_keys(H.gpu_codes_key(cache, S, cap, d, cfg.k_bits, rows), cache["norm"].cpu().numpy()[rows],
                         enc, ol, name, H.gpu_signs(cache, S, cap, d, rows), cache["rnorm"].cpu().numpy()[rows])
    keep = np.array([s * n + 1 for s in range(S)], dtype=np.int64)
    ref = codec.reconstruct_prod(kf["idx"][keep], kf["norm"][keep], kf["sign"][keep], kf["rnorm"][keep],
                                 ol.R, ol.ck, ol.S)
    for dt in (torch.float32, torch.float16):
        empty = B.dequantize(layer, B.TQ_KEYS, cache, 0, out_dtype=dt, prod=True)
        assert tuple(empty.shape) == (S, 0, d)
        two = B.dequantize(layer, B.TQ_KEYS, cache, 2, out_dtype=dt, prod=True).cpu().double().numpy()
        assert np.all(two[:, 0] == 0), f"{name}: zero rows came back nonzero"
        err = np.abs(two[:, 1] - ref) / kf["norm"][keep][:, None]
        bar = 2e-6 if dt == torch.float32 else 2.0 ** -11 * np.abs(ref).max() / kf["norm"][keep].min() + 2e-4
        assert err.max() < bar, f"{name} {dt}: token 1 off by {err.max():.2e} of the norm"
    H.log(f"  zero rows exact, token 1 within the bars")


APPEND_CASES = {
    "haar-d128-f16": workloads.CONFIGS["C2"].with_(N=40),
    "dithered-hadamard-d128-f16": workloads.CONFIGS["C5"].with_(B=1, Hq=4, Hkv=2, N=40, d=128, k_bits=2,
                                                                 v_bits=3, dither=1),
    "hadamard-d256-f16": workloads.CONFIGS["C5"].with_(B=1, Hq=4, Hkv=2, N=40),
    "hadamard-d64-f32": workloads.CONFIGS["C5"].with_(B=1, Hq=4, Hkv=2, N=40, d=64, dtype="f32",
                                                       k_bits=2, v_bits=3),
}


@pytest.mark.parametrize("case", list(APPEND_CASES))
def test_append_in_pieces_matches_one_call(case):
    """Quantizing tokens in several calls (starting inside a value tile) gives
    the same bytes as one call, and leaves other tokens untouched."""
    cfg = APPEND_CASES[case]
    layer = H.gpu_layer(cfg)
    x = torch.from_numpy(_kv(cfg, "V", seed=4)).cuda()
    S = x.shape[0]
    for which in (B.TQ_KEYS, B.TQ_VALUES):
        one = B.Cache(layer, which, S, 48)
        B.quantize_kv(layer, which, x, one)
        parts = B.Cache(layer, which, S, 48)
        for a, b in ((0, 13), (13, 14), (14, 27), (27, 40)):
            B.quantize_kv(layer, which, x[:, a:b].contiguous(), parts, t0=a)
        torch.cuda.synchronize()
        for k in ("idx", "norm", "sign", "rnorm"):
            if one[k] is not None:
                assert torch.equal(one[k], parts[k]), (which, k)
        # a single-token append into the middle of a tile changes only that token
        before = parts["idx"].clone()
        B.quantize_kv(layer, which, torch.zeros_like(x[:, 21:22]), parts, t0=21)
        torch.cuda.synchronize()
        d = cfg.d
        if which == B.TQ_VALUES:
            g0 = codec.unpack_value_codes(before.cpu().numpy(), cfg.v_bits, S, 48, d)
            g1 = codec.unpack_value_codes(parts["idx"].cpu().numpy(), cfg.v_bits, S, 48, d)
            changed = (g0 != g1).any(axis=2)
            assert not changed[:, :21].any() and not changed[:, 22:40].any()
            if cfg.dither:
                # zero row of the dithered variant: the codes of -delta (token 21's offset)
                ol = H.OracleLayer(cfg)
                dl = ol.offsets(B.TQ_VALUES, S, 1, t0=21)
                exp = codec.encode_rows(np.zeros((S, d)), ol.R, ol.cv, ol.bv, dither=dl)["idx"]
                assert (g1[:, 21] == exp).all()
            else:
                assert (g1[:, 21] == (1 << (cfg.v_bits - 1)) - 1).all()  # zero row: lower-middle code
        assert torch.equal(parts["norm"].view(S, 48)[:, 21], torch.zeros(S, device="cuda"))


def test_edge_shapes_single_key_zero_rows_and_head_dims():
    """N=1, zero input rows, d=64 and d=256 with 1- and 4-bit codes, Hadamard
    with QJL, fp32 inputs, and a causal chunk as long as the cache."""
    cases = [
        workloads.CONFIGS["C1"].with_(N=1),
        workloads.CONFIGS["C2"].with_(d=64, N=37, k_bits=1, v_bits=4, Hq=8, Hkv=2),
        workloads.CONFIGS["C5"].with_(B=1, Hq=4, Hkv=1, N=21, k_qjl=1, k_bits=3, v_bits=1),
        workloads.CONFIGS["C4"].with_(B=1, N=16, Tq=16),
        workloads.CONFIGS["C1"].with_(N=9, Tq=3, causal=1, Hq=2, Hkv=1, rot="hadamard"),
    ]
    for cfg in cases:
        H.log(f"[edge] {cfg}")
        xk, xv = _kv(cfg, "K", seed=5), _kv(cfg, "V", seed=5)
        xk[:, 0] = 0  # a zero key row
        rel, err = _decode_check(cfg, xk, xv, workloads.q_numpy(cfg, seed=5), str(cfg))


def test_decode_is_deterministic():
    cfg = REDUCED["C2"]
    cap = (cfg.N + 7) // 8 * 8
    packed = workloads.random_packed_numpy(cfg, cfg.B * cfg.Hkv, cap, seed=6)
    layer = H.gpu_layer(cfg)
    K, V = H.upload_packed(layer, cfg, packed, cfg.B * cfg.Hkv, cap)
    q = torch.from_numpy(workloads.q_numpy(cfg, seed=6)).cuda()
    a, _ = B.attn_decode(layer, q, K, V, cfg.N, cfg.Hkv)
    b, _ = B.attn_decode(layer, q, K, V, cfg.N, cfg.Hkv)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("dtype", ["f16", "f32"])
def test_hadamard_quantize_all_widths(d, dtype):
    """Randomized-Hadamard rotation without QJL (the transform path): every code
    width, head dimension and input dtype, keys and values, ragged length."""
    for bits in (1, 2, 3, 4):
        cfg = workloads.CONFIGS["C5"].with_(B=1, Hq=4, Hkv=2, N=77, d=d, dtype=dtype, k_bits=bits,
                                            v_bits=5 - bits)
        H.log(f"[hadamard quantize] d={d} {dtype} k_bits={bits} v_bits={5 - bits}")
        for which, bnd_bits in ((B.TQ_KEYS, cfg.k_bits), (B.TQ_VALUES, cfg.v_bits)):
            x = _kv(cfg, "K" if which == B.TQ_KEYS else "V", seed=7)
            S, n, _ = x.shape
            layer, ol, cache, enc, cap = H.run_quantize_both(cfg, x, which)
            rows = np.array([s * cap + t for s in range(S) for t in range(n)])
            if which == B.TQ_KEYS:
                gidx = H.gpu_codes_key(cache, S, cap, d, bnd_bits, rows)
                bnd = ol.bk
            else:
                gidx = H.gpu_codes_value(cache, S, cap, d, bnd_bits)[rows]
                bnd = ol.bv
            flipped = H.compare_codes(gidx, enc, bnd, f"d={d} {dtype} bits={bnd_bits}")
            assert flipped.mean() < 0.02
            np.testing.assert_allclose(cache["norm"].cpu().numpy()[rows], enc["norm"], rtol=2e-6)

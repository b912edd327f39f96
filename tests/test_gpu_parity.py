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


@pytest.mark.parametrize("name", list(REDUCED))
def test_quantize_keys_parity(name):
    cfg = REDUCED[name]
    H.log(f"[quantize K] {name} {cfg}")
    x = _kv(cfg, "K")
    S, n, d = x.shape
    layer, ol, cache, enc, cap = H.run_quantize_both(cfg, x, B.TQ_KEYS)
    rows = np.array([s * cap + t for s in range(S) for t in range(n)])
    gidx = H.gpu_codes_key(cache, S, cap, d, cfg.k_bits, rows)
    flipped = H.compare_codes(gidx, enc, ol.bk, f"{name} K codes")
    assert flipped.mean() < 0.01
    np.testing.assert_allclose(cache["norm"].cpu().numpy()[rows], enc["norm"], rtol=2e-6)
    # packed bytes are identical for every row without a band difference
    rb = d * cfg.k_bits // 8
    gbytes = cache["idx"].cpu().numpy().reshape(S * cap, rb)[rows]
    obytes = codec.pack_key_codes(enc["idx"], cfg.k_bits)
    assert np.array_equal(gbytes[~flipped], obytes[~flipped])
    if cfg.k_qjl:
        gs = H.gpu_signs(cache, S, cap, d, rows)
        H.compare_key_extras(gs, cache["rnorm"].cpu().numpy()[rows], enc, flipped, f"{name} K")
    H.log(f"  rows={len(rows)} band-flipped rows={int(flipped.sum())}")


@pytest.mark.parametrize("name", list(REDUCED))
def test_quantize_values_parity(name):
    cfg = REDUCED[name]
    H.log(f"[quantize V] {name}")
    x = _kv(cfg, "V")
    S, n, d = x.shape
    layer, ol, cache, enc, cap = H.run_quantize_both(cfg, x, B.TQ_VALUES)
    rows = np.array([s * cap + t for s in range(S) for t in range(n)])
    gidx = H.gpu_codes_value(cache, S, cap, d, cfg.v_bits)[rows]
    flipped = H.compare_codes(gidx, enc, ol.bv, f"{name} V codes")
    assert flipped.mean() < 0.01
    np.testing.assert_allclose(cache["norm"].cpu().numpy()[rows], enc["norm"], rtol=2e-6)


def _decode_both(cfg, packed, q_np, N, want_scores=True):
    S = cfg.B * cfg.Hkv
    cap = (N + 7) // 8 * 8
    layer = H.gpu_layer(cfg)
    ol = H.OracleLayer(cfg)
    K, V = H.upload_packed(layer, cfg, packed, S, cap)
    q = torch.from_numpy(q_np).cuda()
    out, scores = B.attn_decode(layer, q, K, V, N, cfg.Hkv, cfg.causal, want_scores=want_scores)
    torch.cuda.synchronize()
    cache = attention.unpack_cache(packed, cfg.B, cfg.Hkv, cap, cfg.d, cfg.k_bits, cfg.v_bits, cfg.k_qjl)
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


@pytest.mark.parametrize("name", list(REDUCED))
def test_end_to_end_from_raw_inputs(name):
    """Quantize K and V and decode on the GPU; the oracle encodes the same raw
    inputs itself.  Keys whose code or sign bit differs inside the boundary band are left
    out of the score comparison; the output must still be within 2e-3."""
    cfg = REDUCED[name]
    H.log(f"[end to end] {name}")
    xk, xv = _kv(cfg, "K", seed=2), _kv(cfg, "V", seed=2)
    S, N, d = xk.shape
    layer = H.gpu_layer(cfg)
    ol = H.OracleLayer(cfg)
    _, _, K, ek, cap = H.run_quantize_both(cfg, xk, B.TQ_KEYS, layer, ol)
    _, _, V, ev, _ = H.run_quantize_both(cfg, xv, B.TQ_VALUES, layer, ol)
    rows = np.array([s * cap + t for s in range(S) for t in range(N)])
    kflip = H.compare_codes(H.gpu_codes_key(K, S, cap, d, cfg.k_bits, rows), ek, ol.bk, "K")
    if cfg.k_qjl:
        kflip = kflip | H.compare_key_extras(H.gpu_signs(K, S, cap, d, rows), K["rnorm"].cpu().numpy()[rows],
                                             ek, kflip, "K")
    q_np = workloads.q_numpy(cfg, seed=2)
    q = torch.from_numpy(q_np).cuda()
    out, scores = B.attn_decode(layer, q, K, V, N, cfg.Hkv, cfg.causal, want_scores=True)
    torch.cuda.synchronize()
    pk = {"k_idx": codec.pack_key_codes(ek["idx"], cfg.k_bits),
          "k_norm": ek["norm"].astype(np.float32),
          "v_idx": codec.pack_value_codes(ev["idx"].reshape(S, N, d), cfg.v_bits) if N % 8 == 0 else None}
    cache = {"k_idx": ek["idx"].reshape(cfg.B, cfg.Hkv, N, d), "k_norm": ek["norm"].reshape(cfg.B, cfg.Hkv, N),
             "v_idx": ev["idx"].reshape(cfg.B, cfg.Hkv, N, d), "v_norm": ev["norm"].reshape(cfg.B, cfg.Hkv, N)}
    if cfg.k_qjl:
        cache["k_sign"] = ek["sign"].reshape(cfg.B, cfg.Hkv, N, d)
        cache["k_rnorm"] = ek["rnorm"].reshape(cfg.B, cfg.Hkv, N)
    ref_out, ref_scores = attention.decode(q_np, ol.R, ol.S, ol.ck, ol.cv, cache, N, cfg.causal)
    scale = H.score_scale(q_np, ol.R, ol.S, ol.ck, cache, N, cfg.G, cfg.k_qjl)
    keep = (~kflip).reshape(cfg.B, cfg.Hkv, N)
    key_mask = np.repeat(keep, cfg.G, axis=1)[:, :, None, :]
    rel = H.compare_scores(scores.cpu().numpy(), ref_scores, scale, name, key_mask)
    err = H.compare_out(out.cpu().numpy(), ref_out, name)
    H.log(f"  flipped keys {int(kflip.sum())}  score rel {rel:.2e}  out abs {err:.2e}")


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
    ref = codec.reconstruct_mse(enc["idx"][keep], enc["norm"][keep], ol.R, c)
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
}


@pytest.mark.parametrize("name", list(DEQUANT_SHAPES))
@pytest.mark.parametrize("which", [B.TQ_KEYS, B.TQ_VALUES])
def test_dequantize_shapes(name, which):
    cfg, n_out = DEQUANT_SHAPES[name]
    H.log(f"[dequantize] {name} which={which}")
    err = _check_dequantize(cfg, which, n_out)
    H.log(f"  max error / norm {err:.2e}")


APPEND_CASES = {
    "haar-d128-f16": workloads.CONFIGS["C2"].with_(N=40),
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
        layer = H.gpu_layer(cfg)
        ol = H.OracleLayer(cfg)
        _, _, K, ek, cap = H.run_quantize_both(cfg, xk, B.TQ_KEYS, layer, ol)
        _, _, V, ev, _ = H.run_quantize_both(cfg, xv, B.TQ_VALUES, layer, ol)
        S, N, d = xk.shape
        rows = np.array([s * cap + t for s in range(S) for t in range(N)])
        kflip = H.compare_codes(H.gpu_codes_key(K, S, cap, d, cfg.k_bits, rows), ek, ol.bk, "K")
        if cfg.k_qjl:
            kflip = kflip | H.compare_key_extras(H.gpu_signs(K, S, cap, d, rows),
                                                 K["rnorm"].cpu().numpy()[rows], ek, kflip, "K")
        assert K["norm"].view(S, cap)[:, 0].abs().max().item() == 0.0
        q_np = workloads.q_numpy(cfg, seed=5)
        out, scores = B.attn_decode(layer, torch.from_numpy(q_np).cuda(), K, V, N, cfg.Hkv,
                                    cfg.causal, want_scores=True)
        cache = {"k_idx": ek["idx"].reshape(cfg.B, cfg.Hkv, N, d), "k_norm": ek["norm"].reshape(cfg.B, cfg.Hkv, N),
                 "v_idx": ev["idx"].reshape(cfg.B, cfg.Hkv, N, d), "v_norm": ev["norm"].reshape(cfg.B, cfg.Hkv, N)}
        if cfg.k_qjl:
            cache["k_sign"] = ek["sign"].reshape(cfg.B, cfg.Hkv, N, d)
            cache["k_rnorm"] = ek["rnorm"].reshape(cfg.B, cfg.Hkv, N)
        ref_out, ref_scores = attention.decode(q_np, ol.R, ol.S, ol.ck, ol.cv, cache, N, cfg.causal)
        scale = H.score_scale(q_np, ol.R, ol.S, ol.ck, cache, N, cfg.G, cfg.k_qjl)
        keep = np.repeat((~kflip).reshape(cfg.B, cfg.Hkv, N), cfg.G, axis=1)[:, :, None, :]
        H.compare_scores(scores.cpu().numpy(), ref_scores, np.maximum(scale, 1e-30), str(cfg), keep)
        H.compare_out(out.cpu().numpy(), ref_out, str(cfg))


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

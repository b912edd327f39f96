"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
and the fp64 oracle on the same seeded inputs, and compare them at the
tolerances the method's target states:
  * codes and sign bits bit-exact, except coordinates whose rotated value lies
    within 1e-5 of a boundary (resp. |(S r)_i| < 1e-5), where either adjacent
    code (either sign) is accepted.  A row whose codes differ inside the band
    has a different residual: the oracle recomputes its residual, gamma and
    S r from the GPU's codes, and its sign bits and gamma are compared with
    those.  The decode checks then run the oracle on the cache the GPU wrote
    (its validated codes and signs, the oracle's own norms and gammas), so
    every key takes part in every score comparison;
  * scores within 1e-4 relative to the score's Cauchy-Schwarz scale
    n_k (||q|| ||c[idx]|| + gamma sqrt(pi/2)/d ||S q||_1) / sqrt(d);
  * attention output within 2e-3 max absolute error.
"""
import math

import numpy as np
import torch

import workloads
from compressed_attention_turboquant_amd import binding as B
from oracle import attention, codebook, codec, transforms

BAND = 1e-5
SCORE_RTOL = 1e-4
OUT_ATOL = 2e-3


def log(msg):
    print(msg, flush=True)


class OracleLayer:
    def __init__(self, cfg):
        self.R = transforms.rotation(cfg.d, cfg.rot, cfg.layer_seed)
        self.S = transforms.gaussian_projection(cfg.d, cfg.layer_seed)
        self.ck, self.bk = codebook.codebook(cfg.k_bits, cfg.d, cfg.codebook)
        self.cv, self.bv = codebook.codebook(cfg.v_bits, cfg.d, cfg.codebook)
        self.seed = cfg.layer_seed
        self.dither = cfg.dither

    def offsets(self, which, S, n, t0=0):
        """Dithered variant: offsets of tokens t0..t0+n-1 of sequences 0..S-1,
        one per row in [S, n] order (None for other layers)."""
        if not self.dither:
            return None
        seq, t = np.meshgrid(np.arange(S), np.arange(t0, t0 + n), indexing="ij")
        c = self.ck if which == B.TQ_KEYS else self.cv
        return codec.dither_offsets(self.seed, "K" if which == B.TQ_KEYS else "V", seq.ravel(), t.ravel(), c)


def gpu_layer(cfg):
    rot = B.TQ_ROT_HAAR if cfg.rot == "haar" else B.TQ_ROT_HADAMARD
    flags = B.TQ_LAYER_BETA_CODEBOOK if cfg.codebook == "beta" else 0
    if cfg.dither:
        flags |= B.TQ_LAYER_DITHER
    if cfg.v_qjl:
        flags |= B.TQ_LAYER_VALUE_QJL
    return B.make_rotation(cfg.d, rot, cfg.layer_seed, cfg.k_bits, cfg.k_qjl, cfg.v_bits, flags=flags)


def torch_dtype(cfg):
    return torch.float16 if cfg.dtype == "f16" else torch.float32


def band_mask(y, boundaries):
    """Coordinates within BAND of some boundary."""
    b = np.asarray(boundaries, np.float64)
    return (np.abs(y[..., None] - b) < BAND).any(axis=-1)


def compare_codes(gpu_idx, enc, boundaries, what):
    """Check codes: exact outside the band; inside, one of the two neighbours.
    Returns a boolean per row: True where the row had a (legal) difference."""
    exp = enc["idx"]
    diff = gpu_idx != exp
    band = band_mask(enc["y"], boundaries)
    bad = diff & ~band
    assert not bad.any(), f"{what}: {int(bad.sum())} codes differ outside the 1e-5 band " \
                          f"(first at {np.argwhere(bad)[0].tolist()})"
    assert (np.abs(gpu_idx.astype(np.int64) - exp)[diff] == 1).all(), f"{what}: band code off by more than 1"
    return diff.any(axis=1)


def check_keys(gpu_idx, gpu_norm, enc, ol, what, gpu_sign=None, gpu_rnorm=None, values=False):
    """Validate the GPU's key fields (values' with `values`, which carry QJL
    when the layer gives them QJL) against the oracle's encoding `enc` of the
    same rows and return the oracle's view of those rows as decode inputs.

    Codes: exact outside the band (compare_codes).  Norms: within 2e-6.  With
    QJL, expected signs and gamma come from the oracle's own codes for rows
    whose codes matched, and from codec.qjl_stage on the GPU's codes for rows
    whose codes differed inside the band; sign bits must then match outside
    |(S r)_i| < BAND and gamma within 1e-5 relative.

    Returns (fields, stats): fields = {"idx", "norm"[, "sign", "rnorm"]} per
    row -- the GPU's codes and signs (validated, so any difference from the
    oracle's is a legal band choice) and the oracle's fp64 norms and gammas;
    stats counts rows with a band code difference and with a band sign
    difference."""
    c, bnd = (ol.cv, ol.bv) if values else (ol.ck, ol.bk)
    flipped = compare_codes(gpu_idx, enc, bnd, what + " codes")
    np.testing.assert_allclose(gpu_norm, enc["norm"], rtol=2e-6, atol=0, err_msg=what + ": norms")
    fields = {"idx": gpu_idx, "norm": enc["norm"]}
    if "dither" in enc:
        fields["dither"] = enc["dither"]
    stats = {"code_rows": int(flipped.sum()), "sign_rows": 0}
    if gpu_sign is not None:
        sign, rnorm, proj = enc["sign"].copy(), enc["rnorm"].copy(), enc["proj"].copy()
        if flipped.any():
            redo = codec.qjl_stage(enc["u"][flipped], gpu_idx[flipped], ol.R, c, ol.S)
            sign[flipped], rnorm[flipped], proj[flipped] = redo["sign"], redo["rnorm"], redo["proj"]
        sdiff = gpu_sign != sign
        bad = sdiff & ~(np.abs(proj) < BAND)
        assert not bad.any(), f"{what}: {int(bad.sum())} sign bits differ outside the band " \
                              f"(first at {np.argwhere(bad)[0].tolist()})"
        np.testing.assert_allclose(gpu_rnorm, rnorm, rtol=1e-5, atol=1e-6, err_msg=what + ": residual norms")
        fields["sign"] = gpu_sign
        fields["rnorm"] = rnorm
        stats["sign_rows"] = int(sdiff.any(axis=1).sum())
    return fields, stats


def check_values(gpu_idx, gpu_norm, enc, ol, what):
    """Validate the GPU's value codes and norms; return the decode inputs
    (the GPU's validated codes, the oracle's norms) and the count of rows with
    a band code difference."""
    flipped = compare_codes(gpu_idx, enc, ol.bv, what + " codes")
    np.testing.assert_allclose(gpu_norm, enc["norm"], rtol=2e-6, atol=0, err_msg=what + ": norms")
    fields = {"idx": gpu_idx, "norm": enc["norm"]}
    if "dither" in enc:
        fields["dither"] = enc["dither"]
    return fields, int(flipped.sum())


def oracle_cache(kf, vf, B, Hkv, N, d):
    """Decode inputs [B, Hkv, N, ...] from per-row key and value fields."""
    cache = {"k_idx": kf["idx"].reshape(B, Hkv, N, d), "k_norm": kf["norm"].reshape(B, Hkv, N),
             "v_idx": vf["idx"].reshape(B, Hkv, N, d), "v_norm": vf["norm"].reshape(B, Hkv, N)}
    if "sign" in kf:
        cache["k_sign"] = kf["sign"].reshape(B, Hkv, N, d)
        cache["k_rnorm"] = kf["rnorm"].reshape(B, Hkv, N)
    if "sign" in vf:
        cache["v_sign"] = vf["sign"].reshape(B, Hkv, N, d)
        cache["v_rnorm"] = vf["rnorm"].reshape(B, Hkv, N)
    if "dither" in kf:
        cache["k_dither"] = kf["dither"].reshape(B, Hkv, N)
    if "dither" in vf:
        cache["v_dither"] = vf["dither"].reshape(B, Hkv, N)
    return cache


def score_scale(q, R, S, ck, cache, N, G, qjl):
    """Per (b, h, t, key) Cauchy-Schwarz scale of the score."""
    Bn, Hq, Tq, d = q.shape
    qn = np.linalg.norm(q.astype(np.float64), axis=-1)                    # [B,Hq,Tq]
    q1 = np.abs(q.astype(np.float64) @ S.T).sum(axis=-1) if qjl else 0.0  # ||S q||_1
    kc = ck[cache["k_idx"][:, :, :N]]
    if "k_dither" in cache:                                               # dithered variant
        kc = kc + cache["k_dither"][:, :, :N, None]
    cn = np.linalg.norm(kc, axis=-1)                                      # [B,Hkv,N]
    kap = math.sqrt(math.pi / 2) / d
    out = np.empty((Bn, Hq, Tq, N))
    for h in range(Hq):
        g = h // G
        term = qn[:, h, :, None] * cn[:, g, None, :]
        if qjl:
            term = term + cache["k_rnorm"][:, g, None, :N] * kap * q1[:, h, :, None]
        out[:, h] = cache["k_norm"][:, g, None, :N] * term / math.sqrt(d)
    return out


def compare_scores(gpu, ref, scale, what):
    finite = np.isfinite(ref)
    assert np.array_equal(finite, np.isfinite(gpu)), f"{what}: mask pattern differs"
    with np.errstate(invalid="ignore"):
        err = np.abs(np.where(finite, gpu - ref, 0.0)) / np.where(finite, scale, 1.0)
    worst = float(err.max()) if err.size else 0.0
    assert worst <= SCORE_RTOL, f"{what}: score relative error {worst:.3e} > {SCORE_RTOL}"
    return worst


def compare_out(gpu, ref, what, scale=1.0):
    """Max absolute error within OUT_ATOL * scale.  scale is 1 for the
    workloads' inputs (output coordinates of order one); rows of much larger
    norm pass their output scale (fp32 cannot hold 2e-3 absolute at 1e4)."""
    assert np.isfinite(gpu).all(), f"{what}: output not finite"
    err = float(np.abs(gpu - ref).max()) if gpu.size else 0.0
    assert err <= OUT_ATOL * scale, f"{what}: output max abs error {err:.3e} > {OUT_ATOL * scale:.3e}"
    return err


def upload_packed(layer, cfg, packed, S, cap, device="cuda"):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
    K = B.Cache(layer, B.TQ_KEYS, S, cap, arrays={
        "idx": t(packed["k_idx"]), "norm": t(packed["k_norm"]),
        "sign": t(packed["k_sign"]) if cfg.k_qjl else None,
        "rnorm": t(packed["k_rnorm"]) if cfg.k_qjl else None})
    V = B.Cache(layer, B.TQ_VALUES, S, cap, arrays={
        "idx": t(packed["v_idx"]), "norm": t(packed["v_norm"]),
        "sign": t(packed["v_sign"]) if cfg.v_qjl else None,
        "rnorm": t(packed["v_rnorm"]) if cfg.v_qjl else None})
    return K, V


def gpu_codes_key(cache, S, cap, d, bits, rows=None):
    """Unpack the GPU's key codes [S*cap, d] (optionally only some rows)."""
    raw = cache["idx"].cpu().numpy().reshape(S * cap, d * bits // 8)
    if rows is not None:
        raw = raw[rows]
    return codec.unpack_key_codes(raw, bits, d)


def gpu_signs(cache, S, cap, d, rows=None):
    raw = cache["sign"].cpu().numpy().reshape(S * cap, d // 8)
    if rows is not None:
        raw = raw[rows]
    return codec.unpack_key_codes(raw, 1, d) == 1


def gpu_codes_value(cache, S, cap, d, bits):
    return codec.unpack_value_codes(cache["idx"].cpu().numpy(), bits, S, cap, d).reshape(S * cap, d)


def run_quantize_both(cfg, x_np, which, layer=None, olayer=None):
    """Quantize [S, n, d] host input on the GPU (cap = n rounded to 8) and in the oracle."""
    layer = layer or gpu_layer(cfg)
    olayer = olayer or OracleLayer(cfg)
    S, n, d = x_np.shape
    cap = (n + 7) // 8 * 8
    cache = B.Cache(layer, which, S, cap)
    x = torch.from_numpy(x_np).cuda()
    B.quantize_kv(layer, which, x, cache)
    torch.cuda.synchronize()
    c, bnd = (olayer.ck, olayer.bk) if which == B.TQ_KEYS else (olayer.cv, olayer.bv)
    Sm = olayer.S if (cfg.k_qjl if which == B.TQ_KEYS else cfg.v_qjl) else None
    dith = olayer.offsets(which, S, n)
    enc = codec.encode_rows(x_np.reshape(-1, d), olayer.R, c, bnd, Sm, dither=dith)
    if dith is not None:
        enc["dither"] = dith
    return layer, olayer, cache, enc, cap


def quantize_and_check(cfg, xk, xv, layer=None, ol=None, what=""):
    """Quantize K and V rows [S, N, d] (host arrays) on the GPU into caches of
    capacity N rounded up to 8 and in the oracle; validate every GPU field
    (check_keys, check_values) and return (layer, ol, K, V, cache, stats) with
    `cache` the oracle's decode inputs [B, Hkv, N, ...] for those keys."""
    layer = layer or gpu_layer(cfg)
    ol = ol or OracleLayer(cfg)
    _, _, K, ek, cap = run_quantize_both(cfg, xk, B.TQ_KEYS, layer, ol)
    _, _, V, ev, _ = run_quantize_both(cfg, xv, B.TQ_VALUES, layer, ol)
    S, N, d = xk.shape
    rows = np.array([s * cap + t for s in range(S) for t in range(N)], dtype=np.int64)
    kn = K["norm"].cpu().numpy()[rows]
    if cfg.k_qjl:
        kf, st = check_keys(gpu_codes_key(K, S, cap, d, cfg.k_bits, rows), kn, ek, ol, what + " K",
                            gpu_signs(K, S, cap, d, rows), K["rnorm"].cpu().numpy()[rows])
    else:
        kf, st = check_keys(gpu_codes_key(K, S, cap, d, cfg.k_bits, rows), kn, ek, ol, what + " K")
    vidx = gpu_codes_value(V, S, cap, d, cfg.v_bits)[rows]
    vn = V["norm"].cpu().numpy()[rows]
    if cfg.v_qjl:
        vf, vst = check_keys(vidx, vn, ev, ol, what + " V", gpu_signs(V, S, cap, d, rows),
                             V["rnorm"].cpu().numpy()[rows], values=True)
        st["value_rows"], st["value_sign_rows"] = vst["code_rows"], vst["sign_rows"]
    else:
        vf, st["value_rows"] = check_values(vidx, vn, ev, ol, what + " V")
    return layer, ol, K, V, oracle_cache(kf, vf, cfg.B, cfg.Hkv, N, d), st

"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
and the fp64 oracle on the same seeded inputs, and compare them at the
tolerances the method's target states:
  * codes and sign bits bit-exact, except coordinates whose rotated value lies
    within 1e-5 of a boundary (resp. |(S r)_i| < 1e-5), where either adjacent
    code is accepted; a row with such a code difference has a different
    residual, so its sign bits and residual norm are not compared;
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
        self.ck, self.bk = codebook.codebook(cfg.k_bits, cfg.d)
        self.cv, self.bv = codebook.codebook(cfg.v_bits, cfg.d)


def gpu_layer(cfg):
    rot = B.TQ_ROT_HAAR if cfg.rot == "haar" else B.TQ_ROT_HADAMARD
    return B.make_rotation(cfg.d, rot, cfg.layer_seed, cfg.k_bits, cfg.k_qjl, cfg.v_bits)


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


def compare_key_extras(gpu_sign, gpu_rnorm, enc, flipped, what):
    """Check sign bits (exact outside the band) and residual norms of the rows
    whose codes matched.  Returns a boolean per row: True where a sign bit
    differed (legally, inside the band) -- such a key's score differs by
    gamma sqrt(pi/2)/d * 2 |(S q)_i|, so score comparisons leave it out."""
    keep = ~flipped
    sdiff = (gpu_sign != enc["sign"]) & keep[:, None]
    sband = np.abs(enc["proj"]) < BAND
    bad = sdiff & ~sband
    assert not bad.any(), f"{what}: {int(bad.sum())} sign bits differ outside the band"
    np.testing.assert_allclose(gpu_rnorm[keep], enc["rnorm"][keep], rtol=1e-5, atol=1e-6,
                               err_msg=f"{what}: residual norms")
    return sdiff.any(axis=1)


def score_scale(q, R, S, ck, cache, N, G, qjl):
    """Per (b, h, t, key) Cauchy-Schwarz scale of the score."""
    Bn, Hq, Tq, d = q.shape
    qn = np.linalg.norm(q.astype(np.float64), axis=-1)                    # [B,Hq,Tq]
    q1 = np.abs(q.astype(np.float64) @ S.T).sum(axis=-1) if qjl else 0.0  # ||S q||_1
    cn = np.linalg.norm(ck[cache["k_idx"][:, :, :N]], axis=-1)            # [B,Hkv,N]
    kap = math.sqrt(math.pi / 2) / d
    out = np.empty((Bn, Hq, Tq, N))
    for h in range(Hq):
        g = h // G
        term = qn[:, h, :, None] * cn[:, g, None, :]
        if qjl:
            term = term + cache["k_rnorm"][:, g, None, :N] * kap * q1[:, h, :, None]
        out[:, h] = cache["k_norm"][:, g, None, :N] * term / math.sqrt(d)
    return out


def compare_scores(gpu, ref, scale, what, key_mask=None):
    finite = np.isfinite(ref)
    assert np.array_equal(finite, np.isfinite(gpu)), f"{what}: mask pattern differs"
    with np.errstate(invalid="ignore"):
        err = np.abs(np.where(finite, gpu - ref, 0.0)) / np.where(finite, scale, 1.0)
    if key_mask is not None:
        err = err * key_mask
    worst = float(err.max()) if err.size else 0.0
    assert worst <= SCORE_RTOL, f"{what}: score relative error {worst:.3e} > {SCORE_RTOL}"
    return worst


def compare_out(gpu, ref, what):
    err = float(np.abs(gpu - ref).max()) if gpu.size else 0.0
    assert err <= OUT_ATOL, f"{what}: output max abs error {err:.3e} > {OUT_ATOL}"
    return err


def upload_packed(layer, cfg, packed, S, cap, device="cuda"):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
    K = B.Cache(layer, B.TQ_KEYS, S, cap, arrays={
        "idx": t(packed["k_idx"]), "norm": t(packed["k_norm"]),
        "sign": t(packed["k_sign"]) if cfg.k_qjl else None,
        "rnorm": t(packed["k_rnorm"]) if cfg.k_qjl else None})
    V = B.Cache(layer, B.TQ_VALUES, S, cap, arrays={"idx": t(packed["v_idx"]), "norm": t(packed["v_norm"])})
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
    Sm = olayer.S if (which == B.TQ_KEYS and cfg.k_qjl) else None
    enc = codec.encode_rows(x_np.reshape(-1, d), olayer.R, c, bnd, Sm)
    return layer, olayer, cache, enc, cap

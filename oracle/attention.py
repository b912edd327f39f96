"""Decode attention over a TurboQuant-compressed cache (fp64).

[cuTile] listing: the asymmetric score estimator (an MSE inner product plus
a QJL correction term), the attention pipeline (scores, softmax, weighted sum
of values) and its test that scores carry the 1/sqrt(d) scale.  [Mobilint], "Two-Stage Approach": the query
is rotated once, <q, x~> = <Pi q, y~>, so each cached token costs one O(d)
inner product; the QJL term uses S q against the stored signs with the
factor sqrt(pi/2)/d.  Per key t and query q:
    s_t = n_t * ( <R q, c_k[idx_t]> + gamma_t * sqrt(pi/2)/d * <S q, sigma_t> ) / sqrt(d)
(the QJL term only when keys carry it), softmax over the visible keys, and
    out = R^T ( sum_t p_t * nv_t * c_v[idxv_t] )
where the value reconstruction n_v R^T c_v[idx] is summed in the rotated
domain and un-rotated once.

In the dithered randomized-Hadamard variant the cache also holds each
token's offset ("k_dither", "v_dither"): the reconstruction is c[idx] + delta.

Values with QJL (TurboQuant_prod on V; [Mobilint] "Two-Stage Approach",
final reconstruction) carry "v_sign" and "v_rnorm": each value is the
two-stage reconstruction n (R^T c[idx] + sqrt(pi/2)/d gamma S^T sigma) and
the output is the softmax-weighted sum of those rows.

Readings (pages silent; parity unpinned by the pages):
  * grouped-query heads: query head h reads KV head h // (Hq / Hkv);
  * with Tq query tokens and `causal`, query i (0-based) sees keys
    t <= N - Tq + i (the query chunk holds the last Tq positions);
  * masked scores are reported as -inf.
"""
import math

import numpy as np

from . import codec


def unpack_cache(packed: dict, B: int, Hkv: int, cap: int, d: int,
                 k_bits: int, v_bits: int, k_qjl: int, v_qjl: int = 0) -> dict:
    """Packed arrays in the library layout -> unpacked [B, Hkv, cap, ...] fields."""
    S = B * Hkv
    out = {
        "k_idx": codec.unpack_key_codes(packed["k_idx"], k_bits, d).reshape(B, Hkv, cap, d),
        "k_norm": np.asarray(packed["k_norm"], np.float64).reshape(B, Hkv, cap),
        "v_idx": codec.unpack_value_codes(packed["v_idx"], v_bits, S, cap, d).reshape(B, Hkv, cap, d),
        "v_norm": np.asarray(packed["v_norm"], np.float64).reshape(B, Hkv, cap),
    }
    if k_qjl:
        out["k_sign"] = codec.unpack_key_codes(packed["k_sign"], 1, d).reshape(B, Hkv, cap, d) == 1
        out["k_rnorm"] = np.asarray(packed["k_rnorm"], np.float64).reshape(B, Hkv, cap)
    if v_qjl:  # sign rows have the same per-token layout for values as for keys
        out["v_sign"] = codec.unpack_key_codes(packed["v_sign"], 1, d).reshape(B, Hkv, cap, d) == 1
        out["v_rnorm"] = np.asarray(packed["v_rnorm"], np.float64).reshape(B, Hkv, cap)
    return out


def decode(q, R, S, ck, cv, cache: dict, N: int, causal: bool,
           heads=None):
    """q [B, Hq, Tq, d] -> (out [B, Hq, Tq, d], scores [B, Hq, Tq, N]).

    `cache` holds unpacked fields (see unpack_cache) for at least N tokens.
    `heads`, if given, is a list of (b, h) pairs to compute; the others are
    left as NaN (used to sample very large layers one head at a time).
    """
    q = np.asarray(q, dtype=np.float64)
    R = np.asarray(R, dtype=np.float64)
    ck = np.asarray(ck, dtype=np.float64)
    cv = np.asarray(cv, dtype=np.float64)
    B, Hq, Tq, d = q.shape
    Hkv = cache["k_idx"].shape[1]
    G = Hq // Hkv
    qjl = "k_sign" in cache
    kappa = math.sqrt(math.pi / 2.0) / d

    q_rot = q @ R.T                                   # R q for every query row
    q_proj = q @ np.asarray(S, np.float64).T if qjl else None

    out = np.full((B, Hq, Tq, d), np.nan)
    scores = np.full((B, Hq, Tq, N), np.nan)
    todo = heads if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]
    for b, h in todo:
        g = h // G
        kc = ck[cache["k_idx"][b, g, :N]]             # [N, d] centroid values
        if "k_dither" in cache:                       # dithered variant: c[idx] + delta
            kc = kc + cache["k_dither"][b, g, :N][:, None]
        t1 = q_rot[b, h] @ kc.T                       # [Tq, N]
        s = t1
        if qjl:
            sigma = np.where(cache["k_sign"][b, g, :N], 1.0, -1.0)
            t2 = q_proj[b, h] @ sigma.T
            s = t1 + cache["k_rnorm"][b, g, :N][None, :] * kappa * t2
        s = cache["k_norm"][b, g, :N][None, :] * s / math.sqrt(d)
        if causal:
            for i in range(Tq):
                s[i, N - Tq + i + 1:] = -np.inf
        m = s.max(axis=1, keepdims=True)
        p = np.exp(s - m)
        p = p / p.sum(axis=1, keepdims=True)
        if "v_sign" in cache:                         # values with QJL: two-stage rows
            v_hat = codec.reconstruct_prod(cache["v_idx"][b, g, :N], cache["v_norm"][b, g, :N],
                                           cache["v_sign"][b, g, :N], cache["v_rnorm"][b, g, :N],
                                           R, cv, S)
            out[b, h] = p @ v_hat
        else:
            vc = cv[cache["v_idx"][b, g, :N]]
            if "v_dither" in cache:
                vc = vc + cache["v_dither"][b, g, :N][:, None]
            v_rot = cache["v_norm"][b, g, :N][:, None] * vc
            acc = p @ v_rot                           # [Tq, d], rotated domain
            out[b, h] = acc @ R                       # row form of R^T acc
        scores[b, h] = s
    return out, scores

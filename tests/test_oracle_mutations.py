"""Planted mistakes in the oracle must make at least one pin fail.

Each case patches one plausible slip into the oracle (on the CPU only) and
runs the pins that should notice it.  If a pin still passes under the slip,
the pin set has a hole.
"""
import math

import numpy as np
import pytest

import oracle.attention as attention
import oracle.codebook as codebook
import oracle.codec as codec
import oracle.transforms as transforms
from tests import test_oracle_pins as pins


def _fails(fn, *args):
    try:
        fn(*args)
    except AssertionError:
        return True
    return False


def _encode_transposed(x, R, centroids, boundaries, S=None):
    return _orig_encode(x, np.asarray(R).T, centroids, boundaries, S)


def _encode_flipped_signs(x, R, centroids, boundaries, S=None):
    out = _orig_encode(x, R, centroids, boundaries, S)
    if S is not None:
        out["sign"] = ~out["sign"]
    return out


def _encode_ge_tie(x, R, centroids, boundaries, S=None):
    x = np.asarray(x, dtype=np.float64)
    n = np.sqrt((x * x).sum(axis=1))
    u = np.where(n[:, None] > 0, x / np.where(n > 0, n, 1)[:, None], 0.0)
    y = u @ np.asarray(R).T
    idx = (y[..., None] >= np.asarray(boundaries, np.float64)).sum(axis=-1)
    return {"idx": idx, "norm": n, "y": y}


def _reconstruct_prod_without_qjl(idx, norm, sign, rnorm, R, centroids, S):
    """The two-stage reconstruction without its QJL term."""
    return codec.reconstruct_mse(idx, norm, R, centroids)


def _reconstruct_prod_wrong_kappa(idx, norm, sign, rnorm, R, centroids, S):
    d = np.asarray(R).shape[0]
    c = np.asarray(centroids, np.float64)
    sigma = np.where(np.asarray(sign, bool), 1.0, -1.0)
    qjl = (math.pi / 2 / d) * np.asarray(rnorm)[:, None] * (sigma @ S)
    return np.asarray(norm)[:, None] * (c[idx] @ R + qjl)


_orig_encode = codec.encode_rows


def _encode_dither_added(x, R, centroids, boundaries, S=None, dither=None):
    """The offset added before quantizing instead of subtracted."""
    return _orig_encode(x, R, centroids, boundaries, S, None if dither is None else -np.asarray(dither))


def _hadamard_signs_after(d, seed):
    """D H instead of H D: the signs scale the rows of the transform."""
    return transforms.rademacher_signs(d, seed)[:, None] * transforms.sylvester_hadamard(d)


def _beta_wrong_exponent(bits, d, tol=1e-15, max_iter=200000):
    """The exact-law solver with the exponent (d-1)/2 instead of (d-3)/2."""
    return _orig_beta.__wrapped__(bits, d + 2, tol, max_iter)


_orig_beta = codebook.lloyd_max_beta
MODULES = {"codec": codec, "transforms": transforms, "codebook": codebook}


def _decode_variant(mutation):
    orig = attention.decode

    def run(q, R, S, ck, cv, cache, N, causal, heads=None):
        cache = dict(cache)
        if mutation == "drop_qjl":
            cache.pop("k_sign", None)
            cache.pop("k_rnorm", None)
        if mutation == "gqa_modulo":
            Hkv = cache["k_idx"].shape[1]
            B, Hq = q.shape[0], q.shape[1]
            # a slip that maps query head h to KV head h % Hkv
            perm = [h % Hkv for h in range(Hq)]
            G = Hq // Hkv
            order = np.argsort([p * G + i // Hkv for i, p in enumerate(perm)], kind="stable")
            q = q[:, order]
        out, s = orig(q, R, S, ck, cv, cache, N, causal, heads)
        if mutation == "no_sqrt_d":
            d = q.shape[-1]
            s = s * math.sqrt(d)
        if mutation == "no_unrotate":
            out = out @ np.asarray(R).T
        return out, s
    return run


@pytest.mark.parametrize("mutation,patch,checks", [
    ("rotation transposed", ("codec", "encode_rows", _encode_transposed),
     [pins.test_mse_bound_and_monotone, pins.test_encode_matches_nearest_centroid_bruteforce]),
    ("QJL sign flipped", ("codec", "encode_rows", _encode_flipped_signs),
     [pins.test_slopes_mse_only_biased_qjl_unbiased]),
    ("ties to the upper index", ("codec", "encode_rows", _encode_ge_tie),
     [pins.test_zero_row_is_lower_middle_index]),
    ("QJL factor pi/2 instead of sqrt(pi/2)", ("codec", "reconstruct_prod", _reconstruct_prod_wrong_kappa),
     [pins.test_slopes_mse_only_biased_qjl_unbiased, pins.test_unbiased_and_variance_bound,
      pins.test_value_qjl_output_unbiased_over_projections]),
    ("QJL term of the two-stage reconstruction dropped", ("codec", "reconstruct_prod", _reconstruct_prod_without_qjl),
     [pins.test_value_qjl_output_unbiased_over_projections]),
    ("Hadamard signs applied after the transform", ("transforms", "hadamard_rotation", _hadamard_signs_after),
     [lambda: pins.test_hadamard_applies_signs_before_transform(64)]),
    ("dither added instead of subtracted", ("codec", "encode_rows", _encode_dither_added),
     [pins.test_dithered_hadamard_mse_within_the_bound, lambda: pins.test_decode_equals_dense_bruteforce("dither")]),
    ("exact-law exponent (d-1)/2", ("codebook", "lloyd_max_beta", _beta_wrong_exponent),
     [lambda: pins.test_beta_codebook_one_bit_closed_form(64), lambda: pins.test_beta_codebook_d3_is_the_uniform_quantizer(2),
      pins.test_beta_codebook_mse_on_rotated_unit_vectors]),
])
def test_planted_codec_mistake_is_caught(monkeypatch, mutation, patch, checks):
    mod, name, fn = patch
    monkeypatch.setattr(MODULES[mod], name, fn)
    assert any(_fails(check) for check in checks), mutation


@pytest.mark.parametrize("mutation", ["drop_qjl", "no_sqrt_d", "no_unrotate", "gqa_modulo"])
def test_planted_decode_mistake_is_caught(monkeypatch, mutation):
    monkeypatch.setattr(attention, "decode", _decode_variant(mutation))
    assert _fails(pins.test_decode_equals_dense_bruteforce, 1), mutation

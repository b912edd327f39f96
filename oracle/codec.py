"""TurboQuant key/value encoding, bit layouts and reconstruction (fp64).

Encoding of one row x ([Mobilint], sections "Coordinates Become Predictable
After Rotation", "Designing the Optimal Codebook Without Data" and
"Two-Stage Approach"; [cuTile] listing, key and value compression functions, values without
QJL):
  1. n = ||x||_2 is stored; u = x / n (u = 0 when n = 0).
  2. y = R u with R the Haar rotation Pi or the randomized Hadamard H D.
  3. idx_j = #{i : beta_i < y_j} over the sorted float32 boundaries.
  4. The codes are bit-packed.
  5. Keys with QJL only: x_mse = R^T c[idx], residual r = u - x_mse,
     gamma = ||r||_2 is stored with the sign bits sigma_i = sign((S r)_i).
Readings: the residual is taken for the unit vector u (the key norm is
applied once, outside, in the score); sign(0) is +1 (a single bit cannot
hold numpy's sign(0) = 0); norms are stored as float32.

Bit layouts (the pages are silent; contract of this project, pinned only by
the hand-worked examples in tests/golden/):
  * a "stream" is little-endian: bit k of a stream is bit (k mod 8) of byte
    k // 8, and a b-bit code occupies stream bits [p*b, p*b + b) with its
    least significant bit first, p being the code's position in the stream;
  * key codes: one stream per token, positions = coordinates 0..d-1;
    token t of sequence s starts at byte (s*cap + t) * d*b/8;
  * key sign bits: same, with b = 1 and bit value 1 meaning sigma = +1;
  * value codes: tokens are grouped in tiles of 8 (t // 8); one stream per
    tile, position of (coordinate j, token t) = 8*j + (t mod 8), i.e. the
    tile is stored coordinate-major; tile k of sequence s starts at byte
    (s*cap/8 + k) * 8*d*b/8.  `cap` (tokens per sequence) is a multiple of 8.
"""
import math

import numpy as np

from . import rng

KAPPA_NUM = math.sqrt(math.pi / 2.0)      # QJL correction sqrt(pi/2); divided by d


# ---------------------------------------------------------------- encoding --

def dither_offsets(seed: int, which: str, seq, t, centroids):
    """Per-token offsets of the dithered randomized-Hadamard variant
    (thelatestinai.com paper page 2606.10458, third abstract: HD, then a random
    scalar offset subtracted before quantizing).  Readings (the abstract fixes
    neither): one offset per token, the same for all its coordinates, uniform
    over the spacing of the two central centroids,
        delta = (c[L/2] - c[L/2 - 1]) * (u - 1/2),
    u the uniform of output seq * 2^32 + t + 1 of the layer's stream with tag
    3 (keys) or 4 (values), so the decoder regenerates it (nothing is stored).
    seq, t: integer arrays of equal shape."""
    c = np.asarray(centroids, dtype=np.float64)
    L = c.size
    width = c[L // 2] - c[L // 2 - 1]
    tag = rng.TAG_DITHER_K if which == "K" else rng.TAG_DITHER_V
    k = np.asarray(seq, dtype=np.int64) * (1 << 32) + np.asarray(t, dtype=np.int64) + 1
    return width * (rng.uniform_at(seed, tag, k) - 0.5)


def encode_rows(x, R, centroids, boundaries, S=None, dither=None) -> dict:
    """Encode rows of x [rows, d].  Returns unpacked fields plus diagnostics.

    idx [rows, d] int64; norm [rows] fp64; u [rows, d] the unit rows; y
    [rows, d] the values compared with the boundaries: the rotated unit
    vectors, minus the per-row offsets `dither` when given (dithered
    variant, keys without QJL and values); with S: sign [rows, d] bool (True
    means +1), rnorm [rows] fp64 and proj [rows, d] = S r (see qjl_stage).
    """
    x = np.asarray(x, dtype=np.float64)
    R = np.asarray(R, dtype=np.float64)
    c = np.asarray(centroids, dtype=np.float64)
    beta = np.asarray(boundaries, dtype=np.float64)

    norm = np.sqrt(np.sum(x * x, axis=1))
    safe = np.where(norm > 0.0, norm, 1.0)
    u = np.where(norm[:, None] > 0.0, x / safe[:, None], 0.0)
    y = u @ R.T                                   # row form of y = R u
    if dither is not None:                        # dithered variant: quantize y - delta
        y = y - np.asarray(dither, dtype=np.float64)[:, None]
    idx = (y[..., None] > beta).sum(axis=-1)      # #{i : beta_i < y_j}
    out = {"idx": idx, "norm": norm, "y": y, "u": u}
    if S is not None:
        out.update(qjl_stage(u, idx, R, c, S))
    return out


def qjl_stage(u, idx, R, centroids, S) -> dict:
    """Stage 2 of [Mobilint], "Two-Stage Approach", for unit rows u [rows, d]
    whose stage-1 codes are idx: residual r = u - R^T c[idx], gamma = ||r||_2,
    sign bits sigma_i = sign((S r)_i) with sign(0) = +1.

    Returns sign [rows, d] bool (True means +1), rnorm [rows] and proj = S r
    [rows, d].  Any codes may be given, so a row can be re-derived from codes
    other than its nearest-centroid ones."""
    c = np.asarray(centroids, dtype=np.float64)
    x_mse = c[np.asarray(idx)] @ np.asarray(R, dtype=np.float64)   # row form of R^T c[idx]
    r = np.asarray(u, dtype=np.float64) - x_mse
    proj = r @ np.asarray(S, dtype=np.float64).T
    return {"sign": proj >= 0.0, "rnorm": np.sqrt(np.sum(r * r, axis=1)), "proj": proj}


def reconstruct_mse(idx, norm, R, centroids, dither=None) -> np.ndarray:
    """x_hat = n * R^T c[idx] ([cuTile] listing, decompression function:
    centroid lookup, inverse rotation, norm rescale); with per-row `dither`,
    x_hat = n * R^T (c[idx] + delta) (the offset added back)."""
    c = np.asarray(centroids, dtype=np.float64)
    yhat = c[idx]
    if dither is not None:
        yhat = yhat + np.asarray(dither, dtype=np.float64)[:, None]
    return np.asarray(norm, dtype=np.float64)[:, None] * (yhat @ np.asarray(R, np.float64))


def reconstruct_prod(idx, norm, sign, rnorm, R, centroids, S) -> np.ndarray:
    """Two-stage reconstruction x_hat = n * (R^T c[idx] + sqrt(pi/2)/d * gamma * S^T sigma)
    ([Mobilint], "Two-Stage Approach", final reconstruction)."""
    d = np.asarray(R).shape[0]
    c = np.asarray(centroids, dtype=np.float64)
    sigma = np.where(np.asarray(sign, bool), 1.0, -1.0)
    mse = c[idx] @ np.asarray(R, np.float64)
    qjl = (KAPPA_NUM / d) * np.asarray(rnorm, np.float64)[:, None] * (sigma @ np.asarray(S, np.float64))
    return np.asarray(norm, dtype=np.float64)[:, None] * (mse + qjl)


# ------------------------------------------------------------- bit streams --

def pack_stream(codes, bits: int) -> np.ndarray:
    """Little-endian packing of a 1-D sequence of b-bit codes into bytes."""
    codes = np.asarray(codes, dtype=np.int64).reshape(-1)
    if codes.size * bits % 8:
        raise ValueError("stream length must be a whole number of bytes")
    bit = (codes[:, None] >> np.arange(bits)[None, :]) & 1      # LSB first
    bit = bit.reshape(-1, 8)
    return (bit << np.arange(8)[None, :]).sum(axis=1).astype(np.uint8)


def unpack_stream(data, bits: int, count: int) -> np.ndarray:
    data = np.asarray(data, dtype=np.uint8).reshape(-1)
    bit = (data[:, None].astype(np.int64) >> np.arange(8)[None, :]) & 1
    bit = bit.reshape(-1)[: count * bits].reshape(count, bits)
    return (bit << np.arange(bits)[None, :]).sum(axis=1)


def pack_key_codes(idx, bits: int) -> np.ndarray:
    """[rows, d] codes -> [rows, d*b/8] bytes, one stream per token."""
    idx = np.asarray(idx, dtype=np.int64)
    rows, d = idx.shape
    return pack_stream(idx.reshape(-1), bits).reshape(rows, d * bits // 8)


def unpack_key_codes(data, bits: int, d: int) -> np.ndarray:
    data = np.asarray(data, dtype=np.uint8).reshape(-1, d * bits // 8)
    return unpack_stream(data, bits, data.shape[0] * d).reshape(-1, d)


def pack_value_codes(idx, bits: int) -> np.ndarray:
    """[S, cap, d] codes -> [S, cap/8, d*b] bytes, 8-token tiles stored coordinate-major."""
    idx = np.asarray(idx, dtype=np.int64)
    S, cap, d = idx.shape
    if cap % 8:
        raise ValueError("capacity must be a multiple of 8")
    tiles = idx.reshape(S, cap // 8, 8, d).transpose(0, 1, 3, 2)   # [S, tile, j, t]: position 8*j + t
    return pack_stream(tiles.reshape(-1), bits).reshape(S, cap // 8, d * bits)


def unpack_value_codes(data, bits: int, S: int, cap: int, d: int) -> np.ndarray:
    data = np.asarray(data, dtype=np.uint8).reshape(-1)
    tiles = unpack_stream(data, bits, S * cap * d).reshape(S, cap // 8, d, 8)
    return tiles.transpose(0, 1, 3, 2).reshape(S, cap, d)


# --------------------------------------------------------- whole tensors --

def encode_cache(x, R, centroids, boundaries, bits: int, S=None, layout: str = "key") -> dict:
    """Encode a tensor [S, cap, d] (rows beyond the valid length may be anything)
    and return packed arrays in the library's layout plus unpacked fields."""
    x = np.asarray(x)
    Sq, cap, d = x.shape
    enc = encode_rows(x.reshape(-1, d), R, centroids, boundaries, S)
    idx = enc["idx"].reshape(Sq, cap, d)
    packed = {
        "idx": (pack_key_codes(idx.reshape(-1, d), bits) if layout == "key"
                else pack_value_codes(idx, bits)).reshape(-1),
        "norm": enc["norm"].astype(np.float32),
    }
    if S is not None:
        packed["sign"] = pack_key_codes(enc["sign"].astype(np.int64), 1).reshape(-1)
        packed["rnorm"] = enc["rnorm"].astype(np.float32)
    packed["enc"] = enc
    return packed

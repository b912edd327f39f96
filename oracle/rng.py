"""Counter-based random stream used to draw the layer's random matrices.

The pages fix only the distributions: a Gaussian matrix whose QR factor is
the Haar rotation, a Gaussian projection S, and random +-1 signs D for the
randomized Hadamard transform ([Mobilint], sections "How JL Matrices Evolved"
and "Two-Stage Approach"; [cuTile] listing, the QJL projection and Haar
rotation functions).  Which generator produces them is not on the pages, so this
stream is a contract of this project (parity unpinned by the pages).

Definition (SplitMix64, Steele, Lea and Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014, with the published 64-bit finaliser):
  start   s0 = seed XOR (tag * 0xD1B54A32D192ED03)        (mod 2^64)
  output  k (k = 1, 2, ...):  z = s0 + k * 0x9E3779B97F4A7C15
          z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9
          z = (z ^ (z >> 27)) * 0x94D049BB133111EB
          z =  z ^ (z >> 31)
  uniform u = ((z >> 11) + 0.5) * 2^-53, in (0, 1)
  normals by Box-Muller on consecutive uniforms (u1, u2):
          rho = sqrt(-2 ln u1);  z0 = rho cos(2 pi u2);  z1 = rho sin(2 pi u2)
  matrices are filled row-major, element 2p from z0 and 2p+1 from z1 of pair p.
  signs:  D_j = +1 when the top bit of output j+1 is 0, else -1.
Tags: 0 = Gaussian matrix for the Haar rotation, 1 = projection S, 2 = signs D,
3 / 4 = per-token dither offsets of keys / values (output number
seq * 2^32 + t + 1 for token t of sequence seq).
"""
import math

MASK64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15
TAG_MUL = 0xD1B54A32D192ED03

TAG_HAAR, TAG_PROJ, TAG_SIGNS = 0, 1, 2
TAG_DITHER_K, TAG_DITHER_V = 3, 4


def _mix(z: int) -> int:
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


def stream(seed: int, tag: int, count: int):
    """The first `count` 64-bit outputs of stream (seed, tag)."""
    s0 = (seed ^ ((tag * TAG_MUL) & MASK64)) & MASK64
    return [_mix((s0 + k * GAMMA) & MASK64) for k in range(1, count + 1)]


def uniforms(seed: int, tag: int, count: int):
    return [((z >> 11) + 0.5) * 2.0 ** -53 for z in stream(seed, tag, count)]


def normals(seed: int, tag: int, count: int):
    """`count` standard normals by Box-Muller, in stream order."""
    pairs = (count + 1) // 2
    u = uniforms(seed, tag, 2 * pairs)
    out = []
    for p in range(pairs):
        rho = math.sqrt(-2.0 * math.log(u[2 * p]))
        ang = 2.0 * math.pi * u[2 * p + 1]
        out.append(rho * math.cos(ang))
        out.append(rho * math.sin(ang))
    return out[:count]


def signs(seed: int, tag: int, count: int):
    return [1 if (z >> 63) == 0 else -1 for z in stream(seed, tag, count)]


def uniform_at(seed: int, tag: int, k):
    """Uniform (0, 1) of output number k (k >= 1, scalar or integer array) of
    stream (seed, tag): counter-based access to the same stream."""
    import numpy as np
    s0 = (seed ^ ((tag * TAG_MUL) & MASK64)) & MASK64
    ks = np.asarray(k, dtype=object)
    z = np.vectorize(lambda kk: _mix((s0 + int(kk) * GAMMA) & MASK64), otypes=[object])(ks)
    return np.vectorize(lambda zz: ((zz >> 11) + 0.5) * 2.0 ** -53, otypes=[float])(z).astype(np.float64)

"""Random rotation, QJL projection and randomized Hadamard transform (fp64).

* Haar rotation Pi: the Q factor of the QR factorisation of a d x d standard
  Gaussian matrix ([cuTile] listing, Haar rotation function; [Mobilint], "Two-Stage Approach", where the
  sample code rotates by the QR factor).  Reading: the columns of Q are signed
  so that diag(R) > 0, which makes Q unique and exactly Haar distributed.
  A unit vector u is rotated as y = Pi u.
* QJL projection S: a d x d matrix of i.i.d. N(0,1) entries, m = d rows,
  unnormalised ([Mobilint], "QJL" estimator and "Two-Stage Approach",
  Stage 2 equation with the factor sqrt(pi/2)/d).
* Randomized Hadamard HD: D is a diagonal of random signs and H the
  normalised Sylvester Walsh-Hadamard matrix ([Mobilint], "How JL Matrices
  Evolved": f(x) = P H D x, with H_2 and H_4 printed there).  Sylvester order
  means H[i, j] = (-1)^popcount(i & j) / sqrt(d).  The rotation is y = H D u
  and its inverse D H y.
"""
import numpy as np

from . import rng


def haar_rotation(d: int, seed: int) -> np.ndarray:
    g = np.array(rng.normals(seed, rng.TAG_HAAR, d * d), dtype=np.float64).reshape(d, d)
    q, r = np.linalg.qr(g)
    # Sign each column so the triangular factor has a positive diagonal.
    return q * np.sign(np.diag(r))[None, :]


def gaussian_projection(d: int, seed: int) -> np.ndarray:
    return np.array(rng.normals(seed, rng.TAG_PROJ, d * d), dtype=np.float64).reshape(d, d)


def rademacher_signs(d: int, seed: int) -> np.ndarray:
    return np.array(rng.signs(seed, rng.TAG_SIGNS, d), dtype=np.float64)


def sylvester_hadamard(d: int) -> np.ndarray:
    """Normalised Walsh-Hadamard matrix, entry (i, j) = (-1)^popcount(i&j)/sqrt(d)."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.empty((d, d))
    for i in range(d):
        for j in range(d):
            h[i, j] = -1.0 if bin(i & j).count("1") % 2 else 1.0
    return h / np.sqrt(d)


def hadamard_rotation(d: int, seed: int) -> np.ndarray:
    """The matrix H D, so that y = (H D) u."""
    return sylvester_hadamard(d) * rademacher_signs(d, seed)[None, :]


def rotation(d: int, kind: str, seed: int) -> np.ndarray:
    if kind == "haar":
        return haar_rotation(d, seed)
    if kind == "hadamard":
        return hadamard_rotation(d, seed)
    raise ValueError(kind)

"""Lloyd-Max scalar codebook for the rotated coordinate law (fp64 solver).

[Mobilint], section "Coordinates Become Predictable After Rotation": each
coordinate of a rotated unit vector follows a Beta law that tends to
N(0, 1/d).  Section "Designing the Optimal Codebook Without Data": the
optimal b-bit scalar quantizer is found by Lloyd-Max -- boundaries at the
midpoints of adjacent centroids, each centroid the conditional mean of its
region under the density, repeated to convergence, with the integrals done
numerically rather than from samples.  [cuTile] listing: the codebook is
returned as sorted float32 centroids (2^b) and boundaries (2^b - 1).

Readings taken here:
* the law is N(0, 1/d) (the Gaussian limit the pages use for the codebook
  sample code and for every printed value);
* the solver runs on N(0,1) with exact conditional means
    E[X | a < X < b] = (phi(a) - phi(b)) / (Phi(b) - Phi(a)),
  starting from linspace(-2, 2, 2^b) as the page's sample version does, and
  stops when no centroid moves by more than 1e-15;
* the converged centroids are made exactly symmetric, scaled by 1/sqrt(d) in
  fp64 and rounded to float32; boundaries are the fp64 midpoints rounded to
  float32 (so the middle boundary is exactly 0).
Assigning y to #{i : boundary_i < y} is the nearest-centroid rule the page
states for the boundary update (ties go to the lower index).
"""
import functools
import math

import numpy as np

SQRT2 = math.sqrt(2.0)


def _pdf(x: float) -> float:
    if math.isinf(x):
        return 0.0
    return math.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)


def _mass(a: float, b: float) -> float:
    """P(a < X < b) for X ~ N(0,1), using the upper tail when a >= 0."""
    if a >= 0.0:
        return 0.5 * math.erfc(a / SQRT2) - 0.5 * math.erfc(b / SQRT2)
    return 0.5 * math.erfc(-b / SQRT2) - 0.5 * math.erfc(-a / SQRT2)


def lloyd_max_normal(bits: int, tol: float = 1e-15, max_iter: int = 200000):
    """Centroids (ascending, fp64) of the b-bit Lloyd-Max quantizer of N(0,1)."""
    levels = 1 << bits
    c = [-2.0 + 4.0 * i / (levels - 1) for i in range(levels)]
    for _ in range(max_iter):
        edges = [-math.inf] + [(c[i] + c[i + 1]) / 2.0 for i in range(levels - 1)] + [math.inf]
        new = [(_pdf(edges[i]) - _pdf(edges[i + 1])) / _mass(edges[i], edges[i + 1])
               for i in range(levels)]
        moved = max(abs(x - y) for x, y in zip(c, new))
        c = new
        if moved <= tol:
            break
    half = [(c[levels - 1 - i] - c[i]) / 2.0 for i in range(levels)]
    return np.array([-half[i] for i in range(levels)], dtype=np.float64)


@functools.lru_cache(maxsize=None)
def lloyd_max_beta(bits: int, d: int, tol: float = 1e-15, max_iter: int = 200000):
    """Centroids (ascending, fp64) of the b-bit Lloyd-Max quantizer of the exact
    coordinate law of a rotated unit vector ([Mobilint], "Coordinates Become
    Predictable After Rotation"): f(t) proportional to (1 - t^2)^((d-3)/2) on
    [-1, 1], i.e. (X + 1) / 2 ~ Beta((d-1)/2, (d-1)/2).

    Same iteration as for the Gaussian ("Designing the Optimal Codebook Without
    Data": midpoint boundaries, conditional-mean centroids, integrals done
    numerically): with a = (d-3)/2,
      P(lo < X < hi)   = I_{(1+hi)/2}(a+1, a+1) - I_{(1+lo)/2}(a+1, a+1)
                         (regularized incomplete beta, scipy.special.betainc),
      E[X; lo < X < hi] = ((1-lo^2)^(a+1) - (1-hi^2)^(a+1)) / (2 (a+1) Z),
      Z = B(1/2, a+1) = the integral of (1 - t^2)^a over [-1, 1].
    Starts from the Gaussian start scaled to the coordinate spread 1/sqrt(d);
    stops when no centroid moves by more than tol; then made exactly symmetric.
    d >= 3."""
    from scipy import special
    if d < 3:
        raise ValueError("the coordinate law needs d >= 3")
    levels = 1 << bits
    a = (d - 3) / 2.0
    Z = special.beta(0.5, a + 1.0)
    # Evenly spaced start over [-2, 2] standard deviations (1/sqrt(d)), kept
    # inside the support so that every cell starts with positive mass.
    top = min(2.0 / math.sqrt(d), 1.0 - 1.0 / levels)
    c = [-top + 2.0 * top * i / (levels - 1) for i in range(levels)]

    def mass(lo, hi):
        return float(special.betainc(a + 1.0, a + 1.0, (1.0 + hi) / 2.0)
                     - special.betainc(a + 1.0, a + 1.0, (1.0 + lo) / 2.0))

    def first_moment(lo, hi):
        return ((1.0 - lo * lo) ** (a + 1.0) - (1.0 - hi * hi) ** (a + 1.0)) / (2.0 * (a + 1.0) * Z)

    for _ in range(max_iter):
        edges = [-1.0] + [(c[i] + c[i + 1]) / 2.0 for i in range(levels - 1)] + [1.0]
        new = [first_moment(edges[i], edges[i + 1]) / mass(edges[i], edges[i + 1]) for i in range(levels)]
        moved = max(abs(x - y) for x, y in zip(c, new))
        c = new
        if moved <= tol:
            break
    half = [(c[levels - 1 - i] - c[i]) / 2.0 for i in range(levels)]
    out = np.array([-half[i] for i in range(levels)], dtype=np.float64)
    out.setflags(write=False)
    return out


def beta_mse(centroids, d: int) -> float:
    """Expected squared error of a codebook (in the coordinate's own units) on
    the exact coordinate law of dimension d: the sum over the nearest-centroid
    cells of E[X^2; cell] - 2 c_i E[X; cell] + c_i^2 P(cell), each moment by
    numerical quadrature of (1 - t^2)^((d-3)/2) / Z."""
    from scipy import integrate, special
    a = (d - 3) / 2.0
    Z = special.beta(0.5, a + 1.0)
    f = lambda t: (1.0 - t * t) ** a / Z
    c = [float(v) for v in centroids]
    edges = [-1.0] + [(c[i] + c[i + 1]) / 2.0 for i in range(len(c) - 1)] + [1.0]
    total = 0.0
    for i, ci in enumerate(c):
        lo, hi = edges[i], edges[i + 1]
        m0 = integrate.quad(f, lo, hi, epsabs=1e-15, epsrel=1e-13, limit=200)[0]
        m1 = integrate.quad(lambda t: t * f(t), lo, hi, epsabs=1e-15, epsrel=1e-13, limit=200)[0]
        m2 = integrate.quad(lambda t: t * t * f(t), lo, hi, epsabs=1e-15, epsrel=1e-13, limit=200)[0]
        total += m2 - 2.0 * ci * m1 + ci * ci * m0
    return total


def codebook(bits: int, d: int, law: str = "gaussian"):
    """(centroids float32 [2^b], boundaries float32 [2^b - 1]) for the
    coordinate law: "gaussian" (N(0, 1/d), the default) or "beta" (the exact
    law of lloyd_max_beta)."""
    if law == "gaussian":
        c = lloyd_max_normal(bits) / math.sqrt(d)
    elif law == "beta":
        c = lloyd_max_beta(bits, d)
    else:
        raise ValueError(law)
    mids = (c[:-1] + c[1:]) / 2.0
    return c.astype(np.float32), mids.astype(np.float32)


def quantize_scalar(y, boundaries) -> np.ndarray:
    """Index #{i : boundary_i < y}: the nearest centroid, ties to the lower index."""
    y = np.asarray(y, dtype=np.float64)
    b = np.asarray(boundaries, dtype=np.float64)
    return (y[..., None] > b).sum(axis=-1)


def normal_mse(centroids_unit) -> float:
    """Expected squared error of a codebook (given for N(0,1)) on X ~ N(0,1).

    E[(X - c(X))^2] = 1 - sum_i c_i^2 P(region_i) when every c_i is the
    conditional mean of its region (cross term E[X c(X)] = E[c(X)^2]).
    Written out in full here instead: sum over regions of
    E[X^2; region] - 2 c_i E[X; region] + c_i^2 P(region).
    """
    c = [float(v) for v in centroids_unit]
    edges = [-math.inf] + [(c[i] + c[i + 1]) / 2.0 for i in range(len(c) - 1)] + [math.inf]
    total = 0.0
    for i, ci in enumerate(c):
        a, b = edges[i], edges[i + 1]
        p = _mass(a, b)
        m1 = _pdf(a) - _pdf(b)                               # E[X; a<X<b]
        m2 = p + (a * _pdf(a) if not math.isinf(a) else 0.0) \
            - (b * _pdf(b) if not math.isinf(b) else 0.0)    # E[X^2; a<X<b]
        total += m2 - 2.0 * ci * m1 + ci * ci * p
    return total

"""Pins of the fp64 oracle to what the pages and the mathematics fix.

Nothing here compares the oracle with itself: each test checks it against a
value printed on the pages, a closed form, a textbook table, a library
routine for a special case, an invariant, or brute force on tiny inputs.

Parity status per oracle function:
  rng.*                 SplitMix64 published outputs; Box-Muller identity.
                        (Which generator is used: parity unpinned by the pages.)
  transforms.haar_*     orthogonality, R-factor sign rule, Haar law (KS).
  transforms.sylvester  scipy.linalg.hadamard, printed H_4, 1/sqrt(d) spread.
  transforms.hadamard_rotation  signs before the transform (H D, not D H):
                        D e_k -> column k of H.
  codebook.*            printed 1-/2-bit codebooks and MSEs, Max (1960) table,
                        conditional-mean fixed point by quadrature,
                        Panter-Dite bound, monotone in b.
  codebook.lloyd_max_beta  d = 3 uniform quantizer, b = 1 closed form,
                        fixed point by quadrature, optimal against the
                        Gaussian codebook on its law, tends to the Gaussian
                        codebook as 1/d, MSE on Haar-rotated unit vectors.
  codec.encode_rows     nearest-centroid brute force, centroid round trip,
                        2/pi bias at b=1, slope 1-D_mse (MSE only) and 1 (QJL),
                        unbiasedness, variance bound.
  codec.pack_*          hand-worked bytes in tests/golden/bit_layouts.txt.
  attention.decode      estimator identity s = <q, x_hat>/sqrt(d), dense
                        softmax brute force (also dithered), N=1, identical
                        keys, retrieval, causal alignment, score error falls
                        with bits.
  codec.dither_offsets  uniform over the central centroid spacing, K / V and
                        sequences independent; dithered HD MSE within the
                        pi sqrt(3)/2 4^-b bound and decreasing in b; the offset
                        moves the reconstruction only along D e_0.
"""
import math
import os

import numpy as np
import pytest
from scipy import integrate, stats
from scipy.linalg import hadamard as scipy_hadamard

from oracle import attention, codebook, codec, rng, transforms

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
PANTER_DITE = math.sqrt(3.0) * math.pi / 2.0


def _golden_lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


def _random_rotation(rs, d):
    q, r = np.linalg.qr(rs.standard_normal((d, d)))
    return q * np.sign(np.diag(r))


def _unit_rows(rs, n, d):
    x = rs.standard_normal((n, d))
    return x / np.linalg.norm(x, axis=1, keepdims=True)


# ------------------------------------------------------------------ rng --

def test_splitmix64_published_outputs():
    want = [int(v, 16) for _, v in _golden_lines("splitmix64.txt")]
    assert rng.stream(0, 0, 3) == want


def test_stream_tag_and_counter():
    # Output k of stream (seed, tag) is the finaliser applied to s0 + k*gamma:
    # stream (seed=g*5, tag=0) starts 5 outputs further along stream (0, 0).
    g = rng.GAMMA
    seed = (5 * g) & rng.MASK64
    assert rng.stream(seed, 0, 3) == rng.stream(0, 0, 8)[5:8]
    assert rng.stream(7, 1, 4) != rng.stream(7, 2, 4)


def test_box_muller_identity_and_moments():
    u = rng.uniforms(11, 1, 2000)
    z = rng.normals(11, 1, 2000)
    for p in range(1000):
        assert z[2 * p] ** 2 + z[2 * p + 1] ** 2 == pytest.approx(-2 * math.log(u[2 * p]), rel=1e-12)
    big = np.array(rng.normals(3, 0, 100000))
    assert abs(big.mean()) < 4 / math.sqrt(1e5)
    assert abs(big.var() - 1) < 4 * math.sqrt(2 / 1e5)
    assert stats.kstest(big, "norm").pvalue > 1e-3


def test_signs_balanced():
    s = np.array(rng.signs(5, 2, 20000))
    assert set(np.unique(s)) == {-1, 1}
    assert abs(s.mean()) < 4 / math.sqrt(2e4)


# ------------------------------------------------------------ rotations --

@pytest.mark.parametrize("d", [8, 64, 128])
def test_haar_orthogonal_and_sign_rule(d):
    P = transforms.haar_rotation(d, seed=3)
    assert np.abs(P.T @ P - np.eye(d)).max() < 1e-13
    # Pi is the Q of G = Q R with diag(R) > 0: R = Q^T G must be upper
    # triangular with a positive diagonal.
    G = np.array(rng.normals(3, rng.TAG_HAAR, d * d)).reshape(d, d)
    R = P.T @ G
    assert np.abs(np.tril(R, -1)).max() < 1e-10 * np.abs(R).max()
    assert (np.diag(R) > 0).all()


def test_haar_column_is_uniform_on_sphere():
    # [Mobilint], "Coordinates Become Predictable After Rotation": a coordinate
    # of a random rotation of a unit vector satisfies (x+1)/2 ~ Beta((d-1)/2, (d-1)/2).
    d, trials = 16, 600
    coords = [transforms.haar_rotation(d, seed=1000 + t)[2, 0] for t in range(trials)]
    a = (d - 1) / 2
    assert stats.kstest((np.array(coords) + 1) / 2, stats.beta(a, a).cdf).pvalue > 1e-3


@pytest.mark.parametrize("d", [2, 4, 16, 128, 256])
def test_sylvester_matches_library(d):
    assert np.array_equal(transforms.sylvester_hadamard(d), scipy_hadamard(d) / np.sqrt(d))


def test_hadamard_printed_h4_and_involution():
    h4 = np.array([[1, 1, 1, 1], [1, -1, 1, -1], [1, 1, -1, -1], [1, -1, -1, 1]]) / 2.0
    assert np.array_equal(transforms.sylvester_hadamard(4), h4)
    H = transforms.sylvester_hadamard(128)
    assert np.abs(H @ H - np.eye(128)).max() < 1e-14


def test_hadamard_spreads_one_hot():
    # [Mobilint] sanity check: a one-hot input ends with max/norm 0.088 at d=128;
    # exactly 1/sqrt(d) for every coordinate.
    d = 128
    HD = transforms.hadamard_rotation(d, seed=9)
    y = HD @ np.eye(d)[0]
    assert np.allclose(np.abs(y), 1 / np.sqrt(d))
    assert round(float(np.abs(y).max()), 3) == 0.088
    assert np.abs(HD.T @ HD - np.eye(d)).max() < 1e-14


@pytest.mark.parametrize("d", [16, 64, 256])
def test_hadamard_applies_signs_before_transform(d):
    # [Mobilint], "How JL Matrices Evolved": f(x) = P H D x, the random signs act
    # on the input before the transform.  Since D D = I, the input D e_k must
    # come out as column k of H (a Walsh function), and D 1 / sqrt(d) as e_0.
    # With the signs applied after the transform (D H) neither holds unless
    # every sign is equal, which the seed below rules out.
    seed = 21
    D = np.array(rng.signs(seed, rng.TAG_SIGNS, d), dtype=np.float64)
    assert 0 < (D > 0).sum() < d
    HD = transforms.hadamard_rotation(d, seed)
    H = scipy_hadamard(d) / np.sqrt(d)
    assert np.allclose(HD @ (D / np.sqrt(d)), np.eye(d)[0], atol=1e-14)
    for k in (0, 1, d // 2 + 3, d - 1):
        assert np.allclose(HD @ (D * np.eye(d)[k]), H[:, k], atol=1e-14)


def test_fwht_op_count_at_128():
    # [Mobilint], "Running TurboQuant on NPUs": 7 stages x 64 butterflies.  A
    # butterfly is one add and one subtract: 896 add/subs, "roughly 900".
    d = 128
    stages = int(math.log2(d))
    assert stages == 7 and stages * (d // 2) * 2 == 896


# ------------------------------------------------------------- codebook --

@pytest.mark.parametrize("line", _golden_lines("lloyd_max_normal.txt"), ids=lambda l: "b" + l[0])
def test_codebook_printed_and_textbook_values(line):
    bits, tol_c, tol_mse, mse = int(line[0]), float(line[1]), float(line[2]), float(line[3])
    want = np.array([float(v) for v in line[4:]])
    c = codebook.lloyd_max_normal(bits)
    half = c[len(c) // 2:]
    assert np.abs(half - want).max() <= tol_c
    assert codebook.normal_mse(c) == pytest.approx(mse, rel=tol_mse)


def test_one_bit_closed_form():
    for d in (64, 128, 256):
        c, beta = codebook.codebook(1, d)
        assert c[1] == np.float32(math.sqrt(2 / (math.pi * d)))
        assert c[0] == -c[1] and beta[0] == 0.0


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_codebook_fixed_point_by_quadrature(bits):
    # Each centroid is the conditional mean of its region and each boundary the
    # midpoint, checked with numerical integration instead of the closed form.
    c = codebook.lloyd_max_normal(bits)
    edges = [-np.inf] + list((c[:-1] + c[1:]) / 2) + [np.inf]
    for i, ci in enumerate(c):
        a, b = edges[i], edges[i + 1]
        m0 = integrate.quad(stats.norm.pdf, a, b, epsabs=1e-14)[0]
        m1 = integrate.quad(lambda x: x * stats.norm.pdf(x), a, b, epsabs=1e-14)[0]
        assert m1 / m0 == pytest.approx(ci, abs=1e-9)
    # MSE by quadrature equals the closed form sum.
    q = sum(integrate.quad(lambda x, ci=ci: (x - ci) ** 2 * stats.norm.pdf(x),
                           edges[i], edges[i + 1], epsabs=1e-14)[0] for i, ci in enumerate(c))
    assert codebook.normal_mse(c) == pytest.approx(q, rel=1e-9)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_codebook_shape_sorted_symmetric(d):
    for bits in (1, 2, 3, 4):
        c, beta = codebook.codebook(bits, d)
        assert c.dtype == np.float32 and beta.dtype == np.float32
        assert c.shape == (2 ** bits,) and beta.shape == (2 ** bits - 1,)
        assert (np.diff(c) > 0).all() and (np.diff(beta) > 0).all()
        assert np.array_equal(c, -c[::-1]) and np.array_equal(beta, -beta[::-1])
        assert beta[len(beta) // 2] == 0.0
        # boundaries lie between their centroids
        assert ((c[:-1] < beta) & (beta < c[1:])).all()


def test_mse_bound_and_monotone():
    # [cuTile] tests: per-vector MSE <= sqrt(3)*pi/2 * 4^-b, strictly lower
    # with more bits; [Mobilint] Panter-Dite bound.  Reading: the bound holds
    # for the expectation over vectors, so the mean is tested.
    exact = [codebook.normal_mse(codebook.lloyd_max_normal(b)) for b in (1, 2, 3, 4)]
    for b, e in zip((1, 2, 3, 4), exact):
        assert e <= PANTER_DITE * 4.0 ** -b
    assert all(exact[i + 1] < exact[i] for i in range(3))
    rs = np.random.default_rng(0)
    d, n = 128, 3000
    u = _unit_rows(rs, n, d)
    P = _random_rotation(rs, d)
    means = []
    for b in (1, 2, 3, 4):
        c, beta = codebook.codebook(b, d)
        enc = codec.encode_rows(u, P, c, beta)
        xh = codec.reconstruct_mse(enc["idx"], enc["norm"], P, c)
        mse = ((xh - u) ** 2).sum(axis=1)
        means.append(mse.mean())
        assert mse.mean() <= PANTER_DITE * 4.0 ** -b
        assert mse.mean() == pytest.approx(exact[b - 1], rel=0.05)
    assert all(means[i + 1] < means[i] for i in range(3))


# ------------------------------------------------- exact-law codebook --
# [Mobilint], "Coordinates Become Predictable After Rotation": a coordinate of
# a rotated unit vector has density proportional to (1 - t^2)^((d-3)/2); the
# codebook "Designing the Optimal Codebook Without Data" solves for is the
# Lloyd-Max quantizer of that law.

@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_beta_codebook_d3_is_the_uniform_quantizer(bits):
    # d = 3: the law is uniform on [-1, 1] (Archimedes), whose Lloyd-Max
    # quantizer is the uniform one: centroids -1 + (2i + 1) / L.
    L = 1 << bits
    c = codebook.lloyd_max_beta(bits, 3)
    assert np.allclose(c, -1 + (2 * np.arange(L) + 1) / L, atol=1e-13)


@pytest.mark.parametrize("d", [16, 64, 128, 256])
def test_beta_codebook_one_bit_closed_form(d):
    # E[X | X > 0] = Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2)) for the density
    # Gamma(d/2) / (sqrt(pi) Gamma((d-1)/2)) (1 - t^2)^((d-3)/2) printed there.
    from scipy import special
    want = math.exp(special.gammaln(d / 2) - special.gammaln((d + 1) / 2)) / math.sqrt(math.pi)
    c = codebook.lloyd_max_beta(1, d)
    assert c[1] == pytest.approx(want, rel=1e-12) and c[0] == -c[1]


@pytest.mark.parametrize("d", [16, 128])
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_beta_codebook_fixed_point_by_quadrature(d, bits):
    # Each centroid is the conditional mean of its cell under the printed
    # density, by numerical integration (not the incomplete beta function the
    # solver uses).
    from scipy import special
    a = (d - 3) / 2
    norm = math.gamma(d / 2) / (math.sqrt(math.pi) * math.gamma((d - 1) / 2)) if d < 300 else None
    f = lambda t: norm * (1 - t * t) ** a
    assert integrate.quad(f, -1, 1)[0] == pytest.approx(1.0, abs=1e-12)
    c = codebook.lloyd_max_beta(bits, d)
    edges = [-1.0] + list((c[:-1] + c[1:]) / 2) + [1.0]
    for i, ci in enumerate(c):
        m0 = integrate.quad(f, edges[i], edges[i + 1], epsabs=1e-15, epsrel=1e-13, limit=200)[0]
        m1 = integrate.quad(lambda t: t * f(t), edges[i], edges[i + 1], epsabs=1e-15, epsrel=1e-13, limit=200)[0]
        assert m1 / m0 == pytest.approx(ci, rel=1e-9, abs=1e-12)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_beta_codebook_beats_gaussian_codebook_on_its_law(bits):
    # The density is log-concave, so its Lloyd-Max quantizer is the unique
    # MSE-optimal one: under the exact law it does strictly better than the
    # N(0, 1/d) codebook, by a small margin at d = 64.
    d = 64
    mb = codebook.beta_mse(codebook.lloyd_max_beta(bits, d), d)
    mg = codebook.beta_mse(codebook.lloyd_max_normal(bits) / math.sqrt(d), d)
    assert mb < mg < mb * 1.01


def test_beta_codebook_tends_to_the_gaussian_one():
    # "In high dimensions this Beta distribution converges to a Gaussian
    # N(0,1/d)": sqrt(d) c_beta -> c_gauss, the gap shrinking like 1/d.
    g = codebook.lloyd_max_normal(3)
    gap = [np.abs(codebook.lloyd_max_beta(3, d) * math.sqrt(d) - g).max() for d in (64, 256, 1024)]
    assert gap[0] > gap[1] > gap[2]
    assert 3.0 < gap[0] / gap[1] < 5.0 and 3.0 < gap[1] / gap[2] < 5.0


def test_beta_codebook_mse_on_rotated_unit_vectors():
    # Monte Carlo on actual Haar rotations of unit vectors at d = 16 (where the
    # exact law and the Gaussian differ most): the per-coordinate squared error
    # of the exact-law codebook matches beta_mse within the sampling error.
    rs = np.random.default_rng(16)
    d, n = 16, 4000
    c = codebook.lloyd_max_beta(2, d)
    beta = (c[:-1] + c[1:]) / 2
    y = np.concatenate([(_random_rotation(rs, d) @ _unit_rows(rs, 1, d)[0])[None] for _ in range(n)])
    err = (y - c[codebook.quantize_scalar(y, beta)]) ** 2
    want = codebook.beta_mse(c, d)
    assert err.mean() == pytest.approx(want, abs=4 * err.std() / math.sqrt(err.size / 2))


# -------------------------------------------- dithered Hadamard variant --
# thelatestinai.com paper page 2606.10458, third abstract: randomized Hadamard
# HD, then a random scalar offset subtracted before quantizing; the dithered
# TurboQuant's MSE is (pi sqrt(3)/2 + o(1)) 4^-b.

def test_dither_offsets_uniform_and_independent():
    c, _ = codebook.codebook(3, 128)
    w = float(c[4]) - float(c[3])
    t = np.arange(20000)
    zero = np.zeros_like(t)
    dk = codec.dither_offsets(11, "K", zero, t, c)
    assert (np.abs(dk) < w / 2).all()
    assert stats.kstest(dk / w + 0.5, "uniform").pvalue > 1e-3
    dv = codec.dither_offsets(11, "V", zero, t, c)
    d1 = codec.dither_offsets(11, "K", zero + 1, t, c)
    assert abs(np.corrcoef(dk, dv)[0, 1]) < 0.05 and abs(np.corrcoef(dk, d1)[0, 1]) < 0.05


def _dithered_mse(bits, d, n, seed):
    rs = np.random.default_rng(seed)
    HD = transforms.hadamard_rotation(d, seed)
    u = _unit_rows(rs, n, d)
    c, beta = codebook.codebook(bits, d)
    dl = codec.dither_offsets(seed, "K", np.zeros(n, np.int64), np.arange(n), c)
    enc = codec.encode_rows(u, HD, c, beta, dither=dl)
    xh = codec.reconstruct_mse(enc["idx"], enc["norm"], HD, c, dither=dl)
    return ((xh - u) ** 2).sum(axis=1).mean()


def test_dithered_hadamard_mse_within_the_bound():
    mses = [_dithered_mse(b, 256, 3000, 21) for b in (1, 2, 3, 4)]
    for b, m in zip((1, 2, 3, 4), mses):
        assert m <= PANTER_DITE * 4.0 ** -b
    assert all(mses[i + 1] < mses[i] for i in range(3))


def test_dithered_reconstruction_moves_only_along_d_e0():
    # The offset is added to every rotated coordinate: (H D)^T (delta 1) =
    # delta D H 1 = delta sqrt(d) D_0 e_0 (H 1 = sqrt(d) e_0 for the Sylvester
    # H), so the dithered reconstruction differs from the plain one only in
    # coordinate 0, by n delta sqrt(d) D_0.
    d, seed = 64, 5
    HD = transforms.hadamard_rotation(d, seed)
    D0 = float(rng.signs(seed, rng.TAG_SIGNS, 1)[0])
    rs = np.random.default_rng(5)
    x = rs.standard_normal((40, d)) * 3.0
    c, beta = codebook.codebook(2, d)
    dl = codec.dither_offsets(seed, "V", np.zeros(40, np.int64), np.arange(40), c)
    enc = codec.encode_rows(x, HD, c, beta, dither=dl)
    diff = (codec.reconstruct_mse(enc["idx"], enc["norm"], HD, c, dither=dl)
            - codec.reconstruct_mse(enc["idx"], enc["norm"], HD, c))
    assert np.abs(diff[:, 1:]).max() < 1e-12
    assert np.allclose(diff[:, 0], enc["norm"] * dl * math.sqrt(d) * D0, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- codec --

def test_encode_matches_nearest_centroid_bruteforce():
    rs = np.random.default_rng(1)
    d = 64
    P = _random_rotation(rs, d)
    x = rs.standard_normal((500, d)) * 3.0
    for b in (1, 2, 3, 4):
        c, beta = codebook.codebook(b, d)
        enc = codec.encode_rows(x, P, c, beta)
        y = (x / np.linalg.norm(x, axis=1, keepdims=True)) @ P.T
        nearest = np.argmin(np.abs(y[..., None] - c.astype(np.float64)), axis=-1)
        assert np.array_equal(enc["idx"], nearest)
        assert np.allclose(enc["norm"], np.linalg.norm(x, axis=1), rtol=1e-14)


def test_centroid_round_trip_and_nearby_values():
    # [cuTile] tests: a centroid survives a quantize/dequantize round trip
    # unchanged, and a value near a centroid takes that centroid's index.
    d = 128
    for b in (1, 2, 3, 4):
        c, beta = codebook.codebook(b, d)
        idx = codebook.quantize_scalar(c, beta)
        assert np.array_equal(idx, np.arange(2 ** b))
        gaps = np.diff(c.astype(np.float64)).min()
        jitter = np.linspace(-0.3, 0.3, 7)[:, None] * gaps
        assert (codebook.quantize_scalar(c[None, :] + jitter, beta) == np.arange(2 ** b)).all()


def test_zero_row_is_lower_middle_index():
    d = 64
    c, beta = codebook.codebook(3, d)
    enc = codec.encode_rows(np.zeros((1, d)), np.eye(d), c, beta, S=np.eye(d))
    assert enc["norm"][0] == 0.0 and (enc["idx"] == 3).all()


def test_one_bit_bias_is_two_over_pi():
    # [Mobilint], "The Bias Problem": with the 1-bit codebook, <x, x_q> has
    # mean 2/pi = 0.6366 over random unit vectors (rotation does not change it).
    rs = np.random.default_rng(2)
    d = 128
    u = _unit_rows(rs, 5000, d)
    c, beta = codebook.codebook(1, d)
    enc = codec.encode_rows(u, np.eye(d), c, beta)
    ratio = (u * c.astype(np.float64)[enc["idx"]]).sum(axis=1)
    assert ratio.mean() == pytest.approx(2 / math.pi, abs=3e-3)
    assert round(float(ratio.mean()), 2) == 0.64


def _estimates(rs, d, b_mse, trials, with_qjl):
    """Estimated and true <y, x> for independent (Pi, S, x, y) draws."""
    c, beta = codebook.codebook(b_mse, d)
    est, truth = [], []
    for _ in range(trials):
        x = _unit_rows(rs, 1, d)
        y = _unit_rows(rs, 1, d)[0]
        P = _random_rotation(rs, d)
        S = rs.standard_normal((d, d))
        enc = codec.encode_rows(x, P, c, beta, S if with_qjl else None)
        if with_qjl:
            xh = codec.reconstruct_prod(enc["idx"], enc["norm"], enc["sign"], enc["rnorm"], P, c, S)
        else:
            xh = codec.reconstruct_mse(enc["idx"], enc["norm"], P, c)
        est.append(float(xh[0] @ y))
        truth.append(float(x[0] @ y))
    return np.array(est), np.array(truth)


def test_slopes_mse_only_biased_qjl_unbiased():
    # [Mobilint], "Two-Stage Approach" experiment (2-bit MSE, d=128): regression
    # slope < 1 without QJL and ~1 with it.  The MSE-only slope has the closed
    # form E[x c(x)] / E[x^2] = 1 - D_mse(b) by the centroid condition.
    rs = np.random.default_rng(3)
    d, trials = 64, 1500
    est, truth = _estimates(rs, d, 2, trials, with_qjl=False)
    slope = est @ truth / (truth @ truth)
    d_mse = codebook.normal_mse(codebook.lloyd_max_normal(2))
    assert slope == pytest.approx(1 - d_mse, abs=0.02)
    est, truth = _estimates(rs, d, 2, trials, with_qjl=True)
    resid = est - truth
    slope = est @ truth / (truth @ truth)
    se = math.sqrt(resid.var() / (truth @ truth))
    assert abs(slope - 1) < 4 * se + 1e-3


def test_unbiased_and_variance_bound():
    # [Mobilint], "Unbiasedness Proof" and "Variance Bound": E[<y, x_hat>] =
    # <y, x>, and Var <= pi/(2d) ||y||^2 E||r||^2 with E||r||^2 = D_mse(b-1).
    rs = np.random.default_rng(4)
    d, trials, b_mse = 64, 2500, 1
    est, truth = _estimates(rs, d, b_mse, trials, with_qjl=True)
    err = est - truth
    assert abs(err.mean()) < 4 * err.std() / math.sqrt(trials)
    bound = math.pi / (2 * d) * codebook.normal_mse(codebook.lloyd_max_normal(b_mse))
    assert err.var() <= 1.1 * bound


def test_qjl_residual_norm_matches_rotated_residual():
    rs = np.random.default_rng(5)
    d = 64
    P = _random_rotation(rs, d)
    S = rs.standard_normal((d, d))
    c, beta = codebook.codebook(2, d)
    x = rs.standard_normal((50, d))
    enc = codec.encode_rows(x, P, c, beta, S)
    # ||u - P^T c|| = ||P u - c|| because P is orthogonal.
    r_rot = enc["y"] - c.astype(np.float64)[enc["idx"]]
    assert np.allclose(enc["rnorm"], np.linalg.norm(r_rot, axis=1), rtol=1e-12)


# ---------------------------------------------------------- bit layouts --

def test_bit_layout_golden_examples():
    for line in _golden_lines("bit_layouts.txt"):
        arrow = line.index("->")
        want = np.array([int(v, 16) for v in line[arrow + 1:]], dtype=np.uint8)
        if line[0] == "stream":
            bits = int(line[1])
            codes = [int(v) for v in line[2:arrow]]
            assert np.array_equal(codec.pack_stream(codes, bits), want)
            assert list(codec.unpack_stream(want, bits, len(codes))) == codes
        else:
            d, bits = int(line[1]), int(line[2])
            codes = np.array([int(v) for v in line[4:arrow]]).reshape(1, 8, d)
            assert np.array_equal(codec.pack_value_codes(codes, bits).reshape(-1), want)
            assert np.array_equal(codec.unpack_value_codes(want, bits, 1, 8, d), codes)


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_pack_round_trip(bits):
    rs = np.random.default_rng(bits)
    d = 128
    codes = rs.integers(0, 2 ** bits, size=(24, d))
    packed = codec.pack_key_codes(codes, bits)
    assert packed.shape == (24, d * bits // 8)
    assert np.array_equal(codec.unpack_key_codes(packed, bits, d), codes)
    v = codes.reshape(3, 8, d)
    assert np.array_equal(codec.unpack_value_codes(codec.pack_value_codes(v, bits), bits, 3, 8, d), v)
    # a token's key codes are contiguous: token 5 only touches its own bytes
    alt = codes.copy()
    alt[5] = (alt[5] + 1) % (2 ** bits)
    diff = np.nonzero((codec.pack_key_codes(alt, bits) != packed).any(axis=1))[0]
    assert list(diff) == [5]


# ------------------------------------------------------------ attention --

def _tiny_layer(rs, d, kb, vb, qjl):
    P = _random_rotation(rs, d)
    S = rs.standard_normal((d, d))
    ck, bk = codebook.codebook(kb, d)
    cv, bv = codebook.codebook(vb, d)
    return P, S, ck, bk, cv, bv


def _encode_tiny(rs, B, Hkv, N, d, kb, vb, qjl, P, S, ck, bk, cv, bv, kscale=1.0):
    K = rs.standard_normal((B * Hkv * N, d)) * kscale
    V = rs.standard_normal((B * Hkv * N, d))
    ek = codec.encode_rows(K, P, ck, bk, S if qjl else None)
    ev = codec.encode_rows(V, P, cv, bv)
    cache = {"k_idx": ek["idx"].reshape(B, Hkv, N, d), "k_norm": ek["norm"].reshape(B, Hkv, N),
             "v_idx": ev["idx"].reshape(B, Hkv, N, d), "v_norm": ev["norm"].reshape(B, Hkv, N)}
    if qjl:
        cache["k_sign"] = ek["sign"].reshape(B, Hkv, N, d)
        cache["k_rnorm"] = ek["rnorm"].reshape(B, Hkv, N)
    return K, V, ek, ev, cache


@pytest.mark.parametrize("qjl", [0, 1, "dither", "values"])
def test_decode_equals_dense_bruteforce(qjl):
    # Estimator identity: s = <q, x_hat_k>/sqrt(d) with the explicit two-stage
    # (or MSE) reconstruction, and out = softmax(s) @ x_hat_v.  Pins the
    # pre-rotation trick, the QJL factor, the 1/sqrt(d) scaling, the GQA map
    # and the un-rotation against a plain dense computation.
    dither = qjl == "dither"
    vqjl = qjl == "values"        # QJL on keys and values
    qjl = 1 if qjl in (1, "values") else 0
    rs = np.random.default_rng(10 + qjl + 2 * dither + 4 * vqjl)
    B, Hq, Hkv, Tq, N, d = 2, 4, 2, 3, 9, 16
    P, S, ck, bk, cv, bv = _tiny_layer(rs, d, 2, 3, qjl)
    if dither:
        P = transforms.hadamard_rotation(d, 4)
        seq = np.repeat(np.arange(B * Hkv), N)
        tok = np.tile(np.arange(N), B * Hkv)
        dk = codec.dither_offsets(4, "K", seq, tok, ck)
        dv = codec.dither_offsets(4, "V", seq, tok, cv)
        K = rs.standard_normal((B * Hkv * N, d))
        V = rs.standard_normal((B * Hkv * N, d))
        ek = codec.encode_rows(K, P, ck, bk, dither=dk)
        ev = codec.encode_rows(V, P, cv, bv, dither=dv)
        cache = {"k_idx": ek["idx"].reshape(B, Hkv, N, d), "k_norm": ek["norm"].reshape(B, Hkv, N),
                 "k_dither": dk.reshape(B, Hkv, N), "v_dither": dv.reshape(B, Hkv, N),
                 "v_idx": ev["idx"].reshape(B, Hkv, N, d), "v_norm": ev["norm"].reshape(B, Hkv, N)}
    else:
        K, V, ek, ev, cache = _encode_tiny(rs, B, Hkv, N, d, 2, 3, qjl, P, S, ck, bk, cv, bv)
    if vqjl:
        ev = codec.encode_rows(V, P, cv, bv, S)
        cache.update({"v_idx": ev["idx"].reshape(B, Hkv, N, d), "v_norm": ev["norm"].reshape(B, Hkv, N),
                      "v_sign": ev["sign"].reshape(B, Hkv, N, d), "v_rnorm": ev["rnorm"].reshape(B, Hkv, N)})
    q = rs.standard_normal((B, Hq, Tq, d))
    out, scores = attention.decode(q, P, S, ck, cv, cache, N, causal=False)
    if qjl:
        kh = codec.reconstruct_prod(ek["idx"], ek["norm"], ek["sign"], ek["rnorm"], P, ck, S)
    else:
        kh = codec.reconstruct_mse(ek["idx"], ek["norm"], P, ck, dither=dk if dither else None)
    if vqjl:
        vh = codec.reconstruct_prod(ev["idx"], ev["norm"], ev["sign"], ev["rnorm"], P, cv, S)
    else:
        vh = codec.reconstruct_mse(ev["idx"], ev["norm"], P, cv, dither=dv if dither else None)
    kh = kh.reshape(B, Hkv, N, d)
    vh = vh.reshape(B, Hkv, N, d)
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            s = q[b, h] @ kh[b, g].T / math.sqrt(d)
            assert np.allclose(scores[b, h], s, rtol=1e-12, atol=1e-12)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            assert np.allclose(out[b, h], p @ vh[b, g], rtol=1e-11, atol=1e-12)


def test_value_qjl_output_unbiased_over_projections():
    # With QJL on values every value row is reconstructed without bias over the
    # projection S (E[sqrt(pi/2)/d ||r|| S^T sign(S r)] = r, [Mobilint]
    # "Two-Stage Approach"), and the keys (MSE-only) do not depend on S, so
    # the decode output averaged over many independent S is the
    # softmax-weighted sum of the exact values.
    rs = np.random.default_rng(21)
    d, N = 16, 5
    P = _random_rotation(rs, d)
    ck, bk = codebook.codebook(2, d)
    cv, bv = codebook.codebook(1, d)
    K = rs.standard_normal((N, d))
    V = rs.standard_normal((N, d))
    ek = codec.encode_rows(K, P, ck, bk)
    q = rs.standard_normal((1, 1, 1, d))
    runs = 4000
    acc = np.zeros(d)
    for _ in range(runs):
        S = rs.standard_normal((d, d))
        ev = codec.encode_rows(V, P, cv, bv, S)
        cache = {"k_idx": ek["idx"].reshape(1, 1, N, d), "k_norm": ek["norm"].reshape(1, 1, N),
                 "v_idx": ev["idx"].reshape(1, 1, N, d), "v_norm": ev["norm"].reshape(1, 1, N),
                 "v_sign": ev["sign"].reshape(1, 1, N, d), "v_rnorm": ev["rnorm"].reshape(1, 1, N)}
        out, scores = attention.decode(q, P, S, ck, cv, cache, N, causal=False)
        acc += out[0, 0, 0]
    s = scores[0, 0, 0]
    p = np.exp(s - s.max())
    p /= p.sum()
    want = p @ V
    # per coordinate, the QJL noise of one run is of order ||V|| / sqrt(d) per row
    err = np.abs(acc / runs - want).max()
    assert err < 0.1, err
    # and the MSE-only value reconstruction is biased for 1-bit codes (pins
    # that the QJL term is there): its error is several times larger
    mse = p @ codec.reconstruct_mse(ev["idx"], ev["norm"], P, cv)
    assert np.abs(mse - want).max() > 3 * err


def test_decode_single_key_and_identical_keys():
    rs = np.random.default_rng(12)
    d = 16
    P, S, ck, bk, cv, bv = _tiny_layer(rs, d, 3, 2, 1)
    K, V, ek, ev, cache = _encode_tiny(rs, 1, 1, 1, d, 3, 2, 1, P, S, ck, bk, cv, bv)
    q = rs.standard_normal((1, 1, 1, d))
    out, _ = attention.decode(q, P, S, ck, cv, cache, 1, causal=False)
    vh = codec.reconstruct_mse(ev["idx"], ev["norm"], P, cv)
    assert np.allclose(out[0, 0, 0], vh[0], atol=1e-13)
    # identical keys: uniform weights, output = mean of the value reconstructions
    N = 6
    K, V, ek, ev, cache = _encode_tiny(rs, 1, 1, N, d, 3, 2, 1, P, S, ck, bk, cv, bv)
    for f in ("k_idx", "k_norm", "k_sign", "k_rnorm"):
        cache[f][:] = cache[f][:, :, :1]
    out, scores = attention.decode(q, P, S, ck, cv, cache, N, causal=False)
    assert np.allclose(scores[0, 0, 0], scores[0, 0, 0, 0])
    vh = codec.reconstruct_mse(ev["idx"], ev["norm"], P, cv)
    assert np.allclose(out[0, 0, 0], vh.mean(axis=0), atol=1e-13)


def test_causal_alignment():
    rs = np.random.default_rng(13)
    d, Tq, N = 16, 4, 7
    P, S, ck, bk, cv, bv = _tiny_layer(rs, d, 2, 2, 1)
    _, _, _, ev, cache = _encode_tiny(rs, 1, 1, N, d, 2, 2, 1, P, S, ck, bk, cv, bv)
    q = rs.standard_normal((1, 1, Tq, d))
    out, scores = attention.decode(q, P, S, ck, cv, cache, N, causal=True)
    for i in range(Tq):
        visible = N - Tq + i + 1
        assert np.isfinite(scores[0, 0, i, :visible]).all()
        assert np.isneginf(scores[0, 0, i, visible:]).all()
    # the last query sees everything: same as the non-causal result
    out_all, _ = attention.decode(q, P, S, ck, cv, cache, N, causal=False)
    assert np.allclose(out[0, 0, Tq - 1], out_all[0, 0, Tq - 1], atol=1e-13)
    # the first query equals decoding over the prefix it can see
    pre = {k: v[:, :, :N - Tq + 1] for k, v in cache.items()}
    out_pre, _ = attention.decode(q[:, :, :1], P, S, ck, cv, pre, N - Tq + 1, causal=False)
    assert np.allclose(out[0, 0, 0], out_pre[0, 0, 0], atol=1e-13)


def test_retrieval_of_planted_key():
    # [cuTile] test: the most-attended key is still found after compression.
    rs = np.random.default_rng(14)
    d, N = 128, 256
    P, S, ck, bk, cv, bv = _tiny_layer(rs, d, 2, 2, 1)
    q = rs.standard_normal((1, 1, 1, d))
    K = rs.standard_normal((N, d))
    K[77] = 3.0 * q[0, 0, 0]
    ek = codec.encode_rows(K, P, ck, bk, S)
    ev = codec.encode_rows(rs.standard_normal((N, d)), P, cv, bv)
    cache = {"k_idx": ek["idx"][None, None], "k_norm": ek["norm"][None, None],
             "k_sign": ek["sign"][None, None], "k_rnorm": ek["rnorm"][None, None],
             "v_idx": ev["idx"][None, None], "v_norm": ev["norm"][None, None]}
    _, scores = attention.decode(q, P, S, ck, cv, cache, N, causal=False)
    assert int(np.argmax(scores[0, 0, 0])) == 77


def test_score_error_falls_with_bits_and_correlates():
    # [cuTile] tests: higher bits give lower score MSE; estimated scores
    # correlate with true q.k/sqrt(d).
    rs = np.random.default_rng(15)
    d, N = 128, 400
    P = _random_rotation(rs, d)
    S = rs.standard_normal((d, d))
    K = rs.standard_normal((N, d))
    q = rs.standard_normal((1, 1, 1, d))
    true = K @ q[0, 0, 0] / math.sqrt(d)
    errs = []
    for b in (1, 2, 3, 4):
        ck, bk = codebook.codebook(b, d)
        ek = codec.encode_rows(K, P, ck, bk, S)
        cache = {"k_idx": ek["idx"][None, None], "k_norm": ek["norm"][None, None],
                 "k_sign": ek["sign"][None, None], "k_rnorm": ek["rnorm"][None, None],
                 "v_idx": ek["idx"][None, None], "v_norm": ek["norm"][None, None]}
        _, s = attention.decode(q, P, S, ck, ck, cache, N, causal=False)
        errs.append(((s[0, 0, 0] - true) ** 2).mean())
        if b >= 2:
            assert np.corrcoef(s[0, 0, 0], true)[0, 1] > 0.9
    assert all(errs[i + 1] < errs[i] for i in range(3))

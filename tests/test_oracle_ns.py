"""Pins of the oracle's normalisation + Newton-Schulz + rescale (CPU only).

Every check here goes through a route other than the oracle's own matrix
iteration: a library SVD (numpy.linalg.svd) or the in-repo Jacobi SVD, the
scalar singular-value map, values the pages print, or closed forms.
"""

import math
import os

import numpy as np
import pytest

import oracle
from oracle import jacobi_svd, newton_schulz, orthogonalized_update, polar_factor

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def _scalar_map(x, schedule):
    """Iterate p(x) = a x + b x^3 + c x^5 on one scalar (the singular-value map)."""
    for a, b, c in schedule:
        x = a * x + b * x ** 3 + c * x ** 5
    return x


def _sigma_map_reference(n_mat, schedule, svd=np.linalg.svd):
    """U diag(f(sigma / ||sigma||)) V^T from a library SVD of N."""
    u, s, vt = svd(np.asarray(n_mat, dtype=np.float64), full_matrices=False) \
        if svd is np.linalg.svd else svd(n_mat)
    fro = math.sqrt(float(np.sum(s * s)))
    f = np.array([_scalar_map(v / fro, schedule) for v in s])
    return (u * f) @ vt


def _rng(seed):
    return np.random.default_rng(seed)


# --------------------------------------------------------------------------- schedule


def test_schedule_matches_pages():
    rows = _read_golden("ns_coefficients.txt")
    assert len(rows) == 10 == len(oracle.DEEPSEEK_V4_SCHEDULE)
    for r, coeffs in zip(rows, oracle.DEEPSEEK_V4_SCHEDULE):
        assert tuple(float(v) for v in r[1:]) == tuple(coeffs)
    assert oracle.QUINTIC5_SCHEDULE == (tuple(float(v) for v in rows[0][1:]),) * 5


def test_aggressive_map_at_one_is_below_one():
    # The book's table says the aggressive polynomial overshoots at x = 1; in fact
    # p(1) = a + b + c = 0.701 (reading recorded in the design notes).
    a, b, c = oracle.DEEPSEEK_V4_SCHEDULE[0]
    assert abs(_scalar_map(1.0, [(a, b, c)]) - 0.701) < 1e-12


# ----------------------------------------------------------------- sigma-map invariant


@pytest.mark.parametrize("shape", [(8, 12), (12, 8), (16, 16), (5, 3), (3, 5), (1, 7), (7, 1),
                                   (40, 64), (64, 40)])
def test_sigma_map_invariant_library_svd(shape):
    """NS(N) == U diag(f(sigma/||N||_F)) V^T: U, V kept, each sigma mapped by the scalar
    polynomial (DeepSeek-V4 book ch. 6, section 3)."""
    n = _rng(sum(shape)).standard_normal(shape)
    got = newton_schulz(n)
    ref = _sigma_map_reference(n, oracle.DEEPSEEK_V4_SCHEDULE)
    assert np.linalg.norm(got - ref) <= 1e-12 * max(1.0, np.linalg.norm(ref))


@pytest.mark.parametrize("shape", [(6, 9), (9, 6), (7, 7)])
def test_sigma_map_invariant_jacobi_svd(shape):
    n = _rng(100 + sum(shape)).standard_normal(shape)
    got = newton_schulz(n)
    ref = _sigma_map_reference(n, oracle.DEEPSEEK_V4_SCHEDULE, svd=jacobi_svd)
    assert np.linalg.norm(got - ref) <= 1e-12 * np.linalg.norm(ref)


def test_sigma_map_invariant_ill_conditioned():
    """Log-uniform spectrum in [1e-4, 1e-1] (the configs' gradient law)."""
    r = _rng(7)
    rows, cols = 24, 40
    u, _ = np.linalg.qr(r.standard_normal((rows, rows)))
    v, _ = np.linalg.qr(r.standard_normal((cols, rows)))
    sig = np.exp(r.uniform(math.log(1e-4), math.log(1e-1), rows))
    n = (u * sig) @ v.T
    got = newton_schulz(n)
    ref = _sigma_map_reference(n, oracle.DEEPSEEK_V4_SCHEDULE)
    assert np.linalg.norm(got - ref) <= 1e-10 * np.linalg.norm(ref)


def test_sigma_map_invariant_quintic5():
    n = _rng(3).standard_normal((10, 14))
    got = newton_schulz(n, oracle.QUINTIC5_SCHEDULE)
    ref = _sigma_map_reference(n, oracle.QUINTIC5_SCHEDULE)
    assert np.linalg.norm(got - ref) <= 1e-12 * np.linalg.norm(ref)


def test_diagonal_worked_example():
    """NS(diag(1, 0.1)) = diag(f(1/sqrt(1.01)), f(0.1/sqrt(1.01)))."""
    got = newton_schulz(np.diag([1.0, 0.1]))
    f1 = _scalar_map(1.0 / math.sqrt(1.01), oracle.DEEPSEEK_V4_SCHEDULE)
    f2 = _scalar_map(0.1 / math.sqrt(1.01), oracle.DEEPSEEK_V4_SCHEDULE)
    assert abs(got[0, 0] - f1) < 1e-14 and abs(got[1, 1] - f2) < 1e-14
    assert got[0, 1] == 0.0 and got[1, 0] == 0.0
    assert abs(f1 - 1.0000265362697844) < 1e-13
    assert abs(f2 - 1.0000474834200586) < 1e-13


# ------------------------------------------------------------------- values the pages print


def test_hybrid_band_from_pages():
    """After the 8 aggressive steps the singular values lie in [0.69, 1.20]; the 2
    standard steps take them into [1.0000, 1.0020] (four printed decimals)."""
    g = {r[0]: float(r[1]) for r in _read_golden("hybrid_band.txt")}
    half = 0.5 * 10 ** (-int(g["printed_decimals"]))
    std2 = oracle.DEEPSEEK_V4_SCHEDULE[8:]
    xs = np.linspace(g["in_lo"], g["in_hi"], 2001)
    ys = np.array([_scalar_map(x, std2) for x in xs])
    assert ys.min() >= g["out_lo"] - half and ys.max() <= g["out_hi"] + half
    # Same claim through the oracle's matrix iteration: a matrix whose normalised
    # singular values are all resolved (>= 1e-3) ends with sigma in the band.
    r = _rng(11)
    u, _ = np.linalg.qr(r.standard_normal((30, 30)))
    v, _ = np.linalg.qr(r.standard_normal((50, 30)))
    sig = np.exp(r.uniform(math.log(1e-3), 0.0, 30))
    out = newton_schulz((u * sig) @ v.T)
    s_out = np.linalg.svd(out, compute_uv=False)
    assert s_out.min() >= g["out_lo"] - half and s_out.max() <= g["out_hi"] + half


def test_shape_rescale_example_from_pages():
    for r in _read_golden("shape_rescale.txt"):
        rows, cols, ns_fro, factor, rescaled = (int(v) for v in r)
        n = _rng(rows + cols).standard_normal((rows, cols))
        x = newton_schulz(n)
        assert abs(np.linalg.norm(x) / ns_fro - 1.0) < 2.2e-3
        assert math.sqrt(max(rows, cols)) == factor
        o = orthogonalized_update(n, gamma=1.0)
        assert abs(np.linalg.norm(o) / rescaled - 1.0) < 2.2e-3


def test_standard_map_drill_from_pages():
    """Pure standard NS from a weakest normalised singular value of 0.05."""
    std = oracle.DEEPSEEK_V4_SCHEDULE[9]
    big = math.sqrt(1.0 - 0.05 ** 2)        # keeps ||N||_F = 1 so sigma_min stays 0.05
    n = np.diag([big, 0.05])
    for r in _read_golden("standard_map_drill.txt"):
        steps, printed, dec = int(r[0]), float(r[1]), int(r[2])
        x = newton_schulz(n, (std,) * steps)
        assert round(float(x[1, 1]), dec) == printed


def test_flops_formula_examples_from_pages():
    for r in _read_golden("flops_overhead.txt"):
        m, batch, steps, pct = int(r[0]), int(r[1]), int(r[2]), float(r[3])
        ns = oracle.ns_flops_dense(m, m, steps)            # square case: 6 T m^3
        assert ns == 6 * steps * m ** 3
        overhead = ns / (6 * m * m * batch)                 # vs 6 n m B forward+backward
        assert round(100 * overhead, 1) == pct


def test_algorithmic_flops_triangle_count():
    # brute-force count of the multiply-adds the symmetric method needs, small sizes
    for rows, cols in [(3, 5), (5, 3), (4, 4)]:
        s, l = min(rows, cols), max(rows, cols)
        gram = sum(1 for i in range(s) for j in range(i + 1)) * l          # one triangle
        sq = sum(1 for i in range(s) for j in range(i + 1)) * s            # one triangle of A A
        apply = s * l * s
        assert oracle.ns_flops_algorithmic(rows, cols, 1) == 2 * (gram + sq + apply)


# --------------------------------------------------------------------------- invariants


def test_transpose_rule():
    n = _rng(5).standard_normal((9, 17))
    assert np.array_equal(newton_schulz(n.T), newton_schulz(n).T)


def test_scale_invariance():
    n = _rng(6).standard_normal((11, 13))
    a = newton_schulz(n)
    for c in (1e-6, 0.37, 2.0 ** 20):
        assert np.linalg.norm(newton_schulz(c * n) - a) <= 1e-12 * np.linalg.norm(a)


def test_orthogonal_equivariance():
    r = _rng(8)
    n = r.standard_normal((10, 15))
    q1, _ = np.linalg.qr(r.standard_normal((10, 10)))
    q2, _ = np.linalg.qr(r.standard_normal((15, 15)))
    lhs = newton_schulz(q1 @ n @ q2)
    rhs = q1 @ newton_schulz(n) @ q2
    assert np.linalg.norm(lhs - rhs) <= 1e-12 * np.linalg.norm(rhs)


def test_zero_matrix_gives_zero():
    assert not np.any(newton_schulz(np.zeros((4, 6))))


def test_rank_deficient_zero_sigma_stays_zero():
    r = _rng(9)
    u, _ = np.linalg.qr(r.standard_normal((8, 3)))
    v, _ = np.linalg.qr(r.standard_normal((12, 3)))
    n = (u * np.array([1.0, 0.5, 0.1])) @ v.T           # rank 3 in 8 x 12
    out = newton_schulz(n)
    s = np.linalg.svd(out, compute_uv=False)
    # rounding noise (~1e-16) in the null space is amplified by at most f(x)/x ~ 8e4
    assert np.all(s[3:] < 1e-9)
    assert np.all(np.abs(s[:3] - 1.0) < 2.1e-3)


# ------------------------------------------------------------------ polar-factor closeness


@pytest.mark.parametrize("shape", [(6, 10), (10, 6), (8, 8)])
def test_close_to_jacobi_polar(shape):
    n = _rng(20 + shape[0]).standard_normal(shape)
    s = np.linalg.svd(n, compute_uv=False)
    assert s.min() / np.linalg.norm(n) >= 3.7e-5   # spectrum resolved by the 10 steps
    gap = newton_schulz(n) - polar_factor(n)
    assert np.linalg.norm(gap, 2) <= 2.1e-3


def test_frobenius_norm_is_sqrt_min_and_rms_is_gamma():
    """||O'||_F ~ sqrt(min(n,m)) (book ch. 6 section 5) and RMS(O) ~ gamma
    (the deep-dive page's update-scale lemma)."""
    for rows, cols in [(64, 128), (128, 64), (96, 96), (32, 256)]:
        n = _rng(rows * cols).standard_normal((rows, cols))
        x = newton_schulz(n)
        assert abs(np.linalg.norm(x) / math.sqrt(min(rows, cols)) - 1.0) < 2.2e-3
        o = orthogonalized_update(n, gamma=0.2)
        rms = math.sqrt(float(np.mean(o * o)))
        assert abs(rms / 0.2 - 1.0) < 2.2e-3


def test_unit_rms_mode_rms_is_gamma_for_any_x():
    """Unit-RMS mode (the deep-dive page's Megatron-Bridge recipe): O = X * gamma / RMS(X)
    has RMS exactly gamma whatever X is, orthogonal or not; RMS here is the plain mean of
    squares over all n*m entries."""
    for rows, cols in [(3, 7), (7, 3), (16, 16), (40, 9)]:
        x = _rng(rows + 31 * cols).standard_normal((rows, cols)) * 3.7
        o = x * oracle.update_scale(x, 0.2, "unit_rms")
        rms = math.sqrt(sum(float(v) ** 2 for v in o.ravel()) / (rows * cols))
        assert abs(rms - 0.2) < 1e-13


def test_unit_rms_mode_equals_sqrt_max_on_orthogonal_x():
    """For X with orthonormal columns (or rows), ||X||_F = sqrt(min(n, m)), so the unit-RMS
    factor gamma * sqrt(n m) / ||X|| is exactly gamma * sqrt(max(n, m)): the two scale modes
    agree on an exact polar factor (the deep-dive page's remark that they are equivalent in
    theory)."""
    for rows, cols in [(12, 5), (5, 12), (9, 9)]:
        q, _ = np.linalg.qr(_rng(rows * cols).standard_normal((max(rows, cols), min(rows, cols))))
        x = q if rows >= cols else q.T
        assert x.shape == (rows, cols)
        got = oracle.update_scale(x, 0.18, "unit_rms")
        assert abs(got / (0.18 * math.sqrt(max(rows, cols))) - 1.0) < 1e-13


def test_unit_rms_mode_zero_and_worked_scalars():
    """X = 0 gives a zero factor (decay-only update); a 2 x 2 case by hand:
    X = diag(3, 4) has ||X|| = 5 and RMS 5/2, so with gamma = 0.25 the factor is 0.1,
    and with lr = 0.5 the update scalar s is fl32(0.05)."""
    assert oracle.update_scale(np.zeros((4, 6)), 0.2, "unit_rms") == 0.0
    x = np.array([[3.0, 0.0], [0.0, 4.0]], dtype=np.float32)
    assert abs(oracle.update_scale(x, 0.25, "unit_rms") - 0.1) < 1e-15
    d, s = oracle.muon_scalars_f32(0.5, 0.2, 0.25, 2, 2, x, "unit_rms")
    assert d == np.float32(0.9) and s == np.float32(0.05)
    w = np.array([[1.0, 2.0], [-1.0, 0.5]], dtype=np.float32)
    got = oracle.apply_update_f32(w, x, 0.5, 0.2, 0.25, False, "unit_rms")
    want = np.array([[np.float32(0.9) * np.float32(1.0) - np.float32(0.05) * np.float32(3.0),
                      np.float32(0.9) * np.float32(2.0)],
                     [np.float32(0.9) * np.float32(-1.0),
                      np.float32(0.9) * np.float32(0.5) - np.float32(0.05) * np.float32(4.0)]], dtype=np.float32)
    assert np.array_equal(got, want)
    with pytest.raises(ValueError):
        oracle.update_scale(x, 0.2, "bogus")


def test_unit_rms_mode_close_to_sqrt_max_after_ns():
    """After the hybrid schedule the singular values sit within the pages' band around 1, so
    the two modes' O differ by the factor sqrt(min)/||O'|| within 2.2e-3."""
    for rows, cols in [(64, 128), (128, 64)]:
        rng = _rng(7 * rows + cols)
        w, g, m = (rng.standard_normal((rows, cols)).astype(np.float32) for _ in range(3))
        a = oracle.muon_step(w, g, m)
        b = oracle.muon_step(w, g, m, scale_mode="unit_rms")
        assert np.array_equal(a["x"], b["x"])
        ratio = np.linalg.norm(b["o"]) / np.linalg.norm(a["o"])
        assert abs(ratio - math.sqrt(min(rows, cols)) / np.linalg.norm(a["x"])) < 1e-12
        assert abs(ratio - 1.0) < 2.2e-3


# --------------------------------------------------------------- the independent polar route


def test_jacobi_svd_against_library():
    r = _rng(30)
    for shape in [(5, 3), (3, 5), (7, 7), (1, 4), (4, 1), (12, 9)]:
        a = r.standard_normal(shape)
        u, s, vt = jacobi_svd(a)
        assert np.allclose(s, np.linalg.svd(a, compute_uv=False), rtol=1e-13, atol=1e-14)
        assert np.linalg.norm(u @ np.diag(s) @ vt - a) <= 1e-13 * np.linalg.norm(a)
        k = min(shape)
        assert np.allclose(u.T @ u, np.eye(k), atol=1e-13)
        assert np.allclose(vt @ vt.T, np.eye(k), atol=1e-13)


def _sym_power(a, p):
    w, q = np.linalg.eigh(a)
    return (q * w ** p) @ q.T


def test_shampoo_identity_matches_jacobi_polar():
    """(G G^T)^{-1/4} G (G^T G)^{-1/4} = U V^T (the deep-dive page, Muon vs Shampoo)."""
    g = _rng(31).standard_normal((7, 7))
    lhs = _sym_power(g @ g.T, -0.25) @ g @ _sym_power(g.T @ g, -0.25)
    assert np.linalg.norm(lhs - polar_factor(g)) <= 1e-12

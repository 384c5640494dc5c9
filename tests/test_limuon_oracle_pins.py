"""Pins for the oracle's LiMuon orthogonaliser (randomized SVD of the
momentum, LiMuon digest "Метод"; Halko, Martinsson & Tropp 2011, Algorithms
4.4 and 5.1), independent of the oracle's own code: a hand-worked fixture,
the exact SVD (a library routine) wherever the randomized range finder is
exact, invariances of the algorithm, and planted mistakes that must fail."""
import numpy as np
import pytest

import oracle
from conftest import load_golden

lim = oracle.limuon_orthogonalize


def rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


def low_rank(r, c, rank, seed, spread=2.0):
    """U diag(s) V^T with Haar factors and distinct singular values in
    [10^-spread, 1]."""
    rng = np.random.default_rng(seed)
    u, _ = np.linalg.qr(rng.standard_normal((r, rank)))
    v, _ = np.linalg.qr(rng.standard_normal((c, rank)))
    s = np.sort(10.0 ** (-spread * rng.random(rank)))[::-1]
    return (u * s) @ v.T, u, s, v


def svd_truncated_polar(m, k, rcond=0.0):
    """U_k V_k^T of the exact SVD (library routine), dropping singular values
    at most rcond * sigma_1."""
    u, s, vt = np.linalg.svd(m, full_matrices=False)
    keep = [i for i in range(min(k, s.size)) if s[i] > rcond * s[0]]
    return u[:, keep] @ vt[keep, :]


def omega_for(m, kp, seed):
    return np.random.default_rng(seed).standard_normal((max(m.shape), kp))


# ---------------------------------------------------------------- hand-worked

def test_golden_hand_worked_2x3():
    g = load_golden("limuon_2x3_hand.txt")
    m = np.array([[3.0, 0.0, 0.0], [0.0, 1.0, 0.0]])
    om = np.ones((3, 1))
    for q, key in ((0, "q0"), (1, "q1")):
        o = lim(m, om, rank=1, power_iters=q)
        want = np.array([[g[key + "_00"], g[key + "_01"], 0.0], [g[key + "_10"], g[key + "_11"], 0.0]])
        np.testing.assert_allclose(o, want, atol=1e-9)
        # the tall orientation sketches the same (long) side: O(M^T) = O(M)^T
        np.testing.assert_allclose(lim(m.T, om, rank=1, power_iters=q), want.T, atol=1e-9)
    om2 = np.array([[1.0, 0.0], [1.0, 1.0], [1.0, 2.0]])
    np.testing.assert_allclose(lim(m, om2, rank=2, power_iters=0), [[1, 0, 0], [0, 1, 0]], atol=1e-12)
    np.testing.assert_allclose(lim(m, om2, rank=1, power_iters=0), [[1, 0, 0], [0, 0, 0]], atol=1e-12)


# ---------------------------------------------------------------- exact cases

@pytest.mark.parametrize("shape", [(40, 90), (90, 40), (64, 64)])
@pytest.mark.parametrize("q", [0, 1, 2])
def test_rank_at_most_k_gives_the_polar_factor(shape, q):
    """rank(M) <= k: the range finder is exact (range(X Omega) = range(X) for
    a Gaussian Omega), so O = U_r V_r^T, the polar factor of M on its
    range."""
    r, c = shape
    for rank, k, p in ((5, 5, 3), (5, 8, 4), (12, 12, 0)):
        m, u, s, v = low_rank(r, c, rank, seed=rank + 7 * q + r)
        o = lim(m, omega_for(m, k + p, 11 + q), rank=k, power_iters=q)
        assert rel(o, u @ v.T) < 1e-10, (shape, rank, k, p)


@pytest.mark.parametrize("shape", [(30, 70), (70, 30), (48, 48)])
def test_full_sketch_gives_truncated_svd(shape):
    """k + p >= s: the sketch spans the whole short side, B = Q^T X has X's
    singular values, and O is U_k V_k^T of the exact SVD (distinct singular
    values, so the truncation is unique); k = s gives polar(M) = U V^T."""
    r, c = shape
    s = min(r, c)
    m, _, _, _ = low_rank(r, c, s, seed=r * c)
    for k in (1, 7, s - 3, s):
        o = lim(m, omega_for(m, s + 2, 5), rank=k, power_iters=0)
        assert rel(o, svd_truncated_polar(m, k)) < 1e-9, k
    u, _, vt = np.linalg.svd(m, full_matrices=False)
    assert rel(lim(m, omega_for(m, s, 6), rank=s, power_iters=1), u @ vt) < 1e-9


def test_rcond_drops_tiny_directions():
    """Directions with sketched singular value <= rcond * sigma_1 map to zero
    (like p(0) = 0 for Newton-Schulz); above the cutoff they map to 1."""
    m = np.diag([1.0, 1e-6, 1e-2])
    om = np.eye(3)
    np.testing.assert_allclose(lim(m, om, rank=3, rcond=1e-4), np.diag([1.0, 0.0, 1.0]), atol=1e-12)
    np.testing.assert_allclose(lim(m, om, rank=3, rcond=1e-8), np.eye(3), atol=1e-9)
    np.testing.assert_allclose(lim(m, om, rank=1, rcond=1e-8), np.diag([1.0, 0.0, 0.0]), atol=1e-12)
    assert not np.any(lim(np.zeros((4, 6)), np.ones((6, 2)), rank=2))


# ---------------------------------------------------------------- invariances

def _generic(shape, seed):
    """Gaussian plus a rank-4 spike (a clear gap after the 4th singular
    value, as in a gradient with a few dominant directions)."""
    rng = np.random.default_rng(seed)
    r, c = shape
    m = 0.1 * rng.standard_normal((r, c))
    u, _ = np.linalg.qr(rng.standard_normal((r, 4)))
    v, _ = np.linalg.qr(rng.standard_normal((c, 4)))
    return m + 3.0 * (u * np.array([4.0, 3.0, 2.5, 2.0])) @ v.T


@pytest.mark.parametrize("shape", [(36, 80), (80, 36)])
def test_invariances(shape):
    """Exact identities of the algorithm (any M, any Gaussian draw):
    positive scale, transpose (the long side is sketched either way), left
    and right orthogonal factors (the right one rotates Omega with it), and
    Omega entering only through the range of X Omega."""
    m = _generic(shape, 3)
    kp, k = 10, 6
    om = omega_for(m, kp, 4)
    o = lim(m, om, rank=k, power_iters=1)
    assert rel(lim(37.5 * m, om, rank=k, power_iters=1), o) < 1e-11
    assert rel(lim(m.T, om, rank=k, power_iters=1), o.T) < 1e-11
    rng = np.random.default_rng(8)
    r, c = m.shape
    p, _ = np.linalg.qr(rng.standard_normal((r, r)))
    q, _ = np.linalg.qr(rng.standard_normal((c, c)))
    # the long side of m is cols when wide, rows when tall: rotate Omega with it
    if r <= c:
        assert rel(lim(p @ m, om, rank=k, power_iters=1), p @ o) < 1e-10
        assert rel(lim(m @ q, q.T @ om, rank=k, power_iters=1), o @ q) < 1e-10
    else:
        assert rel(lim(m @ q, om, rank=k, power_iters=1), o @ q) < 1e-10
        assert rel(lim(p @ m, p @ om, rank=k, power_iters=1), p @ o) < 1e-10
    g = rng.standard_normal((kp, kp)) + 3.0 * np.eye(kp)     # invertible
    assert rel(lim(m, om @ g, rank=k, power_iters=1), o) < 1e-10


def test_power_iteration_identity():
    """One power iteration sketches with (X^T X) Omega: O(M; Omega, q = 1)
    equals O(M; X^T X Omega, q = 0) (X = M, wide), and q iterations approach
    U_k V_k^T of the exact SVD monotonically on a matrix with a gap."""
    m = _generic((40, 90), 12)
    om = omega_for(m, 7, 13)
    assert rel(lim(m, om, rank=4, power_iters=1), lim(m, m.T @ m @ om, rank=4, power_iters=0)) < 1e-9
    target = svd_truncated_polar(m, 4)
    errs = [rel(lim(m, om, rank=4, power_iters=q), target) for q in range(7)]
    assert all(b <= a * (1 + 1e-9) for a, b in zip(errs, errs[1:])), errs
    assert errs[-1] < 1e-8


def test_limuon_step_is_muon_update_with_limuon_o():
    """The full step: momentum as in Muon, O from the randomized SVD, the
    decoupled update; a zero gradient with zero momentum is pure decay."""
    rng = np.random.default_rng(21)
    w = rng.standard_normal((20, 50))
    g = _generic((20, 50), 22)
    om = omega_for(g, 8, 23)
    r = oracle.muon_step_matrix(w, g, np.zeros_like(g), lr=0.02, mu=0.95, weight_decay=0.01, coeffs=None,
                                variant="limuon", omega=om, rank=4, power_iters=1)
    np.testing.assert_array_equal(r["momentum"], g)
    o = lim(g, om, rank=4, power_iters=1)
    np.testing.assert_allclose(r["ortho"], o, rtol=0, atol=0)
    np.testing.assert_allclose(r["weight"], w - 0.02 * (o + 0.01 * w), rtol=1e-15)
    z = oracle.muon_step_matrix(w, np.zeros_like(g), np.zeros_like(g), lr=0.02, mu=0.95, weight_decay=0.01,
                                coeffs=None, variant="limuon", omega=om, rank=4)
    np.testing.assert_allclose(z["weight"], (1 - 0.02 * 0.01) * w, rtol=1e-15)


# ---------------------------------------------------------------- planted mistakes

def _passes_pins(f):
    """The exact pins above, applied to a candidate orthogonaliser."""
    try:
        for shape in ((30, 70), (70, 30)):
            m, u, s, v = low_rank(*shape, 5, seed=99)
            if rel(f(m, omega_for(m, 8, 1), 5, 1), u @ v.T) > 1e-9:
                return False
            m, _, _, _ = low_rank(*shape, 30, seed=98)
            if rel(f(m, omega_for(m, 32, 2), 6, 0), svd_truncated_polar(m, 6)) > 1e-9:
                return False
            m = _generic(shape, 97)
            om = omega_for(m, 10, 3)
            if rel(f(1e-7 * m, om, 6, 1), f(m, om, 6, 1)) > 1e-9:
                return False
        m = np.array([[3.0, 0.0, 0.0], [0.0, 1.0, 0.0]])
        g = load_golden("limuon_2x3_hand.txt")
        if abs(f(m, np.ones((3, 1)), 1, 1)[0, 0] - g["q1_00"]) > 1e-9:
            return False
    except (ValueError, np.linalg.LinAlgError):
        return False
    return True


def test_planted_mistakes_are_caught():
    assert _passes_pins(lambda m, om, k, q: lim(m, om, k, q))

    def no_truncation(m, om, k, q):          # keeps every sketched direction
        return lim(m, om, om.shape[1], q)

    def short_side_sketch(m, om, k, q):       # sketches the short side instead
        x = m if m.shape[0] <= m.shape[1] else m.T
        o = lim(x.T, om[: x.shape[0]] if om.shape[0] >= x.shape[0] else om, k, q)
        return o.T if m.shape[0] <= m.shape[1] else o

    def absolute_cutoff(m, om, k, q):         # rcond applied to sigma, not sigma / sigma_1
        x = m if m.shape[0] <= m.shape[1] else m.T
        qq, _ = np.linalg.qr(x @ om)
        for _ in range(q):
            qt, _ = np.linalg.qr(x.T @ qq)
            qq, _ = np.linalg.qr(x @ qt)
        ub, sv, vt = np.linalg.svd(qq.T @ x, full_matrices=False)
        keep = [i for i in range(min(k, sv.size)) if sv[i] > 1e-4]
        o = (qq @ ub[:, keep]) @ vt[keep, :]
        return o if m.shape[0] <= m.shape[1] else o.T

    def transposed_factor(m, om, k, q):       # V from the wrong side of B
        x = m if m.shape[0] <= m.shape[1] else m.T
        qq, _ = np.linalg.qr(x @ om)
        ub, sv, vt = np.linalg.svd(qq.T @ x, full_matrices=False)
        o = (qq @ vt[:k, : qq.shape[1]].T) @ vt[:k, :]
        return o if m.shape[0] <= m.shape[1] else o.T

    def no_power_iteration(m, om, k, q):
        return lim(m, om, k, 0)

    for bad in (no_truncation, short_side_sketch, absolute_cutoff, transposed_factor, no_power_iteration):
        assert not _passes_pins(bad), bad.__name__

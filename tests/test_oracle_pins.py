"""Pins for the fp64 oracle, independent of the oracle's own code.

Each check compares the oracle against something fixed by the pages or by the
mathematics: hand-worked examples (tests/golden), the singular-value closed
form obtained from a library SVD, convergence to the polar factor, invariants
and special cases.  A planted mistake in any step of the oracle fails at least
one of them (see test_planted_mistakes_are_caught).
"""
import math

import numpy as np
import pytest

import oracle
from oracle import muon_oracle as om
from conftest import load_golden

RNG = np.random.default_rng(12345)


def scalar_map(sigma, coeffs, divisor, restart_every):
    """Closed form on singular values: normalise by the 2-norm of sigma (the
    Frobenius norm of the matrix) and the divisor, then apply the scalar odd
    polynomials, dividing by sqrt(d) at each restart."""
    s = np.asarray(sigma, dtype=np.float64)
    nrm = math.sqrt(float(np.sum(s * s)))
    if nrm == 0:
        return np.zeros_like(s)
    x = s / (math.sqrt(divisor) * nrm)
    for k in range(1, coeffs.shape[0] + 1):
        if restart_every > 0 and k > 1 and (k - 1) % restart_every == 0:
            x = x / math.sqrt(divisor)
        a, b, c = coeffs[k - 1]
        x = a * x + b * x ** 3 + c * x ** 5
    return x


def closed_form(m, coeffs, divisor=1.0, restart_every=0):
    u, s, vt = np.linalg.svd(m, full_matrices=False)
    return (u * scalar_map(s, coeffs, divisor, restart_every)) @ vt


def rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


# ---------------------------------------------------------------- golden

@pytest.mark.parametrize("variant", ["direct", "gram"])
@pytest.mark.parametrize("kind", ["cubic", "quintic"])
def test_golden_scalar_mona_two_steps(variant, kind):
    g = load_golden("mona_scalar_two_steps.txt")
    coeffs = oracle.coefficient_table(kind, 5)
    hp = dict(lr=g["lr"], mu=g["mu"], weight_decay=g["weight_decay"], coeffs=coeffs,
              variant=variant, beta_a=g["beta_a"], alpha=g["alpha"])
    w = np.array([[g["w0"]]])
    m = np.zeros((1, 1))
    a = np.zeros((1, 1))
    prev = np.zeros((1, 1))
    r0 = oracle.muon_step_matrix(w, np.array([[g["g0"]]]), m, accel=a, prev_grad=prev, step=0, **hp)
    assert r0["accel"][0, 0] == pytest.approx(g["a1"], abs=1e-15)
    assert r0["momentum"][0, 0] == pytest.approx(g["m1"], abs=1e-15)
    assert r0["ortho"][0, 0] == pytest.approx(g["o1"], abs=1e-15)
    assert r0["weight"][0, 0] == pytest.approx(g["w1"], abs=1e-14)
    r1 = oracle.muon_step_matrix(r0["weight"], np.array([[g["g1"]]]), r0["momentum"], accel=r0["accel"],
                                 prev_grad=r0["prev_grad"], step=1, **hp)
    assert r1["accel"][0, 0] == pytest.approx(g["a2"], abs=1e-14)
    assert r1["momentum"][0, 0] == pytest.approx(g["m2"], abs=1e-14)
    assert r1["ortho"][0, 0] == pytest.approx(g["o2"], abs=1e-14)
    assert r1["weight"][0, 0] == pytest.approx(g["w2"], abs=1e-12)


@pytest.mark.parametrize("variant", ["direct", "gram"])
def test_golden_diag_2x2_cubic(variant):
    g = load_golden("diag_2x2_cubic.txt")
    m = np.diag([g["m00"], g["m11"]])
    x0 = oracle.frobenius_normalize(m)
    np.testing.assert_allclose(np.diag(x0), [g["x00"], g["x11"]], atol=1e-15)
    o1 = oracle.newton_schulz(x0, oracle.coefficient_table("cubic", 1), variant)
    np.testing.assert_allclose(o1, np.diag([g["o00"], g["o11"]]), atol=1e-15)
    o2 = oracle.newton_schulz(x0, oracle.coefficient_table("cubic", 2), variant)
    np.testing.assert_allclose(o2, np.diag([g["o00_two"], g["o11_two"]]), atol=1e-15)


# ---------------------------------------------------------------- closed form

SHAPES = [(7, 13), (13, 7), (16, 16), (40, 9), (5, 64), (1, 9), (9, 1)]


def _coeff_sets():
    custom = np.array([[2.0, -1.4, 0.45], [1.9, -1.3, 0.4], [1.7, -0.9, 0.2], [1.5, -0.5, 0.0]])
    return [("cubic", oracle.coefficient_table("cubic", 5)),
            ("quintic", oracle.coefficient_table("quintic", 5)),
            ("custom", custom)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("variant", ["direct", "gram"])
def test_closed_form_matches_svd(shape, variant):
    m = RNG.standard_normal(shape)
    for name, coeffs in _coeff_sets():
        for d, r in [(1.0, 0), (1.03, 0), (1.03, 3), (1.05, 1), (1.02, 2)]:
            x0 = oracle.frobenius_normalize(m, d)
            o = oracle.newton_schulz(x0, coeffs, variant, d, r)
            ref = closed_form(m, coeffs, d, r)
            assert o.shape == m.shape
            assert rel(o, ref) < 1e-12, (name, d, r, rel(o, ref))


def test_closed_form_wide_spectrum():
    """Singular values spread over 10 decades, like the synthetic gradients."""
    u, _ = np.linalg.qr(RNG.standard_normal((48, 24)))
    v, _ = np.linalg.qr(RNG.standard_normal((24, 24)))
    s = 10.0 ** RNG.uniform(-10, 0, 24)
    m = (u * s) @ v.T
    coeffs = oracle.coefficient_table("quintic", 5)
    for variant in ("direct", "gram"):
        o = oracle.newton_schulz(oracle.frobenius_normalize(m, 1.03), coeffs, variant, 1.03, 3)
        ref = (u * scalar_map(s, coeffs, 1.03, 3)) @ v.T
        assert rel(o, ref) < 1e-12


# ---------------------------------------------------------------- polar factor

@pytest.mark.parametrize("variant", ["direct", "gram"])
@pytest.mark.parametrize("shape", [(8, 16), (16, 8), (12, 12)])
def test_converges_to_polar_factor(variant, shape):
    """polar(X) = U V^T (Gram Newton-Schulz post): many steps reach it."""
    k = min(shape)
    u, _ = np.linalg.qr(RNG.standard_normal((shape[0], k)))
    v, _ = np.linalg.qr(RNG.standard_normal((shape[1], k)))
    s = np.linspace(1.0, 3.0, k)  # condition number 3
    m = (u * s) @ v.T
    uu, _, vvt = np.linalg.svd(m, full_matrices=False)
    polar = uu @ vvt
    for kind, steps in [("cubic", 40), ("quintic", 25)]:
        o = oracle.newton_schulz(oracle.frobenius_normalize(m), oracle.coefficient_table(kind, steps), variant)
        assert np.linalg.norm(o - polar) < 1e-12
        assert np.linalg.norm(o.T @ o - np.eye(shape[1]) if shape[0] >= shape[1] else o @ o.T - np.eye(shape[0])) < 1e-12


@pytest.mark.parametrize("variant", ["direct", "gram"])
def test_orthogonal_input_is_fixed_up_to_scalar(variant):
    """M = Q with orthonormal rows: all singular values 1, so O = phi(1/sqrt(s)) Q
    exactly, and polar(Q) = Q is reached as the step count grows."""
    q, _ = np.linalg.qr(RNG.standard_normal((32, 8)))
    q = q.T  # 8 x 32, orthonormal rows
    coeffs = oracle.coefficient_table("quintic", 5)
    o = oracle.newton_schulz(oracle.frobenius_normalize(q), coeffs, variant)
    x = 1.0 / math.sqrt(8.0)
    for _ in range(5):
        x = 15 / 8 * x - 5 / 4 * x ** 3 + 3 / 8 * x ** 5
    np.testing.assert_allclose(o, x * q, atol=1e-14)
    o_long = oracle.newton_schulz(oracle.frobenius_normalize(q), oracle.coefficient_table("quintic", 30), variant)
    np.testing.assert_allclose(o_long, q, atol=1e-13)


# ---------------------------------------------------------------- direct == gram

@pytest.mark.parametrize("shape", [(10, 30), (30, 10), (17, 17), (3, 50)])
def test_direct_equals_gram(shape):
    m = RNG.standard_normal(shape)
    for name, coeffs in _coeff_sets():
        for d, r in [(1.0, 0), (1.03, 3), (1.05, 2)]:
            x0 = oracle.frobenius_normalize(m, d)
            od = oracle.newton_schulz_direct(x0, coeffs, d, r)
            og = oracle.newton_schulz_gram(x0, coeffs, d, r)
            assert rel(od, og) < 1e-13, (name, d, r)


def test_restart_without_divisor_is_noop():
    m = RNG.standard_normal((12, 20))
    coeffs = oracle.coefficient_table("quintic", 6)
    x0 = oracle.frobenius_normalize(m)
    base = oracle.newton_schulz_gram(x0, coeffs, 1.0, 0)
    for r in (1, 2, 3, 5):
        assert rel(oracle.newton_schulz_gram(x0, coeffs, 1.0, r), base) < 1e-13


# ---------------------------------------------------------------- invariants

@pytest.mark.parametrize("variant", ["direct", "gram"])
def test_invariants(variant):
    m = RNG.standard_normal((9, 21))
    coeffs = oracle.coefficient_table("quintic", 5)

    def ns(x):
        return oracle.newton_schulz(oracle.frobenius_normalize(x, 1.03), coeffs, variant, 1.03, 3)

    o = ns(m)
    # transpose
    assert rel(ns(m.T), o.T) < 1e-13
    # orthogonal equivariance
    p, _ = np.linalg.qr(RNG.standard_normal((9, 9)))
    q, _ = np.linalg.qr(RNG.standard_normal((21, 21)))
    assert rel(ns(p @ m @ q), p @ o @ q) < 1e-12
    # permutation equivariance
    pr, pc = RNG.permutation(9), RNG.permutation(21)
    assert rel(ns(m[pr][:, pc]), o[pr][:, pc]) < 1e-13
    # positive scale invariance (exact reading: no epsilon)
    for c in (1e-8, 3.0, 1e6):
        assert rel(ns(c * m), o) < 1e-13
    # sign flips the output
    assert rel(ns(-m), -o) < 1e-14


@pytest.mark.parametrize("variant", ["direct", "gram"])
def test_singular_values_driven_toward_one(variant):
    """Cubic and quintic satisfy x <= p(x) <= 1 on [0, 1]: singular values rise
    toward 1 monotonically, keep their order, and ||O^T O - I|| never grows."""
    m = RNG.standard_normal((16, 40))
    x0 = oracle.frobenius_normalize(m)
    s0 = np.linalg.svd(x0, compute_uv=False)
    for kind in ("cubic", "quintic"):
        prev_dev, prev_s = np.inf, s0
        for k in range(0, 9):
            o = oracle.newton_schulz(x0, oracle.coefficient_table(kind, k), variant)
            s = np.linalg.svd(o, compute_uv=False)
            assert np.all(s <= 1.0 + 1e-13)
            assert np.all(s >= prev_s - 1e-13)
            assert np.all(np.diff(s) <= 1e-13)  # order kept (descending)
            dev = np.linalg.norm(o @ o.T - np.eye(16))
            assert dev <= prev_dev + 1e-13
            prev_dev, prev_s = dev, s


# ---------------------------------------------------------------- special cases

def test_zero_steps_returns_normalised_input():
    m = RNG.standard_normal((6, 11))
    x0 = oracle.frobenius_normalize(m, 1.03)
    assert math.isclose(np.linalg.norm(x0), 1 / math.sqrt(1.03), rel_tol=1e-14)
    for variant in ("direct", "gram"):
        o = oracle.newton_schulz(x0, oracle.coefficient_table("quintic", 0), variant, 1.03, 3)
        np.testing.assert_array_equal(o, x0)


def test_zero_gradient_is_pure_decay():
    w = RNG.standard_normal((5, 7))
    r = oracle.muon_step_matrix(w, np.zeros((5, 7)), np.zeros((5, 7)), lr=0.1, mu=0.9, weight_decay=0.01,
                                coeffs=oracle.coefficient_table("quintic", 5))
    np.testing.assert_array_equal(r["ortho"], 0.0)
    np.testing.assert_allclose(r["weight"], (1 - 0.1 * 0.01) * w, rtol=0, atol=1e-15)


@pytest.mark.parametrize("variant", ["direct", "gram"])
def test_alpha_zero_recovers_plain_muon(variant):
    """With alpha = 0 the acceleration buffer never reaches the momentum."""
    shape = (8, 12)
    coeffs = oracle.coefficient_table("quintic", 5)
    w = RNG.standard_normal(shape)
    hp = dict(lr=0.02, mu=0.95, weight_decay=0.01, coeffs=coeffs, variant=variant)
    m_a, m_p, a, prev, wa, wp = np.zeros(shape), np.zeros(shape), np.zeros(shape), np.zeros(shape), w, w
    for step in range(3):
        g = RNG.standard_normal(shape)
        ra = oracle.muon_step_matrix(wa, g, m_a, accel=a, prev_grad=prev, step=step, beta_a=0.9, alpha=0.0, **hp)
        rp = oracle.muon_step_matrix(wp, g, m_p, **hp)
        np.testing.assert_array_equal(ra["momentum"], rp["momentum"])
        np.testing.assert_array_equal(ra["ortho"], rp["ortho"])
        np.testing.assert_array_equal(ra["weight"], rp["weight"])
        m_a, a, prev, wa = ra["momentum"], ra["accel"], ra["prev_grad"], ra["weight"]
        m_p, wp = rp["momentum"], rp["weight"]
    assert np.any(a != 0)  # the EMA itself did run


def test_mona_first_step_has_no_difference():
    g = RNG.standard_normal((4, 4))
    gt, a, prev = oracle.mona_acceleration(g, np.zeros((4, 4)), np.full((4, 4), 7.0), 0, 0.9, 0.5)
    np.testing.assert_array_equal(a, 0.0)
    np.testing.assert_array_equal(gt, g)
    np.testing.assert_array_equal(prev, g)


def test_mona_ema_closed_form():
    """Over a gradient sequence the EMA equals its unrolled sum
    A_k = (1 - beta) sum_j beta^(k-j) D_j, with D_0 = 0."""
    beta, alpha = 0.9, 0.5
    gs = [RNG.standard_normal((3, 5)) for _ in range(6)]
    a, prev = np.zeros((3, 5)), np.zeros((3, 5))
    for k, g in enumerate(gs):
        gt, a, prev = oracle.mona_acceleration(g, a, prev, k, beta, alpha)
        ds = [np.zeros((3, 5))] + [gs[j] - gs[j - 1] for j in range(1, k + 1)]
        unrolled = (1 - beta) * sum(beta ** (k - j) * ds[j] for j in range(k + 1))
        np.testing.assert_allclose(a, unrolled, atol=1e-14)
        np.testing.assert_allclose(gt, g + alpha * unrolled, atol=1e-14)


def test_momentum_closed_form():
    mu = 0.95
    gs = [RNG.standard_normal((3, 3)) for _ in range(5)]
    m = np.zeros((3, 3))
    for k, g in enumerate(gs):
        m = oracle.momentum_update(m, g, mu)
        np.testing.assert_allclose(m, sum(mu ** (k - j) * gs[j] for j in range(k + 1)), atol=1e-14)


def test_nan_stays_in_its_matrix():
    coeffs = oracle.coefficient_table("quintic", 5)
    params = [dict(weight=np.ones((3, 4)), grad=np.full((3, 4), np.nan), momentum=np.zeros((3, 4))),
              dict(weight=np.ones((3, 4)), grad=RNG.standard_normal((3, 4)), momentum=np.zeros((3, 4)))]
    res = oracle.muon_step(params, lr=0.02, mu=0.95, weight_decay=0.01, coeffs=coeffs)
    assert np.all(np.isnan(res[0]["weight"]))
    assert np.all(np.isfinite(res[1]["weight"]))


# ---------------------------------------------------------------- planted mistakes

def _check_all(ns_fn):
    """Run the closed-form and golden checks against a candidate NS function."""
    m = RNG.standard_normal((7, 13))
    sq = RNG.standard_normal((9, 9))
    for name, coeffs in _coeff_sets():
        for d, r in [(1.0, 0), (1.03, 3)]:
            for mm in (m, m.T, sq):
                try:
                    o = ns_fn(oracle.frobenius_normalize(mm, d), coeffs, d, r)
                except ValueError:   # shape mismatch
                    return False
                if o.shape != mm.shape or rel(o, closed_form(mm, coeffs, d, r)) > 1e-10:
                    return False
    return True


def test_planted_mistakes_are_caught():
    """Each plausible slip in the matrix iteration fails the closed-form pin."""
    assert _check_all(om.newton_schulz_direct) and _check_all(om.newton_schulz_gram)

    def wrong_gram_side(x0, coeffs, d, r):      # X^T X where X X^T belongs
        x = x0.copy()
        for k in range(1, coeffs.shape[0] + 1):
            a, b, c = coeffs[k - 1]
            if om.restart_due(k, r):
                x = x / math.sqrt(d)
            g = x.T @ x
            x = a * x + (b * g + c * g @ g) @ x
        return x

    def dropped_square(x0, coeffs, d, r):
        c0 = coeffs.copy()
        c0[:, 2] = 0.0
        return om.newton_schulz_direct(x0, c0, d, r)

    def gram_rp_only(x0, coeffs, d, r):       # R <- R P instead of P R P
        y = x0.T if x0.shape[0] < x0.shape[1] else x0
        n = y.shape[1]
        rr, q = y.T @ y, np.eye(n)
        for k in range(1, coeffs.shape[0] + 1):
            a, b, c = coeffs[k - 1]
            if om.restart_due(k, r):
                y = (y @ q) / math.sqrt(d)
                rr, q = y.T @ y, np.eye(n)
            p = a * np.eye(n) + b * rr + c * rr @ rr
            q = q @ p
            rr = rr @ p
        o = y @ q
        return o.T if x0.shape[0] < x0.shape[1] else o

    def divisor_on_gram_not_iterate(x0, coeffs, d, r):   # restart divides X by d, not sqrt(d)
        x = x0.T if x0.shape[0] > x0.shape[1] else x0
        for k in range(1, coeffs.shape[0] + 1):
            a, b, c = coeffs[k - 1]
            if om.restart_due(k, r):
                x = x / d
            g = x @ x.T
            x = a * x + (b * g + c * g @ g) @ x
        return x.T if x0.shape[0] > x0.shape[1] else x

    def sign_slip(x0, coeffs, d, r):
        c0 = coeffs.copy()
        c0[:, 1] = -c0[:, 1]
        return om.newton_schulz_direct(x0, c0, d, r)

    for bad in (wrong_gram_side, dropped_square, gram_rp_only, divisor_on_gram_not_iterate, sign_slip):
        assert not _check_all(bad), bad.__name__


# ---------------------------------------------------------------- MONA-Lite

BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def test_round_bf16_hand_values():
    """bfloat16 rounding from its definition: 8 significant bits, ties to even,
    float32's exponent range, fixed spacing 2^-133 below 2^-126."""
    r = oracle.round_bf16
    cases = [
        (1.0, 1.0),
        (1.0 + 2.0 ** -8, 1.0),                       # tie -> even (1.0000000)
        (1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -6),       # tie -> even (1.0000010)
        (1.0 + 2.0 ** -8 + 2.0 ** -20, 1.0 + 2.0 ** -7),
        (-(1.0 + 2.0 ** -8 + 2.0 ** -20), -(1.0 + 2.0 ** -7)),
        (0.1, 0.10009765625),
        (2.0 ** -130, 2.0 ** -130),                   # subnormal, exact
        (2.0 ** -134, 0.0),                           # half the subnormal spacing -> even (0)
        (3 * 2.0 ** -134, 2.0 ** -132),               # 1.5 spacings -> 2
        (BF16_MAX, BF16_MAX),                          # (2 - 2^-7) 2^127, largest finite
        (BF16_MAX + 2.0 ** 118, BF16_MAX),             # below half a spacing (2^120)
        (BF16_MAX + 2.0 ** 119, np.inf),               # tie -> even -> 2^128 overflows
        (4.0e38, np.inf),
        (-4.0e38, -np.inf),
        (0.0, 0.0),
    ]
    for x, want in cases:
        assert r(np.array([x]))[0] == want, (x, r(np.array([x]))[0], want)
    assert np.isnan(r(np.array([np.nan]))[0])
    assert r(np.array([np.inf]))[0] == np.inf


def test_round_bf16_matches_torch_on_float32_inputs():
    """Float32 inputs round once to bfloat16: torch's conversion must agree."""
    import torch
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(20000) * 10.0 ** rng.uniform(-30, 30, 20000)).astype(np.float32).astype(np.float64)
    want = torch.from_numpy(x).float().to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(oracle.round_bf16(x), want)


def test_mona_lite_exact_state_equals_mona():
    """Without the bfloat16 rounding, the Lite state reproduces MONA's A_k and
    G~_k exactly (the identity A_{k+1} = C_k + (1 - beta_a) G_{k+1})."""
    rng = np.random.default_rng(6)
    beta, alpha = 0.9, 0.5
    a = np.zeros((5, 7))
    prev = np.zeros((5, 7))
    c = None
    for step in range(6):
        g = rng.standard_normal((5, 7))
        gt_m, a, prev = oracle.mona_acceleration(g, a, prev, step, beta, alpha)
        gt_l, a_l, c = oracle.mona_lite_acceleration(g, c, step, beta, alpha, store=lambda v: v)
        np.testing.assert_allclose(a_l, a, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(gt_l, gt_m, rtol=1e-12, atol=1e-13)


def test_mona_lite_rounded_state_stays_close():
    """With the bfloat16 state the acceleration differs from MONA's by the
    state's rounding only: relative Frobenius error below 1e-2 after 8 steps."""
    rng = np.random.default_rng(7)
    beta, alpha = 0.9, 0.5
    a = np.zeros((16, 24))
    prev = np.zeros((16, 24))
    c = None
    for step in range(8):
        g = rng.standard_normal((16, 24))
        _, a, prev = oracle.mona_acceleration(g, a, prev, step, beta, alpha)
        _, a_l, c = oracle.mona_lite_acceleration(g, c, step, beta, alpha)
        assert np.all(oracle.round_bf16(c) == c)        # the stored state is bfloat16
    assert np.linalg.norm(a_l - a) / np.linalg.norm(a) < 1e-2
    assert np.linalg.norm(a_l - a) > 0                   # and the rounding is visible


@pytest.mark.parametrize("variant", ["direct", "gram"])
def test_golden_scalar_mona_lite_two_steps(variant):
    g = load_golden("mona_lite_scalar_two_steps.txt")
    coeffs = oracle.coefficient_table("quintic", 5)
    w, m, c = np.array([[g["w0"]]]), np.zeros((1, 1)), None
    for step, (gk, a_want, m_want, w_want, c_want) in enumerate(
            [(g["g0"], g["a1"], g["m1"], g["w1"], g["c1"]), (g["g1"], g["a2"], g["m2"], g["w2"], g["c2"])]):
        r = oracle.muon_step_matrix(w, np.array([[gk]]), m, lr=g["lr"], mu=g["mu"], weight_decay=g["weight_decay"],
                                    coeffs=coeffs, variant=variant, gamma=g["gamma"], beta_a=g["beta_a"],
                                    alpha=g["alpha"], step=step, lite_state=c if c is not None else np.zeros((1, 1)))
        assert r["accel"][0, 0] == pytest.approx(a_want, abs=1e-15)
        assert r["momentum"][0, 0] == pytest.approx(m_want, abs=1e-14)
        assert r["weight"][0, 0] == pytest.approx(w_want, abs=1e-12)
        assert r["lite_state"][0, 0] == c_want
        w, m, c = r["weight"], r["momentum"], r["lite_state"]


def test_mona_lite_alpha_zero_is_plain_muon():
    """alpha = 0: the momentum, and so the step, equal plain Muon's bitwise."""
    rng = np.random.default_rng(8)
    coeffs = oracle.coefficient_table("quintic", 5)
    w = rng.standard_normal((6, 9))
    m_l = m_p = np.zeros((6, 9))
    w_l = w_p = w
    c = np.zeros((6, 9))
    for step in range(3):
        g = rng.standard_normal((6, 9))
        rl = oracle.muon_step_matrix(w_l, g, m_l, lr=0.02, mu=0.95, weight_decay=0.01, coeffs=coeffs, beta_a=0.9,
                                     alpha=0.0, step=step, lite_state=c)
        rp = oracle.muon_step_matrix(w_p, g, m_p, lr=0.02, mu=0.95, weight_decay=0.01, coeffs=coeffs)
        np.testing.assert_array_equal(rl["momentum"], rp["momentum"])
        np.testing.assert_array_equal(rl["weight"], rp["weight"])
        w_l, m_l, c = rl["weight"], rl["momentum"], rl["lite_state"]
        w_p, m_p = rp["weight"], rp["momentum"]


# ---------------------------------------------------------------- AdamW (vector parameters)

def test_adamw_matches_torch_adamw_float64():
    """The textbook decoupled AdamW against torch.optim.AdamW (an independent
    implementation) in float64 over 5 steps."""
    import torch
    rng = np.random.default_rng(9)
    hp = dict(lr=3e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
    p0 = rng.standard_normal(257)
    tp = torch.nn.Parameter(torch.from_numpy(p0.copy()))
    opt = torch.optim.AdamW([tp], lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
                            weight_decay=hp["weight_decay"])
    p, m, v = p0.copy(), np.zeros(257), np.zeros(257)
    for step in range(5):
        g = rng.standard_normal(257) * 10.0 ** rng.uniform(-3, 1)
        tp.grad = torch.from_numpy(g.copy())
        opt.step()
        p, m, v = oracle.adamw_step(p, g, m, v, step=step, **hp)
        np.testing.assert_allclose(p, tp.detach().numpy(), rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(m, opt.state[tp]["exp_avg"].numpy(), rtol=1e-13, atol=1e-16)
        np.testing.assert_allclose(v, opt.state[tp]["exp_avg_sq"].numpy(), rtol=1e-13, atol=1e-18)


def test_adamw_first_step_is_signed_step():
    """At t = 1 the bias corrections give m^ = g and v^ = g^2, so the update
    is lr g / (|g| + eps): a step of ~lr against the gradient's sign."""
    g = np.array([3.0, -0.5, 1e-3, 0.0])
    p, m, v = oracle.adamw_step(np.zeros(4), g, np.zeros(4), np.zeros(4), step=0, lr=0.01, beta1=0.9,
                                beta2=0.999, eps=1e-8, weight_decay=0.0)
    np.testing.assert_allclose(p, -0.01 * g / (np.abs(g) + 1e-8), rtol=1e-14, atol=0)
    np.testing.assert_allclose(m, 0.1 * g)
    np.testing.assert_allclose(v, 0.001 * g * g)


def test_adamw_zero_gradient_is_pure_decay():
    p0 = np.array([1.0, -2.0])
    p, _, _ = oracle.adamw_step(p0, np.zeros(2), np.zeros(2), np.zeros(2), step=3, lr=0.1, beta1=0.9,
                                beta2=0.99, eps=1e-8, weight_decay=0.5)
    np.testing.assert_allclose(p, p0 * (1 - 0.1 * 0.5))

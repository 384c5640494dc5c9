"""fp64 reference (oracle) for one Muon / MONA optimizer step.

TEST INFRASTRUCTURE ONLY -- imported by ``tests/``, ``__graft_entry__.smoke()``
and ``bench.py``'s ``cpu_baseline`` leg, never by the product path.  It shares
no code with the HIP library.

Sources (the pages this follows):

* "Technische Samenvatting: MONA - Muon-optimizer met Nesterov-versnelling"
  (gist.science, paper 2605.26842), section 2 "Methodologie", sub-section
  "Kernalgoritme", steps 1-4: the gradient difference, the acceleration EMA,
  the curvature-aware gradient, heavy-ball momentum, Newton-Schulz
  orthogonalisation and the decoupled weight-decay update.  Sub-section
  "Ontwerprichtlijnen": the acceleration is applied before orthogonalisation.
* The same MONA summary, "Efficiëntie en Implementatie" (MONA-Lite): the
  auxiliary state is stored in bfloat16 and the gradient difference is
  formed in place, so no separate previous-gradient buffer is kept.
* The Telegram post on Gram Newton-Schulz (quant_prune_distill, post 677),
  main body: polar(X) = U V^T for X = U S V^T; the Gram form
  X (X^T X)^{-1/2} with the inverse square root found by Newton-Schulz on the
  smaller Gram matrix; restarts to control the Gram's eigenvalues; a 1.02-1.05
  safety divisor so that the eigenvalues land in [0, 1].
* The same MONA summary, "Ontwerprichtlijnen": vector-shaped parameters
  (embeddings, biases) keep AdamW, as in Muon.  The pages give AdamW no
  formula or hyper-parameters; the oracle follows the textbook decoupled
  form (I. Loshchilov, F. Hutter, "Decoupled Weight Decay Regularization",
  ICLR 2019, Algorithm 2, with the bias corrections of Adam).
* Textbook Newton-Schulz for the polar factor (N. J. Higham, "Functions of
  Matrices", 2008, section 8.3): the cubic map X <- (3X - X X^T X)/2, which
  needs sigma_max(X) < sqrt(3); Frobenius normalisation guarantees
  sigma_max <= 1.
* "LiMuon: Light and Fast Muon Optimizer for Large Models" (digest,
  arxiv.sitesynth.xyz 2509.14562v1), section "Метод": momentum as in Muon,
  with the orthogonalisation done through a randomized SVD of the momentum.
  The randomized SVD is the textbook one (N. Halko, P.-G. Martinsson,
  J. A. Tropp, "Finding structure with randomness", SIAM Review 53(2),
  2011): Algorithm 4.4 (randomized subspace iteration: a Gaussian test
  matrix, power iterations with re-orthonormalisation) followed by
  Algorithm 5.1 (direct SVD of the small projected matrix).

Readings of points the pages leave open (each is listed with its reason in the
design notes):

* Polynomial step k is p_k(x) = a_k x + b_k x^3 + c_k x^5, applied to the
  matrix as X <- a_k X + (b_k A + c_k A^2) X with A = X X^T.  The cubic family
  member is (1.5, -0.5, 0); the quintic one is (15/8, -5/4, 3/8), the next
  member of the same family with p(1) = 1, p'(1) = p''(1) = 0.
* No epsilon in the normalisation: X0 = M / (sqrt(d) ||M||_F), and the zero
  matrix gives O = 0.
* The safety divisor d scales the Gram's eigenvalues by 1/d (the iterate by
  1/sqrt(d)) at the start and at every restart.  The direct variant applies the
  identical scalar schedule, so both variants compute the same function.
* A restart, with period r > 0, happens before 1-based step k when k > 1 and
  (k - 1) mod r == 0: the iterate Y Q is materialised (and divided by
  sqrt(d)), its Gram recomputed, and the accumulated factor reset to I.
* MONA's first step has no previous gradient: D_0 = 0.
* MONA-Lite keeps one bfloat16 state C_k = beta_a A_k - (1 - beta_a) G_k, so
  that A_{k+1} = C_k + (1 - beta_a) G_{k+1} is MONA's A_{k+1} exactly in real
  arithmetic and G_{k-1} is never stored; C is rounded to bfloat16 (nearest,
  ties to even) each time it is stored.
* gamma (the scale on O in the update) is a per-matrix number, default 1.
* LiMuon (the digest names the method only): O = U_k V_k^T built from the
  rank-k randomized SVD of the momentum, sketching the long side (the wide
  orientation X, s x l, s <= l: Y = X Omega with a Gaussian test matrix
  Omega of l x (k + p), drawn by the caller and passed in), q power
  iterations, and directions whose sketched singular value is at most
  rcond * sigma_1 dropped (a null direction maps to zero, as p(0) = 0 does
  for Newton-Schulz).  Rank k, oversampling p, q and rcond are arguments.

Everything is computed in float64 from inputs upcast exactly from their stored
dtype.  There is no blocking, fusion or reordering beyond what the steps
state; every matrix product is a plain numpy ``@``.
"""
from __future__ import annotations

import math
from typing import Iterable

import numpy as np

# Cubic member: p(x) = (3x - x^3)/2, textbook Newton-Schulz (Higham 2008, 8.3).
CUBIC = (1.5, -0.5, 0.0)
# Quintic member: p(x) = (15x - 10x^3 + 3x^5)/8.
QUINTIC = (15.0 / 8.0, -5.0 / 4.0, 3.0 / 8.0)


def coefficient_table(kind, steps: int) -> np.ndarray:
    """Return a [steps, 3] float64 table of (a, b, c) per Newton-Schulz step.

    ``kind`` is "cubic", "quintic", or an explicit sequence of (a, b, c)
    triples (one per step).
    """
    if isinstance(kind, str):
        base = {"cubic": CUBIC, "quintic": QUINTIC}[kind]
        return np.tile(np.asarray(base, dtype=np.float64), (steps, 1))
    table = np.asarray(kind, dtype=np.float64).reshape(-1, 3)
    if table.shape[0] != steps:
        raise ValueError("coefficient table has %d rows, expected %d" % (table.shape[0], steps))
    return table


def restart_due(k: int, restart_every: int) -> bool:
    """True when a restart precedes 1-based Newton-Schulz step ``k``."""
    return restart_every > 0 and k > 1 and (k - 1) % restart_every == 0


def mona_acceleration(grad, accel, prev_grad, step: int, beta_a: float, alpha: float):
    """MONA steps 1-3 (MONA summary, section 2, Kernalgoritme).

    D_k = G_k - G_{k-1}           (D_0 = 0: there is no previous gradient)
    A_k = beta_a A_{k-1} + (1 - beta_a) D_k
    G~_k = G_k + alpha A_k
    Returns (G~_k, A_k, new previous gradient = G_k).
    """
    g = np.asarray(grad, dtype=np.float64)
    if step == 0:
        diff = np.zeros_like(g)
    else:
        diff = g - np.asarray(prev_grad, dtype=np.float64)
    a_new = beta_a * np.asarray(accel, dtype=np.float64) + (1.0 - beta_a) * diff
    g_tilde = g + alpha * a_new
    return g_tilde, a_new, g.copy()


def round_bf16(x) -> np.ndarray:
    """Round to the nearest bfloat16 value (ties to even), returned as float64.

    bfloat16 keeps float32's exponent range with 8 significant bits: normal
    numbers are multiples of 2^(e-7) for 2^e <= |x| < 2^(e+1), e >= -126;
    below 2^-126 the spacing is the fixed 2^-133; magnitudes that round
    beyond the largest finite value (2 - 2^-7) 2^127 become infinity.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, dtype=np.float64, copy=True)
    finite = np.isfinite(x) & (x != 0.0)
    v = x[finite]
    _, e = np.frexp(v)                      # v = f 2^e, 0.5 <= |f| < 1, so 2^(e-1) <= |v|
    exp = np.maximum(e - 1, -126)           # exponent of the leading bit (subnormals: -126)
    quantum = np.ldexp(1.0, exp - 7)
    r = np.rint(v / quantum) * quantum      # rint rounds halves to even
    big = np.ldexp(2.0 - 2.0 ** -7, 127)
    r = np.where(np.abs(r) > big, np.copysign(np.inf, v), r)
    out[finite] = r
    return out


def mona_lite_acceleration(grad, state, step: int, beta_a: float, alpha: float, store=round_bf16):
    """MONA-Lite (MONA summary, "Efficiëntie en Implementatie"): MONA steps
    1-3 with a single bfloat16 state instead of A and G_{k-1}.

    The state is C_{k-1} = beta_a A_{k-1} - (1 - beta_a) G_{k-1}, so
        A_k  = C_{k-1} + (1 - beta_a) G_k      (= beta_a A_{k-1} + (1 - beta_a) D_k)
        G~_k = G_k + alpha A_k
        C_k  = store(beta_a A_k - (1 - beta_a) G_k)
    with A_0 = 0 on the first step (no previous gradient).  ``store`` is the
    state's storage rounding (bfloat16).  Returns (G~_k, A_k, C_k).
    """
    g = np.asarray(grad, dtype=np.float64)
    if step == 0:
        a_new = np.zeros_like(g)
    else:
        a_new = np.asarray(state, dtype=np.float64) + (1.0 - beta_a) * g
    g_tilde = g + alpha * a_new
    c_new = store(beta_a * a_new - (1.0 - beta_a) * g)
    return g_tilde, a_new, c_new


def momentum_update(momentum, g_tilde, mu: float):
    """Heavy-ball momentum M_k = mu M_{k-1} + G~_k (MONA summary, step 4)."""
    return mu * np.asarray(momentum, dtype=np.float64) + np.asarray(g_tilde, dtype=np.float64)


def frobenius_normalize(m, divisor: float = 1.0):
    """X0 = M / (sqrt(d) ||M||_F); the zero matrix maps to zero.

    With ||X0||_F = 1/sqrt(d), every singular value of X0 is at most
    1/sqrt(d) <= 1, so every eigenvalue of the Gram matrix lies in [0, 1/d]
    (Gram Newton-Schulz post: eigenvalues must land in [0, 1]).
    """
    m = np.asarray(m, dtype=np.float64)
    norm = math.sqrt(float(np.sum(m * m)))
    if norm == 0.0:
        return np.zeros_like(m)
    return m / (math.sqrt(divisor) * norm)


def newton_schulz_direct(x0, coeffs: np.ndarray, divisor: float = 1.0, restart_every: int = 0):
    """Direct Newton-Schulz on X (MONA summary step 4 'Newton-Schulz(M_k)';
    Gram Newton-Schulz post: odd matrix polynomials in X).

    Works in the wide orientation (rows <= cols), so A = X X^T is the smaller
    square; a tall input is transposed in and out.
    """
    x = np.asarray(x0, dtype=np.float64)
    tall = x.shape[0] > x.shape[1]
    if tall:
        x = x.T
    x = x.copy()
    inv_sqrt_d = 1.0 / math.sqrt(divisor)
    for k in range(1, coeffs.shape[0] + 1):
        a, b, c = coeffs[k - 1]
        if restart_due(k, restart_every):
            x = x * inv_sqrt_d
        gram = x @ x.T
        x = a * x + (b * gram + c * (gram @ gram)) @ x
    return x.T if tall else x


def newton_schulz_gram(x0, coeffs: np.ndarray, divisor: float = 1.0, restart_every: int = 0):
    """Gram Newton-Schulz: polar(X) = X (X^T X)^{-1/2} with the inverse square
    root built by Newton-Schulz on the smaller Gram matrix (Gram Newton-Schulz
    post, main body), with restarts and the safety divisor.

    Works in the tall orientation Y (rows >= cols), so R = Y^T Y is the smaller
    square.  The accumulated right factor Q is the product of the step
    polynomials P_k = a_k I + b_k R + c_k R^2, and R is carried along as
    P R P, so the tall iterate Y Q is only formed at restarts and at the end.
    """
    y = np.asarray(x0, dtype=np.float64)
    wide = y.shape[0] < y.shape[1]
    if wide:
        y = y.T
    y = y.copy()
    n = y.shape[1]
    eye = np.eye(n)
    inv_sqrt_d = 1.0 / math.sqrt(divisor)
    r = y.T @ y
    q = eye.copy()
    for k in range(1, coeffs.shape[0] + 1):
        a, b, c = coeffs[k - 1]
        if restart_due(k, restart_every):
            y = (y @ q) * inv_sqrt_d
            r = y.T @ y
            q = eye.copy()
        p = a * eye + b * r + c * (r @ r)
        q = q @ p
        r = p @ r @ p
    out = y @ q
    return out.T if wide else out


def newton_schulz(x0, coeffs, variant: str = "direct", divisor: float = 1.0, restart_every: int = 0):
    if variant == "direct":
        return newton_schulz_direct(x0, coeffs, divisor, restart_every)
    if variant == "gram":
        return newton_schulz_gram(x0, coeffs, divisor, restart_every)
    raise ValueError("unknown variant %r" % (variant,))


def limuon_orthogonalize(m, omega, rank: int, power_iters: int = 1, rcond: float = 1e-4):
    """LiMuon's orthogonaliser (LiMuon digest, "Метод": a randomized SVD of
    the momentum in place of Newton-Schulz), as the textbook randomized SVD
    (Halko, Martinsson & Tropp 2011, Algorithms 4.4 and 5.1):

      X = M in its wide orientation (s x l, s <= l; a tall M is transposed
          in and the result transposed back), Omega: l x (k + p) Gaussian
      Y = X Omega,  Q = qr(Y)                       range finder
      q times:  Q~ = qr(X^T Q),  Q = qr(X Q~)       power iterations
      B = Q^T X = U~ S V^T                          SVD of the small matrix
      O = sum over i < k with S_i > rcond S_1 of (Q U~)_i V_i^T

    O is scale-invariant in M (the rcond cutoff is relative) and depends on
    Omega only through the range of X Omega.  M = 0 gives O = 0.
    """
    m = np.asarray(m, dtype=np.float64)
    om = np.asarray(omega, dtype=np.float64)
    tall = m.shape[0] > m.shape[1]
    x = m.T if tall else m
    s, l = x.shape
    if om.shape[0] != l:
        raise ValueError("omega has %d rows, the long side is %d" % (om.shape[0], l))
    if rank < 1 or rank > om.shape[1]:
        raise ValueError("rank must lie in [1, columns of omega]")
    q, _ = np.linalg.qr(x @ om)
    for _ in range(power_iters):
        qt, _ = np.linalg.qr(x.T @ q)
        q, _ = np.linalg.qr(x @ qt)
    b = q.T @ x
    ub, sv, vt = np.linalg.svd(b, full_matrices=False)
    out = np.zeros_like(x)
    if sv.size and sv[0] > 0.0:
        keep = [i for i in range(min(rank, sv.size)) if sv[i] > rcond * sv[0]]
        if keep:
            out = (q @ ub[:, keep]) @ vt[keep, :]
    return out.T if tall else out


def decoupled_update(weight, ortho, lr: float, weight_decay: float, gamma: float = 1.0):
    """W_{k+1} = W_k - eta (gamma O_k + lambda W_k) (MONA summary, step 4)."""
    w = np.asarray(weight, dtype=np.float64)
    return w - lr * (gamma * np.asarray(ortho, dtype=np.float64) + weight_decay * w)


def muon_step_matrix(weight, grad, momentum, *, lr, mu, weight_decay, coeffs,
                     variant="direct", divisor=1.0, restart_every=0, gamma=1.0,
                     accel=None, prev_grad=None, beta_a=0.0, alpha=0.0, step=0, lite_state=None,
                     omega=None, rank=None, power_iters=1, rcond=1e-4):
    """One optimizer step for one weight matrix, in the pages' order.

    MONA (if ``accel`` is given) or MONA-Lite (if ``lite_state`` is given) ->
    momentum -> normalise -> Newton-Schulz (``variant`` "direct" or "gram")
    or LiMuon's randomized SVD (``variant`` "limuon": ``omega``, ``rank``,
    ``power_iters``, ``rcond``; ``coeffs`` unused) -> decoupled update.  The
    acceleration enters before orthogonalisation (MONA summary,
    "Ontwerprichtlijnen").  Returns a dict with every stage's output, all
    float64.
    """
    out = {}
    if lite_state is not None:
        g_tilde, a_new, c_new = mona_lite_acceleration(grad, lite_state, step, beta_a, alpha)
        out["accel"] = a_new
        out["lite_state"] = c_new
    elif accel is not None:
        g_tilde, a_new, prev_new = mona_acceleration(grad, accel, prev_grad, step, beta_a, alpha)
        out["accel"] = a_new
        out["prev_grad"] = prev_new
    else:
        g_tilde = np.asarray(grad, dtype=np.float64)
    m_new = momentum_update(momentum, g_tilde, mu)
    x0 = frobenius_normalize(m_new, divisor)
    if variant == "limuon":
        o = limuon_orthogonalize(m_new, omega, rank, power_iters, rcond)
    else:
        o = newton_schulz(x0, coeffs, variant, divisor, restart_every)
    out["momentum"] = m_new
    out["x0"] = x0
    out["ortho"] = o
    out["weight"] = decoupled_update(weight, o, lr, weight_decay, gamma)
    return out


def adamw_step(param, grad, exp_avg, exp_avg_sq, *, step: int, lr: float, beta1: float, beta2: float,
               eps: float, weight_decay: float):
    """Decoupled AdamW (Loshchilov & Hutter 2019, Algorithm 2) for one tensor;
    ``step`` is 0-based, so t = step + 1 in the bias corrections:
        m = beta1 m + (1 - beta1) g,       v = beta2 v + (1 - beta2) g^2
        m^ = m / (1 - beta1^t),            v^ = v / (1 - beta2^t)
        p = p - lr (m^ / (sqrt(v^) + eps) + weight_decay p)
    Returns (p, m, v) in float64.
    """
    g = np.asarray(grad, dtype=np.float64)
    p = np.asarray(param, dtype=np.float64)
    m = beta1 * np.asarray(exp_avg, dtype=np.float64) + (1.0 - beta1) * g
    v = beta2 * np.asarray(exp_avg_sq, dtype=np.float64) + (1.0 - beta2) * g * g
    t = step + 1
    m_hat = m / (1.0 - beta1 ** t)
    v_hat = v / (1.0 - beta2 ** t)
    p_new = p - lr * (m_hat / (np.sqrt(v_hat) + eps) + weight_decay * p)
    return p_new, m, v


def muon_step(params: Iterable[dict], *, lr, mu, weight_decay, coeffs, variant="direct",
              divisor=1.0, restart_every=0, beta_a=0.0, alpha=0.0, step=0) -> list:
    """Apply :func:`muon_step_matrix` to each param dict independently.

    Each dict holds ``weight``, ``grad``, ``momentum`` and optionally
    ``accel`` and ``prev_grad`` (MONA), ``lite_state`` (MONA-Lite) and
    ``gamma`` (numpy arrays / floats).
    """
    results = []
    for p in params:
        results.append(muon_step_matrix(
            p["weight"], p["grad"], p["momentum"], lr=lr, mu=mu, weight_decay=weight_decay,
            coeffs=coeffs, variant=variant, divisor=divisor, restart_every=restart_every,
            gamma=p.get("gamma", 1.0), accel=p.get("accel"), prev_grad=p.get("prev_grad"),
            beta_a=beta_a, alpha=alpha, step=step, lite_state=p.get("lite_state")))
    return results

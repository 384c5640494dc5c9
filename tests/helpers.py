"""Shared helpers for the GPU parity tests: run libmuon and the oracle on the
same seeded inputs and compare them per matrix."""
import numpy as np
import torch

import oracle

TOL_F32 = 1e-5      # relative Frobenius, fp32 Newton-Schulz operands
TOL_16 = 2e-2       # relative Frobenius, fp16 / bf16 operands with fp32 accumulation
TOL_STATE = 1e-6    # momentum and acceleration buffers (fp32 arithmetic)

# Block-local bound on top of the per-matrix relative Frobenius error: for
# every 64 x 64 block, ||dX_blk||_F / (sqrt(#blk) * rms(X_ref)) -- the block's
# rms error in units of the whole matrix's rms value -- must stay within
# BLOCK_FACTOR times the matrix tolerance.  Rounding error spreads over the
# matrix (a block at the tolerance would hold BLOCK_FACTOR times the
# matrix's average error density), while one wrong 16 x 16 MFMA block or one
# wrong output tile lands in a single block: a zeroed 16 x 16 sub-block alone
# reads 0.25, far above both bounds, where it moves a 1024 x 1024 matrix's
# relative Frobenius error by only 1.6e-2.
BLOCK = 64
BLOCK_FACTOR = 3.0


def rel_fro(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    if nb == 0:
        return float(np.linalg.norm(a))
    return float(np.linalg.norm(a - b) / nb)


def block_errors(a, b, block=BLOCK):
    """Per-block rms error of ``a`` against the reference ``b`` (2-D), in
    units of ``b``'s rms over the whole matrix; ragged edge blocks are
    normalised by their own element count."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape and a.ndim == 2
    r, c = b.shape
    rms = float(np.sqrt(np.mean(b * b))) if b.size else 0.0
    d2 = (a - b) ** 2
    nbr, nbc = -(-r // block), -(-c // block)
    pad = np.zeros((nbr * block, nbc * block))
    pad[:r, :c] = d2
    cnt = np.zeros_like(pad)
    cnt[:r, :c] = 1.0
    sums = pad.reshape(nbr, block, nbc, block).sum(axis=(1, 3))
    cnts = cnt.reshape(nbr, block, nbc, block).sum(axis=(1, 3))
    blk = np.sqrt(sums / np.maximum(cnts, 1.0))
    if rms == 0.0:
        return blk
    return blk / rms


def check_close(a, b, tol, what):
    """Per-matrix relative Frobenius error <= tol, and every 64 x 64 block's
    rms error <= BLOCK_FACTOR * tol in units of the matrix's rms value.
    Returns the relative Frobenius error."""
    err = rel_fro(a, b)
    assert err <= tol, "%s: rel err %.3g > %.3g" % (what, err, tol)
    blk = block_errors(a, b)
    worst = float(blk.max()) if blk.size else 0.0
    if worst > BLOCK_FACTOR * tol:
        i, j = np.unravel_index(int(np.argmax(blk)), blk.shape)
        raise AssertionError("%s: block (%d, %d) rms err %.3g of the matrix rms > %.3g (matrix rel err %.3g)"
                             % (what, i * BLOCK, j * BLOCK, worst, BLOCK_FACTOR * tol, err))
    return err


# dW = W_new - W_old is measured on fp32 master weights: W_new is stored in
# fp32, so the GPU's dW carries the rounding of that store (the update's
# fp32 arithmetic rounds at most twice), which no orthogonaliser precision
# removes.  When the update is tiny next to W (a low-rank O), that floor
# alone can exceed 1e-5 of ||dW||.  The dW checks discount, per element, up
# to DW_STORE_ULPS fp32 spacings of the oracle's W_new before applying the
# tolerance.
DW_STORE_ULPS = 2.0


def dw_discounted(dw_gpu, dw_ref, w_new_ref):
    """dw_gpu with each element's difference from dw_ref shrunk toward zero by
    DW_STORE_ULPS spacings of fp32 at w_new_ref (the storage rounding of
    W_new)."""
    dw_gpu = np.asarray(dw_gpu, dtype=np.float64)
    dw_ref = np.asarray(dw_ref, dtype=np.float64)
    allow = DW_STORE_ULPS * np.abs(np.spacing(np.asarray(w_new_ref, dtype=np.float32))).astype(np.float64)
    d = dw_gpu - dw_ref
    return dw_ref + np.sign(d) * np.maximum(np.abs(d) - allow, 0.0)


def to64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def tol_for(ns_dtype):
    return TOL_F32 if ns_dtype in ("f32", torch.float32) else TOL_16


def make_params(shapes, grad_dtype, mona, seed, device="cuda", gammas=None):
    """Seeded state + one gradient per matrix (values drawn on the CPU).
    ``mona``: False, True (MONA: A and the previous gradient) or "lite"
    (MONA-Lite: one bfloat16 state)."""
    gen = torch.Generator().manual_seed(seed)
    dt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[grad_dtype]
    out = []
    for i, (r, c) in enumerate(shapes):
        p = {
            "weight": (0.02 * torch.randn(r, c, generator=gen, dtype=torch.float64)).float().to(device),
            "momentum": torch.zeros(r, c, dtype=torch.float32, device=device),
            "gamma": 1.0 if gammas is None else gammas[i],
        }
        if mona == "lite":
            p["mona_lite"] = torch.zeros(r, c, dtype=torch.bfloat16, device=device)
        elif mona:
            p["accel"] = torch.zeros(r, c, dtype=torch.float32, device=device)
            p["prev_grad"] = torch.zeros(r, c, dtype=dt, device=device)
        out.append(p)
    return out


def draw_grads(shapes, grad_dtype, seed, kind="gaussian", device="cuda"):
    gen = torch.Generator().manual_seed(seed)
    dt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[grad_dtype]
    gs = []
    for (r, c) in shapes:
        if kind == "gaussian":
            g = torch.randn(r, c, generator=gen, dtype=torch.float64)
        else:  # spread singular values over 4 decades
            k = min(r, c)
            u, _ = torch.linalg.qr(torch.randn(r, k, generator=gen, dtype=torch.float64))
            v, _ = torch.linalg.qr(torch.randn(c, k, generator=gen, dtype=torch.float64))
            s = 10.0 ** (-4.0 * torch.rand(k, generator=gen, dtype=torch.float64))
            g = (u * s) @ v.T
        gs.append(g.to(dt).to(device))
    return gs


def snapshot(params):
    return [{k: (v.detach().clone() if isinstance(v, torch.Tensor) else v) for k, v in p.items()} for p in params]


def f32(v):
    """A scalar as the C ABI receives it (float)."""
    return float(np.float32(v))


def _f64(v):
    return to64(v) if isinstance(v, torch.Tensor) else v


def sketch_for(sketch, shape):
    """The oracle's test matrix for one matrix: the first l = long side
    columns of the kp x L sketch, transposed (l x kp)."""
    sk = to64(sketch) if isinstance(sketch, torch.Tensor) else np.asarray(sketch, dtype=np.float64)
    return sk[:, :max(shape)].T


def oracle_step(snap, grads, *, lr, mu, wd, coeffs, variant, divisor, restart_every, beta_a, alpha, step,
                sketch=None, rank=None, power_iters=1, rcond=1e-4):
    """One oracle step per matrix from ``snap`` (seeded inputs, or the oracle's
    own previous outputs -- never the GPU's).  LiMuon: ``sketch`` is the
    kp x L test matrix the GPU received."""
    # the oracle gets the same float32 hyper-parameters libmuon receives
    lr, mu, wd, beta_a, alpha, divisor = f32(lr), f32(mu), f32(wd), f32(beta_a), f32(alpha), f32(divisor)
    rcond = f32(rcond)
    res = []
    for p, g in zip(snap, grads):
        lm = {}
        if variant == "limuon":
            lm = dict(omega=sketch_for(sketch, tuple(p["weight"].shape)), rank=rank, power_iters=power_iters,
                      rcond=rcond)
        res.append(oracle.muon_step_matrix(
            _f64(p["weight"]), _f64(g), _f64(p["momentum"]), lr=lr, mu=mu, weight_decay=wd, coeffs=coeffs,
            variant=variant, divisor=divisor, restart_every=restart_every, gamma=p.get("gamma", 1.0),
            accel=_f64(p["accel"]) if "accel" in p else None,
            prev_grad=_f64(p["prev_grad"]) if "prev_grad" in p else None,
            lite_state=_f64(p["mona_lite"]) if "mona_lite" in p else None,
            beta_a=beta_a, alpha=alpha, step=step, **lm))
    return res


def oracle_state(snap):
    """The oracle's copy of a parameter list's state (float64)."""
    return [{k: _f64(v) for k, v in p.items() if k != "ortho_out" and k != "grad"} for p in snap]


def advance_oracle_state(state, ref):
    """The oracle's own state after a step (its outputs, never the GPU's)."""
    out = []
    for s, r in zip(state, ref):
        n = dict(s)
        n["weight"], n["momentum"] = r["weight"], r["momentum"]
        if "prev_grad" in s:
            n["accel"], n["prev_grad"] = r["accel"], r["prev_grad"]
        if "mona_lite" in s:
            n["mona_lite"] = r["lite_state"]
        out.append(n)
    return out


# Momentum / acceleration tolerance after the first MONA-Lite step: the
# bfloat16 state C is evaluated in fp32 on the GPU and fp64 in the oracle, so
# up to ~1% of its elements may be stored one spacing (2^-8 relative) apart
# (see compare); through alpha A = alpha (C + (1 - beta_a) G) that moves M by
# at most alpha 2^-8 sqrt(0.01) ||C|| <= 1e-3 ||M|| for these workloads.
TOL_STATE_LITE = 1e-3


def compare(params, before, ref, grads, ns_dtype, label="", ref_before=None, tol_state=TOL_STATE, beta_a=0.9,
            lite_bounds=None):
    """Per-matrix checks; returns the worst O and dW errors.

    ``before``: the GPU's state before the step; ``ref_before``: the oracle's
    own state before the step (defaults to ``before`` on a first step, when
    both hold the same seeded inputs).  ``lite_bounds`` (dict, matrix index ->
    array) carries the elementwise bound on the MONA-Lite state difference
    from step to step."""
    tol = tol_for(ns_dtype)
    ref_before = ref_before if ref_before is not None else [
        {k: (to64(v) if isinstance(v, torch.Tensor) else v) for k, v in b.items()} for b in before]
    worst_o = worst_dw = 0.0
    for i, (p, b, r) in enumerate(zip(params, before, ref)):
        m_err = rel_fro(to64(p["momentum"]), r["momentum"])
        assert m_err <= tol_state, "%s matrix %d: momentum rel err %.3g" % (label, i, m_err)
        if "accel" in p:
            a_err = rel_fro(to64(p["accel"]), r["accel"])
            assert a_err <= tol_state, "%s matrix %d: accel rel err %.3g" % (label, i, a_err)
            assert torch.equal(p["prev_grad"], grads[i]), "%s matrix %d: prev_grad is not the gradient" % (label, i)
        if "mona_lite" in p:
            # the bfloat16 state C = beta_a A - (1 - beta_a) G: the GPU evaluates
            # it in fp32 and the oracle in fp64 before the same rounding, so an
            # element may differ by one bfloat16 spacing plus the fp32 evaluation
            # error of the expression (a few ulp of |A| + |G|, which matters
            # where the two terms cancel)
            # After a step the difference carries on: C_k = beta_a C_{k-1} -
            # (1 - beta_a)^2 G_k, so the bound is this step's rounding plus
            # beta_a times the previous step's bound.
            c_gpu, c_ref = to64(p["mona_lite"]), r["lite_state"]
            g64 = to64(grads[i])
            spacing = np.ldexp(1.0, np.frexp(np.maximum(np.abs(c_ref), 2.0 ** -126))[1] - 8)
            bound = spacing + 2.0 ** -21 * (np.abs(r["accel"]) + np.abs(g64))
            if lite_bounds is not None:
                bound = bound + f32(beta_a) * lite_bounds.get(i, 0.0)
                lite_bounds[i] = bound
            bad = np.abs(c_gpu - c_ref) > bound
            assert not bad.any(), "%s matrix %d: MONA-Lite state off at %d elements (worst %.3g)" % (
                label, i, int(bad.sum()), float(np.max(np.abs(c_gpu - c_ref) - bound)))
            frac = float(np.mean(c_gpu != c_ref))
            assert frac <= 0.05, "%s matrix %d: %.2g of the MONA-Lite state differs" % (label, i, frac)

        if "ortho_out" in p:
            o_err = check_close(to64(p["ortho_out"]), r["ortho"], tol, "%s matrix %d: O" % (label, i))
            worst_o = max(worst_o, o_err)
        dw_gpu = to64(p["weight"]) - to64(b["weight"])
        dw_ref = r["weight"] - ref_before[i]["weight"]
        dw_err = check_close(dw_discounted(dw_gpu, dw_ref, r["weight"]), dw_ref, tol, "%s matrix %d: dW" % (label, i))
        worst_dw = max(worst_dw, dw_err)
    return worst_o, worst_dw

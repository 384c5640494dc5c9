"""Shared helpers for the GPU parity tests: run libmuon and the oracle on the
same seeded inputs and compare them per matrix."""
import numpy as np
import torch

import oracle

TOL_F32 = 1e-5      # relative Frobenius, fp32 Newton-Schulz operands
TOL_16 = 2e-2       # relative Frobenius, fp16 / bf16 operands with fp32 accumulation
TOL_STATE = 1e-6    # momentum and acceleration buffers (fp32 arithmetic)


def rel_fro(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    if nb == 0:
        return float(np.linalg.norm(a))
    return float(np.linalg.norm(a - b) / nb)


def to64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def tol_for(ns_dtype):
    return TOL_F32 if ns_dtype in ("f32", torch.float32) else TOL_16


def make_params(shapes, grad_dtype, mona, seed, device="cuda", gammas=None):
    """Seeded state + one gradient per matrix (values drawn on the CPU)."""
    gen = torch.Generator().manual_seed(seed)
    dt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[grad_dtype]
    out = []
    for i, (r, c) in enumerate(shapes):
        p = {
            "weight": (0.02 * torch.randn(r, c, generator=gen, dtype=torch.float64)).float().to(device),
            "momentum": torch.zeros(r, c, dtype=torch.float32, device=device),
            "gamma": 1.0 if gammas is None else gammas[i],
        }
        if mona:
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


def oracle_step(snap, grads, *, lr, mu, wd, coeffs, variant, divisor, restart_every, beta_a, alpha, step):
    res = []
    for p, g in zip(snap, grads):
        res.append(oracle.muon_step_matrix(
            to64(p["weight"]), to64(g), to64(p["momentum"]), lr=lr, mu=mu, weight_decay=wd, coeffs=coeffs,
            variant=variant, divisor=divisor, restart_every=restart_every, gamma=p.get("gamma", 1.0),
            accel=to64(p["accel"]) if "accel" in p else None,
            prev_grad=to64(p["prev_grad"]) if "prev_grad" in p else None,
            beta_a=beta_a, alpha=alpha, step=step))
    return res


def compare(params, before, ref, grads, ns_dtype, label=""):
    """Per-matrix checks; returns the worst O and dW errors."""
    tol = tol_for(ns_dtype)
    worst_o = worst_dw = 0.0
    for i, (p, b, r) in enumerate(zip(params, before, ref)):
        m_err = rel_fro(to64(p["momentum"]), r["momentum"])
        assert m_err <= TOL_STATE, "%s matrix %d: momentum rel err %.3g" % (label, i, m_err)
        if "accel" in p:
            a_err = rel_fro(to64(p["accel"]), r["accel"])
            assert a_err <= TOL_STATE, "%s matrix %d: accel rel err %.3g" % (label, i, a_err)
            assert torch.equal(p["prev_grad"], grads[i]), "%s matrix %d: prev_grad is not the gradient" % (label, i)
        if "ortho_out" in p:
            o_err = rel_fro(to64(p["ortho_out"]), r["ortho"])
            worst_o = max(worst_o, o_err)
            assert o_err <= tol, "%s matrix %d: O rel err %.3g > %.3g" % (label, i, o_err, tol)
        dw_gpu = to64(p["weight"]) - to64(b["weight"])
        dw_ref = r["weight"] - to64(b["weight"])
        dw_err = rel_fro(dw_gpu, dw_ref)
        worst_dw = max(worst_dw, dw_err)
        assert dw_err <= tol, "%s matrix %d: dW rel err %.3g > %.3g" % (label, i, dw_err, tol)
    return worst_o, worst_dw

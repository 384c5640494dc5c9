"""The largest matrix muon_step accepts (2^31 - 1 elements at most), in both
orientations: 32768 x 65535 (direct, bf16) and 65535 x 32768 (Gram, fp16,
restart every 3, divisor 1.03) -- element offsets past 2^31 inside one matrix
in every stage, and workspace offsets past 4 GiB.

The oracle cannot run a Newton-Schulz step at this size, so the gradient is
built so that the answer is known exactly: a few nonzero entries G[a_i, b_i]
on distinct rows and columns.  Its singular vectors are coordinate vectors,
so every iterate keeps that support, O[a_i, b_i] is what the oracle gives
for the compact r x r matrix with the same values, and every other entry of
O -- hence of W with W_0 = 0 -- is exactly zero (products of zeros).  The
direct case runs two MONA steps on the same support, so momentum, MONA's
acceleration and the stored previous gradient follow the compact problem's
too, and are zero elsewhere.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import rel_fro, tol_for

pytestmark = pytest.mark.gpu

ROWS_IDX = [0, 7, 1000, 20000, 32766, 32767]          # along the short side (32768)
COLS_IDX = [65534, 3, 40000, 65533, 12345, 0]         # along the long side (65535)
SIGMAS = [1.0, 0.5, 0.1, 0.03, 1e-2, 3e-3]


SIGMAS_STEP1 = [0.2, 0.9, 0.05, 0.3, 2e-3, 1e-2]       # second step (MONA): same support


def _run(rows, cols, variant, ns_dtype, divisor, restart, mona=False):
    import newton_schulz_matrix_momentum_amd as nsm
    dev = torch.device("cuda:0")
    tall = rows > cols
    ai, bi = (COLS_IDX, ROWS_IDX) if tall else (ROWS_IDX, COLS_IDX)
    steps = 2 if mona else 1
    print("max-size case: %d x %d, %s, %s, %d step(s)%s" % (rows, cols, variant, ns_dtype, steps,
                                                            ", MONA" if mona else ""), flush=True)
    r_idx = torch.tensor(ai, device=dev)
    c_idx = torch.tensor(bi, device=dev)
    p = {"weight": torch.zeros(rows, cols, dtype=torch.float32, device=dev),
         "grad": torch.zeros(rows, cols, dtype=torch.bfloat16, device=dev),
         "momentum": torch.zeros(rows, cols, dtype=torch.float32, device=dev)}
    if mona:
        p["accel"] = torch.zeros(rows, cols, dtype=torch.float32, device=dev)
        p["prev_grad"] = torch.zeros(rows, cols, dtype=torch.bfloat16, device=dev)
    lr, mu, wd, beta_a, alpha = 0.02, 0.95, 0.01, 0.9, 0.5
    coeffs = oracle.coefficient_table("quintic", 5)
    # the compact problem: value i at (i, i), advanced from its own outputs
    n = len(SIGMAS)
    z = np.zeros((n, n))
    st = {"weight": z, "momentum": z, "accel": z if mona else None, "prev_grad": z if mona else None}
    for step in range(steps):
        sig = torch.tensor(SIGMAS if step == 0 else SIGMAS_STEP1, dtype=torch.float32).to(torch.bfloat16)
        p["grad"][r_idx, c_idx] = sig.to(dev)
        nsm.muon_step([p], lr=lr, mu=mu, beta_a=beta_a, alpha=alpha, weight_decay=wd, ns_steps=5, variant=variant,
                      ns_dtype=ns_dtype, divisor=divisor, restart_every=restart, step=step)
        g_small = np.zeros((n, n))
        g_small[np.arange(n), np.arange(n)] = sig.double().numpy()
        ref = oracle.muon_step_matrix(st["weight"], g_small, st["momentum"], lr=lr, mu=mu, weight_decay=wd,
                                      coeffs=coeffs, variant=variant, divisor=divisor, restart_every=restart,
                                      accel=st["accel"], prev_grad=st["prev_grad"], beta_a=beta_a, alpha=alpha,
                                      step=step)
        st = {"weight": ref["weight"], "momentum": ref["momentum"], "accel": ref.get("accel"),
              "prev_grad": ref.get("prev_grad")}
    torch.cuda.synchronize()
    sup = lambda k: p[k][r_idx, c_idx].double().cpu().numpy()
    err = rel_fro(sup("weight"), np.diag(st["weight"]))
    print("  W on the support: rel err %.3g (tol %.0e)" % (err, tol_for(ns_dtype)), flush=True)
    assert err <= tol_for(ns_dtype)
    assert rel_fro(sup("momentum"), np.diag(st["momentum"])) <= 1e-6
    if mona:
        assert rel_fro(sup("accel"), np.diag(st["accel"])) <= 1e-6
        assert np.array_equal(sup("prev_grad"), np.diag(st["prev_grad"]))
    # everything off the support is exactly zero
    for k in [k for k in ("weight", "momentum", "accel", "prev_grad") if k in p]:
        p[k][r_idx, c_idx] = 0
        assert float(p[k].abs().max()) == 0.0, k
    del p
    torch.cuda.empty_cache()


def test_max_size_wide_direct_bf16_mona():
    assert 32768 * 65535 <= (1 << 31) - 1
    _run(32768, 65535, "direct", "bf16", 1.0, 0, mona=True)


def test_max_size_tall_gram_f16():
    _run(65535, 32768, "gram", "f16", 1.03, 3)


def test_max_size_wide_limuon():
    """LiMuon (rank 8 >= the gradient's rank 6, so the range finder is exact
    and O is the polar factor: 1 at every (a_i, b_i)) at the largest size; O
    is computed in fp32 and is zero outside the 6 x 6 block of the support's
    rows and columns."""
    import newton_schulz_matrix_momentum_amd as nsm
    from workloads import make_sketch
    rows, cols = 32768, 65535
    dev = torch.device("cuda:0")
    print("max-size case: %d x %d, limuon, f32" % (rows, cols), flush=True)
    sig = torch.tensor(SIGMAS, dtype=torch.float32).to(torch.bfloat16)
    grad = torch.zeros(rows, cols, dtype=torch.bfloat16, device=dev)
    r_idx = torch.tensor(ROWS_IDX, device=dev)
    c_idx = torch.tensor(COLS_IDX, device=dev)
    grad[r_idx, c_idx] = sig.to(dev)
    p = {"weight": torch.zeros(rows, cols, dtype=torch.float32, device=dev), "grad": grad,
         "momentum": torch.zeros(rows, cols, dtype=torch.float32, device=dev)}
    lr = 0.02
    sketch = make_sketch(16, cols, 91, device=dev)
    nsm.muon_step([p], lr=lr, mu=0.95, weight_decay=0.01, variant="limuon", ns_dtype="f32", sketch=sketch, rank=8,
                  oversample=8, power_iters=1, step=0)
    torch.cuda.synchronize()
    block = p["weight"][r_idx[:, None], c_idx[None, :]].double().cpu().numpy()
    err = rel_fro(block, -lr * np.eye(len(SIGMAS)))
    print("  O on the support block: rel err %.3g (tol 1e-05)" % err, flush=True)
    assert err <= 1e-5
    p["weight"][r_idx[:, None], c_idx[None, :]] = 0.0
    assert float(p["weight"].abs().max()) == 0.0
    del p, grad
    torch.cuda.empty_cache()

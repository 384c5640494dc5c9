"""LiMuon variant (randomized SVD of the momentum in place of Newton-Schulz)
on the GPU against the fp64 oracle: shapes spanning several 64 tiles with
ragged tails, both orientations, vectors, an exactly low-rank gradient, odd
and maximal sketch widths, zero to two power iterations, MONA over two steps,
a zero gradient, and bitwise determinism.  fp32 operands: O and dW within
1e-5 relative Frobenius per matrix and the per-block bound."""
import numpy as np
import pytest
import torch

import oracle
from helpers import (advance_oracle_state, compare, make_params, oracle_state, oracle_step, snapshot, to64,
                     check_close)
from workloads import make_sketch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import newton_schulz_matrix_momentum_amd as nsm
    nsm.load()
    yield


def spike_grads(shapes, seed, rank=8, noise=0.05, dtype=torch.float32, exact_rank=False):
    """Gaussian noise plus a rank-`rank` spike 10x the noise's top singular
    value (a clear gap after the spike), or (exact_rank) the spike alone."""
    gen = torch.Generator().manual_seed(seed)
    out = []
    for (r, c) in shapes:
        k = min(rank, r, c)
        u, _ = torch.linalg.qr(torch.randn(r, k, generator=gen, dtype=torch.float64))
        v, _ = torch.linalg.qr(torch.randn(c, k, generator=gen, dtype=torch.float64))
        s = 10.0 * noise * (r ** 0.5 + c ** 0.5) * (1.0 + torch.rand(k, generator=gen, dtype=torch.float64))
        g = (u * s) @ v.T
        if not exact_rank:
            g = g + noise * torch.randn(r, c, generator=gen, dtype=torch.float64)
        out.append(g.to(dtype).cuda())
    return out


def run_limuon(shapes, *, rank=8, oversample=8, power_iters=1, rcond=1e-4, mona=False, steps=1, seed=0,
               grads_fn=None, label=""):
    import newton_schulz_matrix_momentum_amd as nsm
    print("limuon case %s: %s k=%d p=%d q=%d mona=%s steps=%d" % (label, shapes, rank, oversample, power_iters,
                                                                  mona, steps), flush=True)
    params = make_params(shapes, "f32", mona, seed)
    for p in params:
        p["ortho_out"] = torch.empty_like(p["weight"])
    ref_state = None
    lmax = max(max(s) for s in shapes)
    worst = 0.0
    for step in range(steps):
        grads = (grads_fn or spike_grads)(shapes, seed + 100 + step)
        sketch = make_sketch(rank + oversample, lmax + 3, seed + 200 + step).cuda()
        for p, g in zip(params, grads):
            p["grad"] = g
        before = snapshot(params)
        ref_before = ref_state if ref_state is not None else oracle_state(before)
        nsm.muon_step(params, lr=0.02, mu=0.95, beta_a=0.9, alpha=0.5, weight_decay=0.01, variant="limuon",
                      ns_dtype="f32", sketch=sketch, rank=rank, oversample=oversample, power_iters=power_iters,
                      rcond=rcond, step=step)
        torch.cuda.synchronize()
        ref = oracle_step(ref_before, grads, lr=0.02, mu=0.95, wd=0.01, coeffs=None, variant="limuon",
                          divisor=1.0, restart_every=0, beta_a=0.9, alpha=0.5, step=step, sketch=sketch,
                          rank=rank, power_iters=power_iters, rcond=rcond)
        o_err, dw_err = compare(params, before, ref, grads, "f32", "limuon step %d" % step,
                                ref_before=ref_before if ref_state is not None else None)
        worst = max(worst, o_err, dw_err)
        ref_state = advance_oracle_state(ref_before, ref)
    print("  worst rel err %.3g" % worst, flush=True)
    return params


SHAPES = [(100, 300), (300, 100), (64, 64), (130, 70), (1, 77), (77, 1), (200, 200), (257, 64)]


@pytest.mark.parametrize("q", [0, 1, 2])
def test_limuon_shapes(q):
    run_limuon(SHAPES, power_iters=q, seed=10 + q, label="shapes")


def test_limuon_exact_low_rank_is_polar():
    """rank(M) <= k: the GPU's O is the polar factor of M on its range (the
    oracle is pinned to the library SVD there)."""
    shapes = [(96, 160), (160, 96)]
    params = run_limuon(shapes, rank=8, oversample=4, seed=31, label="exact rank 5",
                        grads_fn=lambda sh, sd: spike_grads(sh, sd, rank=5, exact_rank=True))
    for p in params:
        u, s, vt = np.linalg.svd(to64(p["momentum"]), full_matrices=False)
        polar = u[:, :5] @ vt[:5]
        check_close(to64(p["ortho_out"]), polar, 1e-5, "exact-rank O vs SVD polar factor")


def test_limuon_odd_and_maximal_sketch_widths():
    run_limuon([(90, 200), (200, 90)], rank=7, oversample=4, seed=41, label="kp 11")
    shapes = [(300, 500), (500, 300)]
    run_limuon(shapes, rank=48, oversample=16, seed=42, label="kp 64",
               grads_fn=lambda sh, sd: spike_grads(sh, sd, rank=48))


def test_limuon_mona_two_steps():
    run_limuon([(128, 384), (384, 128), (192, 192)], mona=True, steps=2, seed=51, label="MONA")


def test_limuon_zero_gradient_is_pure_decay():
    import newton_schulz_matrix_momentum_amd as nsm
    params = make_params([(64, 200)], "f32", False, 61)
    params[0]["grad"] = torch.zeros(64, 200, device="cuda")
    params[0]["ortho_out"] = torch.full((64, 200), 7.0, device="cuda")
    w0 = params[0]["weight"].clone()
    nsm.muon_step(params, lr=0.02, mu=0.95, weight_decay=0.01, variant="limuon", ns_dtype="f32",
                  sketch=make_sketch(16, 200, 62).cuda(), rank=8)
    torch.cuda.synchronize()
    assert torch.count_nonzero(params[0]["ortho_out"]) == 0
    torch.testing.assert_close(params[0]["weight"], w0 - 0.02 * 0.01 * w0, rtol=1e-6, atol=0)


def test_limuon_bitwise_deterministic():
    a = run_limuon([(150, 250), (250, 150)], seed=71, label="det a")
    b = run_limuon([(150, 250), (250, 150)], seed=71, label="det b")
    for pa, pb in zip(a, b):
        assert torch.equal(pa["weight"], pb["weight"]) and torch.equal(pa["ortho_out"], pb["ortho_out"])

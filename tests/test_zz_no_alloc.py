"""muon_step_static (the entry point that allocates nothing: its workspace is
the library's static per-GPU array) against muon_step with an allocated
workspace, through the C ABI: two calls in a row, the second on a smaller
input, both bitwise equal to muon_step and within the oracle tolerance."""
import numpy as np
import pytest
import torch

import oracle
from helpers import check_close, compare, draw_grads, make_params, oracle_step, snapshot, to64

pytestmark = pytest.mark.gpu


def _clone(params):
    return [{k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in p.items()} for p in params]


def _run_pair(shapes, *, grad_dtype, ns_dtype, variant, mona, seed, divisor=1.0, restart_every=0):
    import newton_schulz_matrix_momentum_amd as nsm
    print("no-alloc case: %s %s/%s %s mona=%s" % (shapes, grad_dtype, ns_dtype, variant, mona), flush=True)
    params = make_params(shapes, grad_dtype, mona, seed)
    grads = draw_grads(shapes, grad_dtype, seed + 1, kind="spectral")
    for p, g in zip(params, grads):
        p["grad"] = g
        p["ortho_out"] = torch.empty_like(p["weight"])
    a, b = _clone(params), _clone(params)
    before = snapshot(params)
    coeffs = oracle.coefficient_table("quintic", 5)
    kw = dict(lr=0.02, mu=0.95, beta_a=0.9, alpha=0.5, weight_decay=0.01, ns_steps=5, variant=variant,
              ns_dtype=ns_dtype, coeffs=coeffs.tolist(), divisor=divisor, restart_every=restart_every, step=0)
    nsm.muon_step(a, **kw)
    nsm.muon_step_static(b, **kw)
    torch.cuda.synchronize()
    for i, (pa, pb) in enumerate(zip(a, b)):
        for key in ("weight", "momentum", "ortho_out", "accel", "prev_grad"):
            if key in pa:
                assert torch.equal(pa[key], pb[key]), "matrix %d: %s differs from muon_step" % (i, key)
    ref = oracle_step(before, grads, lr=0.02, mu=0.95, wd=0.01, coeffs=coeffs, variant=variant, divisor=divisor,
                      restart_every=restart_every, beta_a=0.9, alpha=0.5, step=0)
    return compare(b, before, ref, grads, ns_dtype, "no-alloc")


def test_static_matches_muon_step_twice_second_smaller():
    big = [(192, 192), (192, 192), (192, 768), (768, 192), (300, 520), (130, 70)]
    _run_pair(big, grad_dtype="bf16", ns_dtype="bf16", variant="direct", mona=True, seed=101)
    # the second call is smaller: whatever the first call left in the static
    # workspace must not leak into it
    small = [(64, 200), (130, 70)]
    _run_pair(small, grad_dtype="f16", ns_dtype="f16", variant="gram", mona=False, seed=202, divisor=1.03,
              restart_every=3)


def test_static_fp32_after_16bit():
    _run_pair([(64, 256), (96, 40)], grad_dtype="f32", ns_dtype="f32", variant="direct", mona=False, seed=303)


def test_static_rejects_oversized_call():
    import newton_schulz_matrix_momentum_amd as nsm
    from newton_schulz_matrix_momentum_amd import _lib
    w = torch.zeros(4096, 4096, device="cuda")
    p = {"weight": w, "grad": torch.zeros(4096, 4096, dtype=torch.bfloat16, device="cuda"),
         "momentum": torch.zeros_like(w)}
    need = nsm.muon_workspace_size([p], ns_dtype="bf16")
    assert need > _lib.STATIC_WORKSPACE_BYTES
    with pytest.raises(_lib.MuonError) as e:
        nsm.muon_step_static([p], lr=0.02, mu=0.95, ns_dtype="bf16")
    assert e.value.status == _lib.MUON_ERR_WORKSPACE_TOO_SMALL
    assert "static workspace" in str(e.value)
    torch.cuda.synchronize()
    assert torch.count_nonzero(w) == 0    # nothing was enqueued

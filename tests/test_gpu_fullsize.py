"""Full-size parity: every synthetic workload at its real size, stepped exactly
as bench.py steps it (all matrices in one call), checked against the fp64
oracle on the first and the last matrix of every shape class (the last one
sits at the class's highest workspace offset) -- every stage: momentum,
acceleration, previous gradient, O and dW, the last two per matrix and per
64 x 64 block -- plus finiteness of every matrix.

The oracle computes full products in fp64 on the host, so only sampled
matrices are re-derived; the elementwise state of every other matrix is
checked on sampled elements.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import check_close, dw_discounted, rel_fro, sketch_for, to64, tol_for, TOL_STATE
from workloads import WORKLOADS, make_grads, make_state, workload_sketch

pytestmark = pytest.mark.gpu


def _setup(w, device, lite=False):
    gen_dev = device if w.name.startswith("gram_tall") else "cpu"
    state = make_state(w, device=gen_dev, mona="lite" if lite else None)
    params = []
    for st in state:
        params.append({k: v.to(device) for k, v in st.items()})
    return params, gen_dev


def _sample_indices(w):
    """First and last matrix of every shape class."""
    first, last = {}, {}
    for i, s in enumerate(w.shapes):
        first.setdefault(s, i)
        last[s] = i
    return sorted(set(first.values()) | set(last.values()))


def _run_workload(name, variant, lite=False):
    import newton_schulz_matrix_momentum_amd as nsm
    w = WORKLOADS[name]
    dev = torch.device("cuda:0")
    print("workload %s variant %s: %d matrices" % (name, variant, len(w.shapes)), flush=True)
    params, gen_dev = _setup(w, dev, lite)
    sample = _sample_indices(w)
    for i in sample:
        params[i]["ortho_out"] = torch.empty_like(params[i]["weight"])
    divisor, restart = w.settings_for(variant)
    coeffs = oracle.coefficient_table(w.coeffs, w.ns_steps)
    ns_dtype = w.ns_dtype_for(variant)
    tol = tol_for(ns_dtype)
    snaps = {i: {k: to64(v) for k, v in params[i].items() if k != "ortho_out"} for i in sample}
    rng = np.random.default_rng(7)
    for step in range(w.steps):
        grads = make_grads(w, step, device=gen_dev)
        for p, g in zip(params, grads):
            p["grad"] = g.to(dev)
        # elementwise spot checks on a few elements of every matrix
        probes = []
        for i, p in enumerate(params):
            n = p["weight"].numel()
            pos = torch.from_numpy(rng.integers(0, n, 16)).to(dev)
            probes.append((i, pos, {k: p[k].flatten()[pos].double().cpu().numpy()
                                    for k in ("grad", "momentum", "accel", "prev_grad", "mona_lite") if k in p}))
        w_gpu_before = {i: to64(params[i]["weight"]) for i in sample}
        lm, lm_ref = {}, {}
        if variant == "limuon":
            sketch = workload_sketch(w, step).to(dev)
            lm = dict(sketch=sketch, **w.limuon_settings())
            lm_ref = dict(rank=lm["rank"], power_iters=lm["power_iters"], rcond=float(np.float32(1e-4)))
        nsm.muon_step(params, lr=w.lr, mu=w.mu, beta_a=w.beta_a, alpha=w.alpha, weight_decay=w.weight_decay,
                      ns_steps=w.ns_steps, variant=variant, ns_dtype=ns_dtype, coeffs=coeffs.tolist(),
                      divisor=divisor, restart_every=restart, step=step, **lm)
        torch.cuda.synchronize()
        for i, pos, before in probes:
            p = params[i]
            beta, alpha, mu = (float(np.float32(v)) for v in (w.beta_a, w.alpha, w.mu))
            m_ref = mu * before["momentum"]
            if "mona_lite" in before:
                g = before["grad"]
                a_ref = np.zeros_like(g) if step == 0 else before["mona_lite"] + (1 - beta) * g
                c_ref = oracle.round_bf16(beta * a_ref - (1 - beta) * g)
                m_ref = m_ref + g + alpha * a_ref
                c_gpu = p["mona_lite"].flatten()[pos].double().cpu().numpy()
                np.testing.assert_allclose(c_gpu, c_ref, rtol=2.0 ** -7, atol=2.0 ** -21 * float(np.max(np.abs(g))))
            elif "accel" in before:
                d = np.zeros_like(before["grad"]) if step == 0 else before["grad"] - before["prev_grad"]
                a_ref = w.beta_a * before["accel"] + (1 - w.beta_a) * d
                m_ref = m_ref + before["grad"] + w.alpha * a_ref
                np.testing.assert_allclose(p["accel"].flatten()[pos].double().cpu().numpy(), a_ref,
                                           rtol=1e-5, atol=1e-7)
                assert torch.equal(p["prev_grad"].flatten()[pos], p["grad"].flatten()[pos])
            else:
                m_ref = m_ref + before["grad"]
            np.testing.assert_allclose(p["momentum"].flatten()[pos].double().cpu().numpy(), m_ref,
                                       rtol=1e-5, atol=1e-6)
            assert torch.isfinite(p["weight"]).all(), "matrix %d has non-finite weights" % i
        for i in sample:
            s = snaps[i]
            g = to64(params[i]["grad"])
            if variant == "limuon":
                lm_ref["omega"] = sketch_for(lm["sketch"], w.shapes[i])
            ref = oracle.muon_step_matrix(s["weight"], g, s["momentum"], lr=w.lr, mu=w.mu,
                                          weight_decay=w.weight_decay, coeffs=coeffs, variant=variant,
                                          divisor=divisor, restart_every=restart, accel=s.get("accel"),
                                          prev_grad=s.get("prev_grad"), lite_state=s.get("mona_lite"),
                                          beta_a=w.beta_a, alpha=w.alpha, step=step, **lm_ref)
            p = params[i]
            assert rel_fro(to64(p["momentum"]), ref["momentum"]) <= TOL_STATE
            if "accel" in p:
                assert rel_fro(to64(p["accel"]), ref["accel"]) <= TOL_STATE
            what = "step %d matrix %d %s" % (step, i, w.shapes[i])
            print("  %s: O err %.3g, dW err %.3g (tol %.0e)"
                  % (what, rel_fro(to64(p["ortho_out"]), ref["ortho"]),
                     rel_fro(to64(p["weight"]) - w_gpu_before[i], ref["weight"] - s["weight"]), tol), flush=True)
            check_close(to64(p["ortho_out"]), ref["ortho"], tol, what + ": O")
            dw_ref = ref["weight"] - s["weight"]
            check_close(dw_discounted(to64(p["weight"]) - w_gpu_before[i], dw_ref, ref["weight"]), dw_ref, tol,
                        what + ": dW")
            # carry the oracle's own state forward (never the GPU's)
            s["weight"], s["momentum"] = ref["weight"], ref["momentum"]
            if "prev_grad" in ref:
                s["accel"], s["prev_grad"] = ref["accel"], ref["prev_grad"]
            if "lite_state" in ref:
                s["mona_lite"] = ref["lite_state"]


def test_full_single_64x256_f32():
    _run_workload("single_64x256_f32", "direct")


def test_full_nanochat_6l_d192():
    _run_workload("nanochat_6l_d192", "direct")


def test_full_llama430m_24l_d1024():
    _run_workload("llama430m_24l_d1024", "direct")


def test_full_llama430m_24l_d1024_limuon():
    _run_workload("llama430m_24l_d1024", "limuon")


def test_full_llama430m_24l_d1024_mona_lite():
    _run_workload("llama430m_24l_d1024", "direct", lite=True)


@pytest.mark.parametrize("variant", ["direct", "gram"])
def test_full_moe_64e_d2048(variant):
    _run_workload("moe_64e_d2048", variant)


@pytest.mark.timeout(600)
def test_full_gram_tall_32x4096x16384():
    _run_workload("gram_tall_32x4096x16384", "gram")

"""HIP path vs the fp64 oracle on seeded inputs.

Sizes span several tiles and ragged tails (64-wide tiles for short sides up to
256, 128-wide above), both orientations, every dtype combination, both
Newton-Schulz variants, MONA on and off, and two consecutive steps.
Tolerances on O and on dW = W_new - W_old: relative Frobenius per matrix
1e-5 with fp32 Newton-Schulz operands, 2e-2 with fp16 / bf16 operands and fp32
accumulation, and every 64 x 64 block's rms error within 3x that in units of
the matrix's rms value (helpers.check_close); momentum and acceleration 1e-6;
the stored previous gradient is bitwise the gradient.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import (advance_oracle_state, compare, draw_grads, make_params, oracle_state, oracle_step, snapshot,
                     to64, rel_fro, check_close, TOL_STATE, TOL_STATE_LITE)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import newton_schulz_matrix_momentum_amd as nsm
    nsm.load()
    yield


def run_case(shapes, *, grad_dtype, ns_dtype, variant="direct", kind="quintic", ns_steps=5, mona=False, steps=1,
             divisor=1.0, restart_every=0, lr=0.02, mu=0.95, wd=0.01, beta_a=0.9, alpha=0.5, seed=0,
             grad_kind="gaussian", gammas=None, coeffs=None):
    import newton_schulz_matrix_momentum_amd as nsm
    label = "%s %s/%s %s mona=%s" % (shapes[:3], grad_dtype, ns_dtype, variant, mona)
    print("case:", label, flush=True)
    params = make_params(shapes, grad_dtype, mona, seed, gammas=gammas)
    for p in params:
        p["ortho_out"] = torch.full(p["weight"].shape, float("nan"), dtype=torch.float32, device="cuda")
    if coeffs is None:
        coeffs = oracle.coefficient_table(kind, ns_steps)
    worst = (0.0, 0.0)
    ostate = oracle_state(snapshot(params))   # the oracle carries its own state
    lite_bounds = {}
    for step in range(steps):
        grads = draw_grads(shapes, grad_dtype, seed * 100 + step, grad_kind)
        for p, g in zip(params, grads):
            p["grad"] = g
        before = snapshot(params)
        ref = oracle_step(ostate, grads, lr=lr, mu=mu, wd=wd, coeffs=coeffs, variant=variant, divisor=divisor,
                          restart_every=restart_every, beta_a=beta_a, alpha=alpha, step=step)
        nsm.muon_step(params, lr=lr, mu=mu, beta_a=beta_a, alpha=alpha, weight_decay=wd, ns_steps=ns_steps,
                      variant=variant, ns_dtype=ns_dtype, coeffs=coeffs.tolist(), divisor=divisor,
                      restart_every=restart_every, step=step)
        torch.cuda.synchronize()
        w = compare(params, before, ref, grads, ns_dtype, label + " step %d" % step, ref_before=ostate,
                    tol_state=TOL_STATE_LITE if (mona == "lite" and step > 0) else TOL_STATE, beta_a=beta_a,
                    lite_bounds=lite_bounds)
        worst = (max(worst[0], w[0]), max(worst[1], w[1]))
        ostate = advance_oracle_state(ostate, ref)
    print("  worst O err %.3g, worst dW err %.3g" % worst, flush=True)
    return worst


SMALL = [(64, 256), (100, 300), (300, 100), (130, 130), (1, 77), (77, 1), (5, 3)]
MEDIUM = [(260, 520), (520, 260), (384, 384), (300, 1000), (600, 900), (1000, 1500), (1500, 1000)]


# ---------------------------------------------------------------- fp32 path

def test_single_64x256_f32_cubic():
    """One fp32 64x256 matrix, N(0,1) grad, 5 cubic steps, direct."""
    run_case([(64, 256)], grad_dtype="f32", ns_dtype="f32", kind="cubic")


@pytest.mark.parametrize("variant", ["direct", "gram"])
def test_f32_small_ragged(variant):
    run_case(SMALL, grad_dtype="f32", ns_dtype="f32", variant=variant, divisor=1.03, restart_every=2)


@pytest.mark.parametrize("variant", ["direct", "gram"])
def test_f32_medium_tiles128(variant):
    run_case(MEDIUM, grad_dtype="f32", ns_dtype="f32", variant=variant, grad_kind="spectral")


# ---------------------------------------------------------------- 16-bit paths

@pytest.mark.parametrize("grad_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("variant", ["direct", "gram"])
def test_bf16_ns(grad_dtype, variant):
    run_case(SMALL + MEDIUM, grad_dtype=grad_dtype, ns_dtype="bf16", variant=variant, grad_kind="spectral",
             divisor=1.03 if variant == "gram" else 1.0, restart_every=3 if variant == "gram" else 0)


@pytest.mark.parametrize("variant", ["direct", "gram"])
def test_f16_ns(variant):
    run_case(SMALL + MEDIUM, grad_dtype="f16", ns_dtype="f16", variant=variant, grad_kind="spectral",
             divisor=1.03, restart_every=3)


@pytest.mark.parametrize("variant,ns_dtype", [("direct", "bf16"), ("gram", "f16"), ("direct", "f16")])
def test_128_tile_classes_next_to_256_tile_classes(variant, ns_dtype):
    """Short sides that pad well to 128 tiles but not to 256 (1408 as in the
    MoE experts, 1664, 640) next to a 256-tile class (1024): both
    orientations, ragged long sides (1900), two matrices of one class, over
    two MONA steps."""
    shapes = [(1408, 2048), (2048, 1408), (1664, 1900), (1900, 1664), (1024, 1024), (640, 1280), (1408, 2048)]
    run_case(shapes, grad_dtype="bf16", ns_dtype=ns_dtype, variant=variant, grad_kind="spectral", seed=17,
             mona=True, steps=2, divisor=1.03 if variant == "gram" else 1.0,
             restart_every=3 if variant == "gram" else 0)


@pytest.mark.parametrize("ns_dtype", ["bf16", "f16"])
def test_fused_square_update_groups(ns_dtype):
    """Short sides <= 192 form B = b A + c A^2 inside the update launch, each
    block serving a group of output row tiles.  About 1450 (row tile, column
    tile) pairs at a padded short side of 192 make the groups 4 tiles long
    with ragged last groups (22 and 11 row tiles); short sides 64 and 128 run
    in launches of their own in the same step."""
    shapes = [(192, 1408)] * 6 + [(1408, 192)] * 6 + [(150, 700)] * 10 + [(700, 150)] * 10 + \
        [(64, 320), (320, 64), (128, 200), (200, 128)]
    run_case(shapes, grad_dtype="bf16", ns_dtype=ns_dtype, grad_kind="spectral", seed=12)


@pytest.mark.parametrize("ns_dtype,variant", [("bf16", "direct"), ("f16", "gram")])
def test_256_tile_classes_mixed_k(ns_dtype, variant):
    """Three classes on the 256 tile whose Gram products run over different
    K (700, 900, 1300) in one launch: the launch deals each XCD a contiguous
    eighth of every class; both orientations."""
    shapes = [(512, 700), (700, 512), (768, 900), (1300, 512)]
    run_case(shapes, grad_dtype="bf16", ns_dtype=ns_dtype, variant=variant, grad_kind="spectral", seed=17,
             divisor=1.03 if variant == "gram" else 1.0, restart_every=3 if variant == "gram" else 0)


def test_256_tile_many_small_classes():
    """Nine one-matrix classes on the 256 tile (short side 512, long sides
    512 .. 900): 3 to 8 tiles per class and product, so most XCDs get an
    empty eighth of a class, and the ninth class opens a second launch."""
    longs = [512, 530, 560, 600, 640, 700, 760, 800, 900]
    shapes = [(512, l) if i % 2 == 0 else (l, 512) for i, l in enumerate(longs)]
    run_case(shapes, grad_dtype="bf16", ns_dtype="bf16", grad_kind="spectral", seed=18)


@pytest.mark.parametrize("ns_dtype", ["f32", "bf16"])
def test_long_thin_matrices(ns_dtype):
    """Extreme aspect ratios: long sides of 9000 to 70001 with short sides 1
    to 17 (over a thousand 64-row tiles per matrix on the fused path, norms
    over several E1 blocks, ragged long-side tails), both orientations."""
    shapes = [(1, 70001), (40003, 3), (17, 9000), (9001, 5)]
    run_case(shapes, grad_dtype="f32", ns_dtype=ns_dtype, grad_kind="gaussian", seed=16)


@pytest.mark.parametrize("ns_dtype", ["bf16", "f16"])
def test_fused_update_launch_split(ns_dtype):
    """Ten classes whose short side pads to 192 (s = 130 .. 184) in one
    call: the fused update's launch takes at most 8 classes, so the step
    runs it as two launches (8 + 2 classes); both orientations."""
    shapes = []
    for i in range(10):
        s, l = 130 + 6 * i, 150 + 37 * i
        shapes.append((s, l) if i % 2 == 0 else (l, s))
    run_case(shapes, grad_dtype="bf16", ns_dtype=ns_dtype, grad_kind="spectral", seed=15)


@pytest.mark.parametrize("ns_dtype,order", [("bf16", "cqcqq"), ("f16", "qcqcq")])
def test_mixed_cubic_quintic_steps(ns_dtype, order):
    """Per-step coefficient tables mixing cubic (c = 0) and quintic steps on
    short sides <= 192: a quintic step runs fused and reads the iterate in
    one layout, a cubic step runs the separate update product that also
    reads X^T, so the layouts written before each step must follow the
    table (X0^T only when step 1 is cubic, X'^T only ahead of a cubic step)."""
    rows = {"c": oracle.coefficient_table("cubic", 1)[0], "q": oracle.coefficient_table("quintic", 1)[0]}
    coeffs = np.array([rows[ch] for ch in order])
    shapes = [(150, 700), (700, 150), (192, 192), (64, 320), (320, 64), (100, 64)]
    run_case(shapes, grad_dtype="f32", ns_dtype=ns_dtype, grad_kind="spectral", ns_steps=len(order), coeffs=coeffs,
             seed=14)


@pytest.mark.parametrize("ns_dtype", ["bf16", "f16"])
def test_long_k_register_stages(ns_dtype):
    """64 tiles whose Gram product runs over more k than the LDS ring holds
    (K = 704: 11 stages of 64, 3 of them carried in registers) in the same
    launch as classes that fit the ring (K = 64 .. 192)."""
    shapes = [(100, 700), (700, 100), (64, 650), (130, 130), (192, 192), (5, 60)]
    run_case(shapes, grad_dtype="bf16", ns_dtype=ns_dtype, grad_kind="spectral", seed=13)


@pytest.mark.parametrize("variant", ["direct", "gram"])
def test_mona_two_steps(variant):
    run_case([(200, 330), (330, 200), (256, 256)], grad_dtype="bf16", ns_dtype="bf16", variant=variant, mona=True,
             steps=2)


def test_mona_two_steps_f32():
    run_case([(96, 160), (160, 96)], grad_dtype="f32", ns_dtype="f32", mona=True, steps=3)


def test_cubic_gram_no_square_term():
    run_case([(100, 260), (260, 100)], grad_dtype="f32", ns_dtype="f32", variant="gram", kind="cubic",
             divisor=1.02, restart_every=2)


def test_zero_steps_returns_x0():
    run_case([(70, 90), (90, 70)], grad_dtype="f32", ns_dtype="f32", ns_steps=0)


def test_per_matrix_gamma():
    run_case([(64, 64), (64, 128)], grad_dtype="f32", ns_dtype="f32", gammas=[0.5, 2.0])


# ---------------------------------------------------------------- special cases

def test_zero_grad_is_pure_decay():
    import newton_schulz_matrix_momentum_amd as nsm
    params = make_params([(64, 96)], "f32", False, 3)
    params[0]["grad"] = torch.zeros(64, 96, device="cuda")
    params[0]["ortho_out"] = torch.full((64, 96), 7.0, device="cuda")
    w0 = params[0]["weight"].clone()
    nsm.muon_step(params, lr=0.1, mu=0.9, weight_decay=0.01, ns_dtype="bf16")
    torch.cuda.synchronize()
    assert torch.all(params[0]["ortho_out"] == 0)
    expect = w0 - 0.1 * (0.01 * w0)
    assert torch.allclose(params[0]["weight"], expect, rtol=0, atol=1e-7)


def test_nan_is_isolated_per_matrix():
    import newton_schulz_matrix_momentum_amd as nsm
    shapes = [(64, 64), (64, 64), (128, 64)]
    params = make_params(shapes, "bf16", False, 4)
    grads = draw_grads(shapes, "bf16", 5)
    grads[1][3, 7] = float("nan")
    for p, g in zip(params, grads):
        p["grad"] = g
    before = snapshot(params)
    nsm.muon_step(params, lr=0.02, mu=0.95, weight_decay=0.01, ns_dtype="bf16")
    torch.cuda.synchronize()
    assert torch.isnan(params[1]["weight"]).any()
    ref = oracle_step([before[0], before[2]], [grads[0], grads[2]], lr=0.02, mu=0.95, wd=0.01,
                      coeffs=oracle.coefficient_table("quintic", 5), variant="direct", divisor=1.0,
                      restart_every=0, beta_a=0.0, alpha=0.0, step=0)
    compare([params[0], params[2]], [before[0], before[2]], ref, [grads[0], grads[2]], "bf16", "nan-isolation")


def test_alpha_zero_equals_plain_muon_bitwise():
    import newton_schulz_matrix_momentum_amd as nsm
    shapes = [(96, 200), (200, 96)]
    pa = make_params(shapes, "bf16", True, 6)
    pp = make_params(shapes, "bf16", False, 6)
    for step in range(2):
        grads = draw_grads(shapes, "bf16", 60 + step)
        for a, p, g in zip(pa, pp, grads):
            a["grad"] = g
            p["grad"] = g
        nsm.muon_step(pa, lr=0.02, mu=0.95, beta_a=0.9, alpha=0.0, weight_decay=0.01, ns_dtype="bf16", step=step)
        nsm.muon_step(pp, lr=0.02, mu=0.95, weight_decay=0.01, ns_dtype="bf16", step=step)
    torch.cuda.synchronize()
    for a, p in zip(pa, pp):
        assert torch.equal(a["weight"], p["weight"])
        assert torch.equal(a["momentum"], p["momentum"])


def test_deterministic_bitwise():
    import newton_schulz_matrix_momentum_amd as nsm
    shapes = [(300, 700), (700, 300), (192, 192)]
    outs = []
    for _ in range(2):
        params = make_params(shapes, "bf16", True, 8)
        for p, g in zip(params, draw_grads(shapes, "bf16", 9)):
            p["grad"] = g
        nsm.muon_step(params, lr=0.02, mu=0.95, beta_a=0.9, alpha=0.5, weight_decay=0.01, ns_dtype="bf16",
                      variant="gram", divisor=1.03, restart_every=3, step=1)
        torch.cuda.synchronize()
        outs.append([p["weight"].clone() for p in params])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_resume_equals_continuous():
    """Two steps == one step + state copy + one step (bitwise)."""
    import newton_schulz_matrix_momentum_amd as nsm
    shapes = [(128, 320), (320, 128)]
    hp = dict(lr=0.02, mu=0.95, beta_a=0.9, alpha=0.5, weight_decay=0.01, ns_dtype="bf16")
    grads = [draw_grads(shapes, "bf16", 70 + s) for s in range(2)]
    cont = make_params(shapes, "bf16", True, 10)
    for s in range(2):
        for p, g in zip(cont, grads[s]):
            p["grad"] = g
        nsm.muon_step(cont, step=s, **hp)
    res = make_params(shapes, "bf16", True, 10)
    for p, g in zip(res, grads[0]):
        p["grad"] = g
    nsm.muon_step(res, step=0, **hp)
    torch.cuda.synchronize()
    saved = [{k: v.detach().cpu().clone() for k, v in p.items() if isinstance(v, torch.Tensor)} for p in res]
    restored = [{k: v.cuda() for k, v in s.items()} for s in saved]
    for p, g in zip(restored, grads[1]):
        p["grad"] = g
        p["gamma"] = 1.0
    nsm.muon_step(restored, step=1, **hp)
    torch.cuda.synchronize()
    for a, b in zip(cont, restored):
        for k in ("weight", "momentum", "accel", "prev_grad"):
            assert torch.equal(a[k], b[k]), k


def test_empty_list_is_noop():
    import newton_schulz_matrix_momentum_amd as nsm
    nsm.muon_step([], lr=0.02, mu=0.95)


def test_stream_ordering_no_hidden_sync():
    """The call enqueues on the current stream and returns; results are right
    after a later synchronize."""
    import newton_schulz_matrix_momentum_amd as nsm
    s = torch.cuda.Stream()
    shapes = [(256, 1024)] * 4
    params = make_params(shapes, "bf16", False, 11)
    grads = draw_grads(shapes, "bf16", 12)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        for p, g in zip(params, grads):
            p["grad"] = g
        before = snapshot(params)
        nsm.muon_step(params, lr=0.02, mu=0.95, weight_decay=0.01, ns_dtype="bf16")
    s.synchronize()
    ref = oracle_step(before, grads, lr=0.02, mu=0.95, wd=0.01, coeffs=oracle.coefficient_table("quintic", 5),
                      variant="direct", divisor=1.0, restart_every=0, beta_a=0.0, alpha=0.0, step=0)
    compare(params, before, ref, grads, "bf16", "side-stream")


def test_symmetric_input_gram_f32():
    """A symmetric gradient through the Gram variant with fp32 operands."""
    import newton_schulz_matrix_momentum_amd as nsm
    g = torch.randn(200, 200, dtype=torch.float64, generator=torch.Generator().manual_seed(13))
    g = (g + g.T).float().cuda()
    params = make_params([(200, 200)], "f32", False, 14)
    params[0]["grad"] = g
    params[0]["ortho_out"] = torch.empty(200, 200, device="cuda")
    nsm.muon_step(params, lr=0.02, mu=0.95, weight_decay=0.0, ns_dtype="f32", variant="gram")
    torch.cuda.synchronize()
    ref = oracle.newton_schulz_gram(oracle.frobenius_normalize(to64(g)), oracle.coefficient_table("quintic", 5))
    check_close(to64(params[0]["ortho_out"]), ref, 1e-5, "symmetric fp32 Gram: O")


# ---------------------------------------------------------------- launch timing

def _traced_step(group):
    import ctypes
    import newton_schulz_matrix_momentum_amd as nsm
    from newton_schulz_matrix_momentum_amd import _lib
    import bench
    shapes = [(192, 192)] * 4 + [(192, 768), (768, 192)]
    params = make_params(shapes, "bf16", False, 31)
    for p, g in zip(params, draw_grads(shapes, "bf16", 32)):
        p["grad"] = g
    cap = 64
    ev = bench.HipEvents(2 * cap)
    stages = (ctypes.c_int32 * cap)()
    work = (ctypes.c_double * cap)()
    nl = (ctypes.c_int32 * cap)()
    tr = _lib.MuonTrace(events=ctypes.cast(ev.arr, ctypes.POINTER(ctypes.c_void_p)),
                        stages=ctypes.cast(stages, ctypes.POINTER(ctypes.c_int32)),
                        work=ctypes.cast(work, ctypes.POINTER(ctypes.c_double)), capacity=cap, count=0,
                        group=group, launches=ctypes.cast(nl, ctypes.POINTER(ctypes.c_int32)))
    nsm.muon_step(params, lr=0.02, mu=0.95, ns_dtype="bf16", trace=tr)
    torch.cuda.synchronize()
    out = [(_lib.STAGE_NAMES[stages[i]], nl[i], work[i], ev.elapsed_ms(2 * i, 2 * i + 1)) for i in range(tr.count)]
    ev.close()
    return out


def test_trace_per_launch_and_grouped():
    """Per-launch mode: one interval per launch (E1, E2, 2 x 5 products: at
    a short side of 192 the square is formed inside the update launch).
    Grouped mode: one interval per run of one stage, launch counts and work
    summed."""
    per = _traced_step(0)
    assert [s for s, _, _, _ in per] == ["e1", "e2"] + ["gemm"] * 10
    assert all(ms > 0 for _, _, _, ms in per)
    grp = _traced_step(1)
    assert [(s, n) for s, n, _, _ in grp] == [("e1", 1), ("e2", 1), ("gemm", 10)]
    assert grp[2][2] == pytest.approx(sum(w for s, _, w, _ in per if s == "gemm"))
    # 5 quintic steps on 4 x 192^2 and 2 x (192 x 768): half Gram, half square, full update
    s = 192.0
    flops = 5 * (4 * (s * (s + 1) * s * 2 + 2 * s * s * s) + 2 * (s * (s + 1) * 768 + s * (s + 1) * s + 2 * s * s * 768))
    assert grp[2][2] == pytest.approx(flops)
    assert grp[2][3] > 0


# ---------------------------------------------------------------- MONA-Lite

@pytest.mark.parametrize("grad_dtype", ["f32", "bf16", "f16"])
def test_mona_lite_three_steps(grad_dtype):
    """MONA-Lite (one bfloat16 state) over three steps, ragged shapes and
    every gradient dtype; the state is checked to one bfloat16 spacing."""
    run_case([(200, 330), (330, 200), (77, 5), (1, 4099), (256, 256)], grad_dtype=grad_dtype, ns_dtype="bf16",
             mona="lite", steps=3, grad_kind="spectral")


def test_mona_lite_gram_fp16():
    run_case([(300, 700), (700, 300)], grad_dtype="f16", ns_dtype="f16", variant="gram", mona="lite", steps=2,
             divisor=1.03, restart_every=3)


def test_mona_lite_alpha_zero_equals_plain_muon_bitwise():
    import newton_schulz_matrix_momentum_amd as nsm
    shapes = [(96, 200), (200, 96)]
    pl = make_params(shapes, "bf16", "lite", 41)
    pp = make_params(shapes, "bf16", False, 41)
    for step in range(2):
        grads = draw_grads(shapes, "bf16", 410 + step)
        for a, p, g in zip(pl, pp, grads):
            a["grad"] = g
            p["grad"] = g
        nsm.muon_step(pl, lr=0.02, mu=0.95, beta_a=0.9, alpha=0.0, weight_decay=0.01, ns_dtype="bf16", step=step)
        nsm.muon_step(pp, lr=0.02, mu=0.95, weight_decay=0.01, ns_dtype="bf16", step=step)
    torch.cuda.synchronize()
    for a, p in zip(pl, pp):
        assert torch.equal(a["weight"], p["weight"])
        assert torch.equal(a["momentum"], p["momentum"])


def test_mona_lite_and_mona_in_one_call():
    """Plain, MONA and MONA-Lite matrices mixed in one call."""
    import newton_schulz_matrix_momentum_amd as nsm
    shapes = [(128, 320), (320, 128), (64, 64)]
    params = make_params(shapes[:1], "bf16", False, 42) + make_params(shapes[1:2], "bf16", True, 43) + \
        make_params(shapes[2:], "bf16", "lite", 44)
    ostate = oracle_state(snapshot(params))
    lite_bounds = {}
    for step in range(2):
        grads = draw_grads(shapes, "bf16", 420 + step)
        for p, g in zip(params, grads):
            p["grad"] = g
        before = snapshot(params)
        ref = oracle_step(ostate, grads, lr=0.02, mu=0.95, wd=0.01, coeffs=oracle.coefficient_table("quintic", 5),
                          variant="direct", divisor=1.0, restart_every=0, beta_a=0.9, alpha=0.5, step=step)
        nsm.muon_step(params, lr=0.02, mu=0.95, beta_a=0.9, alpha=0.5, weight_decay=0.01, ns_dtype="bf16", step=step)
        torch.cuda.synchronize()
        compare(params, before, ref, grads, "bf16", "mixed step %d" % step, ref_before=ostate,
                tol_state=TOL_STATE_LITE if step > 0 else TOL_STATE, lite_bounds=lite_bounds)
        ostate = advance_oracle_state(ostate, ref)


# ---------------------------------------------------------------- AdamW (vector parameters)

def _adam_case(sizes, grad_dtype, steps, hp, seed, offset_first=False):
    import newton_schulz_matrix_momentum_amd as nsm
    from helpers import f32
    dt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[grad_dtype]
    gen = torch.Generator().manual_seed(seed)
    params, ref = [], []
    for k, n in enumerate(sizes):
        p0 = torch.randn(n, generator=gen, dtype=torch.float64).float()
        if offset_first and k == 0:
            # a view 4 bytes into its buffer: the unaligned element-wise path
            p = torch.zeros(n + 1, device="cuda")[1:]
            p.copy_(p0.cuda())
        else:
            p = p0.cuda()
        params.append({"param": p, "exp_avg": torch.zeros(n, device="cuda"), "exp_avg_sq": torch.zeros(n, device="cuda")})
        ref.append((p0.double().numpy(), np.zeros(n), np.zeros(n)))
    for step in range(steps):
        for q in params:
            n = q["param"].numel()
            q["grad"] = (torch.randn(n, generator=gen, dtype=torch.float64) * 10.0 ** (3 * torch.rand(1, generator=gen).item() - 2)).to(dt).cuda()
        nsm.adamw_step(params, lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
                       weight_decay=hp["weight_decay"], step=step)
        torch.cuda.synchronize()
        new_ref = []
        for q, (p, m, v) in zip(params, ref):
            p, m, v = oracle.adamw_step(p, to64(q["grad"]), m, v, step=step, lr=f32(hp["lr"]), beta1=f32(hp["beta1"]),
                                        beta2=f32(hp["beta2"]), eps=f32(hp["eps"]), weight_decay=f32(hp["weight_decay"]))
            # fp32 arithmetic: each quantity within a few fp32 ulp of its size per step
            np.testing.assert_allclose(to64(q["exp_avg"]), m, rtol=1e-5, atol=1e-6 * np.abs(m).max())
            np.testing.assert_allclose(to64(q["exp_avg_sq"]), v, rtol=1e-5, atol=1e-6 * np.abs(v).max())
            dp_gpu = to64(q["param"]) - p                       # vs the oracle's own trajectory
            assert np.max(np.abs(dp_gpu)) <= 1e-5 * (np.abs(p).max() + hp["lr"] * (step + 1)), (step, np.max(np.abs(dp_gpu)))
            new_ref.append((p, m, v))
        ref = new_ref


@pytest.mark.parametrize("grad_dtype", ["f32", "bf16", "f16"])
def test_adamw_matches_oracle(grad_dtype):
    """Ragged sizes (1, 3, one block, one block +/- 1, multi-block), three steps."""
    hp = dict(lr=3e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
    _adam_case([1, 3, 4095, 4096, 4097, 100003, 192], grad_dtype, 3, hp, seed=51, offset_first=True)


def test_adamw_many_tensors_and_late_step():
    """More tensors than one launch holds (64), and bias corrections at a
    large step count."""
    hp = dict(lr=1e-3, beta1=0.8, beta2=0.999, eps=1e-6, weight_decay=0.0)
    _adam_case([17 + 13 * k for k in range(70)], "bf16", 2, hp, seed=52)


def test_optimizer_routes_vectors_to_adamw():
    """The torch.optim wrapper: 2-D weights take the Muon step, a bias and a
    norm vector take AdamW, in one optimizer step."""
    import newton_schulz_matrix_momentum_amd as nsm
    from helpers import f32
    torch.manual_seed(53)
    w = torch.nn.Parameter(torch.randn(96, 160, device="cuda") * 0.02)
    b = torch.nn.Parameter(torch.randn(96, device="cuda"))
    w0, b0 = w.detach().clone(), b.detach().clone()
    opt = nsm.Muon([w, b], lr=0.02, momentum=0.95, weight_decay=0.01, ns_dtype="bf16", adamw_lr=1e-3,
                   adamw_betas=(0.9, 0.95), adamw_eps=1e-8, adamw_weight_decay=0.05)
    w.grad = torch.randn(96, 160, device="cuda")
    b.grad = torch.randn(96, device="cuda")
    opt.step()
    torch.cuda.synchronize()
    r = oracle.muon_step_matrix(to64(w0), to64(w.grad), np.zeros((96, 160)), lr=f32(0.02), mu=f32(0.95),
                                weight_decay=f32(0.01), coeffs=oracle.coefficient_table("quintic", 5))
    check_close(to64(w) - to64(w0), r["weight"] - to64(w0), 2e-2, "optimizer wrapper: dW")
    pb, _, _ = oracle.adamw_step(to64(b0), to64(b.grad), np.zeros(96), np.zeros(96), step=0, lr=f32(1e-3),
                                 beta1=f32(0.9), beta2=f32(0.95), eps=f32(1e-8), weight_decay=f32(0.05))
    np.testing.assert_allclose(to64(b), pb, rtol=1e-6, atol=1e-7)
    assert opt.state[b]["step"] == 1 and "exp_avg" in opt.state[b] and "momentum" in opt.state[w]


# ---------------------------------------------------------------- graphs and the default workspace

def test_graph_survives_workspace_growth():
    """Capture a step on one set, then step and capture a larger set (the
    default workspace grows, and the second capture empties torch's cache):
    replays of the first graph must still match eager steps bitwise, i.e.
    its workspace buffer was kept alive."""
    import newton_schulz_matrix_momentum_amd as nsm
    small = [(128, 256), (256, 128)]
    big = [(512, 1024), (1024, 512)]
    kw = dict(lr=0.02, mu=0.95, weight_decay=0.01, ns_dtype="bf16")
    pa = make_params(small, "bf16", False, 51)
    ref = make_params(small, "bf16", False, 51)
    ga_grads = draw_grads(small, "bf16", 52)
    for p, q, g in zip(pa, ref, ga_grads):
        p["grad"] = g
        q["grad"] = g.clone()
    nsm.muon_step(pa, **kw)                      # warm-up, eager
    nsm.muon_step(ref, **kw)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    ga = torch.cuda.CUDAGraph()
    with torch.cuda.graph(ga, stream=s):
        nsm.muon_step(pa, **kw)
    torch.cuda.synchronize()
    pb = make_params(big, "bf16", False, 53)
    for p, g in zip(pb, draw_grads(big, "bf16", 54)):
        p["grad"] = g
    nsm.muon_step(pb, **kw)                      # grows the default workspace
    gb = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gb, stream=s):         # empties torch's cache first
        nsm.muon_step(pb, **kw)
    torch.cuda.synchronize()
    for _ in range(3):
        ga.replay()
        gb.replay()
        torch.cuda.synchronize()
        nsm.muon_step(ref, **kw)                 # the same step, eager
        torch.cuda.synchronize()
    for p, q in zip(pa, ref):
        assert torch.equal(p["weight"], q["weight"])
        assert torch.equal(p["momentum"], q["momentum"])


# ---------------------------------------------------------------- tile-selection boundaries

BOUNDARY = [(63, 130), (64, 64), (65, 200), (127, 70), (128, 300), (129, 129), (191, 400), (192, 193),
            (193, 260), (255, 256), (256, 700), (257, 300), (383, 384), (384, 500), (385, 900), (511, 512),
            (512, 520), (513, 600), (547, 700), (548, 640), (1024, 1100), (1096, 1200)]


@pytest.mark.parametrize("ns_dtype,variant", [("bf16", "direct"), ("f16", "gram")])
def test_tile_selection_boundaries(ns_dtype, variant):
    """Short sides just below, at and above every tile and fused-update
    threshold (64-tile padding to 64/128/192/256+, the 128 and 256 tiles and
    their 7% padding limit), both orientations, many shape classes in one
    call (launches split past 8 classes)."""
    shapes = []
    for i, (s, l) in enumerate(BOUNDARY):
        shapes.append((s, l) if i % 2 == 0 else (l, s))
    run_case(shapes, grad_dtype="bf16", ns_dtype=ns_dtype, variant=variant, grad_kind="spectral", seed=14,
             divisor=1.03 if variant == "gram" else 1.0, restart_every=3 if variant == "gram" else 0)

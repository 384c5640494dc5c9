"""The C-ABI library without a GPU: it loads, exports every entry point that
include/muon.h declares, its structs match the header byte for byte, and every
argument error is reported before anything would be enqueued."""
import ctypes
import math
import os
import re
import subprocess

import pytest

from conftest import ROOT
from newton_schulz_matrix_momentum_amd import _lib

HEADER = os.path.join(ROOT, "include", "muon.h")


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(muon_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTS), names
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], stdout=subprocess.PIPE, text=True).stdout
    exported = set(re.findall(r"\bT (muon_\w+)", out))
    for n in names:
        assert n in exported, n
        assert hasattr(lib, n)


def test_struct_layout_matches_header(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text(r'''
#include <stdio.h>
#include <stddef.h>
#include "muon.h"
int main(void) {
  printf("%zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu\n", sizeof(muon_param), offsetof(muon_param, grad),
         offsetof(muon_param, prev_grad), offsetof(muon_param, rows), offsetof(muon_param, gamma),
         offsetof(muon_param, ortho_out), sizeof(muon_options), offsetof(muon_options, coeffs),
         offsetof(muon_options, divisor), offsetof(muon_options, step), offsetof(muon_options, trace),
         sizeof(muon_trace), offsetof(muon_trace, capacity), offsetof(muon_trace, group),
         offsetof(muon_trace, launches), offsetof(muon_param, mona_lite));
  printf("%zu %zu %zu %zu %zu %zu\n", offsetof(muon_options, sketch), offsetof(muon_options, sketch_ld),
         offsetof(muon_options, rank), offsetof(muon_options, oversample), offsetof(muon_options, power_iters),
         offsetof(muon_options, rcond));
  return 0;
}
''')
    exe = tmp_path / "layout"
    subprocess.check_call(["gcc", "-std=c99", "-Wall", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)])
    got = [int(v) for v in subprocess.check_output([str(exe)]).split()]
    P, O = _lib.MuonParam, _lib.MuonOptions
    want = [ctypes.sizeof(P), P.grad.offset, P.prev_grad.offset, P.rows.offset, P.gamma.offset, P.ortho_out.offset,
            ctypes.sizeof(O), O.coeffs.offset, O.divisor.offset, O.step.offset, O.trace.offset,
            ctypes.sizeof(_lib.MuonTrace), _lib.MuonTrace.capacity.offset, _lib.MuonTrace.group.offset,
            _lib.MuonTrace.launches.offset, P.mona_lite.offset,
            O.sketch.offset, O.sketch_ld.offset, O.rank.offset, O.oversample.offset, O.power_iters.offset,
            O.rcond.offset]
    assert got == want


def test_header_compiles_as_cxx(tmp_path):
    src = tmp_path / "h.cpp"
    src.write_text('#include "muon.h"\nint main() { muon_options o; muon_options_init(&o); return 0; }\n')
    subprocess.check_call(["g++", "-std=c++11", "-fsyntax-only", "-I", os.path.join(ROOT, "include"), str(src)])


def test_version_and_strings(lib):
    assert b"gfx950" in lib.muon_version()
    for s in range(5):
        assert lib.muon_status_string(s)
    assert lib.muon_status_string(99) == b"unknown status"


# ---------------------------------------------------------------- validation
# Fake device addresses: validation fails before any pointer is touched.
BASE = 1 << 40


def param(i, rows=8, cols=16, mona=False, gamma=1.0):
    p = _lib.MuonParam()
    step = 1 << 28
    p.weight = BASE + i * 8 * step
    p.grad = BASE + (i * 8 + 1) * step
    p.momentum = BASE + (i * 8 + 2) * step
    if mona:
        p.accel = BASE + (i * 8 + 3) * step
        p.prev_grad = BASE + (i * 8 + 4) * step
    p.rows, p.cols, p.gamma = rows, cols, gamma
    return p


def arr(*ps):
    a = (_lib.MuonParam * max(len(ps), 1))()
    for i, p in enumerate(ps):
        a[i] = p
    return a


def opts(lib, **kw):
    o = _lib.MuonOptions()
    lib.muon_options_init(ctypes.byref(o))
    for k, v in kw.items():
        setattr(o, k, v)
    return o


def step(lib, ps, n=None, o=None, ns_steps=5, variant=0, ws=BASE * 4, ws_bytes=1 << 40, lr=0.02, mu=0.95,
         beta=0.9, alpha=0.5, wd=0.01):
    n = len(ps) if n is None else n
    return lib.muon_step(arr(*ps), n, lr, mu, beta, alpha, wd, ns_steps, variant,
                         ctypes.byref(o) if o is not None else None, ws, ws_bytes, None)


def test_empty_call_is_ok(lib):
    assert lib.muon_step(None, 0, 0.02, 0.95, 0.9, 0.5, 0.01, 5, 0, None, None, 0, None) == _lib.MUON_OK


def test_invalid_arguments(lib):
    E = _lib.MUON_ERR_INVALID_ARG
    assert step(lib, [param(0)], n=-1) == E
    assert lib.muon_step(None, 2, 0.02, 0.95, 0.9, 0.5, 0.01, 5, 0, None, BASE, 1 << 30, None) == E
    p = param(0, rows=0)
    assert step(lib, [p]) == E
    p = param(0)
    p.weight = None
    assert step(lib, [p]) == E
    p = param(0, mona=True)
    p.prev_grad = None
    assert step(lib, [p]) == E
    assert "prev_grad" in _lib.last_error()
    assert step(lib, [param(0)], ns_steps=-1) == E
    assert step(lib, [param(0)], ns_steps=65) == E
    assert step(lib, [param(0)], variant=7) == E
    assert step(lib, [param(0)], o=opts(lib, divisor=0.5)) == E
    assert step(lib, [param(0)], o=opts(lib, divisor=float("nan"))) == E
    assert step(lib, [param(0)], o=opts(lib, restart_every=-1)) == E
    assert step(lib, [param(0)], o=opts(lib, step=-3)) == E
    assert step(lib, [param(0)], lr=float("inf")) == E
    assert step(lib, [param(0)], alpha=float("nan")) == E
    assert step(lib, [param(0, gamma=float("nan"))]) == E
    bad = (ctypes.c_float * 15)(*([1.0] * 14 + [math.inf]))
    assert step(lib, [param(0)], o=opts(lib, coeffs=ctypes.cast(bad, ctypes.POINTER(ctypes.c_float)))) == E
    assert step(lib, [param(0)], ws=None) == E
    assert step(lib, [param(0)], ws=BASE * 4 + 8) == E     # unaligned workspace
    p = param(0, mona=True)
    p.mona_lite = BASE + 7 * (1 << 28)
    assert step(lib, [p]) == E                             # MONA-Lite and MONA state together
    assert "mona_lite" in _lib.last_error()
    p = param(0)
    p.mona_lite = p.momentum + 16                          # overlaps momentum
    assert step(lib, [p]) == E
    assert "overlap" in _lib.last_error()


def test_unsupported(lib):
    U = _lib.MUON_ERR_UNSUPPORTED
    assert step(lib, [param(0)], o=opts(lib, grad_dtype=9)) == U
    assert step(lib, [param(0)], o=opts(lib, ns_dtype=-1)) == U
    assert step(lib, [param(0, rows=1 << 21, cols=2)]) == U
    assert step(lib, [param(0, rows=2, cols=(1 << 20) + 1)]) == U
    assert step(lib, [param(0, rows=46341, cols=46341)]) == U      # 2^31 + 4633 elements
    assert "exceeds the supported size" in _lib.last_error()


def test_overlap_rejected(lib):
    E = _lib.MUON_ERR_INVALID_ARG
    p = param(0)
    p.momentum = p.weight + 4 * 8   # inside weight's 8x16 fp32 range
    assert step(lib, [p]) == E
    a, b = param(0), param(1)
    b.grad = a.grad                  # two params sharing a gradient
    assert step(lib, [a, b]) == E
    assert "overlap" in _lib.last_error()


def test_limuon_argument_checks(lib):
    """MUON_LIMUON: every setting is checked before anything would run."""
    E, U = _lib.MUON_ERR_INVALID_ARG, _lib.MUON_ERR_UNSUPPORTED
    L = _lib.MUON_LIMUON
    sk = BASE * 3
    good = dict(sketch=sk, sketch_ld=16, rank=4, oversample=4)
    ws = lib.muon_workspace_size(arr(param(0)), 1, 5, L, ctypes.byref(opts(lib, **good)))
    assert ws > 0, _lib.last_error()
    assert lib.muon_workspace_size(arr(param(0)), 1, 5, L, ctypes.byref(opts(lib, **dict(good, rank=0)))) == 0
    assert step(lib, [param(0)], variant=L, o=opts(lib, **dict(good, sketch=None))) == E
    assert "sketch" in _lib.last_error()
    assert step(lib, [param(0)], variant=L, o=opts(lib, **dict(good, rank=0))) == E
    assert step(lib, [param(0)], variant=L, o=opts(lib, **dict(good, oversample=-1))) == E
    assert step(lib, [param(0)], variant=L, o=opts(lib, **dict(good, rank=40, oversample=25))) == E
    assert "64" in _lib.last_error()
    assert step(lib, [param(0)], variant=L, o=opts(lib, **dict(good, power_iters=17))) == E
    assert step(lib, [param(0)], variant=L, o=opts(lib, **dict(good, rcond=1.0))) == E
    assert step(lib, [param(0)], variant=L, o=opts(lib, **dict(good, rcond=float("nan")))) == E
    assert step(lib, [param(0)], variant=L, o=opts(lib, **dict(good, sketch_ld=15))) == E   # long side 16
    assert "sketch_ld" in _lib.last_error()
    p = param(0)
    assert step(lib, [p], variant=L, o=opts(lib, **dict(good, sketch=p.weight + 64))) == E   # inside W
    assert "overlap" in _lib.last_error()
    assert step(lib, [param(0)], variant=L, o=opts(lib, **dict(good, ns_dtype=_lib.MUON_BF16))) == U
    # the LiMuon settings are ignored by the Newton-Schulz variants
    assert lib.muon_workspace_size(arr(param(0)), 1, 5, 0, ctypes.byref(opts(lib, rank=0, sketch=None))) > 0


def test_workspace_size_and_too_small(lib):
    ps = [param(0, 100, 300), param(1, 300, 100), param(2, 64, 64)]
    o = opts(lib, ns_dtype=_lib.MUON_BF16)
    need = lib.muon_workspace_size(arr(*ps), 3, 5, 0, ctypes.byref(o))
    assert need > 0 and need % 256 == 0
    # independent of pointer values
    moved = [param(i + 5, p.rows, p.cols) for i, p in enumerate(ps)]
    assert lib.muon_workspace_size(arr(*moved), 3, 5, 0, ctypes.byref(o)) == need
    gram = lib.muon_workspace_size(arr(*ps), 3, 5, 1, ctypes.byref(o))
    assert gram > need
    f32 = lib.muon_workspace_size(arr(*ps), 3, 5, 0, None)
    assert f32 > need
    assert step(lib, ps, o=o, ws_bytes=need - 1) == _lib.MUON_ERR_WORKSPACE_TOO_SMALL
    assert lib.muon_workspace_size(arr(param(0, rows=0)), 1, 5, 0, None) == 0
    assert lib.muon_workspace_size(None, 0, 5, 0, None) > 0


def test_product_path_has_no_oracle_import():
    """The package never imports the oracle or any CPU fallback."""
    pkg = os.path.join(ROOT, "newton_schulz_matrix_momentum_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith(".py"):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text, f
                assert "numpy" not in text, f


# ---------------------------------------------------------------- AdamW entry point

def test_adamw_param_layout_matches_header(tmp_path):
    src = tmp_path / "adam_layout.c"
    src.write_text(r'''
#include <stdio.h>
#include <stddef.h>
#include "muon.h"
int main(void) {
  printf("%zu %zu %zu %zu %zu\n", sizeof(muon_adamw_param), offsetof(muon_adamw_param, grad),
         offsetof(muon_adamw_param, exp_avg), offsetof(muon_adamw_param, exp_avg_sq), offsetof(muon_adamw_param, numel));
  return 0;
}
''')
    exe = tmp_path / "adam_layout"
    subprocess.check_call(["gcc", "-std=c99", "-Wall", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)])
    got = [int(v) for v in subprocess.check_output([str(exe)]).split()]
    A = _lib.MuonAdamwParam
    assert got == [ctypes.sizeof(A), A.grad.offset, A.exp_avg.offset, A.exp_avg_sq.offset, A.numel.offset]


def adam_param(i, numel=1000):
    a = _lib.MuonAdamwParam()
    step = 1 << 28
    a.param = BASE + i * 8 * step
    a.grad = BASE + (i * 8 + 1) * step
    a.exp_avg = BASE + (i * 8 + 2) * step
    a.exp_avg_sq = BASE + (i * 8 + 3) * step
    a.numel = numel
    return a


def adam(lib, ps, n=None, dtype=_lib.MUON_F32, lr=1e-3, b1=0.9, b2=0.999, eps=1e-8, wd=0.0, step=0):
    arr_ = (_lib.MuonAdamwParam * max(len(ps), 1))(*ps)
    return lib.muon_adamw_step(arr_, len(ps) if n is None else n, dtype, lr, b1, b2, eps, wd, step, None, None)


def test_adamw_validation(lib):
    E, U = _lib.MUON_ERR_INVALID_ARG, _lib.MUON_ERR_UNSUPPORTED
    assert lib.muon_adamw_step(None, 0, 0, 1e-3, 0.9, 0.999, 1e-8, 0.0, 0, None, None) == _lib.MUON_OK
    assert adam(lib, [adam_param(0)], n=-1) == E
    assert adam(lib, [adam_param(0, numel=0)]) == E
    p = adam_param(0)
    p.exp_avg = None
    assert adam(lib, [p]) == E
    assert adam(lib, [adam_param(0)], b1=1.0) == E
    assert adam(lib, [adam_param(0)], b2=-0.1) == E
    assert adam(lib, [adam_param(0)], eps=-1e-8) == E
    assert adam(lib, [adam_param(0)], lr=float("nan")) == E
    assert adam(lib, [adam_param(0)], step=-1) == E
    assert adam(lib, [adam_param(0)], dtype=7) == U
    assert adam(lib, [adam_param(0, numel=1 << 31)]) == U
    a, b = adam_param(0), adam_param(1)
    b.exp_avg_sq = a.param + 8          # inside a's param
    assert adam(lib, [a, b]) == E
    assert "overlap" in _lib.last_error()


def test_workspace_keeps_buffers_used_under_graph_capture(monkeypatch):
    """A workspace buffer handed out during a graph capture stays alive when the
    workspace grows (the captured graph keeps its address); one never used
    under capture is dropped."""
    import torch
    from newton_schulz_matrix_momentum_amd.api import Workspace
    ws = Workspace()
    capturing = {"on": False}
    monkeypatch.setattr(Workspace, "_capturing", staticmethod(lambda device: capturing["on"]))
    a = ws.get(1000, torch.device("cpu"))
    assert ws.get(500, torch.device("cpu")) is a          # big enough: reused
    b = ws.get(5000, torch.device("cpu"))                  # grows; a was never captured
    assert b is not a and ws.retired == []
    capturing["on"] = True
    assert ws.get(100, torch.device("cpu")) is b          # handed out during a capture
    capturing["on"] = False
    c = ws.get(10000, torch.device("cpu"))                 # grows again: b must survive
    assert c is not b and len(ws.retired) == 1 and ws.retired[0] is b
    assert ws.get(20000, torch.device("cpu")) is not c and len(ws.retired) == 1   # c never captured


def test_static_entry_point_rejects_oversized_call_before_any_device_call(lib):
    """muon_step_static sizes the call on the host first: a request beyond
    its static workspace fails without touching the device (so this runs
    without a GPU)."""
    big = param(0, 4096, 4096)
    o = opts(lib, ns_dtype=_lib.MUON_BF16)
    need = lib.muon_workspace_size(arr(big), 1, 5, 0, ctypes.byref(o))
    assert need > _lib.STATIC_WORKSPACE_BYTES
    st = lib.muon_step_static(arr(big), 1, 0.02, 0.95, 0.0, 0.0, 0.0, 5, 0, ctypes.byref(o), None)
    assert st == _lib.MUON_ERR_WORKSPACE_TOO_SMALL
    assert "static workspace" in _lib.last_error()
    assert lib.muon_step_static(arr(param(0, rows=0)), 1, 0.02, 0.95, 0.0, 0.0, 0.0, 5, 0, None, None) \
        == _lib.MUON_ERR_INVALID_ARG

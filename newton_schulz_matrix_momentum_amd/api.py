"""Python entry points with the C ABI's names, over torch tensors.

``muon_step`` and ``muon_workspace_size`` marshal torch tensors into
``muon_param`` records and call libmuon; ``adamw_step`` does the same for
``muon_adamw_param``.  The stream is torch's current stream on the tensors'
device.  Tensors must be contiguous and live on the GPU.
"""
from __future__ import annotations

import ctypes
from typing import Dict, List, Optional, Sequence

import torch

from . import _lib

_DT = {torch.float32: _lib.MUON_F32, torch.float16: _lib.MUON_F16, torch.bfloat16: _lib.MUON_BF16}
_DT_NAMES = {"f32": _lib.MUON_F32, "fp32": _lib.MUON_F32, "float32": _lib.MUON_F32,
             "f16": _lib.MUON_F16, "fp16": _lib.MUON_F16, "float16": _lib.MUON_F16,
             "bf16": _lib.MUON_BF16, "bfloat16": _lib.MUON_BF16}
_VARIANTS = {"direct": _lib.MUON_NS_DIRECT, "gram": _lib.MUON_NS_GRAM, "limuon": _lib.MUON_LIMUON}


def _ptr(t: Optional[torch.Tensor], name: str, dtype=None, shape=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a GPU tensor (got %s)" % (name, t.device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must be %s (got %s)" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    return t.data_ptr()


def _dtype_code(x):
    if x is None:
        return None
    if isinstance(x, torch.dtype):
        return _DT[x]
    return _DT_NAMES[str(x).lower()]


def _marshal(params: Sequence[Dict], ns_dtype, coeffs, divisor, restart_every, step, trace=None, limuon=None):
    n = len(params)
    arr = (_lib.MuonParam * max(n, 1))()
    grad_dtype = None
    device = None
    for i, p in enumerate(params):
        w = p["weight"]
        if w.dim() != 2:
            raise ValueError("param %d: weight must be 2-D" % i)
        rows, cols = w.shape
        g = p["grad"]
        if grad_dtype is None:
            grad_dtype = g.dtype
        elif g.dtype != grad_dtype:
            raise ValueError("all grads of one call must share a dtype (param %d is %s, expected %s)"
                             % (i, g.dtype, grad_dtype))
        device = device or w.device
        for key in ("grad", "momentum", "accel", "prev_grad", "ortho_out", "mona_lite"):
            t = p.get(key)
            if t is not None and t.device != w.device:
                raise ValueError("param %d: %s is on %s, weight on %s" % (i, key, t.device, w.device))
        arr[i].weight = _ptr(w, "weight", torch.float32)
        arr[i].grad = _ptr(g, "grad", None, (rows, cols))
        arr[i].momentum = _ptr(p["momentum"], "momentum", torch.float32, (rows, cols))
        arr[i].accel = _ptr(p.get("accel"), "accel", torch.float32, (rows, cols))
        arr[i].prev_grad = _ptr(p.get("prev_grad"), "prev_grad", grad_dtype, (rows, cols))
        arr[i].rows = rows
        arr[i].cols = cols
        arr[i].gamma = float(p.get("gamma", 1.0))
        arr[i].ortho_out = _ptr(p.get("ortho_out"), "ortho_out", torch.float32, (rows, cols))
        arr[i].mona_lite = _ptr(p.get("mona_lite"), "mona_lite", torch.bfloat16, (rows, cols))
    opts = _lib.MuonOptions()
    _lib.load().muon_options_init(ctypes.byref(opts))
    if grad_dtype is not None:
        opts.grad_dtype = _DT[grad_dtype]
    nsd = _dtype_code(ns_dtype)
    opts.ns_dtype = nsd if nsd is not None else opts.grad_dtype
    keep = None
    if coeffs is not None:
        flat = [float(v) for row in coeffs for v in row]
        keep = (ctypes.c_float * len(flat))(*flat)
        opts.coeffs = ctypes.cast(keep, ctypes.POINTER(ctypes.c_float))
    opts.divisor = float(divisor)
    opts.restart_every = int(restart_every)
    opts.step = int(step)
    if trace is not None:
        opts.trace = ctypes.pointer(trace)
    if limuon:
        sk = limuon.get("sketch")
        if sk is not None:
            if sk.dim() != 2:
                raise ValueError("sketch must be 2-D: (rank + oversample) x sketch_ld")
            if device is not None and sk.device != device:
                raise ValueError("sketch is on %s, the weights on %s" % (sk.device, device))
            opts.sketch = _ptr(sk, "sketch", torch.float32)
            opts.sketch_ld = int(sk.shape[1])
            if "oversample" not in limuon and limuon.get("rank") is not None:
                opts.oversample = int(sk.shape[0]) - int(limuon["rank"])
        for key in ("rank", "oversample", "power_iters"):
            if limuon.get(key) is not None:
                setattr(opts, key, int(limuon[key]))
        if limuon.get("rcond") is not None:
            opts.rcond = float(limuon["rcond"])
        if sk is not None and int(sk.shape[0]) != opts.rank + opts.oversample:
            raise ValueError("sketch has %d rows, rank + oversample is %d" % (sk.shape[0], opts.rank + opts.oversample))
    return arr, n, opts, keep, device


def muon_workspace_size(params: Sequence[Dict], *, ns_steps: int = 5, variant: str = "direct", ns_dtype=None,
                        coeffs=None, divisor: float = 1.0, restart_every: int = 0, step: int = 0,
                        sketch=None, rank=None, oversample=None, power_iters=None, rcond=None) -> int:
    lm = dict(sketch=sketch, rank=rank, power_iters=power_iters, rcond=rcond)
    if oversample is not None:
        lm["oversample"] = oversample
    arr, n, opts, keep, _ = _marshal(params, ns_dtype, coeffs, divisor, restart_every, step, limuon=lm)
    size = _lib.load().muon_workspace_size(arr, n, int(ns_steps), _VARIANTS[variant], ctypes.byref(opts))
    if size == 0 and n > 0:
        raise _lib.MuonError(_lib.MUON_ERR_INVALID_ARG, _lib.last_error())
    return int(size)


def debug_square_buffer(params: Sequence[Dict], index: int, which: int, *, ns_steps: int = 5,
                        variant: str = "direct", ns_dtype=None, coeffs=None, divisor: float = 1.0,
                        restart_every: int = 0, step: int = 0):
    """(byte offset, leading dimension, side) of square work buffer ``which``
    of param ``index`` in the workspace of the described call
    (``muon_debug_square_buffer``)."""
    arr, n, opts, keep, _ = _marshal(params, ns_dtype, coeffs, divisor, restart_every, step)
    off, ld, side = ctypes.c_size_t(), ctypes.c_int64(), ctypes.c_int64()
    _lib.check(_lib.load().muon_debug_square_buffer(arr, n, int(ns_steps), _VARIANTS[variant], ctypes.byref(opts),
                                                    int(index), int(which), ctypes.byref(off), ctypes.byref(ld),
                                                    ctypes.byref(side)))
    return off.value, ld.value, side.value


class Workspace:
    """A reusable device byte buffer for ``muon_step`` (grows on demand).

    A buffer handed out while a HIP graph was being captured is never freed
    when the workspace grows: the captured graph keeps using its address on
    every replay, and torch releases cached blocks to the driver when the
    next capture starts, so freeing it would leave the old graph writing
    into unmapped memory.  Such buffers are kept in ``retired`` for the
    life of the workspace."""

    def __init__(self):
        self.buf = None
        self.captured = False   # self.buf was handed out during a capture
        self.retired = []

    @staticmethod
    def _capturing(device) -> bool:
        try:
            return torch.device(device).type == "cuda" and torch.cuda.is_current_stream_capturing()
        except Exception:  # pragma: no cover - no HIP runtime
            return False

    def get(self, nbytes: int, device) -> torch.Tensor:
        if self.buf is None or self.buf.numel() < nbytes or self.buf.device != torch.device(device):
            if self.buf is not None and self.captured:
                self.retired.append(self.buf)
            self.buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
            self.captured = False
        if self._capturing(device):
            self.captured = True
        return self.buf


# Default workspaces, one per (device, stream): a workspace is written by the
# kernels of the stream it is used on, so two streams never share one, and the
# caching allocator (which hands a freed block only to allocations on the
# stream it was allocated on) cannot give a grown-out buffer to another
# stream while kernels of its own stream still use it.
_default_ws: Dict = {}


def muon_step(params: Sequence[Dict], *, lr: float, mu: float, beta_a: float = 0.0, alpha: float = 0.0,
              weight_decay: float = 0.0, ns_steps: int = 5, variant: str = "direct", ns_dtype=None, coeffs=None,
              divisor: float = 1.0, restart_every: int = 0, step: int = 0,
              workspace: Optional[torch.Tensor] = None, trace=None, sketch=None, rank=None, oversample=None,
              power_iters=None, rcond=None) -> None:
    """One Muon / MONA step over ``params`` (list of dicts of tensors).

    Each dict holds ``weight`` (fp32, updated), ``grad``, ``momentum`` (fp32,
    updated) and optionally ``accel`` + ``prev_grad`` (MONA state, updated) or
    ``mona_lite`` (bfloat16 MONA-Lite state, updated), ``gamma`` (float) and
    ``ortho_out`` (fp32, receives O).  Enqueued on the
    current stream; returns without synchronising.  ``trace`` is an optional
    ``_lib.MuonTrace`` for per-launch HIP-event timing.

    ``variant="limuon"`` orthogonalises by a randomized SVD instead of
    Newton-Schulz: ``sketch`` is the Gaussian test matrix, a float32 GPU
    tensor of (rank + oversample) x L (L >= every matrix's long side), with
    ``rank``, ``power_iters`` (default 1) and ``rcond`` (default 1e-4);
    ``ns_dtype`` must be f32.
    """
    lm = dict(sketch=sketch, rank=rank, power_iters=power_iters, rcond=rcond)
    if oversample is not None:
        lm["oversample"] = oversample
    arr, n, opts, keep, device = _marshal(params, ns_dtype, coeffs, divisor, restart_every, step, trace, lm)
    lib = _lib.load()
    if n == 0:
        _lib.check(lib.muon_step(arr, 0, lr, mu, beta_a, alpha, weight_decay, int(ns_steps), _VARIANTS[variant],
                                 ctypes.byref(opts), None, 0, None))
        return
    need = lib.muon_workspace_size(arr, n, int(ns_steps), _VARIANTS[variant], ctypes.byref(opts))
    if need == 0:
        raise _lib.MuonError(_lib.MUON_ERR_INVALID_ARG, _lib.last_error())
    cur = torch.cuda.current_stream(device)
    if workspace is None:
        ws = _default_ws.setdefault((device, cur.cuda_stream), Workspace()).get(need, device)
    else:
        if workspace.device != device or workspace.dtype != torch.uint8:
            raise ValueError("workspace must be a uint8 tensor on %s" % device)
        ws = workspace
        # a caller's workspace allocated on another stream stays reserved
        # until this stream's kernels are done with it (outside captures: a
        # captured graph's memory lives as long as the graph)
        if not Workspace._capturing(device):
            ws.record_stream(cur)
    stream = cur.cuda_stream
    _lib.check(lib.muon_step(arr, n, float(lr), float(mu), float(beta_a), float(alpha), float(weight_decay),
                             int(ns_steps), _VARIANTS[variant], ctypes.byref(opts), ctypes.c_void_p(ws.data_ptr()),
                             ws.numel(), ctypes.c_void_p(stream)))


def muon_step_static(params: Sequence[Dict], *, lr: float, mu: float, beta_a: float = 0.0, alpha: float = 0.0,
                     weight_decay: float = 0.0, ns_steps: int = 5, variant: str = "direct", ns_dtype=None,
                     coeffs=None, divisor: float = 1.0, restart_every: int = 0, step: int = 0, trace=None,
                     sketch=None, rank=None, oversample=None, power_iters=None, rcond=None) -> None:
    """``muon_step`` through ``muon_step_static``: the same step with the
    library's static per-GPU workspace (64 MiB) instead of an allocated one,
    for callers that cannot allocate.  Calls on one GPU share that workspace:
    order them on one stream.  Raises when the call needs a larger workspace."""
    lm = dict(sketch=sketch, rank=rank, power_iters=power_iters, rcond=rcond)
    if oversample is not None:
        lm["oversample"] = oversample
    arr, n, opts, keep, device = _marshal(params, ns_dtype, coeffs, divisor, restart_every, step, trace, lm)
    lib = _lib.load()
    stream = torch.cuda.current_stream(device).cuda_stream if device is not None else None
    _lib.check(lib.muon_step_static(arr, n, float(lr), float(mu), float(beta_a), float(alpha), float(weight_decay),
                                    int(ns_steps), _VARIANTS[variant], ctypes.byref(opts),
                                    ctypes.c_void_p(stream) if stream else None))


def adamw_step(params: Sequence[Dict], *, lr: float, betas=(0.9, 0.999), eps: float = 1e-8,
               weight_decay: float = 0.0, step: int = 0, trace=None) -> None:
    """One decoupled AdamW step (``muon_adamw_step``) over ``params``: dicts of
    ``param`` (fp32, updated), ``grad``, ``exp_avg`` and ``exp_avg_sq`` (fp32,
    updated; zero before step 0), any shape, all grads of one dtype.
    ``step`` is 0-based.  Enqueued on the current stream."""
    n = len(params)
    arr = (_lib.MuonAdamwParam * max(n, 1))()
    grad_dtype = None
    device = None
    for i, p in enumerate(params):
        t = p["param"]
        g = p["grad"]
        if grad_dtype is None:
            grad_dtype = g.dtype
        elif g.dtype != grad_dtype:
            raise ValueError("all grads of one call must share a dtype (param %d is %s, expected %s)"
                             % (i, g.dtype, grad_dtype))
        device = device or t.device
        for key in ("grad", "exp_avg", "exp_avg_sq"):
            if p[key].device != t.device:
                raise ValueError("adamw param %d: %s is on %s, param on %s" % (i, key, p[key].device, t.device))
        arr[i].param = _ptr(t, "param", torch.float32)
        arr[i].grad = _ptr(g, "grad", None, tuple(t.shape))
        arr[i].exp_avg = _ptr(p["exp_avg"], "exp_avg", torch.float32, tuple(t.shape))
        arr[i].exp_avg_sq = _ptr(p["exp_avg_sq"], "exp_avg_sq", torch.float32, tuple(t.shape))
        arr[i].numel = t.numel()
    lib = _lib.load()
    stream = torch.cuda.current_stream(device).cuda_stream if device is not None else 0
    _lib.check(lib.muon_adamw_step(arr, n, _DT[grad_dtype] if grad_dtype is not None else _lib.MUON_F32,
                                   float(lr), float(betas[0]), float(betas[1]), float(eps), float(weight_decay),
                                   int(step), ctypes.pointer(trace) if trace is not None else None,
                                   ctypes.c_void_p(stream)))

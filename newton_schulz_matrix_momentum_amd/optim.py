"""``torch.optim``-style wrapper around ``muon_step``.

Holds the per-matrix state (momentum M; for MONA the acceleration A and the
previous gradient; for MONA-Lite one bfloat16 state) as tensors in
``self.state`` so that ``state_dict`` checkpoints and resumes them.  Only 2-D parameters are accepted: the MONA
summary ("Ontwerprichtlijnen") leaves vector parameters (embeddings, biases)
to AdamW.
"""
from __future__ import annotations

import torch

from .api import muon_step


class Muon(torch.optim.Optimizer):
    def __init__(self, params, lr=0.02, momentum=0.95, weight_decay=0.01, ns_steps=5, variant="direct",
                 ns_dtype="bf16", coeffs=None, mona=False, beta_a=0.9, alpha=0.5, divisor=1.0,
                 restart_every=0, gamma=1.0, mona_lite=False):
        """``mona=True`` keeps MONA's fp32 A and previous gradient;
        ``mona_lite=True`` (MONA summary, "Efficiëntie en Implementatie")
        keeps one bfloat16 state instead."""
        if mona and mona_lite:
            raise ValueError("choose one of mona and mona_lite")
        defaults = dict(lr=lr, momentum=momentum, weight_decay=weight_decay, ns_steps=ns_steps, variant=variant,
                        ns_dtype=ns_dtype, coeffs=coeffs, mona=mona, beta_a=beta_a, alpha=alpha, divisor=divisor,
                        restart_every=restart_every, gamma=gamma, mona_lite=mona_lite)
        super().__init__(params, defaults)
        for group in self.param_groups:
            for p in group["params"]:
                if p.dim() != 2:
                    raise ValueError("Muon handles 2-D weight matrices only (got shape %s)" % (tuple(p.shape),))
                if p.dtype != torch.float32:
                    raise ValueError("Muon keeps fp32 master weights (got %s)" % p.dtype)

    @torch.no_grad()
    def step(self, closure=None):
        loss = None
        if closure is not None:
            with torch.enable_grad():
                loss = closure()
        for group in self.param_groups:
            by_dtype = {}
            for p in group["params"]:
                if p.grad is None:
                    continue
                st = self.state[p]
                if not st:
                    st["step"] = 0
                    st["momentum"] = torch.zeros_like(p, dtype=torch.float32)
                    if group["mona"]:
                        st["accel"] = torch.zeros_like(p, dtype=torch.float32)
                        st["prev_grad"] = torch.zeros_like(p.grad)
                    if group["mona_lite"]:
                        st["mona_lite"] = torch.zeros_like(p, dtype=torch.bfloat16)
                g = p.grad if p.grad.is_contiguous() else p.grad.contiguous()
                rec = {"weight": p, "grad": g, "momentum": st["momentum"], "gamma": group["gamma"]}
                if group["mona"]:
                    rec["accel"] = st["accel"]
                    rec["prev_grad"] = st["prev_grad"]
                if group["mona_lite"]:
                    rec["mona_lite"] = st["mona_lite"]
                by_dtype.setdefault((g.dtype, st["step"]), []).append((p, rec))
            for (_, step), items in by_dtype.items():
                muon_step([r for _, r in items], lr=group["lr"], mu=group["momentum"], beta_a=group["beta_a"],
                          alpha=group["alpha"], weight_decay=group["weight_decay"], ns_steps=group["ns_steps"],
                          variant=group["variant"], ns_dtype=group["ns_dtype"], coeffs=group["coeffs"],
                          divisor=group["divisor"], restart_every=group["restart_every"], step=step)
                for p, _ in items:
                    self.state[p]["step"] = step + 1
        return loss

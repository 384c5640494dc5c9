"""``torch.optim``-style wrapper around ``muon_step``.

Holds the per-matrix state (momentum M; for MONA the acceleration A and the
previous gradient; for MONA-Lite one bfloat16 state) as tensors in
``self.state`` so that ``state_dict`` checkpoints and resumes them.  As the MONA summary ("Ontwerprichtlijnen")
prescribes, parameters that are not 2-D (biases, norm weights) -- and every
parameter of a group created with ``adamw=True`` (e.g. embeddings) -- are
updated by the fused AdamW of libmuon (``muon_adamw_step``) instead.
"""
from __future__ import annotations

import torch

from .api import adamw_step, muon_step


class Muon(torch.optim.Optimizer):
    def __init__(self, params, lr=0.02, momentum=0.95, weight_decay=0.01, ns_steps=5, variant="direct",
                 ns_dtype="bf16", coeffs=None, mona=False, beta_a=0.9, alpha=0.5, divisor=1.0,
                 restart_every=0, gamma=1.0, mona_lite=False, adamw=False, adamw_lr=3e-4,
                 adamw_betas=(0.9, 0.95), adamw_eps=1e-8, adamw_weight_decay=0.0):
        """``mona=True`` keeps MONA's fp32 A and previous gradient;
        ``mona_lite=True`` (MONA summary, "Efficiëntie en Implementatie")
        keeps one bfloat16 state instead.  ``adamw=True`` sends every
        parameter of the group to AdamW with the ``adamw_*`` settings, which
        non-2-D parameters always use."""
        if mona and mona_lite:
            raise ValueError("choose one of mona and mona_lite")
        defaults = dict(lr=lr, momentum=momentum, weight_decay=weight_decay, ns_steps=ns_steps, variant=variant,
                        ns_dtype=ns_dtype, coeffs=coeffs, mona=mona, beta_a=beta_a, alpha=alpha, divisor=divisor,
                        restart_every=restart_every, gamma=gamma, mona_lite=mona_lite, adamw=adamw,
                        adamw_lr=adamw_lr, adamw_betas=adamw_betas, adamw_eps=adamw_eps,
                        adamw_weight_decay=adamw_weight_decay)
        super().__init__(params, defaults)
        for group in self.param_groups:
            for p in group["params"]:
                if p.dtype != torch.float32:
                    raise ValueError("Muon keeps fp32 master weights (got %s)" % p.dtype)

    @staticmethod
    def _uses_adamw(group, p):
        return group["adamw"] or p.dim() != 2

    @torch.no_grad()
    def step(self, closure=None):
        loss = None
        if closure is not None:
            with torch.enable_grad():
                loss = closure()
        for group in self.param_groups:
            by_dtype = {}
            adam = {}
            for p in group["params"]:
                if p.grad is None:
                    continue
                st = self.state[p]
                if self._uses_adamw(group, p):
                    if not st:
                        st["step"] = 0
                        st["exp_avg"] = torch.zeros_like(p, dtype=torch.float32)
                        st["exp_avg_sq"] = torch.zeros_like(p, dtype=torch.float32)
                    g = p.grad if p.grad.is_contiguous() else p.grad.contiguous()
                    rec = {"param": p, "grad": g, "exp_avg": st["exp_avg"], "exp_avg_sq": st["exp_avg_sq"]}
                    adam.setdefault((g.dtype, st["step"]), []).append((p, rec))
                    continue
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
            for (_, step), items in adam.items():
                adamw_step([r for _, r in items], lr=group["adamw_lr"], betas=group["adamw_betas"],
                           eps=group["adamw_eps"], weight_decay=group["adamw_weight_decay"], step=step)
                for p, _ in items:
                    self.state[p]["step"] = step + 1
        return loss

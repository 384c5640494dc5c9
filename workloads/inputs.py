"""Seeded synthetic inputs shaped like the transformer layers the pages train.

The pages train on corpora and checkpoints that are not available here
(NanoChat in the Ringmaster LMO summary; Llama-430M, Qwen-600M, Gemma-1B and a
MoE in the Gram Newton-Schulz post; MoE-1B/6B/68B in the MONA summary).  These
generators stand in for their gradients: the same shapes, with value
distributions chosen to stress the orthogonaliser (wide singular-value
spreads, low-rank spikes, per-expert scale differences).

Seeds: ``seed_for(workload_index, matrix_index, step)`` =
1000 * workload_index + 10 * matrix_index + step.  Values are drawn in float64
and rounded once (round-to-nearest-even) to the gradient dtype, so every
consumer sees identical stored values.  Generation runs on any torch device; a
given device type always reproduces the same values for the same seed.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import torch

_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclass
class Workload:
    """One synthetic parameter set and its optimizer settings."""

    name: str
    index: int                       # used in the seed
    shapes: List[Tuple[int, int]]    # (rows, cols) per matrix, row-major
    grad_dtype: str                  # "f32" | "bf16" | "f16"
    ns_dtype: str                    # dtype of the Newton-Schulz operands
    grad_kind: str                   # "gaussian" | "spectral" | "spike" | "expert"
    coeffs: str = "quintic"          # "cubic" | "quintic"
    ns_steps: int = 5
    variants: Tuple[str, ...] = ("direct",)
    lr: float = 0.02
    mu: float = 0.95
    weight_decay: float = 0.01
    mona: bool = False
    beta_a: float = 0.9
    alpha: float = 0.5
    steps: int = 1                   # consecutive optimizer steps
    divisor: float = 1.0             # Gram variant's safety divisor
    restart_every: int = 0           # Gram variant's restart period
    grad_std: float = 1.0
    log10_sv: Tuple[float, float] = (-4.0, 0.0)   # singular-value range (spectral)
    spike_rank: int = 8
    expert_of: Optional[List[int]] = None        # per matrix: expert id or -1
    note: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def numel(self) -> int:
        return sum(r * c for r, c in self.shapes)

    def settings_for(self, variant: str) -> Tuple[float, int]:
        """(divisor, restart_every) used with a given NS variant."""
        if variant == "gram":
            return self.divisor, self.restart_every
        return self.extra.get("direct_divisor", 1.0), self.extra.get("direct_restart_every", 0)

    def ns_dtype_for(self, variant: str) -> str:
        """Operand dtype of the orthogonaliser's products (LiMuon: fp32)."""
        return "f32" if variant == "limuon" else self.ns_dtype

    def limuon_settings(self) -> dict:
        """rank, oversample and power_iters of the LiMuon variant."""
        return {"rank": self.extra.get("limuon_rank", 8), "oversample": self.extra.get("limuon_oversample", 8),
                "power_iters": self.extra.get("limuon_power_iters", 1)}


def seed_for(workload_index: int, matrix_index: int, step: int) -> int:
    return 1000 * workload_index + 10 * matrix_index + step


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _orthonormal(rows: int, cols: int, gen: torch.Generator, device) -> torch.Tensor:
    """rows x cols with orthonormal columns (cols <= rows): QR of a Gaussian,
    signs fixed by the diagonal of R so the draw is Haar-distributed."""
    z = torch.randn(rows, cols, generator=gen, dtype=torch.float64, device=device)
    q, r = torch.linalg.qr(z)
    d = torch.sign(torch.diagonal(r))
    d[d == 0] = 1.0
    return q * d


def _spectral(rows: int, cols: int, lo: float, hi: float, seed: int, device) -> torch.Tensor:
    """U diag(s) V^T with Haar U, V and log10(s) ~ U(lo, hi)."""
    gen = _gen(seed, device)
    k = min(rows, cols)
    u = _orthonormal(rows, k, gen, device)
    v = _orthonormal(cols, k, gen, device)
    s = torch.pow(10.0, lo + (hi - lo) * torch.rand(k, generator=gen, dtype=torch.float64, device=device))
    return (u * s) @ v.T


def _spike(rows: int, cols: int, std: float, rank: int, seed: int, device) -> torch.Tensor:
    """Rank-``rank`` component sum_i s u_i v_i^T with orthonormal u, v and
    s = 10x the Gaussian noise's top singular value std (sqrt(r) + sqrt(c))."""
    gen = _gen(seed, device)
    rank = min(rank, rows, cols)
    u = _orthonormal(rows, rank, gen, device)
    v = _orthonormal(cols, rank, gen, device)
    s = 10.0 * std * (math.sqrt(rows) + math.sqrt(cols))
    return s * (u @ v.T)


def make_grads(w: Workload, step: int, device="cpu", shapes=None) -> List[torch.Tensor]:
    """Gradients for optimizer step ``step`` (0-based), in ``w.grad_dtype``."""
    shapes = shapes or w.shapes
    out = []
    dt = _DTYPES[w.grad_dtype]
    for i, (r, c) in enumerate(shapes):
        seed = seed_for(w.index, i, step)
        if w.grad_kind == "gaussian":
            g = w.grad_std * torch.randn(r, c, generator=_gen(seed, device), dtype=torch.float64, device=device)
        elif w.grad_kind == "spectral":
            g = _spectral(r, c, w.log10_sv[0], w.log10_sv[1], seed, device)
        elif w.grad_kind == "spike":
            g = w.grad_std * torch.randn(r, c, generator=_gen(seed, device), dtype=torch.float64, device=device)
            # spike directions belong to the matrix, not the step: seed without the step
            g = g + _spike(r, c, w.grad_std, w.spike_rank, seed_for(w.index, i, 9), device)
        elif w.grad_kind == "expert":
            g = torch.randn(r, c, generator=_gen(seed, device), dtype=torch.float64, device=device)
            e = w.expert_of[i] if w.expert_of else -1
            if e >= 0:
                # per-expert scale 10^U(-3, 0), shared by the expert's matrices, fixed over steps
                ge = _gen(seed_for(w.index + 500, e, 0), "cpu")
                g = g * float(10.0 ** (-3.0 * torch.rand(1, generator=ge, dtype=torch.float64).item()))
        else:
            raise ValueError(w.grad_kind)
        out.append(g.to(dt))
    return out


def make_sketch(kp: int, cols: int, seed: int, device="cpu") -> torch.Tensor:
    """Gaussian test matrix for the LiMuon variant: kp rows of ``cols``
    N(0, 1) values (one test vector per row), drawn in float64 and rounded
    once to float32."""
    g = torch.randn(kp, cols, generator=_gen(seed, device), dtype=torch.float64, device=device)
    return g.to(torch.float32)


def workload_sketch(w: Workload, step: int, device="cpu") -> torch.Tensor:
    """The test matrix of optimizer step ``step`` for workload ``w``: wide
    enough for its longest side, seeded per step."""
    st = w.limuon_settings()
    lmax = max(max(r, c) for r, c in w.shapes)
    return make_sketch(st["rank"] + st["oversample"], lmax, seed_for(w.index + 700, 0, step), device)


def make_state(w: Workload, device="cpu", shapes=None, mona=None):
    """Initial optimizer state: W ~ N(0, 0.02^2) fp32, M = 0 (fp32), and for
    MONA A = 0 (fp32) and a previous-gradient buffer (grad dtype, zeros), or
    for mona="lite" one bfloat16 MONA-Lite state (zeros)."""
    shapes = shapes or w.shapes
    mona = w.mona if mona is None else mona
    dt = _DTYPES[w.grad_dtype]
    state = []
    for i, (r, c) in enumerate(shapes):
        gen = _gen(seed_for(w.index + 100, i, 0), device)
        p = {
            "weight": (0.02 * torch.randn(r, c, generator=gen, dtype=torch.float64, device=device)).float(),
            "momentum": torch.zeros(r, c, dtype=torch.float32, device=device),
        }
        if mona == "lite":
            p["mona_lite"] = torch.zeros(r, c, dtype=torch.bfloat16, device=device)
        elif mona:
            p["accel"] = torch.zeros(r, c, dtype=torch.float32, device=device)
            p["prev_grad"] = torch.zeros(r, c, dtype=dt, device=device)
        state.append(p)
    return state


def _nanochat_shapes(layers=6, d=192):
    shapes = []
    for _ in range(layers):
        shapes += [(d, d)] * 4            # Q, K, V, O
        shapes += [(d, 4 * d), (4 * d, d)]  # MLP in, out
    return shapes


def _llama_shapes(layers=24, d=1024, ff=2816):
    shapes = []
    for _ in range(layers):
        shapes += [(d, d)] * 4
        shapes += [(d, ff), (d, ff), (ff, d)]   # gate, up, down
    return shapes


def _moe_shapes(experts=64, d=2048, ff=1408, attn=4):
    shapes, owner = [], []
    for e in range(experts):
        shapes += [(d, ff), (ff, d)]
        owner += [e, e]
    shapes += [(d, d)] * attn
    owner += [-1] * attn
    return shapes, owner


_moe, _moe_owner = _moe_shapes()

WORKLOADS = {
    "single_64x256_f32": Workload(
        name="single_64x256_f32", index=1, shapes=[(64, 256)], grad_dtype="f32", ns_dtype="f32",
        grad_kind="gaussian", coeffs="cubic", ns_steps=5, lr=0.02, mu=0.95, weight_decay=0.01,
        note="one fp32 64x256 matrix, N(0,1) grad, 5 cubic steps, direct"),
    "nanochat_6l_d192": Workload(
        name="nanochat_6l_d192", index=2, shapes=_nanochat_shapes(), grad_dtype="f32", ns_dtype="bf16",
        grad_kind="spectral", log10_sv=(-4.0, 0.0), coeffs="quintic", ns_steps=5,
        note="NanoChat-shaped 6-layer d=192: 24x192^2, 6x192x768, 6x768x192; fp32 grads, bf16 NS"),
    "llama430m_24l_d1024": Workload(
        name="llama430m_24l_d1024", index=3, shapes=_llama_shapes(), grad_dtype="bf16", ns_dtype="bf16",
        grad_kind="spike", grad_std=1e-2, spike_rank=8, coeffs="quintic", ns_steps=5,
        variants=("direct", "limuon"), mona=True, beta_a=0.9, alpha=0.5, steps=2,
        extra={"limuon_rank": 8, "limuon_oversample": 8, "limuon_power_iters": 1},
        note="Llama-430M-style 24 layers d=1024 ff=2816; bf16 N(0,1e-2^2) + rank-8 spike; MONA, 2 steps; "
             "direct NS (bf16) or LiMuon (rank 8, oversampling 8, one power iteration, fp32)"),
    "gram_tall_32x4096x16384": Workload(
        name="gram_tall_32x4096x16384", index=4, shapes=[(4096, 16384)] * 16 + [(16384, 4096)] * 16,
        grad_dtype="f16", ns_dtype="f16", grad_kind="spectral", log10_sv=(-5.0, 0.0),
        coeffs="quintic", ns_steps=5, variants=("gram",), divisor=1.03, restart_every=3,
        note="16x 4096x16384 + 16x 16384x4096 fp16, log-uniform singular values in [1e-5, 1]; Gram r=3 d=1.03"),
    "moe_64e_d2048": Workload(
        name="moe_64e_d2048", index=5, shapes=_moe, expert_of=_moe_owner, grad_dtype="bf16", ns_dtype="bf16",
        grad_kind="expert", coeffs="quintic", ns_steps=5, variants=("direct", "gram"),
        mona=True, beta_a=0.9, alpha=0.5, steps=2, divisor=1.03, restart_every=3,
        note="MoE block: 64 experts x (2048x1408 up + 1408x2048 down) + 4x 2048^2 attention; bf16; MONA; both variants"),
}

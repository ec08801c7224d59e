"""Seeded synthetic workloads: shapes of the layer sets and value generators.

This module holds no arithmetic of the method.  It only defines the workload
shapes and draws seeded Gaussian inputs, so that the HIP library and the CPU
oracle can be fed identical bits.

Workloads (the paper's own runs are RL post-training of Qwen-family models on
maths and reasoning data with 4,096-token contexts and one response per
microbatch -- "LoGRA: Scaling LLM Reinforcement Learning with Low-Rank
Gradient Sketches", paperpeel.com, §3.1, §3.2 and App. D.1 Table 4).  Those
datasets and weights are not used: seeded Gaussian values of the same shapes
stand in for them.  Value recipe: X ~ N(0, 1), D ~ N(0, 1e-3), W ~ N(0, 0.02),
logits z ~ N(0, 4), directional derivatives zdot ~ N(0, 1), where N(0, s)
means standard deviation s.  bf16 inputs are fp32 draws rounded to nearest.

Matrix ids: matrix_id = 7 * layer + {q:0, k:1, v:2, o:3, gate:4, up:5, down:6}.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

KINDS = ("q", "k", "v", "o", "gate", "up", "down")
TAG = {"X": 0, "D": 1, "W": 2, "z": 3, "zdot": 4, "S": 5, "v": 6, "U": 7}


def _qwen_like(hidden, q_out, kv_out, inter):
    """(d, k) of the seven projections of one decoder layer, W is [d x k] = out x in."""
    return {
        "q": (q_out, hidden), "k": (kv_out, hidden), "v": (kv_out, hidden),
        "o": (hidden, q_out), "gate": (inter, hidden), "up": (inter, hidden),
        "down": (hidden, inter),
    }


@dataclass
class Workload:
    name: str
    index: int
    layers: int
    shapes: dict            # kind -> (d, k)
    r: int
    T: int
    microbatches: int
    dtype: str              # "f32" or "bf16" for X, D, W (and z, zdot)
    optimizer: str          # "sgd" or "rowadam"
    beta: float = 0.95
    eps: float = 1e-8
    rounding: str = "nearest"
    eta: float = 1e-3
    alpha: float | None = 1.0   # None: alpha from predicted KL
    P: int = 0
    V: int = 0
    delta: float = 2e-3
    alpha_max: float = 4.0
    tau: float = 1.0
    seed: int = 1
    sr_seed: int = 2
    step: int = 0
    kinds: tuple = field(default=KINDS)

    def matrices(self, layers=None):
        """(layer, kind, matrix_id, d, k) for every selected matrix."""
        out = []
        for layer in (range(self.layers) if layers is None else layers):
            for kind in self.kinds:
                d, k = self.shapes[kind]
                out.append((layer, kind, 7 * layer + KINDS.index(kind), d, k))
        return out


WORKLOADS = [
    Workload("single-256-r8-fp32", 1, 1, {"q": (256, 256)}, r=8, T=512, microbatches=2,
             dtype="f32", optimizer="sgd", P=4, V=512, kinds=("q",)),
    Workload("single-4096-r64", 2, 1, {"q": (4096, 4096)}, r=64, T=4096, microbatches=4,
             dtype="bf16", optimizer="rowadam", beta=0.999, rounding="nearest", kinds=("q",)),
    Workload("qwen2.5-1.5b-set-r64", 3, 28, _qwen_like(1536, 1536, 256, 8960), r=64, T=4096,
             microbatches=8, dtype="bf16", optimizer="rowadam", beta=0.95, rounding="stochastic"),
    Workload("qwen2.5-7b-set-r64", 4, 28, _qwen_like(3584, 3584, 512, 18944), r=64, T=4096,
             microbatches=8, dtype="bf16", optimizer="rowadam", beta=0.95, rounding="nearest",
             alpha=None, P=64, V=152064),
    Workload("dense-27b-set-r256", 5, 64, _qwen_like(5120, 6144, 1024, 17408), r=256, T=4096,
             microbatches=16, dtype="bf16", optimizer="rowadam", beta=0.95,
             rounding="stochastic", alpha=None, P=128, V=152064),
]
BY_NAME = {w.name: w for w in WORKLOADS}


def rng(*words) -> np.random.Generator:
    return np.random.default_rng([int(w) for w in words])


def to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round fp32 draws to bf16 (nearest-even) and return the uint16 bit patterns."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def normal(shape, std, seed_words, dtype: str):
    """Seeded N(0, std) draws: fp32 array for dtype "f32", bf16 bits (uint16) for "bf16"."""
    x = (rng(*seed_words).standard_normal(shape, dtype=np.float32) * np.float32(std))
    if dtype == "f32":
        return x.astype(np.float32)
    if dtype == "bf16":
        return to_bf16_bits(x)
    raise ValueError(dtype)


def layer_input(w: Workload, layer, kind, mb, T=None, k=None):
    """X [T x k] of one microbatch for one matrix."""
    d_, k_ = w.shapes[kind]
    return normal((T or w.T, k or k_), 1.0, (w.index, layer, KINDS.index(kind), mb, TAG["X"]), w.dtype)


def output_grad(w: Workload, layer, kind, mb, T=None, d=None):
    """D [T x d] of one microbatch for one matrix."""
    d_, k_ = w.shapes[kind]
    return normal((T or w.T, d or d_), 1e-3, (w.index, layer, KINDS.index(kind), mb, TAG["D"]), w.dtype)


def weight(w: Workload, layer, kind, d=None, k=None):
    """W [d x k] of one matrix."""
    d_, k_ = w.shapes[kind]
    return normal((d or d_, k or k_), 0.02, (w.index, layer, KINDS.index(kind), 0, TAG["W"]), w.dtype)


def kl_inputs(w: Workload, P=None, V=None):
    """Logits z ~ N(0, 4) and directional derivatives zdot ~ N(0, 1), [P x V]."""
    P, V = P or w.P, V or w.V
    z = normal((P, V), 4.0, (w.index, 0, 0, 0, TAG["z"]), w.dtype)
    zd = normal((P, V), 1.0, (w.index, 0, 0, 0, TAG["zdot"]), w.dtype)
    return z, zd


def fp32_matrix(shape, std, seed_words):
    """Generic fp32 N(0, std) matrix (sketches, optimiser state, update factors)."""
    return normal(shape, std, seed_words, "f32")

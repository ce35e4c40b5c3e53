"""Seeded synthetic inputs for the MoE layout / dispatch / combine path.

This module only draws inputs: it holds none of the method's arithmetic and is
shared by the oracle-side tests and the GPU-side tests and bench, which each
receive the same bytes. All draws use numpy's PCG64 generator with a fixed
seed per workload; bf16 inputs are produced by torch's fp32 -> bf16 cast.

The five workloads (S tokens, H hidden, E experts over P virtual ranks, K
experts per token) mirror the shapes the pages discuss: DeepSeek-V3-shaped
prefill (H=7168, E=256, K=8), a decode batch spread over 128 ranks, an fp8
dynamic-quant dispatch with outliers, and a Zipf-skewed wide expert-parallel
batch. Expert ids per token are distinct: Gumbel-top-K over log p_e (uniform
p, or p_e proportional to (e+1)^-s), which is sampling without replacement.
Weights are a softmax over K of N(0,1) logits, computed in float64 and stored
as fp32.
"""

from dataclasses import dataclass
from typing import Optional

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    S: int
    H: int
    E: int
    P: int
    K: int
    seed: int
    x_std: float = 1.0
    outlier_prob: float = 0.0
    outlier_mul: float = 1.0
    zipf_s: Optional[float] = None
    quant: int = 0  # 0 = bf16 slots, 1 = fp8 e4m3 dynamic quant, 2 = int8 dynamic quant

    @property
    def C(self):
        """Channel count used by the bench and full-size tests."""
        return min(self.S, 128)

    def describe(self):
        q = {0: "bf16", 1: "fp8-e4m3-dyn", 2: "int8-dyn"}[self.quant]
        skew = f" zipf{self.zipf_s}" if self.zipf_s else ""
        return f"{self.name} S={self.S} H={self.H} E={self.E} P={self.P} K={self.K} {q}{skew}"


WORKLOADS = {
    1: Workload("tiny", 128, 1024, 16, 4, 2, 101),
    2: Workload("low_latency_decode", 128, 7168, 256, 128, 8, 102),
    3: Workload("dsv3_prefill", 4096, 7168, 256, 8, 8, 103),
    4: Workload("fp8_dynquant", 4096, 7168, 256, 8, 8, 104, x_std=2.0,
                outlier_prob=0.01, outlier_mul=50.0, quant=1),
    5: Workload("skewed_wide_ep", 8192, 7168, 256, 128, 8, 105, zipf_s=1.2),
}


def f32_to_bf16_input(a):
    """fp32 array -> bf16 bit patterns (uint16) via torch's cast (input drawing only)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def draw_routing(rng, S, E, K, zipf_s=None):
    """Distinct expert ids per token (Gumbel-top-K) and softmax weights."""
    if zipf_s is None:
        logp = np.zeros(E)
    else:
        logp = -zipf_s * np.log(np.arange(1, E + 1, dtype=np.float64))
    keys = logp[None, :] + rng.gumbel(size=(S, E))
    topk_idx = np.argsort(-keys, axis=1, kind="stable")[:, :K].astype(np.int32)
    logits = rng.standard_normal((S, K))
    ex = np.exp(logits - logits.max(axis=1, keepdims=True))
    weights = (ex / ex.sum(axis=1, keepdims=True)).astype(np.float32)
    return np.ascontiguousarray(topk_idx), np.ascontiguousarray(weights)


def make_inputs(w: Workload, with_expert_out=True):
    """Inputs of one workload: dict with x (uint16 bf16 bits [S,H]), topk_idx
    (int32 [S,K]), topk_weights (fp32 [S,K]) and, optionally, expert_out
    (uint16 bf16 bits [S*K, H], one row per slot)."""
    rng = np.random.Generator(np.random.PCG64(w.seed))
    x = rng.standard_normal((w.S, w.H), dtype=np.float32)
    if w.x_std != 1.0:
        x *= np.float32(w.x_std)
    if w.outlier_prob:
        hit = rng.random((w.S, w.H)) < w.outlier_prob
        x = np.where(hit, x * np.float32(w.outlier_mul), x).astype(np.float32)
    topk_idx, weights = draw_routing(rng, w.S, w.E, w.K, w.zipf_s)
    out = {"x": f32_to_bf16_input(x), "topk_idx": topk_idx, "topk_weights": weights}
    if with_expert_out:
        out["expert_out"] = draw_expert_out(w.seed + 1000, w.S * w.K, w.H)
    return out


def draw_expert_out(seed, rows, H, chunk=4096):
    """N(0,1) bf16 rows standing in for expert FFN outputs, drawn in chunks."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = np.empty((rows, H), dtype=np.uint16)
    for r0 in range(0, rows, chunk):
        r1 = min(rows, r0 + chunk)
        out[r0:r1] = f32_to_bf16_input(rng.standard_normal((r1 - r0, H), dtype=np.float32))
    return out


def random_tiny_routing(rng, S, K, E, p_mask=0.1, p_bad=0.0, distinct=False):
    """Small adversarial routing tables: duplicates, -1 masks, optional bad ids."""
    if distinct and K <= E:
        idx = np.stack([rng.permutation(E)[:K] for _ in range(S)]).astype(np.int32)
    else:
        idx = rng.integers(0, E, size=(S, K)).astype(np.int32)
    idx[rng.random((S, K)) < p_mask] = -1
    if p_bad:
        bad = rng.random((S, K)) < p_bad
        idx[bad] = rng.choice(np.array([-7, -2, E, E + 5], dtype=np.int32), size=int(bad.sum()))
    return np.ascontiguousarray(idx)

"""Seeded synthetic inputs for MoE dispatch / combine.

This module only *generates inputs*: router outputs (top-k expert ids and
weights), token activations, and stand-in expert outputs.  It holds none of
the dispatch/combine arithmetic, so both the HIP path and the CPU oracle can
consume the same arrays.

The shapes follow the workloads the pages describe: DeepSeek-V3 dimensions
(hidden 7168, 256 routed experts, top-8, 8 expert groups with top-4 group
selection) and Qwen3-MoE-like decode dimensions (hidden 2048, 128 experts,
top-8); token counts stand in for the decode batch cap and prefill chunks
(page "moe: add DeepEP V2 ElasticBuffer support to MoE token dispatcher",
num_max_tokens_per_rank sizing commit; page "[Feature] Add DeepEPv2
(ElasticBuffer) MoE A2A backend", Capacity and fail-fast behavior).  The
router itself is not on the pages: the group-limited router follows the
DeepSeek-V3 convention and the skewed router samples experts without
replacement from a Zipf popularity by Gumbel-top-k.

All randomness comes from numpy's PCG64 with a fixed seed and a fixed draw
order: routing, activations, outlier rows, weights, expert outputs.
Activations are drawn in fp32 and rounded to bf16 (round to nearest even) by
torch's CPU cast; bf16 values are carried as uint16 bit patterns.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

LAYOUT_CONTIGUOUS = 0
LAYOUT_MASKED = 1
QUANT_NONE = 0
QUANT_FP8_F32 = 1
QUANT_FP8_UE8M0 = 2
QUANT_MXFP8 = 3


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic dispatch/combine problem."""

    name: str
    T: int            # tokens on this rank
    H: int            # hidden size
    E: int            # routed experts
    K: int            # top-k
    R: int            # virtual destination ranks (E % R == 0)
    layout: int       # LAYOUT_CONTIGUOUS or LAYOUT_MASKED
    align: int = 1    # contiguous: expert segments padded to this many rows
    capacity: int = 1 # masked: rows per expert
    quant: int = QUANT_NONE
    routing: str = "softmax"  # softmax | group | zipf
    seed: int = 0
    outlier_frac: float = 0.0
    outlier_scale: float = 50.0
    n_groups: int = 8
    topk_groups: int = 4
    zipf_s: float = 1.2
    expert_output: str = "random"  # random | scaled  (see expert_outputs)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def rows_capacity(self) -> int:
        """Rows the dispatched buffer must hold for T = self.T tokens."""
        if self.layout == LAYOUT_CONTIGUOUS:
            return self.T * self.K + self.E * (self.align - 1)
        return self.E * self.capacity


# The workloads, named by what they are; the field starting with T is the
# token count.
WORKLOADS = {
    "tiny_T64": Workload(
        "tiny_T64", T=64, H=256, E=8, K=2, R=2, layout=LAYOUT_CONTIGUOUS,
        align=1, quant=QUANT_NONE, routing="softmax", seed=1,
        expert_output="scaled"),
    "qwen3moe_decode_T128": Workload(
        "qwen3moe_decode_T128", T=128, H=2048, E=128, K=8, R=8,
        layout=LAYOUT_MASKED, capacity=128, quant=QUANT_FP8_F32,
        routing="softmax", seed=2),
    "deepseekv3_decode_T256": Workload(
        "deepseekv3_decode_T256", T=256, H=7168, E=256, K=8, R=8,
        layout=LAYOUT_MASKED, capacity=256, quant=QUANT_FP8_F32,
        routing="group", seed=3, outlier_frac=0.01),
    "deepseekv3_prefill_T8192": Workload(
        "deepseekv3_prefill_T8192", T=8192, H=7168, E=256, K=8, R=8,
        layout=LAYOUT_CONTIGUOUS, align=128, quant=QUANT_FP8_UE8M0,
        routing="group", seed=4, outlier_frac=0.01),
    # The DeepSeek-V3 prefill batch (same seed, same inputs) dispatched as 1x32 MXFP8.
    "deepseekv3_prefill_T8192_mxfp8": Workload(
        "deepseekv3_prefill_T8192_mxfp8", T=8192, H=7168, E=256, K=8, R=8,
        layout=LAYOUT_CONTIGUOUS, align=128, quant=QUANT_MXFP8,
        routing="group", seed=4, outlier_frac=0.01),
    # Skewed prefill: four variants of one input set (same seed).
    "skewed_prefill_T16384_contig_bf16": Workload(
        "skewed_prefill_T16384_contig_bf16", T=16384, H=7168, E=256, K=8,
        R=8, layout=LAYOUT_CONTIGUOUS, align=128, quant=QUANT_NONE,
        routing="zipf", seed=5),
    "skewed_prefill_T16384_contig_fp8": Workload(
        "skewed_prefill_T16384_contig_fp8", T=16384, H=7168, E=256, K=8,
        R=8, layout=LAYOUT_CONTIGUOUS, align=128, quant=QUANT_FP8_F32,
        routing="zipf", seed=5),
    "skewed_prefill_T16384_masked_bf16": Workload(
        "skewed_prefill_T16384_masked_bf16", T=16384, H=7168, E=256, K=8,
        R=8, layout=LAYOUT_MASKED, capacity=1024, quant=QUANT_NONE,
        routing="zipf", seed=5),
    "skewed_prefill_T16384_masked_fp8": Workload(
        "skewed_prefill_T16384_masked_fp8", T=16384, H=7168, E=256, K=8,
        R=8, layout=LAYOUT_MASKED, capacity=1024, quant=QUANT_FP8_F32,
        routing="zipf", seed=5),
}

HEADLINE = "deepseekv3_prefill_T8192"


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 array -> bf16 bit patterns (uint16), round to nearest even."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 values (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _topk_desc(score: np.ndarray, K: int) -> np.ndarray:
    """Indices of the K largest entries per row; ties go to the lower index."""
    order = np.argsort(-score, axis=1, kind="stable")
    return order[:, :K]


def route_softmax(rng: np.random.Generator, T: int, E: int, K: int):
    """Logits ~ N(0,1) -> softmax -> top-k -> weights renormalised to sum 1."""
    logits = rng.standard_normal((T, E), dtype=np.float32)
    z = logits - logits.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    idx = _topk_desc(p, K)
    w = np.take_along_axis(p, idx, axis=1)
    w = (w / w.sum(axis=1, keepdims=True)).astype(np.float32)
    return idx.astype(np.int32), w


def route_group_limited(rng: np.random.Generator, T: int, E: int, K: int,
                        n_groups: int, topk_groups: int):
    """DeepSeek-V3-style router: sigmoid scores, groups of E/n_groups
    consecutive experts scored by the sum of their two best scores, the best
    `topk_groups` groups kept, top-k experts inside them, weights = selected
    scores normalised to sum 1 (no bias, scaling factor 1)."""
    logits = rng.standard_normal((T, E), dtype=np.float32)
    s = (1.0 / (1.0 + np.exp(-logits.astype(np.float64)))).astype(np.float32)
    g = s.reshape(T, n_groups, E // n_groups)
    top2 = -np.sort(-g, axis=2)[:, :, :2].sum(axis=2)
    keep = _topk_desc(top2, topk_groups)
    mask = np.zeros((T, n_groups), dtype=bool)
    np.put_along_axis(mask, keep, True, axis=1)
    masked = np.where(np.repeat(mask, E // n_groups, axis=1), s, -1.0)
    idx = _topk_desc(masked, K)
    w = np.take_along_axis(s, idx, axis=1)
    w = (w / w.sum(axis=1, keepdims=True)).astype(np.float32)
    return idx.astype(np.int32), w


def route_zipf(rng: np.random.Generator, T: int, E: int, K: int, s: float):
    """Skewed routing: a seeded permutation pi of the experts, popularity
    p_e proportional to (pi(e)+1)^-s, and K distinct experts per token drawn
    without replacement proportionally to p by Gumbel-top-k (keys
    log p_e + Gumbel noise).  Weights ~ U(0,1), renormalised per token."""
    pi = rng.permutation(E)
    logp = -s * np.log(pi.astype(np.float64) + 1.0)
    gumbel = rng.gumbel(size=(T, E))
    idx = _topk_desc(logp[None, :] + gumbel, K)
    w = rng.random((T, K), dtype=np.float32)
    w = (w / w.sum(axis=1, keepdims=True)).astype(np.float32)
    return idx.astype(np.int32), w


@dataclasses.dataclass
class Inputs:
    topk_idx: np.ndarray   # int32 [T, K]
    topk_w: np.ndarray     # float32 [T, K]
    x: np.ndarray          # uint16 (bf16 bits) [T, H]
    rng: np.random.Generator  # continues the draw sequence (expert outputs)


def make_inputs(wl: Workload) -> Inputs:
    """Routing, activations and outlier rows for a workload, in draw order."""
    rng = np.random.Generator(np.random.PCG64(wl.seed))
    if wl.routing == "softmax":
        idx, w = route_softmax(rng, wl.T, wl.E, wl.K)
    elif wl.routing == "group":
        idx, w = route_group_limited(rng, wl.T, wl.E, wl.K, wl.n_groups, wl.topk_groups)
    elif wl.routing == "zipf":
        idx, w = route_zipf(rng, wl.T, wl.E, wl.K, wl.zipf_s)
    else:
        raise ValueError(f"unknown routing {wl.routing!r}")
    x = rng.standard_normal((wl.T, wl.H), dtype=np.float32)
    n_out = int(round(wl.outlier_frac * wl.T))
    if n_out > 0:
        rows = rng.choice(wl.T, size=n_out, replace=False)
        x[rows] *= np.float32(wl.outlier_scale)
    return Inputs(topk_idx=np.ascontiguousarray(idx), topk_w=np.ascontiguousarray(w),
                  x=f32_to_bf16_bits(x), rng=rng)


def expert_outputs(wl: Workload, inp: Inputs, row_to_pair: Optional[np.ndarray] = None,
                   rows: Optional[int] = None) -> np.ndarray:
    """Stand-in expert outputs y, bf16 bits [rows, H], in the dispatched layout.

    "random": every row is a window of H consecutive values of a seeded
    N(0,1) bf16 pool (2^22 values) at a seeded random offset, so rows differ
    and generation stays fast at full size (layout independent; rows
    defaults to the workload's rows_capacity).
    "scaled": row r holding pair p = row_to_pair[r] of token t = p // K routed
    to expert e gets bf16((e + 1) * 0.5 * x[t]); rows holding no pair are 0.
    This needs the layout's row_to_pair map.
    """
    n = wl.rows_capacity if rows is None else rows
    if wl.expert_output == "random":
        pool_n = 1 << 22
        pool = f32_to_bf16_bits(inp.rng.standard_normal(pool_n + wl.H, dtype=np.float32))
        offs = inp.rng.integers(0, pool_n, n)
        y = np.empty((n, wl.H), np.uint16)
        for r in range(n):
            y[r] = pool[offs[r]:offs[r] + wl.H]
        return y
    if wl.expert_output == "scaled":
        if row_to_pair is None:
            raise ValueError("scaled expert outputs need row_to_pair")
        y = np.zeros((n, wl.H), dtype=np.float32)
        kept = np.nonzero(row_to_pair[:n] >= 0)[0]
        p = row_to_pair[kept].astype(np.int64)
        t = p // wl.K
        e = inp.topk_idx.reshape(-1)[p].astype(np.float32)
        y[kept] = ((e + 1.0) * 0.5)[:, None] * bf16_bits_to_f32(inp.x[t])
        return f32_to_bf16_bits(y)
    raise ValueError(f"unknown expert_output {wl.expert_output!r}")

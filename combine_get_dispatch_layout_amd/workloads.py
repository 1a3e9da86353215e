"""Seeded synthetic inputs for the MoE dispatch / combine path.

This module only draws inputs: token activations ``x``, routing ``topk_idx`` and
gate weights ``topk_weights``.  It holds none of the dispatch, layout or combine
arithmetic, so both the CPU oracle (in the tests) and the HIP path can consume
the same arrays without sharing any of the method's code.

Every draw comes from ``torch.Generator('cpu').manual_seed(seed)`` in a fixed
order: ``x`` first, then the routing scores, then the weight logits.  Routing
selections use a stable descending sort, so ties go to the lower expert index.

The routing shapes follow the workloads the pages describe:
* uniform distinct top-k (plain MoE gating),
* group-limited top-k (the DeepSeek-V3 gating the GCU-port README names: pick
  the best expert groups first, then the top-k experts inside them),
* Zipf-skewed expert choice (a hot-expert stress case),
* per-expert fixed-capacity decode batches (the low-latency kernels, whose
  README recommends fewer than 256 tokens per rank).
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic configuration.

    ``channels`` is the number of contiguous token ranges the layout reports
    per bucket; ``ll_capacity`` is ``num_max_dispatch_tokens_per_rank`` for the
    low-latency layout (0 when the workload is a normal dispatch).
    """

    name: str
    tokens: int
    hidden: int
    experts: int
    topk: int
    ranks: int
    channels: int
    routing: str  # "uniform" | "group_limited" | "zipf"
    seed: int
    quant: str = "none"  # "none" | "fp8_e4m3_1x128"
    ll_capacity: int = 0
    reuse_seeds: tuple = ()


# The five workloads the path is checked and measured on.
TINY = Workload("tiny_128x256_e16_top2_r4", 128, 256, 16, 2, 4, 2, "uniform", 1)
LL_DECODE = Workload("ll_decode_128x7168_e256_top8_r8_cap128", 128, 7168, 256, 8, 8, 0,
                     "uniform", 2, ll_capacity=128)
PREFILL = Workload("prefill_4096x7168_e256_top8_grouped_r8_c24", 4096, 7168, 256, 8, 8, 24,
                   "group_limited", 3)
FP8_SKEWED = Workload("fp8_zipf_8192x7168_e256_top8_r8_c24", 8192, 7168, 256, 8, 8, 24,
                      "zipf", 4, quant="fp8_e4m3_1x128")
HANDLE_REUSE = Workload("reuse_16384x4096_e64_top6_r16_c32", 16384, 4096, 64, 6, 16, 32,
                        "uniform", 5, reuse_seeds=tuple(range(501, 511)))

ALL = (TINY, LL_DECODE, PREFILL, FP8_SKEWED, HANDLE_REUSE)
BY_NAME = {w.name: w for w in ALL}


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator("cpu")
    g.manual_seed(int(seed))
    return g


def draw_x(g: torch.Generator, tokens: int, hidden: int) -> torch.Tensor:
    """x ~ N(0,1) drawn in fp32, then rounded to bf16 (round-to-nearest-even)."""
    return torch.randn(tokens, hidden, generator=g, dtype=torch.float32).to(torch.bfloat16)


def _stable_desc(scores: torch.Tensor) -> torch.Tensor:
    # Stable descending sort: equal scores keep ascending index order.
    return torch.sort(scores, dim=-1, descending=True, stable=True).indices


def route_uniform(g: torch.Generator, tokens: int, experts: int, topk: int) -> tuple:
    """Top-k of N(0,1) scores per token: k distinct experts, uniform over experts."""
    scores = torch.randn(tokens, experts, generator=g, dtype=torch.float32)
    idx = _stable_desc(scores)[:, :topk].contiguous()
    return idx.to(torch.int64), torch.gather(scores, 1, idx)


def route_group_limited(g: torch.Generator, tokens: int, experts: int, topk: int,
                        groups: int = 8, groups_kept: int = 4) -> tuple:
    """Group-limited gating.

    Scores ~ N(0,1) [tokens, experts]; experts form ``groups`` contiguous groups.
    A group's score is the sum of its two best expert scores; the ``groups_kept``
    best groups are kept, and the token's top-k experts are the best-scoring
    experts inside the kept groups, in descending score order.
    """
    assert experts % groups == 0
    scores = torch.randn(tokens, experts, generator=g, dtype=torch.float32)
    per = experts // groups
    grouped = scores.view(tokens, groups, per).to(torch.float64)
    top2 = torch.sort(grouped, dim=-1, descending=True, stable=True).values[..., :2]
    group_score = top2.sum(-1)
    kept = _stable_desc(group_score)[:, :groups_kept]
    keep = torch.zeros(tokens, groups, dtype=torch.bool)
    keep.scatter_(1, kept, True)
    masked = scores.clone()
    masked.view(tokens, groups, per)[~keep] = float("-inf")
    idx = _stable_desc(masked)[:, :topk].contiguous()
    return idx.to(torch.int64), torch.gather(scores, 1, idx)


def route_zipf(g: torch.Generator, tokens: int, experts: int, topk: int, s: float = 1.2) -> tuple:
    """Zipf(s) expert choice without replacement (Gumbel-top-k).

    Expert e has weight (e+1)^-s (no permutation, so expert 0 is the hottest);
    the token's experts are the top-k of log(weight) + Gumbel noise.
    """
    logw = -s * torch.log(torch.arange(1, experts + 1, dtype=torch.float64))
    u = torch.rand(tokens, experts, generator=g, dtype=torch.float64)
    u = u.clamp(min=1e-300, max=1.0 - 1e-16)
    keys = logw[None, :] - torch.log(-torch.log(u))
    idx = _stable_desc(keys)[:, :topk].contiguous()
    return idx.to(torch.int64), torch.gather(keys, 1, idx)


def softmax_weights(logits: torch.Tensor) -> torch.Tensor:
    """Softmax along the last axis computed in float64, stored as fp32."""
    return torch.softmax(logits.to(torch.float64), dim=-1).to(torch.float32)


@dataclasses.dataclass
class Inputs:
    x: torch.Tensor            # [T, H] bf16 (CPU)
    topk_idx: torch.Tensor     # [T, K] int64 (CPU)
    topk_weights: torch.Tensor  # [T, K] fp32 (CPU)


def make_inputs(w: Workload, seed: Optional[int] = None, tokens: Optional[int] = None) -> Inputs:
    """Draw (x, topk_idx, topk_weights) for a workload.

    ``tokens`` overrides the token count (for reduced-size parity cases with the
    same routing structure).
    """
    seed = w.seed if seed is None else seed
    T = w.tokens if tokens is None else tokens
    g = _gen(seed)
    x = draw_x(g, T, w.hidden)
    if w.routing == "uniform":
        idx, _ = route_uniform(g, T, w.experts, w.topk)
    elif w.routing == "group_limited":
        idx, sel = route_group_limited(g, T, w.experts, w.topk)
    elif w.routing == "zipf":
        idx, _ = route_zipf(g, T, w.experts, w.topk)
    else:
        raise ValueError(w.routing)
    if w.routing == "group_limited":
        # Gate weights are the softmax over the selected experts' scores.
        weights = softmax_weights(sel)
    else:
        weights = softmax_weights(torch.randn(T, w.topk, generator=g, dtype=torch.float32))
    return Inputs(x, idx, weights)


def fresh_x(w: Workload, seed: int, tokens: Optional[int] = None) -> torch.Tensor:
    """A new activation batch for the same routing (handle reuse)."""
    T = w.tokens if tokens is None else tokens
    return draw_x(_gen(seed), T, w.hidden)


def random_routing(rng: np.random.Generator, tokens: int, experts: int, topk: int,
                   p_empty: float = 0.0) -> np.ndarray:
    """Distinct experts per token with some slots set to -1 (empty).

    Used for small edge-case and property tests.
    """
    out = np.empty((tokens, topk), dtype=np.int64)
    for t in range(tokens):
        out[t] = rng.permutation(experts)[:topk]
    if p_empty > 0:
        out[rng.random((tokens, topk)) < p_empty] = -1
    return out

"""Seeded synthetic inputs for the blockwise FP8 GEMM workloads.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no activation quantization, no GEMM). Both the HIP path
and the CPU oracle receive the same bytes from here. Weights arrive already in
e4m3 (as a checkpoint would), cast by torch's CPU ``float8_e4m3fn`` conversion
after clamping, which is the weight recipe of the vLLM test on page
"prhub.com.cn ... vllm/pull/49932" (section "关键源码片段").

Workloads (all sizes N x K are weight shapes, A is [M, K]):
  * page2_case: M=83, N=576, K=7168; torch.manual_seed(0); A, B ~ U(-448, 448)
    fp32; B clamped and cast to e4m3; Bs ~ U(0, 1e-2) of shape [5, 56]. The
    same RNG call sequence as the page's test.
  * square sweep: N = K = 4096, one fixed weight (seed 1), A ~ U(-448, 448)
    fp32 with seed 100 + M.
  * dense-transformer linears at hidden 5120: QKV (K=5120, N=10240),
    o_proj (K=8192, N=5120), gate+up (K=5120, N=51200), down (K=25600,
    N=5120); weights like the sweep's, activations bf16 N(0, 1) with seed 300 + M.
  * UE8M0 weights (power-of-two block scales, the page "transformers/integrations/
    deepgemm.py" checkpoints with float8_e8m0fnu scale factors): the e4m3 codes of
    ``weight``, with scale codes drawn uniformly from [113, 121], i.e. scales 2**-14 ..
    2**-6, the binades that U(0, 1e-2) mostly covers.
  * MoE routing for the expert chain: per token, top_k distinct experts drawn with
    Dirichlet(1) expert probabilities (numpy), router weights U(0, 1) normalized per token;
    expert weights: gate+up [E, 2I, H] and down [E, H, I] like ``weight``.
  * M-grouped contiguous MoE: 16 experts with weights [4096, 7168]; token counts
    ~ Multinomial(4096, Dirichlet(1)) (seed 4); each expert's rows padded up to a
    multiple of 128; a per-row int32 expert id, -1 on padding rows; bf16 N(0, 1)
    activations on real rows and zeros on padding rows.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

FP8_MAX = 448.0
BLOCK = 128

SQUARE_N = SQUARE_K = 4096
SQUARE_SMALL_M = (1, 8, 9, 16, 24, 32, 64, 128, 160, 192, 224, 256)
SQUARE_LARGE_M = (512, 1024, 2048, 4096, 8192)
TRANSFORMER_LAYERS = {
    "qkv": (10240, 5120),  # (N, K)
    "o_proj": (5120, 8192),
    "gate_up": (51200, 5120),
    "down": (5120, 25600),
}
TRANSFORMER_M = (1, 16, 128, 2048)
MOE_GROUPS, MOE_N, MOE_K, MOE_TOKENS, MOE_ALIGN = 16, 4096, 7168, 4096, 128


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


def _fp8_codes_from_uniform(u: torch.Tensor) -> torch.Tensor:
    """U(0,1) fp32 -> U(-448, 448) -> clamp -> e4m3fn codes (uint8), via torch's CPU cast."""
    w = (u - 0.5) * 2 * FP8_MAX
    return w.clamp(min=-FP8_MAX, max=FP8_MAX).to(torch.float8_e4m3fn).view(torch.uint8)


@dataclass
class Weight:
    """e4m3 weight codes [N, K] (uint8) and float32 block scales [ceil(N/128), ceil(K/128)]."""

    q: torch.Tensor
    s: torch.Tensor


def weight(n: int, k: int, seed: int) -> Weight:
    g = torch.Generator().manual_seed(seed)
    q = _fp8_codes_from_uniform(torch.rand(n, k, generator=g, dtype=torch.float32))
    s = torch.rand(_cdiv(n, BLOCK), _cdiv(k, BLOCK), generator=g, dtype=torch.float32) * 1e-2
    return Weight(q.contiguous(), s.contiguous())


def weight_ue8m0(n: int, k: int, seed: int) -> Weight:
    """e4m3 weight codes [N, K] and UE8M0 scale codes [ceil(N/128), ceil(K/128)] (uint8)."""
    g = torch.Generator().manual_seed(seed)
    q = _fp8_codes_from_uniform(torch.rand(n, k, generator=g, dtype=torch.float32))
    e = torch.randint(113, 122, (_cdiv(n, BLOCK), _cdiv(k, BLOCK)), generator=g, dtype=torch.int32).to(torch.uint8)
    return Weight(q.contiguous(), e.contiguous())


def weight_1x64(n: int, k: int, seed: int) -> Weight:
    """The weight of weight(n, k, seed) (same codes) with 128x64 block scales U(0, 1e-2)
    [ceil(n/128), ceil(k/64)], for the 1x64 / 128x64 layout."""
    w = weight(n, k, seed)
    g = torch.Generator().manual_seed(seed + 1_000_003)
    s = torch.rand(_cdiv(n, BLOCK), _cdiv(k, 64), generator=g, dtype=torch.float32) * 1e-2
    return Weight(w.q, s.contiguous())


def act_uniform(m: int, k: int, seed: int) -> torch.Tensor:
    """fp32 activations ~ U(-448, 448)."""
    g = torch.Generator().manual_seed(seed)
    return (torch.rand(m, k, generator=g, dtype=torch.float32) - 0.5) * 2 * FP8_MAX


def act_normal_bf16(m: int, k: int, seed: int) -> torch.Tensor:
    """bf16 activations ~ N(0, 1)."""
    g = torch.Generator().manual_seed(seed)
    return torch.randn(m, k, generator=g, dtype=torch.float32).to(torch.bfloat16)


def page2_case():
    """(A fp32 [83, 7168], Weight [576, 7168]) drawn exactly like the page's test."""
    m, n, k = 83, 576, 7168
    torch.manual_seed(0)
    a = (torch.rand(m, k, dtype=torch.float32) - 0.5) * 2 * FP8_MAX
    b = (torch.rand(n, k, dtype=torch.float32) - 0.5) * 2 * FP8_MAX
    bq = b.clamp(min=-FP8_MAX, max=FP8_MAX).to(torch.float8_e4m3fn).view(torch.uint8)
    bs = torch.rand(_cdiv(n, BLOCK), _cdiv(k, BLOCK), dtype=torch.float32) * 1e-2
    return a, Weight(bq.contiguous(), bs.contiguous())


def square_weight() -> Weight:
    return weight(SQUARE_N, SQUARE_K, seed=1)


def square_act(m: int) -> torch.Tensor:
    return act_uniform(m, SQUARE_K, seed=100 + m)


def transformer_weight(layer: str) -> Weight:
    n, k = TRANSFORMER_LAYERS[layer]
    return weight(n, k, seed=200 + list(TRANSFORMER_LAYERS).index(layer))


def transformer_act(layer: str, m: int) -> torch.Tensor:
    _, k = TRANSFORMER_LAYERS[layer]
    return act_normal_bf16(m, k, seed=300 + m)


@dataclass
class MoeCase:
    counts: np.ndarray  # tokens per expert [G]
    layout: torch.Tensor  # int32 [M_pad]: expert id per row, -1 on padding
    act: torch.Tensor  # bf16 [M_pad, K]; zeros on padding rows
    weights: list  # G x Weight([N, K])


def moe_counts(groups: int = MOE_GROUPS, tokens: int = MOE_TOKENS, seed: int = 4) -> np.ndarray:
    rng = np.random.default_rng(seed)
    p = rng.dirichlet(np.ones(groups))
    return rng.multinomial(tokens, p)


def moe_layout(counts, align: int = MOE_ALIGN) -> np.ndarray:
    """Per-row expert id for the contiguous layout: each expert's rows, then -1 up to a multiple of `align`."""
    parts = []
    for g, c in enumerate(counts):
        padded = _cdiv(int(c), align) * align
        parts.append(np.full(int(c), g, dtype=np.int32))
        parts.append(np.full(padded - int(c), -1, dtype=np.int32))
    return np.concatenate(parts) if parts else np.zeros(0, np.int32)


def moe_case(groups: int = MOE_GROUPS, n: int = MOE_N, k: int = MOE_K, tokens: int = MOE_TOKENS,
             seed: int = 4, with_weights: bool = True) -> MoeCase:
    counts = moe_counts(groups, tokens, seed)
    layout = moe_layout(counts)
    act = act_normal_bf16(layout.size, k, seed=seed + 1000)
    act[torch.from_numpy(layout < 0)] = 0
    weights = [weight(n, k, seed=seed * 100 + g) for g in range(groups)] if with_weights else []
    return MoeCase(counts, torch.from_numpy(layout), act, weights)


def moe_routing(tokens: int, top_k: int, experts: int, seed: int, sentinel_frac: float = 0.0):
    """(topk_ids [T, top_k] int32, topk_weights [T, top_k] float32); with sentinel_frac > 0, that
    share of the pairs is replaced by the id `experts` (an expert-parallel sentinel)."""
    rng = np.random.default_rng(seed)
    p = rng.dirichlet(np.ones(experts))
    ids = np.stack([rng.choice(experts, top_k, replace=False, p=p) for _ in range(tokens)]).astype(np.int32)
    if sentinel_frac > 0:
        ids[rng.random(ids.shape) < sentinel_frac] = experts
    w = rng.uniform(0.0, 1.0, (tokens, top_k))
    w = (w / w.sum(axis=1, keepdims=True)).astype(np.float32)
    return torch.from_numpy(ids), torch.from_numpy(w)


def moe_experts(experts: int, hidden: int, inter: int, seed: int):
    """(w_up [E, 2I, H], s_up, w_down [E, H, I], s_down): e4m3 codes and float32 128x128 scales."""
    up = [weight(2 * inter, hidden, seed=seed + 2 * g) for g in range(experts)]
    down = [weight(hidden, inter, seed=seed + 2 * g + 1) for g in range(experts)]
    return (torch.stack([w.q for w in up]), torch.stack([w.s for w in up]),
            torch.stack([w.q for w in down]), torch.stack([w.s for w in down]))

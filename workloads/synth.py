"""Seeded synthetic weights, activations and MoE routing for the five linear-layer workloads.

Recipe (the pages ship no weights or datasets, so these stand in for them):

* weights: bf16 draws of N(0, 0.02); for the dense Qwen3-8B / Llama-3.1-8B shapes a fraction
  0.1 % of the entries (``round(0.001 * numel)`` distinct flat indices) is multiplied by 10;
* activations: bf16 draws of N(0, 1); ``max(1, round(0.01 * K))`` distinct channels (columns) are
  multiplied by 20 for every token, which is the channel-wise outlier pattern of LLM activations;
* MoE routing: ``E`` experts ranked by a seeded permutation, expert of rank r gets logit
  ``-s * ln(r)`` (Zipf exponent s = 1.1); each token picks ``top_k`` distinct experts by
  Gumbel-top-k sampling (i.e. sampling without replacement with probability proportional to
  r^-s). The per-expert counts are the histogram of those picks.

Every draw comes from a ``torch.Generator`` seeded with ``seed`` on the device the tensor is made
on; values are drawn in float32 and rounded to bf16 (round to nearest even) by torch's cast.
The same (seed, shape, device) always returns the same tensor. Tensors are returned as torch
tensors of dtype bfloat16 (callers that want the raw bits use ``.view(torch.int16)``).
"""

from __future__ import annotations

import math

import torch

# ---------------------------------------------------------------------------------------------
# Layer shapes, as (name, N_out, K_in) with y = x @ W^T and W stored [N][K].
# ---------------------------------------------------------------------------------------------

#: One Qwen3-8B decoder block: hidden 4096, 32 q heads and 8 kv heads of width 128, MLP 12288.
DENSE_LINEARS_QWEN3_8B = (
    ("q_proj", 4096, 4096),
    ("k_proj", 1024, 4096),
    ("v_proj", 1024, 4096),
    ("o_proj", 4096, 4096),
    ("gate_proj", 12288, 4096),
    ("up_proj", 12288, 4096),
    ("down_proj", 4096, 12288),
)

#: One Llama-3.1-8B decoder block: hidden 4096, 8 kv heads of width 128, MLP 14336.
LLAMA31_8B_LAYER_LINEARS = (
    ("q_proj", 4096, 4096),
    ("k_proj", 1024, 4096),
    ("v_proj", 1024, 4096),
    ("o_proj", 4096, 4096),
    ("gate_proj", 14336, 4096),
    ("up_proj", 14336, 4096),
    ("down_proj", 4096, 14336),
)

CONFIGS = {
    1: dict(
        name="tiny W8A8 linear 256x256, M=4",
        linears=(("w", 256, 256),),
        M=(4,),
        weight_outliers=0.0,
    ),
    2: dict(
        name="Qwen3-8B decoder block linears, decode M=64",
        linears=DENSE_LINEARS_QWEN3_8B,
        M=(64,),
        weight_outliers=0.001,
    ),
    3: dict(
        name="Qwen3-8B decoder block linears, prefill M=8192",
        linears=DENSE_LINEARS_QWEN3_8B,
        M=(8192,),
        weight_outliers=0.001,
    ),
    4: dict(
        name="Llama-3.1-8B MLP at M in {256, 4096}; weight sync of 32 layers",
        linears=LLAMA31_8B_LAYER_LINEARS,
        mlp=LLAMA31_8B_LAYER_LINEARS[4:],
        M=(256, 4096),
        layers=32,
        weight_outliers=0.001,
    ),
    5: dict(
        name="Qwen3-30B-A3B MoE layer: T=4096, hidden 2048, 128 experts, top-8",
        tokens=4096,
        hidden=2048,
        moe_inter=768,
        experts=128,
        top_k=8,
        zipf_s=1.1,
        weight_outliers=0.0,
    ),
}


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def weight_bf16(N: int, K: int, seed: int, *, std: float = 0.02, outlier_frac: float = 0.0,
                outlier_mult: float = 10.0, device="cpu", batch: int | None = None) -> torch.Tensor:
    """bf16 weight ``[N][K]`` (or ``[batch][N][K]``) drawn from N(0, std) with sparse x10 outliers."""
    shape = (N, K) if batch is None else (batch, N, K)
    g = _gen(seed, device)
    w = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    w.mul_(std)
    n_out = int(round(outlier_frac * w.numel()))
    if n_out > 0:
        idx = torch.randperm(w.numel(), generator=g, device=device)[:n_out]
        flat = w.view(-1)
        flat[idx] = flat[idx] * outlier_mult
    return w.to(torch.bfloat16)


def act_bf16(M: int, K: int, seed: int, *, outlier_frac: float = 0.01, outlier_mult: float = 20.0,
             device="cpu") -> torch.Tensor:
    """bf16 activation ``[M][K]`` drawn from N(0, 1) with ~1 % of channels scaled x20."""
    g = _gen(seed, device)
    x = torch.randn((M, K), generator=g, device=device, dtype=torch.float32)
    n_ch = max(1, int(round(outlier_frac * K))) if outlier_frac > 0 else 0
    if n_ch > 0:
        cols = torch.randperm(K, generator=g, device=device)[:n_ch]
        x[:, cols] *= outlier_mult
    return x.to(torch.bfloat16)


def _moe_picks(tokens: int, experts: int, top_k: int, seed: int, zipf_s: float) -> torch.Tensor:
    """The experts each token picks, [tokens][top_k] int64 (CPU)."""
    g = _gen(seed, "cpu")
    perm = torch.randperm(experts, generator=g)  # expert id of rank 1, 2, ...
    rank = torch.empty(experts, dtype=torch.float64)
    rank[perm] = torch.arange(1, experts + 1, dtype=torch.float64)
    logits = -zipf_s * torch.log(rank)  # [E]
    u = torch.rand((tokens, experts), generator=g, dtype=torch.float64)
    u = u.clamp_min(1e-300)
    gumbel = -torch.log(-torch.log(u))
    return torch.topk(logits[None, :] + gumbel, top_k, dim=1).indices  # [T][top_k]


def moe_routing_counts(tokens: int, experts: int, top_k: int, seed: int, *,
                       zipf_s: float = 1.1) -> torch.Tensor:
    """Per-expert row counts (int64, length ``experts``) of a Zipf-skewed top-k router.

    Computed on the CPU; the counts sum to ``tokens * top_k``.
    """
    picks = _moe_picks(tokens, experts, top_k, seed, zipf_s)
    return torch.bincount(picks.reshape(-1), minlength=experts)


def moe_routing(tokens: int, experts: int, top_k: int, seed: int, *,
                zipf_s: float = 1.1) -> tuple[torch.Tensor, torch.Tensor]:
    """The same router as ``moe_routing_counts`` (same seed, same picks) with the token of every
    grouped row: returns ``(counts, row_ids)``, ``row_ids`` int32 of length ``tokens * top_k``
    listing, expert by expert, the tokens that picked that expert in increasing order (so grouped
    row r of an expert-sorted layout holds token ``row_ids[r]``). CPU tensors."""
    picks = _moe_picks(tokens, experts, top_k, seed, zipf_s)
    flat = picks.reshape(-1)
    token = torch.arange(tokens, dtype=torch.int64).repeat_interleave(top_k)
    order = torch.argsort(flat * tokens + token)  # distinct keys: a token picks distinct experts
    counts = torch.bincount(flat, minlength=experts)
    return counts, token[order].to(torch.int32)


def offsets_from_counts(counts) -> torch.Tensor:
    """Exclusive prefix sum of ``counts`` with the total appended (int32, length E + 1)."""
    counts = torch.as_tensor(counts, dtype=torch.int64)
    off = torch.zeros(counts.numel() + 1, dtype=torch.int64)
    off[1:] = torch.cumsum(counts, 0)
    return off.to(torch.int32)


def seed_of(cfg: int, tensor: int, sub: int = 0) -> int:
    """Deterministic seed for tensor ``tensor`` (and sub-index ``sub``) of workload ``cfg``."""
    return (cfg * 1_000_003 + tensor * 10_007 + sub) & 0x7FFFFFFF


def moe_expected_padding(counts, tile_m: int = 128) -> float:
    """Fraction of padded rows when each expert segment is rounded up to ``tile_m`` rows."""
    counts = [int(c) for c in counts]
    padded = sum(int(math.ceil(c / tile_m)) * tile_m for c in counts)
    return 1.0 - sum(counts) / max(padded, 1)

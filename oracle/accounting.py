"""KV-cache and projection-parameter accounting (closed forms).

TEST INFRASTRUCTURE ONLY (part of the oracle package).

Sources:
  * "MHA, MQA và GQA" (coregenaihub interactive e-book), the accounting simulator
    and its mode table: bytes per token are K and V, times the number of KV groups,
    the head dimension, the bytes per element and the layer count; the buffer is
    that times the context length (one sequence, paging not counted); the saving
    against MHA is query heads over KV groups, independent of context and dtype;
    a 4-bit type gives half a byte per element, so byte counts may be fractional;
    K and V projections shrink by the same factor while Q and O do not; a group
    count that does not divide the query-head count is an error, never rounded,
    and the valid counts are the divisors.
  * "Attention Architecture Experiments" (MiniMind docs), section Benchmark: the
    default GQA cache holds 2*4*96 elements per token and layer, MLA with
    kv_lora_rank 128 and rope_dim 48 holds 128+48, about 4.4x fewer.

Readings: the projection counts use hidden = query_heads * head_dim (this is
what makes the e-book's K+V figure 1 073 741 824 for 32 heads of 128 over 32
layers come out), and projection biases are ignored, as the e-book says it does.
All results are exact (``fractions.Fraction`` where a 4-bit type can make them
fractional).
"""
from __future__ import annotations

from fractions import Fraction


class GroupCountError(ValueError):
    """KV group count does not divide the query-head count."""

    def __init__(self, q_heads: int, kv_groups: int):
        self.q_heads = q_heads
        self.kv_groups = kv_groups
        self.remainder = q_heads % kv_groups if kv_groups > 0 else None
        self.valid = valid_group_counts(q_heads)
        super().__init__(
            f"{q_heads} query heads cannot be split into {kv_groups} equal KV groups "
            f"(remainder {self.remainder}); valid group counts: {self.valid}")


def valid_group_counts(q_heads: int) -> list[int]:
    """Every KV group count that splits ``q_heads`` into equal groups (its divisors)."""
    if q_heads <= 0:
        raise ValueError("q_heads must be positive")
    return [g for g in range(1, q_heads + 1) if q_heads % g == 0]


def check_groups(q_heads: int, kv_groups: int) -> int:
    """Return query heads per group; raise GroupCountError when the split is not exact."""
    if kv_groups <= 0 or q_heads <= 0 or q_heads % kv_groups != 0:
        raise GroupCountError(q_heads, kv_groups)
    return q_heads // kv_groups


def mode_name(q_heads: int, kv_groups: int) -> str:
    check_groups(q_heads, kv_groups)
    if kv_groups == q_heads:
        return "MHA"
    if kv_groups == 1:
        return "MQA"
    return "GQA"


def kv_elems_per_token_layer(kv_groups: int, head_dim: int) -> int:
    """Cached elements per token per layer for GQA/MQA/MHA: one K and one V row per group."""
    return 2 * kv_groups * head_dim


def mla_elems_per_token_layer(kv_lora_rank: int, rope_dim: int) -> int:
    """Cached elements per token per layer for MLA: the latent plus the shared RoPE key."""
    return kv_lora_rank + rope_dim


def kv_bytes_per_token(kv_groups: int, head_dim: int, bits: int, layers: int) -> Fraction:
    return Fraction(kv_elems_per_token_layer(kv_groups, head_dim) * bits * layers, 8)


def kv_buffer_bytes(kv_groups: int, head_dim: int, bits: int, layers: int, context: int) -> Fraction:
    return kv_bytes_per_token(kv_groups, head_dim, bits, layers) * context


def savings_vs_mha(q_heads: int, kv_groups: int) -> Fraction:
    check_groups(q_heads, kv_groups)
    return Fraction(q_heads, kv_groups)


def kv_proj_params(q_heads: int, kv_groups: int, head_dim: int, layers: int) -> int:
    """K and V projection weights over all layers (hidden = q_heads * head_dim, no bias)."""
    hidden = q_heads * head_dim
    return 2 * hidden * kv_groups * head_dim * layers


def qo_proj_params(q_heads: int, head_dim: int, layers: int) -> int:
    """Q and output projection weights over all layers; independent of the grouping."""
    hidden = q_heads * head_dim
    return 2 * hidden * q_heads * head_dim * layers


def mode_row(q_heads: int, kv_groups: int, layers: int, head_dim: int, context: int,
             bits: int) -> dict:
    """One row of the e-book's mode table for the given six inputs."""
    per_group = check_groups(q_heads, kv_groups)
    kv_p = kv_proj_params(q_heads, kv_groups, head_dim, layers)
    qo_p = qo_proj_params(q_heads, head_dim, layers)
    return {
        "mode": mode_name(q_heads, kv_groups),
        "kv_groups": kv_groups,
        "q_per_group": per_group,
        "kv_bytes_per_token": kv_bytes_per_token(kv_groups, head_dim, bits, layers),
        "buffer_bytes": kv_buffer_bytes(kv_groups, head_dim, bits, layers, context),
        "savings_vs_mha": savings_vs_mha(q_heads, kv_groups),
        "kv_proj_params": kv_p,
        "qo_proj_params": qo_p,
        "all4_proj_params": kv_p + qo_p,
    }

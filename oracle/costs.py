"""Closed-form byte and FLOP counts of MLA decode -- TEST INFRASTRUCTURE ONLY.

Each function restates a count the pages derive, in this file's own words;
``tests/golden/closed_forms.txt`` holds the values the pages print, with the
passage each comes from, and the tests check these functions against them.

Conventions: one multiply-add is 2 FLOPs (M5.8 0x02 parameter ledger counts
FLOPs that way; zdszero counts multiply-adds, i.e. half).  bf16 = 2 bytes.
"""
from __future__ import annotations


def latent_bytes_per_token_layer(r=512, d_rope=64, elem_bytes=2):
    """Cached latent row: c (r wide) plus the shared rope key ("MLA in full
    detail", the two cached nodes: 576 values, 1152 bytes in bf16)."""
    return (r + d_rope) * elem_bytes


def decompressed_bytes_per_token_layer(heads, d_nope=128, d_rope=64, d_v=128, elem_bytes=2):
    """Per-head 192-wide key plus 128-wide value that the Normal path builds
    (mlxcel bytes table; "MLA in full detail", Step 1)."""
    return heads * (d_nope + d_rope + d_v) * elem_bytes


def naive_upprojection_flops_per_token(heads=128, r=512, d_nope=128, d_v=128):
    """Up-projecting one cached latent into all heads' keys and values
    ("MLA in full detail", Step 1: 2 * r * h * (d_nope + d_v))."""
    return 2 * r * heads * (d_nope + d_v)


def absorbed_core_flops_per_pair(heads=128, r=512, d_rope=64):
    """Attention core per (query, key) pair in the absorbed form: a 576-wide
    score and a 512-wide latent accumulation per head."""
    return 2 * heads * ((r + d_rope) + r)


def normal_core_flops_per_pair(heads=128, d_nope=128, d_rope=64, d_v=128):
    """Attention core per (query, key) pair over expanded 192/128-wide heads."""
    return 2 * heads * ((d_nope + d_rope) + d_v)


def fold_flops_per_query(heads=128, r=512, d_nope=128, d_v=128):
    """The two absorbed bmms per query token: W_UK^T q_nope and W_UV latent."""
    return 2 * heads * d_nope * r + 2 * heads * r * d_v


def decode_intensity(heads=128, r=512, d_rope=64, elem_bytes=2, tp=1):
    """FLOPs per cache byte of one-token absorbed decode; heads shard by the
    tensor-parallel degree while every rank reads the full latent row."""
    return absorbed_core_flops_per_pair(heads // tp, r, d_rope) / latent_bytes_per_token_layer(
        r, d_rope, elem_bytes)


def model_cache_bytes_per_token(layers, r=512, d_rope=64, elem_bytes=2):
    return layers * latent_bytes_per_token_layer(r, d_rope, elem_bytes)


def causal_pairs(queries, prefix):
    """(query, key) pairs when `queries` new tokens follow `prefix` cached ones
    and each new token also sees the earlier new tokens and itself."""
    return queries * prefix + queries * (queries + 1) // 2


def fp8_row_bytes(r=512, n_scales=4, d_rope=64):
    """FP8 latent + fp32 scales + bf16 rope (M5.8 0x0B)."""
    return r * 1 + n_scales * 4 + d_rope * 2


def teaching_crossover(d_nope=128, d_c=512):
    """T_k where materialised and absorbed NoPE-score costs meet at T_q = 1 (M5.8 0x04)."""
    return d_nope * d_c / (d_c * d_nope + d_nope - d_c)


def rectangular_query_bound(heads=128, r=512, d_nope=128, d_rope=64, d_v=128):
    """Largest query block for which absorption wins against all-pairs MHA as
    the context grows: naive up-projection cost / extra core cost per pair."""
    extra = absorbed_core_flops_per_pair(heads, r, d_rope) - normal_core_flops_per_pair(
        heads, d_nope, d_rope, d_v)
    return naive_upprojection_flops_per_token(heads, r, d_nope, d_v) / extra

"""Closed-form cache-size and FLOP accounting -- TEST INFRASTRUCTURE ONLY.

Plain definitions of the sizes and costs the pages state, pinned in the tests
against the numbers the pages print (tests/golden/page_numbers.json).
"""
from __future__ import annotations


def kv_cache_bytes(S: int, n_layers: int, n_kv_heads: int, d_head: int, n_bytes: int) -> int:
    """S x 2 (K and V) x layers x KV heads x head dim x bytes per value.

    "Attention Optimizations", "KV cache size".
    """
    return S * 2 * n_layers * n_kv_heads * d_head * n_bytes


def mla_values_per_token(d_latent: int, d_rope: int) -> int:
    """Values one MLA layer caches per token: the c_KV latent plus the shared RoPE key.

    "Attention Optimizations", "DSA: DeepSeek Sparse Attention" (512 + 64).
    """
    return d_latent + d_rope


def mla_cache_bytes(S: int, d_latent: int, d_rope: int, n_bytes: int) -> int:
    return S * mla_values_per_token(d_latent, d_rope) * n_bytes


def attention_flops(S: int, n_heads: int, d_head: int) -> int:
    """Decode attention FLOPs per token per layer: 4 S n_h d_h (half QK^T, half PV).

    "Long context, KV eviction and sparse attention", "The cost of long context".
    """
    return 4 * S * n_heads * d_head


def attention_linear_crossover(params: float, n_layers: int, n_heads: int, d_head: int) -> float:
    """Context length S at which one token's attention FLOPs over all layers,
    n_layers x attention_flops(S, ...), equal the linear layers' 2 x params.

    "Long context, KV eviction and sparse attention", "The cost of long context".
    attention_flops is linear in S, so S = 2 params / (n_layers x the FLOPs of
    one attended token); the page's printed crossovers (~38K, ~54K) therefore
    pin attention_flops as well.
    """
    per_attended_token = n_layers * attention_flops(1, n_heads, d_head)
    return 2 * params / per_attended_token


def mla_kv_up_projection_bytes(d_latent: int, n_heads: int, d_nope: int, d_v: int,
                               n_bytes: int) -> int:
    """Bytes of W_kv, the map from the latent to per-head keys and values.

    "Attention Optimizations", "Computation Path": (S, 512) -> (S, 2, 128, 128).
    """
    return d_latent * n_heads * (d_nope + d_v) * n_bytes


def mla_over_gqa_groups(d_head: int) -> float:
    """MLA cache per token per layer over one KV group's (2 d_h), at d_c = 4 d_h, d_R = d_h / 2.

    "Overview of Attention Mechanism", MLA "Comparison of KV Cache": (9/2) d_h,
    i.e. MLA caches as much as GQA with 2.25 groups.
    """
    d_c, d_r = 4 * d_head, d_head // 2
    return (d_c + d_r) / (2 * d_head)

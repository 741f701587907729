"""Work and traffic counters of the method (plain integer arithmetic).

"Prefill Optimisation ...", section 4 ("Worked mathematical derivations"):
a fresh chunk of U tokens over K cached tokens computes U*K suffix-to-prefix
pairs plus U(U+1)/2 causal suffix-to-suffix pairs, and attention costs
4 * L * H_Q * pairs * d_head FLOPs (2*d for QK^T and 2*d for PV per pair;
softmax excluded).  Section 6 prices the KV cache per token.
"""
from __future__ import annotations


def pairs(n_new: int, n_cached: int) -> int:
    """Attention pairs of a chunk of ``n_new`` tokens over ``n_cached`` cached ones."""
    return n_new * n_cached + n_new * (n_new + 1) // 2


def full_prefix_blocks(prefix_len: int, block_size: int) -> int:
    """Full blocks a prefix hit can reuse (full-block-only policy, section 3)."""
    return prefix_len // block_size


def attention_flops(n_pairs: int, num_heads: int, head_dim: int, num_layers: int = 1) -> int:
    return 4 * num_layers * num_heads * n_pairs * head_dim


def kv_bytes_per_token(num_kv_heads: int, head_dim: int, elem_bytes: int,
                       num_layers: int = 1) -> int:
    """K and V bytes one token occupies in the cache (section 6)."""
    return 2 * num_layers * num_kv_heads * head_dim * elem_bytes


def chunk_bytes(n_new: int, n_cached: int, num_heads: int, num_kv_heads: int,
                head_dim: int, elem_bytes: int) -> int:
    """Algorithmic HBM bytes of one chunk: read Q, read the new K/V, write them
    to the cache, read the cached K/V once, write O.  Block-table and
    descriptor integers are not counted."""
    q = n_new * num_heads * head_dim * elem_bytes
    new_kv = 2 * n_new * num_kv_heads * head_dim * elem_bytes
    cached_kv = 2 * n_cached * num_kv_heads * head_dim * elem_bytes
    return q + new_kv + new_kv + cached_kv + q

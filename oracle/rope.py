"""Oracle for rotary position embedding (RoPE) at absolute positions, and the
cache write of rotated keys.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix:
* "Prefill Optimisation: Prefix Caching, Chunked Prefill, and
  Disaggregation", section 2, "Causal equivalence and numerical tolerance":
  positional encodings such as RoPE take each token's absolute position in
  the whole sequence, so chunking does not move any token's geometry.
* "Chunked Prefill" (blog note), section "From scratch": the step of a
  sequence passes the number of tokens already in its cache as the position
  offset of its new tokens.

What they leave open, and the reading taken here (the standard rotary
embedding of the RoFormer paper, Su et al. 2021):
* the frequencies: pair i of a head of size D turns by ``p * theta**(-2i/D)``
  radians at position p, i = 0 .. D/2 - 1; ``theta`` is a parameter (10000
  is the usual base; the pages name none);
* the pairing: ``interleaved=False`` pairs element i with element i + D/2
  (the "rotate half" layout); ``interleaved=True`` pairs 2i with 2i + 1;
* the direction: (x, y) -> (x cos a - y sin a, x sin a + y cos a), i.e. the
  pair as the complex number x + iy multiplied by exp(i a).

All arithmetic is float64.
"""
from __future__ import annotations

import numpy as np

from . import attention as _attn


def inv_freq(head_dim: int, theta: float) -> np.ndarray:
    """Angle per position of each of the head_dim / 2 pairs: theta**(-2i/D)."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * i / head_dim)


def pair_index(head_dim: int, interleaved: bool):
    """(first, second) element indices of each rotated pair."""
    i = np.arange(head_dim // 2)
    if interleaved:
        return 2 * i, 2 * i + 1
    return i, i + head_dim // 2


def rotate(x, positions, theta: float, interleaved: bool = False) -> np.ndarray:
    """Rotary embedding of ``x`` ``[T, heads, D]`` at integer ``positions``
    ``[T]`` (one absolute position per token, shared by all its heads)."""
    x = np.asarray(x, dtype=np.float64)
    head_dim = x.shape[-1]
    a = np.asarray(positions, dtype=np.float64)[:, None] * inv_freq(head_dim, theta)[None, :]
    cos = np.cos(a)[:, None, :]
    sin = np.sin(a)[:, None, :]
    i0, i1 = pair_index(head_dim, interleaved)
    out = np.empty_like(x)
    out[..., i0] = x[..., i0] * cos - x[..., i1] * sin
    out[..., i1] = x[..., i0] * sin + x[..., i1] * cos
    return out


def token_positions(cu_seqlens_q, cached_seq_len) -> np.ndarray:
    """Absolute position of every active token of a packed batch (int64
    ``[T]``): token t of sequence b sits at ``cached_seq_len[b] + t``."""
    total = int(cu_seqlens_q[-1])
    pos = np.empty(total, dtype=np.int64)
    for b in range(len(cu_seqlens_q) - 1):
        q0, q1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
        pos[q0:q1] = int(cached_seq_len[b]) + np.arange(q1 - q0)
    return pos


def rope_cache_write(q, k_pool, v_pool, k_new, v_new, block_tables, cu_seqlens_q,
                     cached_seq_len, block_size: int, theta: float, interleaved: bool = False):
    """Rotate this call's queries and keys at their absolute positions, then
    write the rotated keys and the unchanged values to their slots.

    Returns ``(q_rot, k_pool', v_pool')``, all float64; the pools use the
    oracle's canonical ``[num_blocks, block_size, G, D]`` layout.
    """
    pos = token_positions(cu_seqlens_q, cached_seq_len)
    q_rot = rotate(q, pos, theta, interleaved)
    k_rot = rotate(k_new, pos, theta, interleaved)
    k_out, v_out = _attn.cache_write(np.asarray(k_pool, dtype=np.float64),
                                     np.asarray(v_pool, dtype=np.float64), k_rot,
                                     np.asarray(v_new, dtype=np.float64), block_tables,
                                     cu_seqlens_q, cached_seq_len, block_size)
    return q_rot, k_out, v_out

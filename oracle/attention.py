"""Oracle for the cache write and the attention of one chunked-prefill call.

Pools here use the canonical logical layout ``[num_blocks, block_size, G, D]``
(slot ``(block, offset)`` holds the K (or V) vectors of all KV heads for one
token).  The GPU library's physical layout is its own business; tests map it
to this canonical form.

All arithmetic is float64.  Inputs that were bfloat16 on the GPU side arrive
here as their exact float64 values.
"""
from __future__ import annotations

import numpy as np


# ---------------------------------------------------------------------------
# Addressing: a logical position of a sequence -> a physical slot.
# "Prefill Processing", section "Block Allocation": a block-table row lists
# the physical block ids of a sequence in logical order; position p lives in
# logical block p // block_size at offset p % block_size.
# ---------------------------------------------------------------------------
def slot_of(block_row, pos: int, block_size: int) -> int:
    """Flat slot id ``block * block_size + offset`` of logical position ``pos``."""
    return int(block_row[pos // block_size]) * block_size + pos % block_size


def slot_mapping(block_tables, cu_seqlens_q, cached_seq_len, block_size: int) -> np.ndarray:
    """Slot of every active token of a packed batch (int64 ``[T]``).

    Token t of sequence b sits at absolute position ``cached_seq_len[b] + t``
    ("Prefill Processing", section "How Segmentation Works with KV Segments":
    iteration m writes positions cached .. cached+active-1).
    """
    total = int(cu_seqlens_q[-1])
    out = np.empty(total, dtype=np.int64)
    for b in range(len(cu_seqlens_q) - 1):
        q0, q1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
        c = int(cached_seq_len[b])
        for t in range(q1 - q0):
            out[q0 + t] = slot_of(block_tables[b], c + t, block_size)
    return out


def cache_write(k_pool, v_pool, k_new, v_new, block_tables, cu_seqlens_q,
                cached_seq_len, block_size: int):
    """Return copies of the pools with every active token's K and V stored at
    its slot; every other slot is left exactly as it was.

    "Prefill Processing", section "How Segmentation Works with KV Segments"
    (each iteration writes the KV of its active tokens to the cache).
    """
    k_out = np.array(k_pool, copy=True)
    v_out = np.array(v_pool, copy=True)
    for b in range(len(cu_seqlens_q) - 1):
        q0, q1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
        c = int(cached_seq_len[b])
        pos = c + np.arange(q1 - q0)
        blocks = np.asarray(block_tables[b])[pos // block_size]
        offs = pos % block_size
        k_out[blocks, offs] = k_new[q0:q1]
        v_out[blocks, offs] = v_new[q0:q1]
    return k_out, v_out


def gather_kv(pool, block_row, length: int, block_size: int) -> np.ndarray:
    """Logical K (or V) of positions 0..length-1 of one sequence, ``[L, G, D]``,
    read through its block-table row."""
    pos = np.arange(length)
    return pool[np.asarray(block_row)[pos // block_size], pos % block_size]


def _group_of(head: int, num_heads: int, num_kv_heads: int) -> int:
    # GQA: query heads are split into num_kv_heads consecutive groups (the
    # pages name GQA without fixing the grouping; this is the consecutive one).
    return head // (num_heads // num_kv_heads)


# ---------------------------------------------------------------------------
# Plain definition of the attention of one call.
# "Prefill Optimisation ...", section 2, "Causal equivalence": token i
# attends to every position j <= i (absolute positions); chunk m attends to
# all cached KV of earlier chunks and causally to itself.
# ---------------------------------------------------------------------------
def attention(q, k_pool, v_pool, block_tables, cu_seqlens_q, cached_seq_len,
              block_size: int, scale: float, num_kv_heads: int,
              q_tile: int = 256, seqs=None, heads=None):
    """Attention output ``[T, H, D]`` (float64) of a packed varlen batch.

    ``k_pool``/``v_pool`` must already hold this call's writes (see
    ``cache_write``).  For token t of sequence b (absolute position
    ``c_b + t``) and query head h with KV head g:
    ``O = sum_j softmax_j(scale * <q, K_j>) V_j`` over ``j <= c_b + t``.
    Evaluated as a dense masked softmax with the row maximum subtracted, per
    (sequence, head, query tile).  ``seqs``/``heads`` restrict the work to a
    subset (the other rows of the result stay zero).
    """
    q = np.asarray(q, dtype=np.float64)
    total, num_heads, head_dim = q.shape
    out = np.zeros((total, num_heads, head_dim), dtype=np.float64)
    seq_ids = range(len(cu_seqlens_q) - 1) if seqs is None else seqs
    head_ids = range(num_heads) if heads is None else heads
    for b in seq_ids:
        q0, q1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
        n, c = q1 - q0, int(cached_seq_len[b])
        if n == 0:
            continue
        keys = gather_kv(k_pool, block_tables[b], c + n, block_size).astype(np.float64)
        vals = gather_kv(v_pool, block_tables[b], c + n, block_size).astype(np.float64)
        key_pos = np.arange(c + n)
        for h in head_ids:
            g = _group_of(h, num_heads, num_kv_heads)
            for t0 in range(0, n, q_tile):
                t1 = min(n, t0 + q_tile)
                s = scale * (q[q0 + t0:q0 + t1, h, :] @ keys[:, g, :].T)
                allowed = key_pos[None, :] <= (c + np.arange(t0, t1))[:, None]
                s = np.where(allowed, s, -np.inf)
                s = s - s.max(axis=1, keepdims=True)
                p = np.exp(s)
                p /= p.sum(axis=1, keepdims=True)
                out[q0 + t0:q0 + t1, h, :] = p @ vals[:, g, :]
    return out


def attention_rows(q_rows, keys, vals, positions, scale: float):
    """Attention of a few query vectors against one sequence's logical K/V.

    ``q_rows [m, D]`` are queries at absolute ``positions [m]``;
    ``keys``/``vals`` ``[L, D]`` are the logical keys/values of one KV head.
    Used to check sampled outputs of full-size runs one by one.
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    s = scale * (q_rows @ np.asarray(keys, dtype=np.float64).T)
    allowed = np.arange(keys.shape[0])[None, :] <= np.asarray(positions)[:, None]
    s = np.where(allowed, s, -np.inf)
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=1, keepdims=True)
    return p @ np.asarray(vals, dtype=np.float64)


# ---------------------------------------------------------------------------
# Oracle B: the pages' segment loop, written out.
# "Prefill Processing", sections "How Segmentation Works with KV Segments",
# "Kernel Interface" and "Partial KV Segment Handling": the cached KV
# (cached_seq_len tokens) is visited in segments of kv_segment_size; the last
# segment is masked past cached_seq_len; then the chunk attends to itself.
# Each part leaves a partial (running max m, sum l, unnormalised O); the
# parts are merged by log-sum-exp.  The pages give no merge formula; this is
# the standard rescaling that "Prefill Optimisation ..." section 2 alludes to
# (online softmax rescales running normalisers across blocks).
# ---------------------------------------------------------------------------
def num_segments(cached_seq_len: int, kv_segment_size: int) -> int:
    """Segments visited over the cached KV: full ones plus one partial one
    when ``cached_seq_len`` is not a multiple of the segment size."""
    return -(-cached_seq_len // kv_segment_size)


def segment_valid_tokens(cached_seq_len: int, kv_segment_size: int):
    """Valid tokens of each segment, e.g. 3584 at 1024 -> [1024, 1024, 1024, 512]."""
    return [min(kv_segment_size, cached_seq_len - s * kv_segment_size)
            for s in range(num_segments(cached_seq_len, kv_segment_size))]


def partial_state(s_scores, vals):
    """(m, l, O~) of one part: ``s_scores [m_rows, L]`` (−inf where masked),
    ``vals [L, D]``.  A row with no valid key gets m = −inf, l = 0, O~ = 0."""
    m = s_scores.max(axis=1) if s_scores.shape[1] else np.full(s_scores.shape[0], -np.inf)
    safe_m = np.where(np.isfinite(m), m, 0.0)
    p = np.exp(s_scores - safe_m[:, None])
    p = np.where(np.isfinite(s_scores), p, 0.0)
    return m, p.sum(axis=1), p @ vals


def merge_states(states):
    """Log-sum-exp merge of partial states into the normalised output."""
    ms = np.stack([s[0] for s in states])          # [P, rows]
    m = ms.max(axis=0)
    w = np.where(np.isfinite(ms), np.exp(ms - np.where(np.isfinite(m), m, 0.0)[None, :]), 0.0)
    l_tot = sum(w[i] * states[i][1] for i in range(len(states)))
    o_tot = sum(w[i][:, None] * states[i][2] for i in range(len(states)))
    return o_tot / l_tot[:, None]


def segmented_attention(q, k_pool, v_pool, block_tables, cu_seqlens_q,
                        cached_seq_len, block_size: int, scale: float,
                        num_kv_heads: int, kv_segment_size: int):
    """Same result as ``attention`` (exactly, up to rounding order), computed
    the pages' way: cached segments with the partial one masked, the causal
    self part, then a log-sum-exp merge of the partials."""
    q = np.asarray(q, dtype=np.float64)
    total, num_heads, head_dim = q.shape
    out = np.zeros((total, num_heads, head_dim), dtype=np.float64)
    for b in range(len(cu_seqlens_q) - 1):
        q0, q1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
        n, c = q1 - q0, int(cached_seq_len[b])
        if n == 0:
            continue
        keys = gather_kv(k_pool, block_tables[b], c + n, block_size).astype(np.float64)
        vals = gather_kv(v_pool, block_tables[b], c + n, block_size).astype(np.float64)
        for h in range(num_heads):
            g = _group_of(h, num_heads, num_kv_heads)
            qh = q[q0:q1, h, :]
            states = []
            for s in range(num_segments(c, kv_segment_size)):
                lo = s * kv_segment_size
                hi = min(lo + kv_segment_size, c + n)   # segment window in the pool
                sc = scale * (qh @ keys[lo:hi, g, :].T)
                valid = np.arange(lo, hi) < c            # partial-segment mask
                sc = np.where(valid[None, :], sc, -np.inf)
                states.append(partial_state(sc, vals[lo:hi, g, :]))
            # self part: positions c..c+n-1, causal within the chunk
            sc = scale * (qh @ keys[c:c + n, g, :].T)
            causal = np.arange(n)[None, :] <= np.arange(n)[:, None]
            sc = np.where(causal, sc, -np.inf)
            states.append(partial_state(sc, vals[c:c + n, g, :]))
            out[q0:q1, h, :] = merge_states(states)
    return out

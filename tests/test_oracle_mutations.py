"""The pins must catch plausible oracle mistakes.  Each case plants one
mistake in the oracle (CPU only, via monkeypatch) and checks that at least one
pin then fails."""
import numpy as np
import pytest

from oracle import attention as oa
from tests import test_oracle_attention_pins as pins

_orig_gather = oa.gather_kv
_orig_group = oa._group_of
_orig_partial = oa.partial_state


def _gather_wrong_block(pool, block_row, length, block_size):
    # swaps // and % when picking the block-table column
    pos = np.arange(length)
    row = np.asarray(block_row)
    return pool[row[(pos % block_size) % len(row)], pos % block_size]


def _group_modulo(head, num_heads, num_kv_heads):
    return head % num_kv_heads


def _partial_no_rescale(s_scores, vals):
    m, l, o = _orig_partial(s_scores, vals)
    return np.zeros_like(m), l, o          # forgets the running max in the merge


def _attention_strict(q, k_pool, v_pool, block_tables, cu_seqlens_q, cached_seq_len,
                      block_size, scale, num_kv_heads, q_tile=256, seqs=None, heads=None):
    # drops the diagonal (j < c+t instead of j <= c+t) for all but the first row
    out = _orig_attention(q, k_pool, v_pool, block_tables, cu_seqlens_q, cached_seq_len,
                          block_size, scale, num_kv_heads, q_tile, seqs, heads)
    q = np.asarray(q, dtype=np.float64)
    for b in range(len(cu_seqlens_q) - 1):
        q0, q1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
        c = int(cached_seq_len[b])
        keys = _orig_gather(k_pool, block_tables[b], c + q1 - q0, block_size)
        vals = _orig_gather(v_pool, block_tables[b], c + q1 - q0, block_size)
        for t in range(q1 - q0):
            if c + t == 0:
                continue
            for h in range(q.shape[1]):
                g = _orig_group(h, q.shape[1], num_kv_heads)
                s = scale * keys[:c + t, g] @ q[q0 + t, h]
                p = np.exp(s - s.max())
                out[q0 + t, h] = p @ vals[:c + t, g] / p.sum()
    return out


def _attention_no_scale(q, k_pool, v_pool, block_tables, cu_seqlens_q, cached_seq_len,
                        block_size, scale, num_kv_heads, q_tile=256, seqs=None, heads=None):
    return _orig_attention(q, k_pool, v_pool, block_tables, cu_seqlens_q, cached_seq_len,
                           block_size, 1.0, num_kv_heads, q_tile, seqs, heads)


_orig_attention = oa.attention

ALL_PINS = [
    pins.test_brute_force_tiny_chunked_paged,
    pins.test_monolithic_equals_torch_sdpa,
    pins.test_zero_keys_give_prefix_mean_of_values,
    pins.test_selector_queries_pick_one_value_row,
]


@pytest.mark.parametrize("name,attr,bad", [
    ("wrong block index", "gather_kv", _gather_wrong_block),
    ("modulo GQA grouping", "_group_of", _group_modulo),
    ("diagonal dropped", "attention", _attention_strict),
    ("scale dropped", "attention", _attention_no_scale),
])
def test_planted_attention_mistake_is_caught(monkeypatch, name, attr, bad):
    monkeypatch.setattr(oa, attr, bad)
    failures = 0
    for pin in ALL_PINS:
        try:
            pin()
        except AssertionError:
            failures += 1
    assert failures >= 1, f"no pin caught: {name}"


def test_planted_merge_mistake_is_caught(monkeypatch):
    monkeypatch.setattr(oa, "partial_state", _partial_no_rescale)
    with pytest.raises(AssertionError):
        pins.test_brute_force_tiny_chunked_paged()


# --------------------------------------------------------------------------
# attention_rows (the checker of sampled rows at full size)
# --------------------------------------------------------------------------
_orig_rows = oa.attention_rows


def _rows_strict(q_rows, keys, vals, positions, scale):
    # the diagonal dropped: row i sees keys < positions[i] (position 0 keeps one key)
    return _orig_rows(q_rows, keys, vals, [max(p - 1, 0) for p in positions], scale)


def _rows_no_scale(q_rows, keys, vals, positions, scale):
    return _orig_rows(q_rows, keys, vals, positions, 1.0)


def _rows_one_past(q_rows, keys, vals, positions, scale):
    # one key too many (clamped to the keys given)
    return _orig_rows(q_rows, keys, vals, [min(p + 1, len(keys) - 1) for p in positions], scale)


def _rows_values_reversed(q_rows, keys, vals, positions, scale):
    # values read in the wrong order (a transposed or flipped gather)
    return _orig_rows(q_rows, keys, np.asarray(vals)[::-1], positions, scale)


ROW_PINS = [
    pins.test_attention_rows_brute_force,
    pins.test_attention_rows_zero_keys_prefix_mean,
    pins.test_attention_rows_selector_picks_value_row,
]


@pytest.mark.parametrize("name,bad", [
    ("diagonal dropped", _rows_strict),
    ("scale dropped", _rows_no_scale),
    ("one key past the position", _rows_one_past),
    ("values reversed", _rows_values_reversed),
])
def test_planted_attention_rows_mistake_is_caught(monkeypatch, name, bad):
    monkeypatch.setattr(oa, "attention_rows", bad)
    failures = 0
    for pin in ROW_PINS:
        try:
            pin()
        except AssertionError:
            failures += 1
    assert failures >= 1, f"no pin caught: {name}"

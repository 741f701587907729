"""Pins of the attention oracle against things other than itself: brute force
on tiny inputs, a library routine, closed forms and the invariants the pages
state.  CPU only."""
import math

import numpy as np
import pytest
import torch

from oracle import attention as oa
from tests.golden_io import ints, rows
from tests.oracle_helpers import chunks_of, empty_pools, run_chunked


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def _brute_force(q, k, v, scale, num_kv_heads):
    """Pure-Python loops with math.exp over the logical (unpaged) prompt:
    token i, head h attends to j <= i."""
    P, H, D = q.shape
    grp = H // num_kv_heads
    out = np.zeros((P, H, D))
    for i in range(P):
        for h in range(H):
            g = h // grp
            logits = []
            for j in range(i + 1):
                acc = 0.0
                for d in range(D):
                    acc += float(q[i, h, d]) * float(k[j, g, d])
                logits.append(scale * acc)
            mx = max(logits)
            w = [math.exp(x - mx) for x in logits]
            z = sum(w)
            for d in range(D):
                out[i, h, d] = sum(w[j] * float(v[j, g, d]) for j in range(i + 1)) / z
    return out


def test_brute_force_tiny_chunked_paged():
    # H=4, G=2, D=8, bs=4, 37 tokens in chunks 8,8,8,8,5, scattered table
    H, G, D, bs, P = 4, 2, 8, 4, 37
    q, k, v = _rand(1, P, H, D), _rand(2, P, G, D), _rand(3, P, G, D)
    num_blocks = 16
    table = np.random.default_rng(4).permutation(num_blocks)[:10]
    scale = 1 / math.sqrt(D)
    got, _, _ = run_chunked(q, k, v, [8, 8, 8, 8, 5], bs, table, num_blocks, G, scale)
    ref = _brute_force(q, k, v, scale, G)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)
    # the segment-loop oracle (S=8: one full segment per earlier chunk) too
    seg, _, _ = run_chunked(q, k, v, [8, 8, 8, 8, 5], bs, table, num_blocks, G, scale, segmented=8)
    np.testing.assert_allclose(seg, ref, rtol=0, atol=1e-12)


def test_monolithic_equals_torch_sdpa():
    # c = 0 over the whole prompt equals the library's causal attention
    # (float64 on the CPU), with each KV head repeated for its query-head group.
    H, G, D, bs, P = 8, 2, 16, 16, 200
    q, k, v = _rand(11, P, H, D), _rand(12, P, G, D), _rand(13, P, G, D)
    table = np.random.default_rng(14).permutation(20)[:13]
    scale = 1 / math.sqrt(D)
    got, _, _ = run_chunked(q, k, v, [P], bs, table, 20, G, scale)
    tq = torch.from_numpy(q).permute(1, 0, 2)                          # [H, P, D]
    tk = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(H // G, dim=0)
    tv = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(H // G, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True,
                                                           scale=scale)
    np.testing.assert_allclose(got, ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def test_zero_keys_give_prefix_mean_of_values():
    # K = 0 makes every logit 0, so O[t] is the plain mean of V over j <= c+t:
    # pins the causal boundary (inclusive) and the gather through the table.
    H, G, D, bs, P = 4, 4, 8, 16, 300
    q, v = _rand(21, P, H, D), _rand(22, P, G, D)
    k = np.zeros((P, G, D))
    table = np.random.default_rng(23).permutation(40)[:19]
    got, _, _ = run_chunked(q, k, v, [100, 77, 123], bs, table, 40, G, 0.125)
    expect = np.cumsum(v, axis=0) / np.arange(1, P + 1)[:, None, None]
    for h in range(H):
        np.testing.assert_allclose(got[:, h, :], expect[:, h, :], rtol=0, atol=1e-12)


@pytest.mark.parametrize("chunk", [64, 128, 256, 512, 1024])
def test_chunked_equals_monolithic_c1_shape(chunk):
    # "Prefill Optimisation ...", section 2: chunked causal attention equals the
    # monolithic pass in exact arithmetic.  c1 shape: H=G=4, D=64, 1024 tokens,
    # bs16, 128-block pool.
    from synth import free_block_order, get_workload, prompt_qkv
    w = get_workload("c1")
    q, k, v = (x.astype(np.float64) for x in prompt_qkv(w))
    table = free_block_order(w.num_blocks, w.seed)[:64]
    mono, _, _ = run_chunked(q, k, v, [w.prompt_len], w.block_size, table, w.num_blocks,
                             w.num_kv_heads, w.scale)
    got, _, _ = run_chunked(q, k, v, chunks_of(w.prompt_len, chunk), w.block_size, table,
                            w.num_blocks, w.num_kv_heads, w.scale)
    np.testing.assert_allclose(got, mono, rtol=0, atol=1e-12)


@pytest.mark.parametrize("seg", [512, 1024, 2048, 4096])
def test_segment_loop_matches_plain_definition(seg):
    # The pages' segment loop (with the partial segment masked) and an LSE
    # merge give the plain result, whatever kv_segment_size.  Small heads, long
    # enough context for up to 9 segments; chunks cross segment boundaries.
    H, G, D, bs, P = 2, 1, 8, 16, 5000
    q, k, v = _rand(31, P, H, D), _rand(32, P, G, D), _rand(33, P, G, D)
    table = np.random.default_rng(34).permutation(400)[:313]
    scale = 1 / math.sqrt(D)
    chunks = [1024, 1024, 1024, 512, 1416]       # cached 0, 1024, 2048, 3072, 3584
    plain, _, _ = run_chunked(q, k, v, chunks, bs, table, 400, G, scale)
    seg_out, _, _ = run_chunked(q, k, v, chunks, bs, table, 400, G, scale, segmented=seg)
    np.testing.assert_allclose(seg_out, plain, rtol=0, atol=1e-12)


def test_segment_counts_match_pages():
    for cached, size, count, valid in rows("segments.txt"):
        cached, size, count = int(cached), int(size), int(count)
        assert oa.num_segments(cached, size) == count
        assert oa.segment_valid_tokens(cached, size) == ints(valid)


def test_prefix_cached_request_equals_recompute():
    # "Prefill Processing", section "Prefix Caching": a request with a cached
    # prefix is a segmented prefill with num_computed_tokens > 0.  Three
    # requests share the prefix's blocks; one varlen call over the suffixes
    # equals each request computed from token 0.
    H, G, D, bs = 4, 2, 16, 16
    prefix, suffixes = 96, [48, 16, 80]
    scale = 1 / math.sqrt(D)
    kp, vp = _rand(41, prefix, G, D), _rand(42, prefix, G, D)
    qp = _rand(43, prefix, H, D)
    num_blocks = 64
    order = list(np.random.default_rng(44).permutation(num_blocks))
    shared = [order.pop() for _ in range(prefix // bs)]
    k_pool, v_pool = empty_pools(num_blocks, bs, G, D)
    k_pool, v_pool = oa.cache_write(k_pool, v_pool, kp, vp, [shared], [0, prefix], [0], bs)
    tables, qs, ks, vs = [], [], [], []
    for i, s in enumerate(suffixes):
        tables.append(shared + [order.pop() for _ in range(s // bs)])
        qs.append(_rand(50 + i, s, H, D))
        ks.append(_rand(60 + i, s, G, D))
        vs.append(_rand(70 + i, s, G, D))
    cu = np.concatenate([[0], np.cumsum(suffixes)])
    cached = [prefix] * len(suffixes)
    width = max(len(t) for t in tables)
    bt = [t + [0] * (width - len(t)) for t in tables]
    k_pool, v_pool = oa.cache_write(k_pool, v_pool, np.concatenate(ks), np.concatenate(vs),
                                    bt, cu, cached, bs)
    got = oa.attention(np.concatenate(qs), k_pool, v_pool, bt, cu, cached, bs, scale, G)
    for i, s in enumerate(suffixes):
        fq = np.concatenate([qp, qs[i]])
        fk = np.concatenate([kp, ks[i]])
        fv = np.concatenate([vp, vs[i]])
        ref, _, _ = run_chunked(fq, fk, fv, [prefix + s], bs, list(range(20)), 20, G, scale)
        np.testing.assert_allclose(got[cu[i]:cu[i + 1]], ref[prefix:], rtol=0, atol=1e-12)


def test_selector_queries_pick_one_value_row():
    # q = alpha * k[tau] with random unit keys: the logit margin exceeds 100,
    # every other weight is below e^-100, so O equals V[tau] (closed form).
    H, G, D, bs, P = 4, 2, 128, 16, 700
    rng = np.random.default_rng(81)
    k = rng.standard_normal((P, G, D))
    k /= np.linalg.norm(k, axis=2, keepdims=True)
    v = rng.standard_normal((P, G, D))
    alpha = 2000.0
    chunks = [300, 250, 150]
    tau = np.zeros((P, H), dtype=np.int64)
    q = np.zeros((P, H, D))
    for i in range(P):
        for h in range(H):
            tau[i, h] = rng.integers(0, i + 1)
            q[i, h] = alpha * k[tau[i, h], h // (H // G)]
    table = rng.permutation(60)[:44]
    got, _, _ = run_chunked(q, k, v, chunks, bs, table, 60, G, 1 / math.sqrt(D))
    for h in range(H):
        np.testing.assert_allclose(got[:, h], v[tau[:, h], h // (H // G)], rtol=0, atol=1e-12)


def test_placement_does_not_matter():
    # The same logical KV behind two different block tables gives identical
    # attention (the gather uses block_row[p // bs], offset p % bs).
    H, G, D, bs, P = 2, 2, 8, 8, 120
    q, k, v = _rand(91, P, H, D), _rand(92, P, G, D), _rand(93, P, G, D)
    a, _, _ = run_chunked(q, k, v, [50, 70], bs, list(range(15)), 32, G, 0.3)
    b, _, _ = run_chunked(q, k, v, [50, 70], bs, list(np.random.default_rng(94).permutation(32)[:15]),
                          32, G, 0.3)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_cache_write_touches_exactly_the_active_slots():
    bs, G, D, nb = 16, 2, 4, 12
    k_pool = _rand(101, nb, bs, G, D)
    v_pool = _rand(102, nb, bs, G, D)
    tables = [[5, 2, 9, 0], [7, 3, 11, 1]]
    cu, cached = [0, 20, 27], [13, 40]            # positions 13..32 and 40..46
    k_new, v_new = _rand(103, 27, G, D), _rand(104, 27, G, D)
    k_out, v_out = oa.cache_write(k_pool, v_pool, k_new, v_new, tables, cu, cached, bs)
    slots = oa.slot_mapping(tables, cu, cached, bs)
    changed = set()
    for t, s in enumerate(slots):
        blk, off = divmod(int(s), bs)
        assert np.array_equal(k_out[blk, off], k_new[t])
        assert np.array_equal(v_out[blk, off], v_new[t])
        changed.add((blk, off))
    assert len(changed) == 27
    for blk in range(nb):
        for off in range(bs):
            if (blk, off) not in changed:
                assert np.array_equal(k_out[blk, off], k_pool[blk, off])
                assert np.array_equal(v_out[blk, off], v_pool[blk, off])
    # closed form of the addressing: sequence 0 position 13 is logical block 0
    # offset 13 -> block 5; position 16 -> logical block 1 -> block 2, offset 0
    assert slots[0] == 5 * 16 + 13 and slots[3] == 2 * 16 + 0
    assert slots[20] == 11 * 16 + 8                # seq 1 position 40 -> block 11, offset 8


# --------------------------------------------------------------------------
# attention_rows: the sampled-row checker of the full-size runs
# --------------------------------------------------------------------------
def _rows_brute_force(qr, keys, vals, positions, scale):
    """Pure-Python loops with math.exp: row i attends to keys 0..positions[i]."""
    out = np.zeros((len(qr), vals.shape[1]))
    for i, pos in enumerate(positions):
        logits = [scale * sum(float(qr[i, d]) * float(keys[j, d]) for d in range(keys.shape[1]))
                  for j in range(pos + 1)]
        mx = max(logits)
        w = [math.exp(x - mx) for x in logits]
        z = sum(w)
        for d in range(vals.shape[1]):
            out[i, d] = sum(w[j] * float(vals[j, d]) for j in range(pos + 1)) / z
    return out


def test_attention_rows_brute_force():
    # rows at the first key, the last key and in between, on large logits
    # (scale 0.9 with N(0, 2^2) entries) so the max subtraction matters
    L, D = 41, 8
    keys, vals = 2 * _rand(201, L, D), _rand(202, L, D)
    positions = [0, 1, 7, 16, 39, 40]
    qr = 2 * _rand(203, len(positions), D)
    got = oa.attention_rows(qr, keys, vals, positions, 0.9)
    np.testing.assert_allclose(got, _rows_brute_force(qr, keys, vals, positions, 0.9),
                               rtol=0, atol=1e-12)


def test_attention_rows_zero_keys_prefix_mean():
    # K = 0: every allowed logit is 0, so row i is the mean of V[0..positions[i]]
    L, D = 300, 16
    vals = _rand(211, L, D)
    positions = [0, 5, 63, 64, 255, 299]
    got = oa.attention_rows(_rand(212, len(positions), D), np.zeros((L, D)), vals, positions, 0.3)
    expect = np.stack([vals[:p + 1].mean(axis=0) for p in positions])
    np.testing.assert_allclose(got, expect, rtol=0, atol=1e-12)


def test_attention_rows_selector_picks_value_row():
    # q = alpha * k[tau] over random unit keys: O equals V[tau] (closed form),
    # including tau equal to the row's own position (the inclusive diagonal)
    L, D = 500, 128
    rng = np.random.default_rng(221)
    keys = rng.standard_normal((L, D))
    keys /= np.linalg.norm(keys, axis=1, keepdims=True)
    vals = rng.standard_normal((L, D))
    positions = [0, 3, 100, 257, 499, 499]
    tau = [0, 3, 17, 257, 0, 499]
    qr = 2000.0 * keys[tau]
    got = oa.attention_rows(qr, keys, vals, positions, 1 / math.sqrt(D))
    np.testing.assert_allclose(got, vals[tau], rtol=0, atol=1e-12)

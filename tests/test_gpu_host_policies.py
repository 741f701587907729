"""The host policies end to end on the GPU: prefix caching by token digest
(config 3's shared prefix found by lookup, not shared by construction) and
preemption with recompute.  The library's scheduler and the oracle's run in
lockstep (every descriptor bit-exact), every step goes through the GPU path,
and every output is checked against the oracle."""
import math

import numpy as np
import pytest
import torch

from oracle import attention as oa
from synth import config3_suffix_lengths, draw_normal, free_block_order, get_workload
from tests.gpu_helpers import Pair, assert_close, gpu_call, need_gpu, quantize, say

pytestmark = pytest.mark.gpu


def test_config3_prefix_found_by_digest_lookup():
    """Config 3 with prefix caching on: a first request computes the
    4096-token system prompt (its 256 full blocks are registered as they are
    computed) and leaves; 16 requests with that prompt and their own
    suffixes find all 256 blocks by lookup at their first scheduling
    ("Prefill Optimisation ...", section 3, "vLLM block hash chain";
    "vLLM Chunked Prefill ...", sections 2.2 and 3.1), compute only their
    suffixes (cached_seq_len 4096) in one varlen call, and match each
    request recomputed from token 0."""
    need_gpu()
    w = get_workload("c3")
    H, G, D, bs = w.num_heads, w.num_kv_heads, w.head_dim, w.block_size
    prefix = w.prompt_len
    suffix = [int(s) for s in config3_suffix_lengths(w)]
    nb = prefix // bs + sum(-(-s // bs) for s in suffix) + 64
    max_blocks = -(-(prefix + 512) // bs)
    pair = Pair(nb, G, bs, D, "bf16", w.max_batched_tokens, max_blocks, free_block_order(nb, w.seed),
                prefix_caching=True)
    rng = np.random.default_rng(w.seed)
    system = [int(x) for x in rng.integers(0, 1 << 31, size=prefix)]
    # the request that computes the shared prompt
    kpt, kp64 = quantize(draw_normal(w.seed * 10 + 1, (prefix, G, D)), "bf16")
    vpt, vp64 = quantize(draw_normal(w.seed * 10 + 2, (prefix, G, D)), "bf16")
    qpt, qp64 = quantize(draw_normal(w.seed * 10 + 3, (prefix, H, D)), "bf16")
    pair.add_request_tokens(999, system)
    pb, ob = pair.step()
    assert list(pb["q_lens"]) == [prefix] and list(pb["cached_seq_len"]) == [0]
    say("config 3 with lookup: the shared prompt")
    out, _ = gpu_call(pair.cache, pb, qpt, kpt, vpt, w.kv_segment_size)
    ref = pair.oracle_batch(ob, qp64, kp64, vp64, w.scale, G)
    assert_close(out.to(torch.float64).numpy(), ref, "bf16", "c3 shared prompt")
    pair.commit()
    shared = list(pair.prod.request_blocks(999))
    assert shared == pair.orc._find(999).blocks and len(shared) == prefix // bs
    pair.free(999)
    assert pair.prod.pool_stats()["reclaimable"] == prefix // bs
    # the 16 requests: the same prompt, then their own tokens
    for i, s in enumerate(suffix):
        own = [int(x) for x in rng.integers(0, 1 << 31, size=s)]
        pair.add_request_tokens(i, system + own)
    pb, ob = pair.step()
    assert list(pb["cached_seq_len"]) == [prefix] * len(suffix)
    assert list(pb["q_lens"]) == suffix
    for i in range(len(suffix)):
        assert list(pb["block_table"][i][:prefix // bs]) == shared      # found by lookup
        assert pair.prod.refcount(shared[0]) == len(suffix)
    T = pb["num_tokens"]
    qs, ks, vs = [], [], []
    for i, s in enumerate(suffix):
        base = w.seed * 100000 + 10 * i
        qs.append(draw_normal(base + 3, (s, H, D)))
        ks.append(draw_normal(base + 4, (s, G, D)))
        vs.append(draw_normal(base + 5, (s, G, D)))
    qt, q64 = quantize(np.concatenate(qs), "bf16")
    kt, k64 = quantize(np.concatenate(ks), "bf16")
    vt, v64 = quantize(np.concatenate(vs), "bf16")
    say(f"config 3 with lookup: {len(suffix)} suffixes, {T} tokens")
    out, _ = gpu_call(pair.cache, pb, qt, kt, vt, w.kv_segment_size)
    got = out.to(torch.float64).numpy()
    ref = pair.oracle_batch(ob, q64, k64, v64, w.scale, G)
    assert_close(got, ref, "bf16", "c3 lookup batch vs oracle")
    # and each request recomputed from token 0 (prefix ++ suffix, no cache)
    cu = pb["cu_seqlens_q"]
    for i, s in enumerate(suffix):
        keys = np.concatenate([kp64, k64[cu[i]:cu[i + 1]]])
        vals = np.concatenate([vp64, v64[cu[i]:cu[i + 1]]])
        pos = prefix + np.arange(s)
        for h in range(H):
            g = h // (H // G)
            rec = oa.attention_rows(q64[cu[i]:cu[i + 1], h], keys[:, g], vals[:, g], pos, w.scale)
            assert_close(got[cu[i]:cu[i + 1], h], rec, "bf16", f"c3 lookup req {i} head {h}")


def test_preempted_request_recomputed_on_the_gpu():
    """"vLLM Chunked Prefill ...", section 4: a request preempted after three
    chunks of 2048 (block size 16) releases its 384 blocks and goes back to
    0 computed tokens; once the running decode leaves, it is recomputed from
    the start.  Every step (the decode rows with the chunks) runs on the GPU
    and every output matches the oracle; the recomputed prompt matches
    causal attention over the whole prompt."""
    need_gpu()
    H, G, D, bs, S = 8, 2, 128, 16, 1024
    prompt, chunk = 6656, 2048                    # 3 chunks of 2048, then 512 more
    ctx = 640                                     # the decode's 40 cached blocks
    # 440 blocks: the decode's 41 and three chunks' 384 fit, the fourth
    # chunk's 32 more do not; the whole prompt's 416 fit once the decode leaves
    nb = -(-prompt // bs) + 24
    scale = 1 / math.sqrt(D)
    rng = np.random.default_rng(4242)
    pair = Pair(nb, G, bs, D, "bf16", chunk + 1, -(-prompt // bs) + 1,
                rng.permutation(nb).astype(np.int32), preemption=True)
    pair.add_decode(1, ctx)
    kct, kc64 = quantize(rng.standard_normal((ctx, G, D)), "bf16")
    vct, vc64 = quantize(rng.standard_normal((ctx, G, D)), "bf16")
    pair.fill_context(1, kc64, vc64, kct, vct)
    pair.add_request(2, prompt)
    # the prompt's q/k/v by absolute position: a recomputed chunk sees the same values
    qpt, qp64 = quantize(rng.standard_normal((prompt, H, D)), "bf16")
    kpt, kp64 = quantize(rng.standard_normal((prompt, G, D)), "bf16")
    vpt, vp64 = quantize(rng.standard_normal((prompt, G, D)), "bf16")
    final = np.full((prompt, H, D), np.nan)
    preempted_at, freed, steps = None, False, 0
    while True:
        pb, ob = pair.step()
        steps += 1
        if pair.orc.preempted:
            assert pair.orc.preempted == [2] and preempted_at is None
            preempted_at = steps
            info = pair.prod.request_info(2)
            assert info["num_computed"] == 0 and info["num_blocks"] == 0
        rows_q, rows_k, rows_v, rows_q64, rows_k64, rows_v64, where = [], [], [], [], [], [], []
        for j, rid in enumerate(pb["req_ids"]):
            n = int(pb["q_lens"][j])
            c = int(pb["cached_seq_len"][j])
            if rid == 2:
                sl = slice(c, c + n)
                rows_q.append(qpt[sl]); rows_k.append(kpt[sl]); rows_v.append(vpt[sl])
                rows_q64.append(qp64[sl]); rows_k64.append(kp64[sl]); rows_v64.append(vp64[sl])
                where.append((int(pb["cu_seqlens_q"][j]), c, n))
            else:                                 # the decode's token of this step
                qt, q64 = quantize(rng.standard_normal((1, H, D)), "bf16")
                kt, k64 = quantize(rng.standard_normal((1, G, D)), "bf16")
                vt, v64 = quantize(rng.standard_normal((1, G, D)), "bf16")
                rows_q.append(qt); rows_k.append(kt); rows_v.append(vt)
                rows_q64.append(q64); rows_k64.append(k64); rows_v64.append(v64)
        say(f"preemption scenario step {steps}: seqs {list(pb['req_ids'])} q_lens {list(pb['q_lens'])}")
        out, _ = gpu_call(pair.cache, pb, torch.cat(rows_q), torch.cat(rows_k), torch.cat(rows_v), S)
        got = out.to(torch.float64).numpy()
        ref = pair.oracle_batch(ob, np.concatenate(rows_q64), np.concatenate(rows_k64),
                                np.concatenate(rows_v64), scale, G)
        assert_close(got, ref, "bf16", f"preemption step {steps}")
        for q0, c, n in where:
            final[c:c + n] = got[q0:q0 + n]
        pair.commit()
        if preempted_at is not None and not freed:
            pair.free(1)                          # the decode leaves: room to recompute
            freed = True
        if freed and pair.prod.request_info(2)["is_decode"]:
            break
        assert steps < 20
    assert preempted_at == 4
    # the recomputed prompt equals causal attention over the whole prompt
    for h in range(H):
        g = h // (H // G)
        rows = np.arange(0, prompt, 97)
        rec = oa.attention_rows(qp64[rows, h], kp64[:, g], vp64[:, g], rows, scale)
        assert_close(final[rows, h], rec, "bf16", f"recomputed prompt head {h}")

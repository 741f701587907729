"""GPU parity on the five workloads at their full sizes.  Configs 1-3 are
checked against the oracle on every output of every head (config 2 also
through the exact path bench.py times); configs 4 and 5 on sampled rows the
oracle computes one by one (all heads for config 4, one head of every KV
group and more for config 5), plus properties that hold at any size."""
import dataclasses
import math

import numpy as np
import pytest
import torch

from chunked_prefill_paged_amd import HostScheduler, cache_shapes
from oracle import attention as oa
from oracle import schedule as osch
from synth import (config3_suffix_lengths, config4_decode_contexts, draw_normal,
                   free_block_order, get_workload, prompt_qkv)
from tests.gpu_helpers import (DEV, GpuCache, Pair, assert_close, bits_of, gpu_call, need_gpu,
                               quantize, same_batches, say)

pytestmark = pytest.mark.gpu


def _chunked_prompt(w, S, split_pre=0, heads=None, with_oracle=True, fill=0.0):
    """Run a single prompt chunk by chunk (the scheduler picks the chunks);
    returns GPU outputs [P, H, D] (float64), oracle outputs, and the pair."""
    q32, k32, v32 = prompt_qkv(w)
    qt, q64 = quantize(q32, w.dtype)
    kt, k64 = quantize(k32, w.dtype)
    vt, v64 = quantize(v32, w.dtype)
    max_blocks = -(-w.prompt_len // w.block_size)
    order = free_block_order(w.num_blocks, w.seed)
    pair = Pair(w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim, w.dtype,
                w.max_batched_tokens, max_blocks, order, fill=fill)
    pair.add_request(0, w.prompt_len)
    outs, refs = [], []
    pos = 0
    while pos < w.prompt_len:
        pb, ob = pair.step()
        n = pb["num_tokens"]
        assert pb["cached_seq_len"][0] == pos
        out, _ = gpu_call(pair.cache, pb, qt[pos:pos + n], kt[pos:pos + n], vt[pos:pos + n], S,
                          split_pre=split_pre)
        outs.append(out.to(torch.float64).numpy())
        if with_oracle:
            refs.append(pair.oracle_batch(ob, q64[pos:pos + n], k64[pos:pos + n], v64[pos:pos + n],
                                          w.scale, w.num_kv_heads, heads=heads))
        pair.commit()
        pos += n
    return np.concatenate(outs), (np.concatenate(refs) if refs else None), pair


def test_config1_fp32_full():
    need_gpu()
    w = get_workload("c1")
    say("config 1")
    got, ref, pair = _chunked_prompt(w, w.kv_segment_size)
    assert_close(got, ref, "fp32", "c1")
    gk, gv = pair.cache.canonical_bits()
    assert np.array_equal(gk, bits_of(pair.k_pool, "fp32"))
    assert np.array_equal(gv, bits_of(pair.v_pool, "fp32"))


def test_config2_full_and_segment_sweep():
    need_gpu()
    w = get_workload("c2")
    heads = list(range(4)) + list(range(28, 32))          # KV groups 0 and 7
    say("config 2, S=1024 vs oracle, every head")
    base, ref, pair = _chunked_prompt(w, 1024)
    assert_close(base, ref, "bf16", "c2 S=1024")
    gk, gv = pair.cache.canonical_bits()
    assert np.array_equal(gk, bits_of(pair.k_pool, "bf16"))
    assert np.array_equal(gv, bits_of(pair.v_pool, "bf16"))
    # results must not depend on kv_segment_size (nor on how rows are split)
    for S in (512, 1024, 2048, 4096):
        for split in (-1, S):
            say(f"config 2 sweep S={S} split={split}")
            got, _, _ = _chunked_prompt(w, S, split_pre=split, with_oracle=False)
            assert_close(got[:, heads], ref[:, heads], "bf16", f"c2 S={S} split={split} vs oracle")
            assert_close(got, base, "bf16", f"c2 S={S} split={split} vs S=1024")


def _timed_path_every_head(w, what):
    """Run the prompt of workload w through bench.PromptBench (the path the
    bench times) and check every output of every head against the oracle
    run chunk by chunk with its own scheduler, and every cache bit.
    Returns the per-chunk plan counts."""
    import bench
    pb = bench.PromptBench(1024, 0, workload=w)
    assert pb.inline
    say(what)
    pb.step()
    torch.cuda.synchronize()
    got = pb.out.to(torch.float64).cpu().numpy()
    q32, k32, v32 = prompt_qkv(w)
    _, q64 = quantize(q32, "bf16")
    _, k64 = quantize(k32, "bf16")
    _, v64 = quantize(v32, "bf16")
    shape = (w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim)
    kp, vp = np.zeros(shape), np.zeros(shape)
    max_blocks = -(-w.prompt_len // w.block_size)
    orc = osch.Scheduler(osch.BlockPool(w.num_blocks, free_block_order(w.num_blocks, w.seed)),
                         w.block_size, w.max_batched_tokens, max_blocks)
    orc.add_request(0, w.prompt_len)
    pos = 0
    while pos < w.prompt_len:
        ob = orc.step()
        n = ob["num_tokens"]
        kp, vp = oa.cache_write(kp, vp, k64[pos:pos + n], v64[pos:pos + n], ob["block_table"],
                                ob["cu_seqlens_q"], ob["cached_seq_len"], w.block_size)
        ref = oa.attention(q64[pos:pos + n], kp, vp, ob["block_table"], ob["cu_seqlens_q"],
                           ob["cached_seq_len"], w.block_size, w.scale, w.num_kv_heads)
        assert_close(got[pos:pos + n], ref, "bf16", f"{what}: chunk at {pos}")
        orc.commit()
        pos += n
    gk = pb.k_cache.view(torch.int16).permute(0, 2, 1, 3).contiguous().cpu().numpy()
    gv = pb.v_cache.view(torch.int16).permute(0, 3, 1, 2).contiguous().cpu().numpy()
    assert np.array_equal(gk, bits_of(kp, "bf16"))
    assert np.array_equal(gv, bits_of(vp, "bf16"))
    return pb.plan


def test_config2_timed_path_every_head():
    """The exact path bench.py times: the 10k prompt through the library's
    host scheduler, the descriptor inline in the prepare launch's arguments,
    slots derived from the block table, the automatic plan (no key split at
    this size); every output of every head against the oracle, and every
    cache bit."""
    need_gpu()
    plan = _timed_path_every_head(get_workload("c2"), "config 2 through the timed path")
    assert all(p["num_merge_rows"] == 0 for p in plan)


def test_config2_tensor_parallel_share_every_head():
    """One GPU's share of the 10k prompt under an eight-way split by KV-head
    group ("Prefill Processing", section "Kernel Interface", tp_q): H 4 /
    G 1, the bench's c2tp mode.  Each chunk's 64 row tiles leave most of the
    GPU idle, so the automatic plan splits the prefill rows into key ranges
    and merges their partial states; every output against the oracle."""
    need_gpu()
    w = get_workload("c2")
    w = dataclasses.replace(w, num_heads=w.num_heads // w.num_kv_heads, num_kv_heads=1)
    plan = _timed_path_every_head(w, "config 2 at one tensor-parallel share")
    assert all(p["num_merge_rows"] > 0 for p in plan)


def test_config3_prefix_shared_blocks():
    need_gpu()
    w = get_workload("c3")
    H, G, D, bs = w.num_heads, w.num_kv_heads, w.head_dim, w.block_size
    prefix = w.prompt_len
    suffix = config3_suffix_lengths(w)
    nb = prefix // bs + int(sum(-(-s // bs) for s in suffix)) + 64
    order = free_block_order(nb, w.seed)
    max_blocks = -(-(prefix + 512) // bs)
    pair = Pair(nb, G, bs, D, "bf16", w.max_batched_tokens, max_blocks, order)
    kp32 = draw_normal(w.seed * 10 + 1, (prefix, G, D))
    vp32 = draw_normal(w.seed * 10 + 2, (prefix, G, D))
    kpt, kp64 = quantize(kp32, "bf16")
    vpt, vp64 = quantize(vp32, "bf16")
    pair.add_decode(999, prefix)               # the request that computed the prefix
    pair.fill_context(999, kp64, vp64, kpt, vpt)
    shared = pair.prod.request_blocks(999)
    assert list(shared) == pair.orc._find(999).blocks
    for i, s in enumerate(suffix):
        pair.add_request(i, prefix + int(s), shared)
    pair.free(999)
    assert all(pair.prod.refcount(int(b)) == len(suffix) for b in shared)
    pb, ob = pair.step()
    assert list(pb["cached_seq_len"]) == [prefix] * len(suffix)
    T = pb["num_tokens"]
    qs, ks, vs = [], [], []
    for i, s in enumerate(suffix):
        base = w.seed * 100000 + 10 * i
        qs.append(draw_normal(base + 3, (int(s), H, D)))
        ks.append(draw_normal(base + 4, (int(s), G, D)))
        vs.append(draw_normal(base + 5, (int(s), G, D)))
    qt, q64 = quantize(np.concatenate(qs), "bf16")
    kt, k64 = quantize(np.concatenate(ks), "bf16")
    vt, v64 = quantize(np.concatenate(vs), "bf16")
    say(f"config 3: {len(suffix)} requests, {T} tokens")
    out, _ = gpu_call(pair.cache, pb, qt, kt, vt, w.kv_segment_size)
    got = out.to(torch.float64).numpy()
    # each request recomputed from token 0 (no cache): prefix ++ suffix, logical order
    cu = pb["cu_seqlens_q"]
    for i, s in enumerate(suffix):
        keys = np.concatenate([kp64, k64[cu[i]:cu[i + 1]]])
        vals = np.concatenate([vp64, v64[cu[i]:cu[i + 1]]])
        pos = prefix + np.arange(int(s))
        for h in range(H):
            g = h // (H // G)
            ref = oa.attention_rows(q64[cu[i]:cu[i + 1], h], keys[:, g], vals[:, g], pos, w.scale)
            assert_close(got[cu[i]:cu[i + 1], h], ref, "bf16", f"c3 req {i} head {h}")


def _big_pool_pair(num_blocks, bs, budget, max_blocks, order):
    prod = HostScheduler(num_blocks, bs, budget, max_blocks, free_order=order)
    orc = osch.Scheduler(osch.BlockPool(num_blocks, order), bs, budget, max_blocks)
    return prod, orc


def _gen(seed, shape, device=DEV):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)


def test_config4_mixed_batch_sampled():
    need_gpu()
    w = get_workload("c4")
    H, G, D, bs = w.num_heads, w.num_kv_heads, w.head_dim, w.block_size
    ctx = config4_decode_contexts(w)
    pf_cached, pf_prompt = 30720, w.prompt_len
    demand = int(sum(-(-(int(c) + 1) // bs) for c in ctx)) + -(-(pf_cached + 1792) // bs)
    nb = math.ceil(1.2 * demand)
    order = free_block_order(nb, w.seed)
    prod, orc = _big_pool_pair(nb, bs, w.max_batched_tokens, pf_prompt // bs, order)
    for i, c in enumerate(ctx):
        prod.add_decode(i, int(c))
        orc.add_decode(i, int(c))
    prod.add_partial(256, pf_prompt, pf_cached)
    orc.add_partial(256, pf_prompt, pf_cached)
    pb = prod.step()
    ob = orc.step()
    same_batches(pb, ob)
    assert list(pb["q_lens"]) == [1] * 256 + [1792]
    say(f"config 4: pool {nb} blocks ({nb * bs * G * D * 4 / 1e9:.1f} GB K+V)")
    cache = GpuCache(nb, G, bs, D, "bf16")
    # cached context: per-sequence seeded draws on the device, written by the
    # library's own cache write
    lens = [int(c) for c in ctx] + [pf_cached]
    for i, L in enumerate(lens):
        kk = _gen(w.seed * 100000 + 2 * i, (L, G, D))
        vv = _gen(w.seed * 100000 + 2 * i + 1, (L, G, D))
        slots = prod.slots(i, 0, L)
        b = {"cu_seqlens_q": np.array([0, L], np.int32), "cached_seq_len": np.array([0], np.int32),
             "block_table": np.zeros((1, 1), np.int32), "slot_mapping": slots}
        gpu_call(cache, b, None, kk, vv, 0, only_cache=True)
        del kk, vv
    T = pb["num_tokens"]
    qt = _gen(w.seed * 100000 + 900001, (T, H, D))
    kt = _gen(w.seed * 100000 + 900002, (T, G, D))
    vt = _gen(w.seed * 100000 + 900003, (T, G, D))
    out, _ = gpu_call(cache, pb, qt, kt, vt, w.kv_segment_size)
    got = out.to(torch.float64).numpy()
    assert np.isfinite(got).all()
    # every decode row, all heads, bit for bit against the decodes alone: the
    # mixed plan places the prefill items among the decode items, and each
    # decode item must still run exactly once with the same partials
    dec = {"cu_seqlens_q": np.ascontiguousarray(pb["cu_seqlens_q"][:257]),
           "cached_seq_len": np.ascontiguousarray(pb["cached_seq_len"][:256]),
           "block_table": np.ascontiguousarray(pb["block_table"][:256]),
           "slot_mapping": np.ascontiguousarray(pb["slot_mapping"][:256])}
    out_dec, _ = gpu_call(cache, dec, qt[:256], kt[:256], vt[:256], w.kv_segment_size)
    assert torch.equal(out_dec, out[:256]), "decode rows differ between the mixed and the decode-only plan"
    # the step's writes, bit for bit, at the oracle's slots
    kb = cache.k.view(torch.int16)
    vb = cache.v.view(torch.int16)
    ref_slots = oa.slot_mapping(ob["block_table"], ob["cu_seqlens_q"], ob["cached_seq_len"], bs)
    sl = torch.from_numpy(ref_slots).to(DEV)
    blk, off = sl // bs, sl % bs
    k_written = kb[blk, :, off, :]                        # [T, G, D]
    v_written = vb[blk, :, :, off]                        # [T, G, D]
    assert torch.equal(k_written.cpu(), kt.cpu().view(torch.int16))
    assert torch.equal(v_written.cpu(), vt.cpu().view(torch.int16))
    q64 = qt.to(torch.float64).cpu().numpy()
    k64n = kt.to(torch.float64).cpu().numpy()
    v64n = vt.to(torch.float64).cpu().numpy()
    # sampled decode rows: 32 rows spread over the context lengths (the
    # shortest, the longest and evenly spaced ranks between)
    by_len = np.argsort(ctx, kind="stable")
    picks = sorted({int(by_len[r]) for r in np.linspace(0, len(ctx) - 1, 32).round().astype(int)})
    assert len(picks) == 32
    for i in picks:
        L = int(ctx[i])
        keys = np.concatenate([_gen(w.seed * 100000 + 2 * i, (L, G, D)).to(torch.float64).cpu().numpy(),
                               k64n[i:i + 1]])
        vals = np.concatenate([_gen(w.seed * 100000 + 2 * i + 1, (L, G, D)).to(torch.float64).cpu().numpy(),
                               v64n[i:i + 1]])
        for h in range(H):
            g = h // (H // G)
            ref = oa.attention_rows(q64[i:i + 1, h], keys[:, g], vals[:, g], [L], w.scale)
            assert_close(got[i:i + 1, h], ref, "bf16", f"c4 decode {i} (L={L}) head {h}")
    # sampled prefill rows
    kp = _gen(w.seed * 100000 + 2 * 256, (pf_cached, G, D)).to(torch.float64).cpu().numpy()
    vp = _gen(w.seed * 100000 + 2 * 256 + 1, (pf_cached, G, D)).to(torch.float64).cpu().numpy()
    keys = np.concatenate([kp, k64n[256:]])
    vals = np.concatenate([vp, v64n[256:]])
    rows = np.array([0, 1, 31, 32, 63, 64, 127, 128, 500, 777, 1023, 1024, 1400, 1663, 1790, 1791])
    for h in range(H):
        g = h // (H // G)
        ref = oa.attention_rows(q64[256 + rows, h], keys[:, g], vals[:, g], pf_cached + rows, w.scale)
        assert_close(got[256 + rows, h], ref, "bf16", f"c4 prefill head {h}")


def test_config5_long_prompt_sampled_and_monolithic():
    need_gpu()
    w = get_workload("c5")
    H, G, D, bs = w.num_heads, w.num_kv_heads, w.head_dim, w.block_size
    q32, k32, v32 = prompt_qkv(w)
    qt, _ = quantize(q32, "bf16")
    del q32
    kt, k64 = quantize(k32, "bf16")
    vt, v64 = quantize(v32, "bf16")
    P = w.prompt_len
    order = free_block_order(w.num_blocks, w.seed)
    prod, orc = _big_pool_pair(w.num_blocks, bs, w.max_batched_tokens, P // bs, order)
    prod.add_request(0, P)
    orc.add_request(0, P)
    cache = GpuCache(w.num_blocks, G, bs, D, "bf16")
    outs = []
    pos = 0
    while pos < P:
        pb = prod.step()
        ob = orc.step()
        same_batches(pb, ob)
        n = pb["num_tokens"]
        assert n == 2048 and pb["cached_seq_len"][0] == pos
        say(f"config 5 chunk at {pos}")
        out, _ = gpu_call(cache, pb, qt[pos:pos + n], kt[pos:pos + n], vt[pos:pos + n],
                          w.kv_segment_size)
        outs.append(out)
        prod.commit()
        orc.commit()
        pos += n
    chunked = torch.cat(outs)
    # sampled rows against the oracle, at every chunk
    got = chunked.to(torch.float64).numpy()
    for c0 in range(0, P, 2048):
        rows = c0 + np.array([0, 1, 31, 32, 63, 64, 255, 256, 777, 1023, 1024, 1500, 1983, 2000,
                              2046, 2047])
        q64 = qt[rows].to(torch.float64).numpy()
        for h in (0, 7, 8, 17, 26, 33, 42, 51, 60, 63):
            g = h // (H // G)
            ref = oa.attention_rows(q64[:, h], k64[:, g], v64[:, g], rows, w.scale)
            assert_close(got[rows, h], ref, "bf16", f"c5 rows {rows.tolist()} head {h}")
    # monolithic 32k causal prefill (one call, nothing cached) gives the same rows
    mono_pool = GpuCache(w.num_blocks, G, bs, D, "bf16")
    b = {"cu_seqlens_q": np.array([0, P], np.int32), "cached_seq_len": np.array([0], np.int32),
         "block_table": np.arange(P // bs, dtype=np.int32)[None, :],
         "slot_mapping": np.arange(P, dtype=np.int64)}
    mono, _ = gpu_call(mono_pool, b, qt, kt, vt, w.kv_segment_size)
    assert_close(mono.to(torch.float64).numpy(), got, "bf16", "c5 monolithic vs chunked")

"""GPU parity on small and ragged batches: every output element against the
oracle, every cache byte against the oracle's expected pool."""
import math

import numpy as np
import pytest
import torch

from chunked_prefill_paged_amd import AttnCall
from oracle import attention as oa

from tests.gpu_helpers import (DEV, Pair, assert_close, bits_of, gpu_call, need_gpu, quantize,
                               say)

pytestmark = pytest.mark.gpu

# name, dtype, H, G, D, bs, S, partial requests [(prompt, computed)], decodes [ctx], budget
CASES = [
    ("c0_single", "bf16", 8, 2, 128, 16, 512, [(300, 0)], [], 4096),
    ("ragged_multi", "bf16", 32, 8, 128, 16, 1024, [(1500, 1000), (17, 0), (600, 511), (2100, 2048)],
     [], 8192),
    ("hpg1_d64", "bf16", 4, 4, 64, 8, 512, [(700, 300), (129, 64)], [], 4096),
    ("hpg8", "bf16", 64, 8, 128, 16, 512, [(900, 700)], [], 4096),
    ("bs128", "bf16", 32, 8, 128, 128, 1024, [(3000, 2048), (130, 0)], [], 4096),
    ("fp32_c1like", "fp32", 4, 4, 64, 16, 512, [(1024, 768)], [], 256),
    ("fp32_hpg2", "fp32", 8, 4, 64, 32, 512, [(400, 111), (65, 0)], [], 4096),
    ("mixed_decodes", "bf16", 32, 8, 128, 16, 512, [(1300, 1024)], [1, 15, 16, 17, 600, 1111, 2049],
     8192),
    ("tiny_rows", "bf16", 32, 8, 128, 16, 512, [(2, 1), (1, 0), (64, 63)], [], 4096),
    # head groups that do not divide a 32-row wave block or a 128-row item,
    # block sizes at and past the 64-key tile and the largest one
    ("hpg3_bs64", "bf16", 24, 8, 128, 64, 1024, [(777, 640), (100, 0)], [5, 300], 4096),
    ("hpg6_bs256", "bf16", 48, 8, 128, 256, 1024, [(1000, 512), (300, 0)], [2000], 4096),
    ("hpg5_d64_bs512", "bf16", 10, 2, 64, 512, 1024, [(1500, 1024)], [700], 4096),
    ("fp32_hpg3", "fp32", 6, 2, 64, 16, 512, [(300, 200)], [40], 4096),
]
SPLITS = {"auto": (0, 0), "never": (-1, -1), "seg": ("S", "S"), "seg2": ("2S", "S")}


def _resolve(v, S):
    return {"S": S, "2S": 2 * S}.get(v, v)


def run_case(case, split, fill=0.0, seed=0, derive_slots=False, inline_desc=False, scale=None):
    name, dtype, H, G, D, bs, S, reqs, decodes, budget = case
    rng = np.random.default_rng(1000 + seed)
    max_blocks = max(-(-(p + 1) // bs) for p, _ in reqs + [(c + 1, 0) for c in decodes]) + 1
    need = sum(-(-p // bs) for p, _ in reqs) + sum(-(-(c + 1) // bs) for c in decodes)
    nb = need + 37
    order = rng.permutation(nb).astype(np.int32)
    pair = Pair(nb, G, bs, D, dtype, budget, max_blocks, order, fill=fill)
    rid = 0
    for ctx in decodes:
        pair.add_decode(rid, ctx)
        k64 = rng.standard_normal((ctx, G, D)).astype(np.float32)
        v64 = rng.standard_normal((ctx, G, D)).astype(np.float32)
        kt, kq = quantize(k64, dtype)
        vt, vq = quantize(v64, dtype)
        pair.fill_context(rid, kq, vq, kt, vt)
        rid += 1
    for prompt, computed in reqs:
        pair.add_partial(rid, prompt, computed)
        if computed:
            kt, kq = quantize(rng.standard_normal((computed, G, D)), dtype)
            vt, vq = quantize(rng.standard_normal((computed, G, D)), dtype)
            pair.fill_context(rid, kq, vq, kt, vt)
        rid += 1
    pb, ob = pair.step()
    T = pb["num_tokens"]
    qt, q64 = quantize(rng.standard_normal((T, H, D)), dtype)
    kt, k64 = quantize(rng.standard_normal((T, G, D)), dtype)
    vt, v64 = quantize(rng.standard_normal((T, G, D)), dtype)
    sp, sd = (_resolve(x, S) for x in SPLITS[split])
    say(f"case {name} split={split} T={T} seqs={pb['num_seqs']}")
    scale = 1 / math.sqrt(D) if scale is None else scale
    out, _ = gpu_call(pair.cache, pb, qt, kt, vt, S, split_pre=sp, split_dec=sd, scale=scale,
                      derive_slots=derive_slots, inline_desc=inline_desc, attention_twice=inline_desc)
    ref = pair.oracle_batch(ob, q64, k64, v64, scale, G)
    return pair, out, ref, dtype


@pytest.mark.parametrize("split", list(SPLITS))
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_small_batches_match_oracle(case, split):
    need_gpu()
    pair, out, ref, dtype = run_case(case, split)
    assert_close(out.to(torch.float64).numpy(), ref, dtype, f"{case[0]}/{split}")
    # every cache byte: written slots hold the new rows, all others untouched
    gk, gv = pair.cache.canonical_bits()
    assert np.array_equal(gk, bits_of(pair.k_pool, dtype))
    assert np.array_equal(gv, bits_of(pair.v_pool, dtype))


@pytest.mark.parametrize("case", [CASES[1], CASES[6], CASES[7], CASES[8]],
                         ids=["ragged", "fp32", "decodes", "tiny"])
def test_slots_derived_from_the_block_table(case):
    # no slot mapping passed: the cache write derives each token's slot from
    # cu_seqlens_q, cached_seq_len and the block table; same bytes, same outputs
    need_gpu()
    pair, out, ref, dtype = run_case(case, "auto", derive_slots=True)
    assert_close(out.to(torch.float64).numpy(), ref, dtype, f"{case[0]}/derived slots")
    gk, gv = pair.cache.canonical_bits()
    assert np.array_equal(gk, bits_of(pair.k_pool, dtype))
    assert np.array_equal(gv, bits_of(pair.v_pool, dtype))


@pytest.mark.parametrize("split", ["auto", "seg2"])
@pytest.mark.parametrize("case", [CASES[1], CASES[6], CASES[8], CASES[9], CASES[10]],
                         ids=["ragged", "fp32", "tiny", "hpg3_bs64", "hpg6_bs256"])
def test_inline_descriptor_matches_oracle(case, split):
    """The descriptor passed as host copies only (kernel arguments of the
    prepare launch, a workspace copy for the attention launch), with slots
    derived from the block table; the attention launch run twice on the one
    prepared workspace gives the same bits."""
    need_gpu()
    pair, out, ref, dtype = run_case(case, split, derive_slots=True, inline_desc=True)
    assert_close(out.to(torch.float64).numpy(), ref, dtype, f"{case[0]}/{split}/inline")
    gk, gv = pair.cache.canonical_bits()
    assert np.array_equal(gk, bits_of(pair.k_pool, dtype))
    assert np.array_equal(gv, bits_of(pair.v_pool, dtype))


@pytest.mark.parametrize("split", ["auto", "seg"])
@pytest.mark.parametrize("case", [CASES[1], CASES[4], CASES[7], CASES[9]],
                         ids=["ragged", "bs128", "decodes", "hpg3_bs64"])
def test_peaked_softmax_stress(case, split):
    """Q, K ~ N(0, 1) with softmax scale 1: logits have a spread of about
    sqrt(D) = 11, so a row's weight sits on a few keys and the running
    maximum moves often; the output stays within the bf16 tolerance."""
    need_gpu()
    pair, out, ref, dtype = run_case(case, split, scale=1.0)
    err = assert_close(out.to(torch.float64).numpy(), ref, dtype, f"{case[0]}/{split}/scale 1")
    say(f"stress {case[0]}/{split}: max-abs {err[0]:.3g} mean-abs {err[1]:.3g}")


@pytest.mark.parametrize("case", [CASES[1], CASES[7], CASES[6]], ids=["ragged", "decodes", "fp32"])
def test_stale_nan_slots_never_leak(case):
    # every slot not written so far is NaN: unreferenced blocks and the unused
    # tail of each sequence's last block
    need_gpu()
    pair, out, ref, dtype = run_case(case, "seg", fill=float("nan"))
    assert_close(out.to(torch.float64).numpy(), ref, dtype, f"{case[0]}/nan")


def test_selector_queries_select_exact_value_rows():
    """Bit-exact check of every index path through attention: q = alpha*k[tau]
    with unit keys gives a logit margin above 100, so P rounds to one-hot and
    out[t, h] must equal V[tau] bit for bit."""
    need_gpu()
    H, G, D, bs, S = 32, 8, 128, 16, 1024
    rng = np.random.default_rng(7)
    computed, n = 3000, 700
    L = computed + n
    k = rng.standard_normal((L, G, D))
    k /= np.linalg.norm(k, axis=2, keepdims=True)
    kt, k64 = quantize(k, "bf16")
    vt, v64 = quantize(rng.standard_normal((L, G, D)), "bf16")
    nb = -(-L // bs) + 20
    pair = Pair(nb, G, bs, D, "bf16", 4096, -(-L // bs) + 1, rng.permutation(nb).astype(np.int32))
    pair.add_partial(0, L, computed)
    pair.fill_context(0, k64[:computed], v64[:computed], kt[:computed], vt[:computed])
    pb, ob = pair.step()
    tau = np.zeros((n, H), dtype=np.int64)
    for t in range(n):
        for h in range(H):
            tau[t, h] = (t * 7919 + h * 104729) % (computed + t + 1)
    # make sure every block of the sequence is picked by some (token, head)
    pinned = set()
    for i in range(-(-L // bs)):
        p = min(i * bs + i % bs, L - 1)
        t, h = max(i, p - computed), i % H
        while (t, h) in pinned:
            h = (h + 1) % H
            t = t + 1 if h == i % H else t
        pinned.add((t, h))
        tau[t, h] = p
    q = np.zeros((n, H, D))
    for t in range(n):
        for h in range(H):
            q[t, h] = 2000.0 * k64[tau[t, h], h // (H // G)]
    qt, _ = quantize(q, "bf16")
    out, _ = gpu_call(pair.cache, pb, qt, kt[computed:], vt[computed:], S)
    got = out.view(torch.int16).numpy()
    want = vt.view(torch.int16).numpy()
    for h in range(H):
        assert np.array_equal(got[:, h], want[tau[:, h], h // (H // G)]), f"head {h}"
    # every physical block of the sequence was selected at least once
    rows = ob["block_table"][0]
    hit = {rows[p // bs] for p in np.unique(tau)}
    assert len(hit) == -(-L // bs)


@pytest.mark.parametrize("split", [-1, 512], ids=["unsplit", "split512"])
def test_growing_scores_move_the_reference(split):
    """Scores that climb along the keys, by a slow ramp and by jumps placed at
    key offsets 5, 20, 35, 40, 55 and 60 of their 64-key tiles (both 32-key
    blocks, whose exp sums the kernel checks one block at a time, with jumps
    in each 16-key half of them), so that the running reference of the
    online softmax moves many times per row and in every block where the
    kernel may move it."""
    need_gpu()
    H, G, D, bs, S = 32, 8, 128, 16, 512
    rng = np.random.default_rng(11)
    computed, n = 2000, 600
    L = computed + n
    u = rng.standard_normal((G, D))
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    jumps = [64 * m + r for m, r in ((4, 5), (11, 40), (17, 55), (23, 20), (32, 60), (37, 35))]
    ramp = 0.01 * np.arange(L) + 8.0 * np.searchsorted(jumps, np.arange(L), side="right")
    k = 0.5 * rng.standard_normal((L, G, D)) + ramp[:, None, None] * u[None]
    kt, k64 = quantize(k, "bf16")
    vt, v64 = quantize(rng.standard_normal((L, G, D)), "bf16")
    nb = -(-L // bs) + 20
    pair = Pair(nb, G, bs, D, "bf16", 4096, -(-L // bs) + 1, rng.permutation(nb).astype(np.int32))
    pair.add_partial(0, L, computed)
    pair.fill_context(0, k64[:computed], v64[:computed], kt[:computed], vt[:computed])
    pb, ob = pair.step()
    alpha = rng.uniform(8.0, 14.0, H)
    q = 0.3 * rng.standard_normal((n, H, D)) + alpha[None, :, None] * u[np.arange(H) // (H // G)][None]
    qt, q64 = quantize(q, "bf16")
    say(f"growing scores split={split}")
    out, _ = gpu_call(pair.cache, pb, qt, kt[computed:], vt[computed:], S, split_pre=split)
    ref = pair.oracle_batch(ob, q64, k64[computed:], v64[computed:], 1 / math.sqrt(D), G)
    assert_close(out.to(torch.float64).numpy(), ref, "bf16", f"growing/{split}")


def test_timed_attention_matches_and_times_the_kernel():
    """cpa_attention_timed: the same output bits as cpa_attention, and a
    positive elapsed time between the two events its dispatch takes."""
    need_gpu()
    import bench
    H, G, D, bs, S = 32, 8, 128, 16, 512
    rng = np.random.default_rng(5)
    pair = Pair(200, G, bs, D, "bf16", 4096, 120, rng.permutation(200).astype(np.int32))
    pair.add_partial(0, 1500, 1000)
    kt, k64 = quantize(rng.standard_normal((1000, G, D)), "bf16")
    vt, v64 = quantize(rng.standard_normal((1000, G, D)), "bf16")
    pair.fill_context(0, k64, v64, kt, vt)
    pb, ob = pair.step()
    qt, _ = quantize(rng.standard_normal((500, H, D)), "bf16")
    kn, _ = quantize(rng.standard_normal((500, G, D)), "bf16")
    vn, _ = quantize(rng.standard_normal((500, G, D)), "bf16")
    out, _ = gpu_call(pair.cache, pb, qt, kn, vn, S)
    q, k, v = qt.to(DEV), kn.to(DEV), vn.to(DEV)
    out2 = torch.full_like(q, float("nan"))
    call = AttnCall(q=q, k_new=k, v_new=v, k_cache=pair.cache.k, v_cache=pair.cache.v, out=out2,
                    cu_seqlens_q=None, cached_seq_len=None, block_table=None, slot_mapping=None,
                    h_cu_seqlens_q=pb["cu_seqlens_q"], h_cached_seq_len=pb["cached_seq_len"],
                    h_block_table=pb["block_table"], kv_segment_size=S)
    call.set_workspace(torch.empty(call.workspace_bytes(), dtype=torch.uint8, device=DEV))
    hip = bench.HipEvents()
    e0, e1 = hip.create(), hip.create()
    call.prepare()
    call.attention_timed(e0, e1)
    torch.cuda.synchronize()
    ms = hip.elapsed_ms(e0, e1)
    hip.destroy(e0)
    hip.destroy(e1)
    assert ms > 0.0
    assert torch.equal(out2.cpu().view(torch.int16), out.view(torch.int16))


def test_empty_sequence_in_batch_and_lse():
    """A batch with a zero-length sequence between two real ones; the optional
    log-sum-exp output matches the closed form for K = 0 (log of the number of
    visible keys), unsplit and split at 512 keys (which goes through the merge)."""
    need_gpu()
    H, G, D, bs, S = 8, 2, 128, 16, 512
    rng = np.random.default_rng(3)
    pair = Pair(80, G, bs, D, "bf16", 4096, 60, rng.permutation(80).astype(np.int32))
    pair.add_partial(0, 800, 600)
    kz = torch.zeros((600, G, D), dtype=torch.bfloat16)
    pair.fill_context(0, np.zeros((600, G, D)), np.zeros((600, G, D)), kz, kz)
    pair.add_partial(1, 50, 0)
    pb, ob = pair.step()
    # insert an empty sequence by hand (same slots; cu repeats an offset)
    batch = dict(pb)
    batch["cu_seqlens_q"] = np.array([0, 200, 200, 250], np.int32)
    batch["cached_seq_len"] = np.array([600, 0, 0], np.int32)
    batch["block_table"] = np.stack([pb["block_table"][0], pb["block_table"][1], pb["block_table"][1]])
    T = 250
    qt, _ = quantize(rng.standard_normal((T, H, D)), "bf16")
    kt = torch.zeros((T, G, D), dtype=torch.bfloat16)
    vt, v64 = quantize(rng.standard_normal((T, G, D)), "bf16")
    for sp in (-1, 512):
        out, lse = gpu_call(pair.cache, batch, qt, kt, vt, S, want_lse=True, split_pre=sp)
        visible = np.concatenate([600 + np.arange(1, 201), np.arange(1, 51)])
        np.testing.assert_allclose(lse.numpy(), np.log(visible)[None, :].repeat(H, 0), rtol=0, atol=1e-5)
        # K = 0: output is the running mean of V over the visible positions
        ctx_v = np.zeros((600, G, D))
        seq0 = np.concatenate([ctx_v, v64[:200]])
        mean0 = np.cumsum(seq0, axis=0)[600:] / np.arange(601, 801)[:, None, None]
        mean1 = np.cumsum(v64[200:], axis=0) / np.arange(1, 51)[:, None, None]
        want = np.concatenate([mean0, mean1])
        got = out.to(torch.float64).numpy()
        for h in range(H):
            assert np.abs(got[:, h] - want[:, h // (H // G)]).max() <= 2e-2


def test_largest_batch_in_one_call():
    """The largest batch one call takes (4096 sequences): 4095 decodes over
    contexts of 1..700 keys (one or two key segments each, so many rows
    merge) and one 1700-token chunk at cached 300, whose prefill items the
    plan spreads in runs among the decode items; every output element
    against the oracle."""
    need_gpu()
    H, G, D, bs, S, dtype = 8, 2, 64, 16, 512, "bf16"
    rng = np.random.default_rng(4096)
    ctx = rng.integers(1, 701, size=4095)
    prompt, computed = 2000, 300
    lens = [int(c) for c in ctx] + [computed]
    max_blocks = -(-(prompt + 1) // bs) + 1
    nb = sum(-(-(L + 1) // bs) for L in ctx) + -(-prompt // bs) + 41
    pair = Pair(nb, G, bs, D, dtype, 8192, max_blocks, rng.permutation(nb).astype(np.int32))
    for i, c in enumerate(ctx):
        pair.add_decode(i, int(c))
    pair.add_partial(4095, prompt, computed)
    # every sequence's context in one cache-write call, and once into the
    # oracle's pools
    tot = sum(lens)
    kt, k64 = quantize(rng.standard_normal((tot, G, D)), dtype)
    vt, v64 = quantize(rng.standard_normal((tot, G, D)), dtype)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    slots = np.concatenate([pair.prod.slots(r, 0, L) for r, L in enumerate(lens)])
    batch = {"cu_seqlens_q": cu, "cached_seq_len": np.zeros(len(lens), np.int32),
             "block_table": np.zeros((len(lens), 1), np.int32), "slot_mapping": slots}
    gpu_call(pair.cache, batch, None, kt, vt, 0, only_cache=True)
    blocks = [pair.orc._find(r).blocks for r in range(len(lens))]
    pair.k_pool, pair.v_pool = oa.cache_write(pair.k_pool, pair.v_pool, k64, v64, blocks, cu,
                                              np.zeros(len(lens), np.int32), bs)
    pb, ob = pair.step()
    assert pb["num_seqs"] == 4096
    T = pb["num_tokens"]
    qt, q64 = quantize(rng.standard_normal((T, H, D)), dtype)
    kt, k64 = quantize(rng.standard_normal((T, G, D)), dtype)
    vt, v64 = quantize(rng.standard_normal((T, G, D)), dtype)
    say(f"largest batch: {pb['num_seqs']} sequences, T={T}, pool {nb} blocks")
    scale = 1 / math.sqrt(D)
    out, _ = gpu_call(pair.cache, pb, qt, kt, vt, S, scale=scale)
    ref = pair.oracle_batch(ob, q64, k64, v64, scale, G)
    assert_close(out.to(torch.float64).numpy(), ref, dtype, "largest batch")

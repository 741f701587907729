"""GPU parity of the rotary-embedding entry points: rotated queries and the
cache of rotated keys against the RoPE oracle, and the attention of a whole
rotary chunk step against the oracle's attention over the same rotated
inputs."""
import math

import numpy as np
import pytest
import torch

from chunked_prefill_paged_amd import AttnCall
from chunked_prefill_paged_amd.attention import Rope
from oracle import attention as oa
from oracle import rope as orope
from tests.gpu_helpers import DEV, GpuCache, Pair, assert_close, need_gpu, quantize, say

pytestmark = pytest.mark.gpu

# name, dtype, H, G, D, bs, S, partial requests [(prompt, computed)], decodes [ctx], budget
CASES = [
    ("single", "bf16", 8, 2, 128, 16, 512, [(300, 0)], [], 4096),
    ("ragged_multi", "bf16", 32, 8, 128, 16, 1024, [(1500, 1000), (17, 0), (600, 511), (2100, 2048)],
     [], 8192),
    ("hpg1_d64", "bf16", 4, 4, 64, 8, 512, [(700, 300), (129, 64)], [], 4096),
    ("bs128", "bf16", 32, 8, 128, 128, 1024, [(3000, 2048), (130, 0)], [], 4096),
    ("fp32_d64", "fp32", 8, 4, 64, 32, 512, [(400, 111), (65, 0)], [], 4096),
    ("mixed_decodes", "bf16", 32, 8, 128, 16, 512, [(1300, 1024)], [1, 15, 16, 17, 600, 1111, 2049],
     8192),
]
# per-element bound on |gpu - exact|: rounding to the element type (half an
# ulp, at most 2^-8 of the value in bf16, 2^-24 in fp32) plus float
# arithmetic on inputs of size ~1 (a few 2^-24)
REL = {"bf16": 2.0 ** -8, "fp32": 2.0 ** -22}
ABS = 4e-6


def assert_rotated(got, ref, dtype, where):
    got = np.asarray(got, dtype=np.float64)
    bound = REL[dtype] * np.abs(ref) + ABS
    err = np.abs(got - ref)
    bad = err > bound
    assert not bad.any(), f"{where}: {int(bad.sum())} elements off, worst {err[bad].max():.3g}"


def _dev(a, dt):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=dt)).to(DEV)


def _call(cache, batch, qd, kd, vd, S, derive_slots, out=None, inline_desc=False):
    if inline_desc:      # host copies only: the descriptor rides in the launch arguments
        desc = dict(cu_seqlens_q=None, cached_seq_len=None, block_table=None,
                    h_block_table=np.asarray(batch["block_table"], np.int32))
    else:
        desc = dict(cu_seqlens_q=_dev(batch["cu_seqlens_q"], np.int32),
                    cached_seq_len=_dev(batch["cached_seq_len"], np.int32),
                    block_table=_dev(batch["block_table"], np.int32))
    return AttnCall(q=qd, k_new=kd, v_new=vd, k_cache=cache.k, v_cache=cache.v,
                    out=out if out is not None else torch.empty_like(qd), **desc,
                    slot_mapping=None if derive_slots else _dev(batch["slot_mapping"], np.int64),
                    h_cu_seqlens_q=batch["cu_seqlens_q"], h_cached_seq_len=batch["cached_seq_len"],
                    kv_segment_size=S)


def _setup(case, seed):
    name, dtype, H, G, D, bs, S, reqs, decodes, budget = case
    rng = np.random.default_rng(4000 + seed)
    max_blocks = max(-(-(p + 1) // bs) for p, _ in reqs + [(c + 1, 0) for c in decodes]) + 1
    need = sum(-(-p // bs) for p, _ in reqs) + sum(-(-(c + 1) // bs) for c in decodes)
    nb = need + 29
    pair = Pair(nb, G, bs, D, dtype, budget, max_blocks, rng.permutation(nb).astype(np.int32))
    rid = 0
    for ctx in decodes:
        pair.add_decode(rid, ctx)
        kt, kq = quantize(rng.standard_normal((ctx, G, D)), dtype)
        vt, vq = quantize(rng.standard_normal((ctx, G, D)), dtype)
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
    return pair, pb, ob, (qt, q64), (kt, k64), (vt, v64)


@pytest.mark.parametrize("derive_slots", [False, True], ids=["slots", "derived"])
@pytest.mark.parametrize("interleaved", [False, True], ids=["half", "interleaved"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_rotated_queries_and_cache_match_oracle(case, interleaved, derive_slots):
    need_gpu()
    name, dtype, H, G, D, bs, S = case[:7]
    theta = 10000.0 if D == 128 else 500000.0
    pair, pb, ob, (qt, q64), (kt, k64), (vt, v64) = _setup(case, 0)
    say(f"rope {name} interleaved={interleaved} derived={derive_slots} T={pb['num_tokens']}")
    qd, kd, vd = qt.to(DEV), kt.to(DEV), vt.to(DEV)
    q_out = torch.full_like(qd, float("nan"))
    call = _call(pair.cache, pb, qd, kd, vd, S, derive_slots)
    call.rope_reshape_and_cache(Rope(q_out, theta, interleaved))
    torch.cuda.synchronize()
    q_rot, k_pool, v_pool = orope.rope_cache_write(q64, pair.k_pool, pair.v_pool, k64, v64,
                                                   ob["block_table"], ob["cu_seqlens_q"],
                                                   ob["cached_seq_len"], bs, theta, interleaved)
    assert_rotated(q_out.to(torch.float64).cpu().numpy(), q_rot, dtype, f"{name} q_out")
    gk, gv = pair.cache.canonical()
    # slots this call wrote: rotated keys; every other slot: unchanged, bit for bit
    written = np.zeros(gk.shape[:2], dtype=bool)
    sl = np.asarray(pb["slot_mapping"])
    written[sl // bs, sl % bs] = True
    assert_rotated(gk[written], k_pool[written], dtype, f"{name} k_cache")
    assert np.array_equal(gk[~written], k_pool[~written])
    assert np.array_equal(gv, v_pool)
    # the input queries were not touched
    assert torch.equal(qd.cpu(), qt)


_STEP = [(1, False), (2, False), (4, False), (5, False), (1, True), (2, True), (4, True)]


@pytest.mark.parametrize("case,inline_desc", [(CASES[i], il) for i, il in _STEP],
                         ids=[CASES[i][0] + ("/inline" if il else "") for i, il in _STEP])
def test_rotary_chunk_step_matches_oracle_attention(case, inline_desc):
    need_gpu()
    name, dtype, H, G, D, bs, S = case[:7]
    theta = 10000.0
    pair, pb, ob, (qt, q64), (kt, k64), (vt, v64) = _setup(case, 1)
    say(f"rope step {name} T={pb['num_tokens']}")
    qd = qt.to(DEV)
    q_out = torch.empty_like(qd)
    out = torch.full_like(qd, float("nan"))
    call = _call(pair.cache, pb, qd, kt.to(DEV), vt.to(DEV), S, derive_slots=True, out=out,
                 inline_desc=inline_desc)
    ws = torch.empty(max(256, call.workspace_bytes()), dtype=torch.uint8, device=DEV)
    call.set_workspace(ws)
    call.rope_call(Rope(q_out, theta))
    torch.cuda.synchronize()
    # the oracle attends over the rotated queries and keys as stored, i.e.
    # rounded to the element type of the cache and of q_out
    pos = orope.token_positions(ob["cu_seqlens_q"], ob["cached_seq_len"])
    _, q_r = quantize(orope.rotate(q64, pos, theta), dtype)
    _, k_r = quantize(orope.rotate(k64, pos, theta), dtype)
    k_pool, v_pool = oa.cache_write(pair.k_pool, pair.v_pool, k_r, v64, ob["block_table"],
                                    ob["cu_seqlens_q"], ob["cached_seq_len"], bs)
    ref = oa.attention(q_r, k_pool, v_pool, ob["block_table"], ob["cu_seqlens_q"],
                       ob["cached_seq_len"], bs, 1 / math.sqrt(D), G)
    assert_close(out.to(torch.float64).cpu().numpy(), ref, dtype, f"rope step {name}")


def test_rotation_in_place_equals_out_of_place():
    need_gpu()
    case = CASES[1]
    name, dtype, H, G, D, bs, S = case[:7]
    pair, pb, ob, (qt, q64), (kt, k64), (vt, v64) = _setup(case, 2)
    kd, vd = kt.to(DEV), vt.to(DEV)
    q_sep = torch.empty(qt.shape, dtype=qt.dtype, device=DEV)
    call = _call(pair.cache, pb, qt.to(DEV), kd, vd, S, derive_slots=True)
    call.rope_reshape_and_cache(Rope(q_sep, 10000.0))
    q_in = qt.to(DEV)
    call2 = _call(pair.cache, pb, q_in, kd, vd, S, derive_slots=True)
    call2.rope_reshape_and_cache(Rope(q_in, 10000.0))
    torch.cuda.synchronize()
    assert torch.equal(q_in.cpu(), q_sep.cpu())


@pytest.mark.parametrize("interleaved", [False, True], ids=["half", "interleaved"])
def test_long_prompt_positions(interleaved):
    """The last 2048-token chunk of a 32,768-token prompt (cached 30,720;
    H64/G8/D128, bs16): angles up to ~32,767 rad, every rotated element
    checked."""
    need_gpu()
    H, G, D, bs, T, c = 64, 8, 128, 16, 2048, 30720
    nb = (c + T) // bs
    rng = np.random.default_rng(77)
    table = rng.permutation(nb).astype(np.int32)[None, :]
    say(f"rope long prompt interleaved={interleaved}")
    qt, q64 = quantize(rng.standard_normal((T, H, D)), "bf16")
    kt, k64 = quantize(rng.standard_normal((T, G, D)), "bf16")
    vt, v64 = quantize(rng.standard_normal((T, G, D)), "bf16")
    cache = GpuCache(nb, G, bs, D, "bf16")
    batch = {"cu_seqlens_q": np.array([0, T], np.int32), "cached_seq_len": np.array([c], np.int32),
             "block_table": table, "slot_mapping": None}
    q_out = torch.empty(qt.shape, dtype=qt.dtype, device=DEV)
    call = _call(cache, batch, qt.to(DEV), kt.to(DEV), vt.to(DEV), 4096, derive_slots=True)
    call.rope_reshape_and_cache(Rope(q_out, 10000.0, interleaved))
    torch.cuda.synchronize()
    pos = c + np.arange(T)
    assert_rotated(q_out.to(torch.float64).cpu().numpy(), orope.rotate(q64, pos, 10000.0, interleaved),
                   "bf16", "long q_out")
    # keys of positions c .. c+T-1 read back through the table
    gk = cache.k.permute(0, 2, 1, 3)[torch.from_numpy(table[0][pos // bs]).long().to(DEV),
                                     torch.from_numpy(pos % bs).long().to(DEV)]
    assert_rotated(gk.to(torch.float64).cpu().numpy(), orope.rotate(k64, pos, 10000.0, interleaved),
                   "bf16", "long k_cache")

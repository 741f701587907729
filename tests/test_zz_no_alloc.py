"""The entry point that allocates nothing (cpa_chunked_prefill_attn_noalloc):
its output against the workspace entry point's (cpa_chunked_prefill_attn) on
the same inputs, and both against the oracle, on two calls in a row, the
second smaller.  Both calls put partial states (split decode rows) into the
library's scratch."""
import math

import numpy as np
import pytest
import torch

from chunked_prefill_paged_amd import AttnCall
from tests.gpu_helpers import DEV, Pair, _dev, assert_close, need_gpu, quantize, say

pytestmark = pytest.mark.gpu


def _batch(seed, H, G, D, bs, S, reqs, decodes, budget):
    rng = np.random.default_rng(seed)
    max_blocks = max(-(-(p + 1) // bs) for p, _ in reqs + [(c + 1, 0) for c in decodes]) + 1
    need = sum(-(-p // bs) for p, _ in reqs) + sum(-(-(c + 1) // bs) for c in decodes)
    nb = need + 19
    pair = Pair(nb, G, bs, D, "bf16", budget, max_blocks, rng.permutation(nb).astype(np.int32))
    rid = 0
    for ctx in decodes:
        pair.add_decode(rid, ctx)
        kt, kq = quantize(rng.standard_normal((ctx, G, D)), "bf16")
        vt, vq = quantize(rng.standard_normal((ctx, G, D)), "bf16")
        pair.fill_context(rid, kq, vq, kt, vt)
        rid += 1
    for prompt, computed in reqs:
        pair.add_partial(rid, prompt, computed)
        if computed:
            kt, kq = quantize(rng.standard_normal((computed, G, D)), "bf16")
            vt, vq = quantize(rng.standard_normal((computed, G, D)), "bf16")
            pair.fill_context(rid, kq, vq, kt, vt)
        rid += 1
    pb, ob = pair.step()
    T = pb["num_tokens"]
    qt, q64 = quantize(rng.standard_normal((T, H, D)), "bf16")
    kt, k64 = quantize(rng.standard_normal((T, G, D)), "bf16")
    vt, v64 = quantize(rng.standard_normal((T, G, D)), "bf16")
    ref = pair.oracle_batch(ob, q64, k64, v64, 1 / math.sqrt(D), G)
    return pair, pb, (qt, kt, vt), ref


def _call(pair, pb, qkv, S, out):
    q, k, v = (x.to(DEV) for x in qkv)
    return AttnCall(q=q, k_new=k, v_new=v, k_cache=pair.cache.k, v_cache=pair.cache.v, out=out,
                    cu_seqlens_q=_dev(pb["cu_seqlens_q"], np.int32),
                    cached_seq_len=_dev(pb["cached_seq_len"], np.int32),
                    block_table=_dev(pb["block_table"], np.int32),
                    slot_mapping=_dev(pb["slot_mapping"], np.int64),
                    h_cu_seqlens_q=pb["cu_seqlens_q"], h_cached_seq_len=pb["cached_seq_len"],
                    kv_segment_size=S, split_keys_decode=S)


# (H, G, D, bs, S, prefill requests [(prompt, computed)], decode contexts, budget)
BIG = (32, 8, 128, 16, 512, [(1500, 1000), (300, 0)], [700, 1600, 2100, 33, 4000], 8192)
SMALL = (16, 4, 128, 16, 512, [(200, 100)], [520, 9], 4096)


def test_no_alloc_entry_point_matches_workspace_entry_point():
    need_gpu()
    for i, case in enumerate((BIG, SMALL)):
        H, G, D, bs, S = case[:5]
        pair, pb, qkv, ref = _batch(300 + i, *case)
        T = pb["num_tokens"]
        say(f"no-alloc call {i}: T={T} seqs={pb['num_seqs']} H={H} G={G}")
        out_ws = torch.full((T, H, D), float("nan"), dtype=torch.bfloat16, device=DEV)
        call = _call(pair, pb, qkv, S, out_ws)
        assert call.plan_info()["num_merge_rows"] > 0          # partials go through the scratch
        ws = torch.empty(max(256, call.workspace_bytes()), dtype=torch.uint8, device=DEV)
        call.set_workspace(ws)
        call()
        torch.cuda.synchronize()
        out_na = torch.full((T, H, D), float("nan"), dtype=torch.bfloat16, device=DEV)
        _call(pair, pb, qkv, S, out_na).call_noalloc()
        torch.cuda.synchronize()
        # same kernels over the same plan: the same bits
        assert torch.equal(out_na.view(torch.int16), out_ws.view(torch.int16)), f"call {i}"
        assert_close(out_na.to(torch.float64).cpu().numpy(), ref, "bf16", f"no-alloc call {i}")

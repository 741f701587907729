"""GPU parity of the FP8 (E4M3) KV cache: every written code against the
oracle's (bit-exact, saturation and the sign of zero included), and the
attention over an fp8 cache against the oracle's attention over the
dequantized cache, on ragged batches with cached context, decodes and
splits."""
import math

import numpy as np
import pytest
import torch

from chunked_prefill_paged_amd import AttnCall, cache_shapes
from oracle import attention as oa
from oracle import fp8 as of8
from tests.gpu_helpers import DEV, Pair, assert_close, need_gpu, quantize, say

pytestmark = pytest.mark.gpu

# name, H, G, D, bs, S, partial requests [(prompt, computed)], decodes [ctx], budget, k_scale, v_scale
CASES = [
    ("single", 8, 2, 128, 16, 512, [(300, 0)], [], 4096, 0.05, 0.02),
    ("ragged_multi", 32, 8, 128, 16, 1024, [(1500, 1000), (17, 0), (600, 511), (2100, 2048)], [],
     8192, 0.05, 0.02),
    ("d64", 4, 4, 64, 32, 512, [(700, 300), (129, 64)], [], 4096, 0.1, 0.1),
    ("bs128", 32, 8, 128, 128, 1024, [(3000, 2048), (130, 0)], [], 4096, 0.05, 0.02),
    ("mixed_decodes", 32, 8, 128, 16, 512, [(1300, 1024)], [1, 15, 16, 17, 600, 1111, 2049], 8192,
     0.05, 0.02),
    ("saturating", 8, 2, 128, 16, 512, [(400, 200)], [33], 4096, 0.004, 0.006),
    # items whose rows all sit in the first wave (n * H/G <= 32) stream their
    # tiles through two loader waves: decodes over larger blocks, short
    # chunks with cached context (causal rows), one query head per KV head
    ("rows_in_one_wave_bs64", 32, 8, 128, 64, 1024, [(308, 300), (5, 0), (132, 129)],
     [64, 65, 127, 128, 129, 700, 2047, 3000], 8192, 0.05, 0.02),
    ("rows_in_one_wave_bs256", 16, 4, 128, 256, 1024, [(1006, 1000)], [100, 255, 256, 257, 1500],
     8192, 0.05, 0.02),
    ("rows_in_one_wave_hpg1", 8, 8, 128, 32, 512, [(132, 100), (20, 0), (95, 64)], [77, 191], 8192,
     0.05, 0.02),
]
SPLITS = {"auto": (0, 0), "never": (-1, -1), "seg": ("S", "S")}


def _dev(a, dt):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=dt)).to(DEV)


class Fp8Pools:
    """Product pools (device, one byte per element) and the oracle's code
    pools (canonical [nb, bs, G, D])."""

    def __init__(self, nb, G, bs, D):
        ks, vs = cache_shapes(nb, G, bs, D)
        self.k = torch.zeros(ks, dtype=torch.uint8, device=DEV)
        self.v = torch.zeros(vs, dtype=torch.uint8, device=DEV)
        self.ok = np.zeros((nb, bs, G, D), dtype=np.uint8)
        self.ov = np.zeros((nb, bs, G, D), dtype=np.uint8)
        self.bs = bs

    def canonical(self):
        return (self.k.permute(0, 2, 1, 3).contiguous().cpu().numpy(),
                self.v.permute(0, 3, 1, 2).contiguous().cpu().numpy())

    def call(self, batch, q, k, v, S, ks, vs, out=None, slots=True, inline_desc=False, **kw):
        if inline_desc:   # host copies only: the descriptor rides in the launch arguments
            desc = dict(cu_seqlens_q=None, cached_seq_len=None, block_table=None,
                        h_block_table=np.asarray(batch["block_table"], np.int32))
        else:
            desc = dict(cu_seqlens_q=_dev(batch["cu_seqlens_q"], np.int32),
                        cached_seq_len=_dev(batch["cached_seq_len"], np.int32),
                        block_table=_dev(batch["block_table"], np.int32))
        return AttnCall(q=q, k_new=k, v_new=v, k_cache=self.k, v_cache=self.v, out=out, **desc,
                        slot_mapping=_dev(batch["slot_mapping"], np.int64) if slots else None,
                        h_cu_seqlens_q=batch["cu_seqlens_q"], h_cached_seq_len=batch["cached_seq_len"],
                        kv_segment_size=S, k_scale=ks, v_scale=vs, **kw)

    def oracle_write(self, batch_rows, cu, cached, k64, v64, ks, vs):
        self.ok, self.ov = of8.cache_write(self.ok, self.ov, k64, v64, batch_rows, cu, cached, self.bs,
                                           ks, vs)


def _run(case, split, derive_slots=False, seed=0, inline_desc=False):
    name, H, G, D, bs, S, reqs, decodes, budget, ks, vs = case
    rng = np.random.default_rng(7000 + seed)
    max_blocks = max(-(-(p + 1) // bs) for p, _ in reqs + [(c + 1, 0) for c in decodes]) + 1
    need = sum(-(-p // bs) for p, _ in reqs) + sum(-(-(c + 1) // bs) for c in decodes)
    nb = need + 23
    pair = Pair(nb, G, bs, 64, "bf16", budget, max_blocks, rng.permutation(nb).astype(np.int32))
    pools = Fp8Pools(nb, G, bs, D)
    rid = 0

    def fill(rid, L):
        kt, k64 = quantize(rng.standard_normal((L, G, D)), "bf16")
        vt, v64 = quantize(rng.standard_normal((L, G, D)), "bf16")
        slots = pair.prod.slots(rid, 0, L)
        batch = {"cu_seqlens_q": np.array([0, L], np.int32), "cached_seq_len": np.array([0], np.int32),
                 "block_table": np.zeros((1, 1), np.int32), "slot_mapping": slots}
        pools.call(batch, None, kt.to(DEV), vt.to(DEV), 0, ks, vs).reshape_and_cache()
        r = pair.orc._find(rid)
        pools.oracle_write([r.blocks], [0, L], [0], k64, v64, ks, vs)

    for ctx in decodes:
        pair.add_decode(rid, ctx)
        fill(rid, ctx)
        rid += 1
    for prompt, computed in reqs:
        pair.add_partial(rid, prompt, computed)
        if computed:
            fill(rid, computed)
        rid += 1
    pb, ob = pair.step()
    T = pb["num_tokens"]
    qt, q64 = quantize(rng.standard_normal((T, H, D)), "bf16")
    kt, k64 = quantize(rng.standard_normal((T, G, D)), "bf16")
    vt, v64 = quantize(rng.standard_normal((T, G, D)), "bf16")
    sp, sd = ({"S": S}.get(x, x) for x in SPLITS[split])
    say(f"fp8 {name} split={split} derived={derive_slots} T={T}")
    qd = qt.to(DEV)
    out = torch.full_like(qd, float("nan"))
    call = pools.call(pb, qd, kt.to(DEV), vt.to(DEV), S, ks, vs, out=out, slots=not derive_slots,
                      inline_desc=inline_desc, split_keys_prefill=sp, split_keys_decode=sd)
    call.set_workspace(torch.empty(max(256, call.workspace_bytes()), dtype=torch.uint8, device=DEV))
    call()
    torch.cuda.synchronize()
    pools.oracle_write(ob["block_table"], ob["cu_seqlens_q"], ob["cached_seq_len"], k64, v64, ks, vs)
    ref = oa.attention(q64, of8.dequantize(pools.ok, ks), of8.dequantize(pools.ov, vs),
                       ob["block_table"], ob["cu_seqlens_q"], ob["cached_seq_len"], bs,
                       1 / math.sqrt(D), G)
    return pools, out, ref


@pytest.mark.parametrize("split", list(SPLITS))
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fp8_cache_attention_matches_oracle(case, split):
    need_gpu()
    pools, out, ref = _run(case, split)
    gk, gv = pools.canonical()
    assert np.array_equal(gk, pools.ok), "K codes differ"
    assert np.array_equal(gv, pools.ov), "V codes differ"
    assert_close(out.to(torch.float64).cpu().numpy(), ref, "bf16", f"fp8 {case[0]}/{split}")


@pytest.mark.parametrize("case", [CASES[1], CASES[3], CASES[5]],
                         ids=[CASES[1][0], CASES[3][0], CASES[5][0]])
def test_fp8_cache_with_inline_descriptor(case):
    """The fp8 cache write and attention with the descriptor given as host
    copies only, slots derived from the block table."""
    need_gpu()
    pools, out, ref = _run(case, "seg", derive_slots=True, seed=2, inline_desc=True)
    gk, gv = pools.canonical()
    assert np.array_equal(gk, pools.ok) and np.array_equal(gv, pools.ov)
    assert_close(out.to(torch.float64).cpu().numpy(), ref, "bf16", f"fp8 inline {case[0]}")


@pytest.mark.parametrize("case", [CASES[1], CASES[4]], ids=[CASES[1][0], CASES[4][0]])
def test_fp8_cache_with_derived_slots(case):
    need_gpu()
    pools, out, ref = _run(case, "auto", derive_slots=True, seed=1)
    gk, gv = pools.canonical()
    assert np.array_equal(gk, pools.ok) and np.array_equal(gv, pools.ov)
    assert_close(out.to(torch.float64).cpu().numpy(), ref, "bf16", f"fp8 derived {case[0]}")


def test_fp8_codes_of_edge_values():
    """Largest, smallest, ties, saturation and negative zero through the
    cache write (one token, one head, D = 128)."""
    need_gpu()
    vals = np.array([448.0, 500.0, -1e6, 1.0, 1.0625, 1.1875, 2.0 ** -9, 2.0 ** -11, -1e-4, 0.0,
                     -0.0, 432.0, 416.0, 0.3, -7.0, 3.0e-3] * 8, dtype=np.float32)
    kt, k64 = quantize(vals.reshape(1, 1, 128), "bf16")
    pools = Fp8Pools(2, 1, 16, 128)
    batch = {"cu_seqlens_q": np.array([0, 1], np.int32), "cached_seq_len": np.array([0], np.int32),
             "block_table": np.zeros((1, 1), np.int32), "slot_mapping": np.array([17], np.int64)}
    pools.call(batch, None, kt.to(DEV), kt.to(DEV), 0, 1.0, 1.0).reshape_and_cache()
    torch.cuda.synchronize()
    gk, gv = pools.canonical()
    want = of8.quantize(k64.reshape(-1), 1.0)
    assert np.array_equal(gk[1, 1, 0], want) and np.array_equal(gv[1, 1, 0], want)


@pytest.mark.parametrize("split", [-1, 512], ids=["unsplit", "split512"])
def test_fp8_growing_scores_move_the_reference(split):
    """The climbing-score rows of the bf16 test over an fp8 cache whose K
    scale is not 1 (it is folded into the softmax scale): a ramp and jumps
    in both 32-key blocks of the tiles move the running reference many
    times, through the same rescale code as a bf16 cache."""
    need_gpu()
    H, G, D, bs, S = 32, 8, 128, 16, 512
    ks, vs = 0.25, 0.02                    # codes of K up to ~300, of V up to ~250: no saturation
    rng = np.random.default_rng(12)
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
    pair = Pair(nb, G, bs, 64, "bf16", 4096, -(-L // bs) + 1, rng.permutation(nb).astype(np.int32))
    pools = Fp8Pools(nb, G, bs, D)
    pair.add_partial(0, L, computed)
    slots = pair.prod.slots(0, 0, computed)
    fill = {"cu_seqlens_q": np.array([0, computed], np.int32), "cached_seq_len": np.array([0], np.int32),
            "block_table": np.zeros((1, 1), np.int32), "slot_mapping": slots}
    pools.call(fill, None, kt[:computed].to(DEV), vt[:computed].to(DEV), 0, ks, vs).reshape_and_cache()
    pools.oracle_write([pair.orc._find(0).blocks], [0, computed], [0], k64[:computed], v64[:computed],
                       ks, vs)
    pb, ob = pair.step()
    alpha = rng.uniform(8.0, 14.0, H)
    q = 0.3 * rng.standard_normal((n, H, D)) + alpha[None, :, None] * u[np.arange(H) // (H // G)][None]
    qt, q64 = quantize(q, "bf16")
    say(f"fp8 growing scores split={split}")
    qd = qt.to(DEV)
    out = torch.full_like(qd, float("nan"))
    call = pools.call(pb, qd, kt[computed:].to(DEV), vt[computed:].to(DEV), S, ks, vs, out=out,
                      split_keys_prefill=split)
    call.set_workspace(torch.empty(max(256, call.workspace_bytes()), dtype=torch.uint8, device=DEV))
    call()
    torch.cuda.synchronize()
    pools.oracle_write(ob["block_table"], ob["cu_seqlens_q"], ob["cached_seq_len"], k64[computed:],
                       v64[computed:], ks, vs)
    gk, gv = pools.canonical()
    assert np.array_equal(gk, pools.ok) and np.array_equal(gv, pools.ov)
    ref = oa.attention(q64, of8.dequantize(pools.ok, ks), of8.dequantize(pools.ov, vs),
                       ob["block_table"], ob["cu_seqlens_q"], ob["cached_seq_len"], bs,
                       1 / math.sqrt(D), G)
    assert_close(out.to(torch.float64).cpu().numpy(), ref, "bf16", f"fp8 growing/{split}")

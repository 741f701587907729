"""Test-side drivers for the GPU path (product) and the oracle on the same
seeded inputs.  The product side gets its block tables and slots from the
library's own scheduler; the oracle side from the oracle's scheduler; the two
are compared for equality before any attention is compared."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from chunked_prefill_paged_amd import AttnCall, HostScheduler, cache_shapes
from oracle import attention as oa
from oracle import schedule as osch

DEV = "cuda"
TORCH_DTYPE = {"bf16": torch.bfloat16, "fp32": torch.float32}
BITS_DTYPE = {"bf16": torch.int16, "fp32": torch.int32}
TOL = {"bf16": (2e-2, 2e-3), "fp32": (1e-4, None)}   # (max-abs, mean-abs)


def need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def quantize(x32, dtype):
    """float32 numpy -> (torch tensor in `dtype` on the CPU, its exact float64 values)."""
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(TORCH_DTYPE[dtype])
    return t, t.to(torch.float64).numpy()


def assert_close(got, ref, dtype, where=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{where}: non-finite output"
    err = np.abs(got - ref)
    max_tol, mean_tol = TOL[dtype]
    assert err.max() <= max_tol, f"{where}: max-abs {err.max():.3g} > {max_tol}"
    if mean_tol is not None:
        assert err.mean() <= mean_tol, f"{where}: mean-abs {err.mean():.3g} > {mean_tol}"
    return float(err.max()), float(err.mean())


class GpuCache:
    """The product's paged pool on the device."""

    def __init__(self, num_blocks, num_kv_heads, block_size, head_dim, dtype, fill=0.0):
        ks, vs = cache_shapes(num_blocks, num_kv_heads, block_size, head_dim)
        td = TORCH_DTYPE[dtype]
        self.dtype = dtype
        self.k = torch.full(ks, fill, dtype=td, device=DEV)
        self.v = torch.full(vs, fill, dtype=td, device=DEV)

    def canonical_bits(self):
        """Pools as raw bits in the canonical [nb, bs, G, D] order (numpy ints)."""
        bd = BITS_DTYPE[self.dtype]
        k = self.k.view(bd).permute(0, 2, 1, 3).contiguous().cpu().numpy()
        v = self.v.view(bd).permute(0, 3, 1, 2).contiguous().cpu().numpy()
        return k, v

    def canonical(self):
        k = self.k.permute(0, 2, 1, 3).to(torch.float64).cpu().numpy()
        v = self.v.permute(0, 3, 1, 2).to(torch.float64).cpu().numpy()
        return k, v


def bits_of(x64, dtype):
    """Exact float64 values -> raw bits of `dtype` (numpy ints)."""
    t = torch.from_numpy(np.ascontiguousarray(x64)).to(TORCH_DTYPE[dtype])
    return t.view(BITS_DTYPE[dtype]).numpy()


def _dev(a, dt):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=dt)).to(DEV)


def gpu_call(cache, batch, q, k_new, v_new, kv_segment_size, *, scale=None, want_lse=False,
             split_pre=0, split_dec=0, dec_thresh=0, only_cache=False, derive_slots=False,
             inline_desc=False, attention_twice=False):
    """Run one batch through the library.  q/k_new/v_new are CPU or device
    tensors of the cache dtype.  derive_slots passes no slot mapping (the
    library derives the slots from the block table).  inline_desc passes
    the descriptor as host copies only (no device cu_seqlens_q,
    cached_seq_len or block_table).  attention_twice runs the attention
    launch a second time on the same prepared workspace and checks that it
    reproduces the first output bit for bit.  Returns (out, lse) as CPU
    tensors."""
    qd = q.to(DEV) if q is not None else None
    kd, vd = k_new.to(DEV), v_new.to(DEV)
    out = torch.empty_like(qd) if qd is not None else None
    lse = None
    if want_lse and qd is not None:
        lse = torch.full((qd.shape[1], qd.shape[0]), float("nan"), dtype=torch.float32, device=DEV)
    if inline_desc:
        desc = dict(cu_seqlens_q=None, cached_seq_len=None, block_table=None,
                    h_block_table=np.asarray(batch["block_table"], np.int32))
    else:
        desc = dict(cu_seqlens_q=_dev(batch["cu_seqlens_q"], np.int32),
                    cached_seq_len=_dev(batch["cached_seq_len"], np.int32),
                    block_table=_dev(batch["block_table"], np.int32))
    call = AttnCall(q=qd, k_new=kd, v_new=vd, k_cache=cache.k, v_cache=cache.v, out=out, **desc,
                    slot_mapping=None if derive_slots else _dev(batch["slot_mapping"], np.int64),
                    h_cu_seqlens_q=batch["cu_seqlens_q"], h_cached_seq_len=batch["cached_seq_len"],
                    kv_segment_size=kv_segment_size, scale=scale, lse=lse,
                    decode_token_threshold=dec_thresh, split_keys_prefill=split_pre,
                    split_keys_decode=split_dec)
    if only_cache:
        call.reshape_and_cache()
        torch.cuda.synchronize()
        return None, None
    ws = torch.empty(max(256, call.workspace_bytes()), dtype=torch.uint8, device=DEV)
    call.set_workspace(ws)
    call()
    torch.cuda.synchronize()
    if attention_twice and out is not None:
        first = out.clone()
        out.fill_(float("nan"))
        call.attention()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16) if out.dtype == torch.bfloat16 else out,
                           first.view(torch.int16) if first.dtype == torch.bfloat16 else first)
    return (out.cpu() if out is not None else None), (lse.cpu() if lse is not None else None)


def same_batches(pb, ob):
    """Product descriptor == oracle descriptor (bit-exact integer work)."""
    assert list(pb["cu_seqlens_q"]) == ob["cu_seqlens_q"]
    assert list(pb["cached_seq_len"]) == ob["cached_seq_len"]
    assert np.array_equal(pb["block_table"], np.array(ob["block_table"], dtype=np.int32))
    assert list(pb["slot_mapping"]) == ob["slot_mapping"]


class Pair:
    """The product scheduler + device pool, and the oracle scheduler + float64
    pool, driven in lockstep."""

    def __init__(self, num_blocks, num_kv_heads, block_size, head_dim, dtype, budget, max_blocks,
                 free_order=None, fill=0.0, cap=0, align=False, prefix_caching=False,
                 preemption=False):
        self.bs, self.dtype = block_size, dtype
        self.prod = HostScheduler(num_blocks, block_size, budget, max_blocks, cap, align, free_order,
                                  prefix_caching=prefix_caching, preemption=preemption)
        self.pool = osch.BlockPool(num_blocks, free_order)
        self.orc = osch.Scheduler(self.pool, block_size, budget, max_blocks, cap, align,
                                  prefix_caching=prefix_caching, preemption=preemption)
        self.cache = GpuCache(num_blocks, num_kv_heads, block_size, head_dim, dtype, fill)
        shape = (num_blocks, block_size, num_kv_heads, head_dim)
        self.k_pool = np.full(shape, fill, dtype=np.float64)
        self.v_pool = np.full(shape, fill, dtype=np.float64)

    def add_partial(self, rid, prompt, computed):
        self.prod.add_partial(rid, prompt, computed)
        self.orc.add_partial(rid, prompt, computed)

    def add_decode(self, rid, ctx):
        self.prod.add_decode(rid, ctx)
        self.orc.add_decode(rid, ctx)

    def add_request(self, rid, prompt, prefix=()):
        self.prod.add_request(rid, prompt, prefix)
        self.orc.add_request(rid, prompt, list(prefix))

    def free(self, rid):
        self.prod.free_request(rid)
        self.orc.free_request(rid)

    def fill_context(self, rid, k64, v64, kt, vt):
        """Place already-computed context (positions 0..L-1) of a request: the
        product writes it with its cache-write entry point, the oracle with its
        own cache write."""
        L = k64.shape[0]
        slots = self.prod.slots(rid, 0, L)
        batch = {"cu_seqlens_q": np.array([0, L], np.int32), "cached_seq_len": np.array([0], np.int32),
                 "block_table": np.zeros((1, 1), np.int32), "slot_mapping": slots}
        gpu_call(self.cache, batch, None, kt, vt, 0, only_cache=True)
        r = self.orc._find(rid)
        self.k_pool, self.v_pool = oa.cache_write(self.k_pool, self.v_pool, k64, v64, [r.blocks],
                                                  [0, L], [0], self.bs)

    def add_request_tokens(self, rid, tokens, namespace="default"):
        self.prod.add_request_tokens(rid, tokens, namespace)
        self.orc.add_request_tokens(rid, tokens, namespace)

    def step(self):
        pb = self.prod.step()
        ob = self.orc.step()
        same_batches(pb, ob)
        assert self.prod.last_preempted() == self.orc.preempted
        return pb, ob

    def commit(self):
        self.prod.commit()
        self.orc.commit()

    def oracle_batch(self, ob, q64, k64, v64, scale, num_kv_heads, heads=None, seqs=None):
        self.k_pool, self.v_pool = oa.cache_write(self.k_pool, self.v_pool, k64, v64,
                                                  ob["block_table"], ob["cu_seqlens_q"],
                                                  ob["cached_seq_len"], self.bs)
        return oa.attention(q64, self.k_pool, self.v_pool, ob["block_table"], ob["cu_seqlens_q"],
                            ob["cached_seq_len"], self.bs, scale, num_kv_heads, heads=heads,
                            seqs=seqs)

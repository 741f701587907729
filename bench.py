#!/usr/bin/env python3
"""Benchmark of the chunked-prefill attention path on one MI355X.

Workload (default): a 10,000-token prompt, GQA 32 query / 8 KV heads,
head_dim 128, bf16, block_size 128, kv_segment_size 1024, token budget 2048,
so the scheduler cuts it into chunks of 2048 x 4 + 1808 at cached lengths
0, 2048, 4096, 6144, 8192 ("Prefill Processing", section "Prefill
Segmentation").  One step is the whole prompt: for every chunk, the host
scheduler builds the descriptor, the descriptor goes to the device, and the
library writes the chunk's K/V into the paged cache and runs the attention.
Q/K/V of the prompt are resident in HBM before timing starts.

Metric: algorithmic attention FLOPs, 4 * H * D * pairs per chunk with
pairs = n*c + n(n+1)/2 ("Prefill Optimisation ...", section 4), over the
wall time of the steps -> TFLOP/s, and as a fraction of the MI355X dense
bf16 MFMA peak.

    python bench.py [--steps K] [--warmup W] [--clock-warmup-s S] [--no-cpu-baseline]

Before the W warmup steps the headline mode runs untimed steps for S seconds
(default 0.25; the count is in the line's "clock_warmup"): an idle GPU's
shader clock ramps up over ~0.1 s of continuous work, so after a few warmup
steps alone the timed steps would measure the ramp.  --clock-warmup-s 0
gives the cold-clock number.
    python bench.py --copy-probe      # one plain 1 GiB device copy, for
                                      # calibrating HBM byte counters

The roofline's "traffic" is the attention kernel's HBM bytes per launch as
measured by hardware counters and recorded, with the hash of the kernel
sources it was measured on, in profiles/attn_kernel_10k_prompt_hbm_traffic.txt;
it is reported only while those sources are unchanged (null otherwise).
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA (published)
PEAK_HBM_GBS = 8000.0
ROOT = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = ("chunked_prefill_paged_amd/csrc/cpa_attn.hip", "chunked_prefill_paged_amd/csrc/cpa_plan.h")
TRAFFIC_FILE = "profiles/attn_kernel_10k_prompt_hbm_traffic.txt"
ROPE_TRAFFIC_FILE = "profiles/prep_kernel_rope_cache_write.txt"
COPY_PROBE_BYTES = 1 << 30
FP8_SCALE = 0.05              # per-tensor K and V scale of an fp8 cache (N(0,1) data: no saturation)


def _args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=100,
                    help="untimed steps first (the first few dozen run below steady state)")
    ap.add_argument("--kv-segment-size", type=int, default=1024)
    ap.add_argument("--split-keys-prefill", type=int, default=0,
                    help="0 automatic, -1 never, else keys per work item")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--event-timing", choices=("dispatch", "records"), default="dispatch",
                    help="per-launch attention timing: events taken by the kernel's own dispatch "
                         "(cpa_attention_timed), or event records around the launch")
    ap.add_argument("--workload", choices=("c2", "c2tp", "c3", "c4", "c5", "rope"), default="c2",
                    help="c2: the 10k prompt (headline line); c2tp: the 10k prompt at one "
                         "tensor-parallel share of eight (H4/G1); c3: 16 prefix-cached requests "
                         "in one varlen call; c5: the 32k prompt, per chunk and against one "
                         "monolithic call; c4: the mixed decode + prefill batch; rope: the cache "
                         "write with rotary embedding fused in, at two chunk shapes")
    ap.add_argument("--clock-warmup-s", type=float, default=0.25,
                    help="seconds of untimed steps before the warmup steps (the 10k-prompt modes): "
                         "an idle GPU's shader clock ramps up over ~0.1 s of continuous work "
                         "(0: none)")
    ap.add_argument("--steady-warmup", type=int, default=100,
                    help="after the timed steps, this many more untimed steps, then the same "
                         "number of timed steps again: the steady-state rate (0: skip)")
    ap.add_argument("--kv-cache", choices=("bf16", "fp8"), default="bf16",
                    help="KV cache element type for c2/c5/c4: bf16, or E4M3 codes under per-tensor "
                         "scales (attention still computes in bf16)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run a plain 1 GiB device-to-device copy 5 times and exit")
    return ap.parse_args()


_COMMENT_OR_STRING = re.compile(r'//[^\n]*|/\*.*?\*/|"(?:\\.|[^"\\])*"', re.S)


def kernel_sources_sha256() -> str:
    """Digest of the kernel sources' code: comments dropped and whitespace
    runs collapsed, so that a recorded counter summary stays valid across
    edits that cannot change the compiled kernels."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel)) as f:
            text = f.read()
        code = _COMMENT_OR_STRING.sub(lambda m: m.group(0) if m.group(0).startswith('"') else " ", text)
        h.update(" ".join(code.split()).encode())
    return h.hexdigest()


def recorded_traffic(rel=TRAFFIC_FILE):
    """HBM bytes per launch of the kernel a committed counter summary covers
    (by default the attention kernel's), or None when the kernel sources
    changed since it was measured."""
    path = os.path.join(ROOT, rel)
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith((" ", "#", "|")):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("source_sha256") != kernel_sources_sha256():
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_probe():
    """A plain device copy of known size: what HBM byte counters read for it
    calibrates what they read for the attention kernel."""
    import torch
    src = torch.ones(COPY_PROBE_BYTES // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": COPY_PROBE_BYTES, "copy_probe_bytes_written":
                      COPY_PROBE_BYTES, "launches": 5}), flush=True)


class PromptBench:
    """One chunked prompt (the 10k prompt by default), its device buffers and
    the per-chunk calls."""

    def __init__(self, kv_segment_size, split_pre, workload="c2", kv_fp8=False):
        import torch
        from chunked_prefill_paged_amd import AttnCall, HostScheduler, cache_shapes
        from synth import free_block_order, get_workload, prompt_qkv

        self.torch = torch
        w = get_workload(workload) if isinstance(workload, str) else workload
        self.w = w
        q32, k32, v32 = prompt_qkv(w)
        dev = "cuda"
        self.q = torch.from_numpy(q32).to(torch.bfloat16).to(dev)
        self.k = torch.from_numpy(k32).to(torch.bfloat16).to(dev)
        self.v = torch.from_numpy(v32).to(torch.bfloat16).to(dev)
        self.out = torch.empty_like(self.q)
        ks, vs = cache_shapes(w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim)
        cache_t = torch.uint8 if kv_fp8 else torch.bfloat16
        self.k_cache = torch.zeros(ks, dtype=cache_t, device=dev)
        self.v_cache = torch.zeros(vs, dtype=cache_t, device=dev)
        self.max_blocks = -(-w.prompt_len // w.block_size)
        self.sched = HostScheduler(w.num_blocks, w.block_size, w.max_batched_tokens,
                                   self.max_blocks, free_order=free_block_order(w.num_blocks, w.seed))
        self.AttnCall = AttnCall
        self.S = kv_segment_size
        self.split_pre = split_pre
        self.rid = 0
        # chunk plan of the prompt (fixed): build one call per chunk index with
        # persistent device descriptor buffers and pinned host staging
        from chunked_prefill_paged_amd import INLINE_DESC_INTS, schedule_prompt
        self.chunks = schedule_prompt(w.max_batched_tokens, 0, w.prompt_len)
        self.calls, self.dev_desc, self.pinned, self.copied = [], [], [], []
        # the per-chunk descriptor (cu_seqlens_q, cached_seq_len, block-table
        # row) rides in the launches' arguments when it fits; otherwise it
        # is uploaded with one copy from pinned memory.  No slot mapping:
        # the library derives the slots from the block table.
        n32 = 2 + 1 + self.max_blocks
        self.inline = n32 <= INLINE_DESC_INTS
        pos = 0
        ws_bytes = 256
        for n in self.chunks:
            if self.inline:
                d_i32 = p_i32 = None
                dev_desc = dict(cu_seqlens_q=None, cached_seq_len=None, block_table=None,
                                h_block_table=np.zeros((1, self.max_blocks), np.int32))
            else:
                d_i32 = torch.zeros(n32, dtype=torch.int32, device=dev)
                p_i32 = torch.zeros(n32, dtype=torch.int32, pin_memory=True)
                dev_desc = dict(cu_seqlens_q=d_i32[0:2], cached_seq_len=d_i32[2:3],
                                block_table=d_i32[3:].view(1, self.max_blocks))
            call = AttnCall(q=self.q[pos:pos + n], k_new=self.k[pos:pos + n], v_new=self.v[pos:pos + n],
                            k_cache=self.k_cache, v_cache=self.v_cache, out=self.out[pos:pos + n],
                            slot_mapping=None, h_cu_seqlens_q=np.array([0, n], np.int32),
                            h_cached_seq_len=np.array([pos], np.int32),
                            kv_segment_size=kv_segment_size, split_keys_prefill=split_pre,
                            k_scale=FP8_SCALE, v_scale=FP8_SCALE, **dev_desc)
            ws_bytes = max(ws_bytes, call.workspace_bytes())
            self.calls.append(call)
            self.dev_desc.append(d_i32)
            self.pinned.append(p_i32)
            self.copied.append(None)
            pos += n
        self.ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        for call in self.calls:
            call.set_workspace(self.ws)
        self.plan = [c.plan_info() for c in self.calls]

    def flops_per_step(self) -> int:
        # 4 * H * D FLOPs per (query, key, head) pair; a chunk of n tokens over
        # c cached ones has n*c + n(n+1)/2 pairs
        w, c, total = self.w, 0, 0
        for n in self.chunks:
            total += 4 * w.num_heads * w.head_dim * (n * c + n * (n + 1) // 2)
            c += n
        return total

    def step(self, events=None):
        """One pass of the whole path over the prompt."""
        torch = self.torch
        sched = self.sched
        sched.add_request(self.rid, self.w.prompt_len)
        for i, call in enumerate(self.calls):
            b = sched.step()
            if self.inline:
                bt = np.ascontiguousarray(b["block_table"], dtype=np.int32)
                call.args.h_block_table = bt.ctypes.data
            else:
                bt = None
                p_i32 = self.pinned[i]
                if self.copied[i] is not None:
                    self.copied[i].synchronize()    # staging buffer of the previous step is free
                a32 = p_i32.numpy()
                a32[0:2] = b["cu_seqlens_q"]
                a32[2] = b["cached_seq_len"][0]
                a32[3:] = b["block_table"][0]
                self.dev_desc[i].copy_(p_i32, non_blocking=True)
                ev = torch.cuda.Event()
                ev.record()
                self.copied[i] = ev
            call.args.h_cu_seqlens_q = b["cu_seqlens_q"].ctypes.data
            call.args.h_cached_seq_len = b["cached_seq_len"].ctypes.data
            call._keep_host = (b["cu_seqlens_q"], b["cached_seq_len"], bt)
            call.prepare()
            if events is None:
                call.attention()
            elif isinstance(events[i][0], int):        # raw events taken by the dispatch
                call.attention_timed(events[i][0], events[i][1])
            else:                                      # event records around the launch
                events[i][0].record()
                call.attention()
                events[i][1].record()
            sched.commit()
        sched.free_request(self.rid)
        self.rid += 1


class HipEvents:
    """Raw hipEvent_t handles from the HIP runtime the process already uses
    (torch's), for launches that take their timing events in the dispatch."""

    def __init__(self):
        import ctypes
        self._c = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so.7")

    def _check(self, err, what):
        if err != 0:
            raise RuntimeError(f"{what} failed ({err})")

    def create(self) -> int:
        ev = self._c.c_void_p()
        self._check(self.hip.hipEventCreate(self._c.byref(ev)), "hipEventCreate")
        return ev.value

    def elapsed_ms(self, a: int, b: int) -> float:
        ms = self._c.c_float()
        self._check(self.hip.hipEventElapsedTime(self._c.byref(ms), self._c.c_void_p(a),
                                                 self._c.c_void_p(b)), "hipEventElapsedTime")
        return ms.value

    def destroy(self, ev: int) -> None:
        self._check(self.hip.hipEventDestroy(self._c.c_void_p(ev)), "hipEventDestroy")


def cpu_baseline(w, max_blocks):
    """The oracle as it stands, timed over two whole steps of the same
    workload: the 10k prompt's five chunks, every query head, with the
    oracle's scheduler, cache write and attention (NumPy float64)."""
    import torch
    from threadpoolctl import threadpool_info

    from oracle import attention as oa
    from oracle import counters
    from oracle import schedule as osch
    from synth import free_block_order, prompt_qkv

    q32, k32, v32 = prompt_qkv(w)
    q64, k64, v64 = (torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
                     for x in (q32, k32, v32))
    shape = (w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim)
    steps, flops = 2, 0
    t0 = time.perf_counter()
    for _ in range(steps):
        kp, vp = np.zeros(shape), np.zeros(shape)
        pool = osch.BlockPool(w.num_blocks, free_block_order(w.num_blocks, w.seed))
        sched = osch.Scheduler(pool, w.block_size, w.max_batched_tokens, max_blocks)
        sched.add_request(0, w.prompt_len)
        pos = 0
        while pos < w.prompt_len:
            b = sched.step()
            n = b["num_tokens"]
            kp, vp = oa.cache_write(kp, vp, k64[pos:pos + n], v64[pos:pos + n], b["block_table"],
                                    b["cu_seqlens_q"], b["cached_seq_len"], w.block_size)
            oa.attention(q64[pos:pos + n], kp, vp, b["block_table"], b["cu_seqlens_q"],
                         b["cached_seq_len"], w.block_size, w.scale, w.num_kv_heads)
            flops += counters.attention_flops(counters.pairs(n, pos), w.num_heads, w.head_dim)
            sched.commit()
            pos += n
    elapsed = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": round(flops / elapsed / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "seconds": round(elapsed, 2),
            "host_cpus": os.cpu_count(), "cpus_available": len(os.sched_getaffinity(0)),
            "cpu_model": cpu_model(),
            "sample": f"{steps} whole steps: the 10k prompt's 5 chunks (2048x4 + 1808), all 32 "
                      "query heads, oracle scheduler + cache write + attention in numpy float64 "
                      f"({flops / 1e9:.2f} GFLOP)"}


def cpu_model() -> str:
    """Model name of the host CPU (as lscpu reports it)."""
    try:
        import subprocess
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _time_steps(torch, fn, steps, warmup):
    gc.collect()
    gc.disable()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    gc.enable()
    return (time.perf_counter() - t0) / steps


def run_long_prompt(args):
    """The 32,768-token prompt (GQA 64/8, bs16, S4096) in 16 chunks of 2048:
    TFLOP/s of every chunk as the cached length grows, and the whole chunked
    prompt against one monolithic causal call over all 32k tokens."""
    import torch
    S = 4096 if args.kv_segment_size == 1024 else args.kv_segment_size
    bench = PromptBench(S, args.split_keys_prefill, workload="c5", kv_fp8=args.kv_cache == "fp8")
    w = bench.w
    steps = max(1, min(args.steps, 5))
    warm = max(1, min(args.warmup, 10))
    for _ in range(warm):
        bench.step()
    torch.cuda.synchronize()
    events = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in bench.chunks] for _ in range(steps)]
    t0 = time.perf_counter()
    for st in range(steps):
        bench.step([list(p) for p in events[st]])
    torch.cuda.synchronize()
    chunked_s = (time.perf_counter() - t0) / steps
    per_chunk_ms = [sum(events[st][i][0].elapsed_time(events[st][i][1]) for st in range(steps)) / steps
                    for i in range(len(bench.chunks))]
    H, D, c, per_chunk_tf = w.num_heads, w.head_dim, 0, []
    for n, ms in zip(bench.chunks, per_chunk_ms):
        per_chunk_tf.append(round(4 * H * D * (n * c + n * (n + 1) // 2) / (ms / 1e3) / 1e12, 1))
        c += n
    # monolithic: one call over the whole prompt, nothing cached (same slots)
    from chunked_prefill_paged_amd import AttnCall
    from synth import free_block_order
    P = w.prompt_len
    # the whole pool (exactly the prompt's 2048 blocks) in its seeded order
    table = np.ascontiguousarray(free_block_order(w.num_blocks, w.seed)[:P // w.block_size])
    dev = "cuda"
    cu = torch.tensor([0, P], dtype=torch.int32, device=dev)
    cached = torch.zeros(1, dtype=torch.int32, device=dev)
    bt = torch.from_numpy(table).view(1, -1).to(dev)
    slots = (torch.from_numpy(table.astype(np.int64)).to(dev).repeat_interleave(w.block_size)
             * w.block_size + torch.arange(P, device=dev) % w.block_size)
    mono = AttnCall(q=bench.q, k_new=bench.k, v_new=bench.v, k_cache=bench.k_cache,
                    v_cache=bench.v_cache, out=bench.out, cu_seqlens_q=cu, cached_seq_len=cached,
                    block_table=bt, slot_mapping=slots, h_cu_seqlens_q=np.array([0, P], np.int32),
                    h_cached_seq_len=np.array([0], np.int32), kv_segment_size=S,
                    split_keys_prefill=args.split_keys_prefill, k_scale=FP8_SCALE, v_scale=FP8_SCALE)
    ws = torch.empty(mono.workspace_bytes(), dtype=torch.uint8, device=dev)
    mono.set_workspace(ws)
    mono_s = _time_steps(torch, mono, steps, warm)
    flops = bench.flops_per_step()
    print(json.dumps({
        "metric": "32k-prompt chunked prefill TFLOP/s per chunk; chunked vs monolithic time",
        "value": round(flops / chunked_s / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": steps, "warmup": warm, "ms_per_step": round(chunked_s * 1e3, 3),
        "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "32,768-token prompt in 16 chunks of 2048 (cached 0..30720), "
                               f"H64/G8/D128, block_size 16, kv_segment_size {S}",
                   "kv_cache": args.kv_cache},
        "gflop_per_step": round(flops / 1e9, 2),
        "attention_ms_per_chunk": [round(x, 4) for x in per_chunk_ms],
        "attention_tflops_per_chunk": per_chunk_tf,
        "monolithic_ms": round(mono_s * 1e3, 3),
        "monolithic_tflops": round(flops / mono_s / 1e12, 2),
        "chunked_over_monolithic": round(chunked_s / mono_s, 4),
    }), flush=True)


def run_mixed_batch(args):
    """The piggybacked batch: 256 decodes (context 16*U{64..2048}) plus a
    1792-token chunk of a 32k prompt at cached 30,720, one varlen call under
    a 2048-token budget (bs16, S2048, GQA 32/8).  Times the mixed call, the
    decode rows alone (achieved HBM GB/s over the KV they read) and the
    prefill rows alone (TFLOP/s)."""
    import math

    import torch
    from chunked_prefill_paged_amd import AttnCall, HostScheduler, cache_shapes
    from synth import config4_decode_contexts, free_block_order, get_workload

    w = get_workload("c4")
    H, G, D, bs = w.num_heads, w.num_kv_heads, w.head_dim, w.block_size
    S = 2048 if args.kv_segment_size == 1024 else args.kv_segment_size
    ctx = [int(x) for x in config4_decode_contexts(w)]
    pf_cached, pf_prompt = 30720, w.prompt_len
    demand = sum(-(-(L + 1) // bs) for L in ctx) + -(-(pf_cached + 1792) // bs)
    nb = math.ceil(1.2 * demand)
    max_blocks = -(-(max(ctx) + 1) // bs) + 1
    sched = HostScheduler(nb, bs, w.max_batched_tokens, max(max_blocks, pf_prompt // bs),
                          free_order=free_block_order(nb, w.seed))
    for i, L in enumerate(ctx):
        sched.add_decode(i, L)
    sched.add_partial(256, pf_prompt, pf_cached)
    b = sched.step()
    T = int(b["num_tokens"])
    dev = "cuda"
    ks, vs = cache_shapes(nb, G, bs, D)
    fp8 = args.kv_cache == "fp8"
    k_cache = torch.empty(ks, dtype=torch.uint8 if fp8 else torch.bfloat16, device=dev)
    v_cache = torch.empty(vs, dtype=torch.uint8 if fp8 else torch.bfloat16, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed)
    for t in (k_cache, v_cache):             # the cached context: seeded N(0,1)
        for i in range(0, nb, 8192):
            if fp8:                          # its E4M3 codes under FP8_SCALE
                blk = torch.randn(t[i:i + 8192].shape, generator=gen, device=dev) / FP8_SCALE
                t[i:i + 8192] = blk.to(torch.float8_e4m3fn).view(torch.uint8)
            else:
                t[i:i + 8192].normal_(generator=gen)
    q = torch.randn((T, H, D), generator=gen, device=dev).to(torch.bfloat16)
    kn = torch.randn((T, G, D), generator=gen, device=dev).to(torch.bfloat16)
    vn = torch.randn((T, G, D), generator=gen, device=dev).to(torch.bfloat16)
    out = torch.empty_like(q)
    cu_h = np.ascontiguousarray(b["cu_seqlens_q"], dtype=np.int32)
    cached_h = np.ascontiguousarray(b["cached_seq_len"], dtype=np.int32)
    table_h = np.ascontiguousarray(b["block_table"], dtype=np.int32)
    slots_h = np.ascontiguousarray(b["slot_mapping"], dtype=np.int64)
    d = lambda a: torch.from_numpy(a).to(dev)
    cu, cached, table, slots = d(cu_h), d(cached_h), d(table_h), d(slots_h)

    def make(seqs):
        lo, hi = seqs
        t0, t1 = int(cu_h[lo]), int(cu_h[hi])
        call = AttnCall(q=q[t0:t1], k_new=kn[t0:t1], v_new=vn[t0:t1], k_cache=k_cache,
                        v_cache=v_cache, out=out[t0:t1],
                        cu_seqlens_q=(cu[lo:hi + 1] - t0).contiguous(),
                        cached_seq_len=cached[lo:hi].contiguous(),
                        block_table=table[lo:hi].contiguous(), slot_mapping=slots[t0:t1].contiguous(),
                        h_cu_seqlens_q=cu_h[lo:hi + 1] - t0, h_cached_seq_len=cached_h[lo:hi],
                        kv_segment_size=S, split_keys_prefill=args.split_keys_prefill,
                        k_scale=FP8_SCALE, v_scale=FP8_SCALE)
        call.set_workspace(torch.empty(call.workspace_bytes(), dtype=torch.uint8, device=dev))
        return call

    B = len(cu_h) - 1
    mixed, decodes, prefill = make((0, B)), make((0, B - 1)), make((B - 1, B))
    steps, warm = max(1, args.steps), max(1, args.warmup)
    t_mixed = _time_steps(torch, mixed, steps, warm)
    t_dec = _time_steps(torch, decodes, steps, warm)
    t_pre = _time_steps(torch, prefill, steps, warm)
    eb = 1 if fp8 else 2
    dec_bytes = sum(2 * (L + 1) * G * D * eb for L in ctx)         # K and V each decode reads
    n_pre = T - 256
    pre_flops = 4 * H * D * (n_pre * pf_cached + n_pre * (n_pre + 1) // 2)
    dec_flops = sum(4 * H * D * (L + 1) for L in ctx)
    print(json.dumps({
        "metric": "mixed decode + prefill batch: decode GB/s, prefill TFLOP/s, mixed call time",
        "value": round(dec_bytes / t_dec / 1e9, 1), "unit": "GB/s (decode rows)", "n_gpus": 1,
        "steps": steps, "warmup": warm, "ms_per_step": round(t_mixed * 1e3, 4),
        "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"256 decodes (context 16*U{{64..2048}}) + 1792-token chunk at "
                               f"cached 30720, budget 2048, bs16, S{S}, H32/G8/D128, "
                               f"pool {nb} blocks ({2 * nb * G * bs * D * eb / 1e9:.1f} GB K+V)",
                   "kv_cache": args.kv_cache},
        "mixed_ms": round(t_mixed * 1e3, 4),
        "decode_only_ms": round(t_dec * 1e3, 4),
        "decode_kv_gb": round(dec_bytes / 1e9, 3),
        "decode_gbps": round(dec_bytes / t_dec / 1e9, 1),
        "decode_frac_of_hbm_peak": round(dec_bytes / t_dec / 1e9 / PEAK_HBM_GBS, 4),
        "prefill_only_ms": round(t_pre * 1e3, 4),
        "prefill_tflops": round(pre_flops / t_pre / 1e12, 1),
        "mixed_tflops": round((pre_flops + dec_flops) / t_mixed / 1e12, 1),
        "roofline_mixed_ms": round(max(dec_bytes / (PEAK_HBM_GBS * 1e9),
                                       (pre_flops + dec_flops) / (PEAK_BF16_TFLOPS * 1e12)) * 1e3, 4),
    }), flush=True)


def run_rope(args):
    """The cache write alone and with rotary embedding fused in (queries
    rotated into a second tensor, keys rotated on their way into the cache),
    at two chunk shapes: a 2048-token chunk of the 10k prompt (H32/G8, bs128,
    cached 2048) and the last 2048-token chunk of the 32k prompt (H64/G8,
    bs16, cached 30,720).  HBM-bound: reports GB/s of the bytes each call
    must move (K/V read and written; with RoPE also Q read and written)."""
    import torch
    from chunked_prefill_paged_amd import AttnCall, cache_shapes
    from chunked_prefill_paged_amd.attention import Rope

    dev = "cuda"
    shapes = [("10k prompt chunk: T2048 at cached 2048, H32/G8/D128, bs128", 2048, 2048, 32, 8, 128, 128),
              ("32k prompt last chunk: T2048 at cached 30720, H64/G8/D128, bs16", 2048, 30720, 64, 8, 128, 16)]
    steps, warm = max(1, args.steps), max(1, args.warmup)
    res = []
    for name, T, c, H, G, D, bs in shapes:
        nb = (c + T) // bs
        ks, vs = cache_shapes(nb, G, bs, D)
        gen = torch.Generator(device=dev)
        gen.manual_seed(11)
        k_cache = torch.zeros(ks, dtype=torch.bfloat16, device=dev)
        v_cache = torch.zeros(vs, dtype=torch.bfloat16, device=dev)
        q = torch.randn((T, H, D), generator=gen, device=dev).to(torch.bfloat16)
        kn = torch.randn((T, G, D), generator=gen, device=dev).to(torch.bfloat16)
        vn = torch.randn((T, G, D), generator=gen, device=dev).to(torch.bfloat16)
        q_out = torch.empty_like(q)
        table = torch.from_numpy(np.random.default_rng(12).permutation(nb).astype(np.int32)[None, :]).to(dev)
        call = AttnCall(q=q, k_new=kn, v_new=vn, k_cache=k_cache, v_cache=v_cache, out=q_out,
                        cu_seqlens_q=torch.tensor([0, T], dtype=torch.int32, device=dev),
                        cached_seq_len=torch.tensor([c], dtype=torch.int32, device=dev),
                        block_table=table, slot_mapping=None,
                        h_cu_seqlens_q=np.array([0, T], np.int32), h_cached_seq_len=np.array([c], np.int32),
                        kv_segment_size=1024 if bs == 128 else 4096)
        rope = Rope(q_out, 10000.0)
        kv_bytes = 2 * 2 * T * G * D * 2              # K and V, read once and written once
        q_bytes = 2 * T * H * D * 2                   # Q read, rotated Q written
        row = {"shape": name}
        for label, fn, nbytes in (("cache_write", lambda: call.reshape_and_cache(), kv_bytes),
                                  ("rope_cache_write", lambda: call.rope_reshape_and_cache(rope),
                                   kv_bytes + q_bytes)):
            # back-to-back launches between two events: the mean launch
            # duration (small kernels; a per-launch pair would add its gap)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            for _ in range(warm):
                fn()
            torch.cuda.synchronize()
            a.record()
            for _ in range(steps):
                fn()
            b.record()
            torch.cuda.synchronize()
            us = a.elapsed_time(b) / steps * 1e3
            row[label] = {"us": round(us, 2), "mb": round(nbytes / 1e6, 2),
                          "gbps": round(nbytes / us / 1e3, 1),
                          "frac_of_hbm_peak": round(nbytes / us / 1e3 / PEAK_HBM_GBS, 4)}
        res.append(row)
    r0 = res[0]["rope_cache_write"]
    print(json.dumps({
        "metric": "cache write with rotary embedding fused: GB/s of the bytes it must move",
        "value": r0["gbps"], "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": warm,
        "ms_per_step": round(r0["us"] / 1e3, 5), "higher_is_better": True, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": res[0]["shape"] + "; RoPE theta 10000, rotate-half pairs"},
        "roofline": {"bound": "hbm", "achieved": r0["gbps"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": r0["frac_of_hbm_peak"], "traffic": recorded_traffic(ROPE_TRAFFIC_FILE),
                     "kernel": "prep_kernel<bf16,128,rope>"},
        "shapes": res,
    }), flush=True)


def main():
    args = _args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_probe:
        copy_probe()
        return
    if args.workload == "c5":
        run_long_prompt(args)
        return
    if args.workload == "c4":
        run_mixed_batch(args)
        return
    if args.workload == "rope":
        run_rope(args)
        return
    if args.workload == "c3":
        run_prefix_batch(args)
        return
    run_prompt(args)


class RunAhead:
    """Keeps the host at most `depth` steps ahead of the GPU: before a step
    is enqueued, the event recorded at the end of the step `depth` back is
    awaited.  A serving loop cannot run further ahead than its outputs allow;
    without a bound the host here enqueues dozens of steps ahead, and the
    runtime's one-time growth of its launch resources then stalls the host
    for ~30 ms with the GPU idle (and its clock falling back)."""

    def __init__(self, torch, depth=2):
        self.torch, self.depth, self.marks = torch, depth, []

    def before(self):
        if len(self.marks) >= self.depth:
            self.marks.pop(0).synchronize()

    def after(self):
        ev = self.torch.cuda.Event()
        ev.record()
        self.marks.append(ev)


def _steps(torch, bench, n):
    """n untimed steps under the run-ahead bound."""
    ra = RunAhead(torch)
    for _ in range(n):
        ra.before()
        bench.step()
        ra.after()


def _clock_warmup(torch, bench, seconds):
    """Untimed steps until `seconds` of wall time have passed, the GPU kept
    busy throughout: the shader clock of an idle MI355X measures ~2.18 GHz
    and climbs to ~2.43 GHz over the first ~0.1 s of continuous work, so a
    short warmup would time the climb.  Returns (steps, seconds)."""
    if seconds <= 0:
        return 0, 0.0
    ra = RunAhead(torch)
    n = 0
    t0 = time.perf_counter()
    while True:
        ra.before()
        bench.step()
        ra.after()
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= seconds:
                break
    torch.cuda.synchronize()
    return n, time.perf_counter() - t0


def _timed_steps(torch, args, bench):
    """K timed steps with the per-launch attention events; returns (wall
    seconds, attention ms summed over launches, mean ms per chunk)."""
    if args.event_timing == "dispatch":
        hip = HipEvents()
        events = [[(hip.create(), hip.create()) for _ in bench.chunks] for _ in range(args.steps)]
        elapsed_ms = hip.elapsed_ms
    else:
        events = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in bench.chunks] for _ in range(args.steps)]
        elapsed_ms = lambda a, b: a.elapsed_time(b)   # noqa: E731
    torch.cuda.synchronize()
    ra = RunAhead(torch)
    t0 = time.perf_counter()
    for s in range(args.steps):
        ev = [list(p) for p in events[s]]
        ra.before()
        bench.step(ev)
        ra.after()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    attn_ms = sum(elapsed_ms(a, b) for step in events for (a, b) in step)
    per_chunk_ms = [sum(elapsed_ms(*events[s][i]) for s in range(args.steps))
                    / args.steps for i in range(len(bench.chunks))]
    if args.event_timing == "dispatch":
        for step in events:
            for a, b in step:
                hip.destroy(a)
                hip.destroy(b)
    return elapsed, attn_ms, per_chunk_ms


def run_prompt(args):
    """The 10k prompt (the headline line), or its tensor-parallel share."""
    import dataclasses

    import torch
    from synth import get_workload
    w = get_workload("c2")
    tp = args.workload == "c2tp"
    if tp:   # one GPU's share of an eight-way split by KV-head group
        w = dataclasses.replace(w, num_heads=w.num_heads // w.num_kv_heads, num_kv_heads=1)
    bench = PromptBench(args.kv_segment_size, args.split_keys_prefill, workload=w,
                        kv_fp8=args.kv_cache == "fp8")
    flops = bench.flops_per_step()
    # no collector pauses in the loops: a full collection over torch's heap
    # stalls the host ~30 ms, with the GPU idle, at an unpredictable step
    gc.collect()
    gc.freeze()
    gc.disable()
    cw_steps, cw_s = _clock_warmup(torch, bench, args.clock_warmup_s)
    _steps(torch, bench, args.warmup)
    torch.cuda.synchronize()
    elapsed, attn_ms, per_chunk_ms = _timed_steps(torch, args, bench)
    value = flops * args.steps / elapsed / 1e12
    achieved = flops * args.steps / (attn_ms / 1e3) / 1e12
    shape = f"H{w.num_heads}/G{w.num_kv_heads}/D{w.head_dim}"
    line = {
        "metric": "chunked-prefill attention TFLOP/s + % of bf16 MFMA peak (10k GQA prompt)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": ("10k-token GQA chunked prefill: chunks 2048x4+1808 (cached 0..8192), "
                         f"{shape}, block_size 128, kv_segment_size {args.kv_segment_size}"
                         + (", one KV-head group of eight (tensor-parallel share)" if tp else "")),
            "global_batch": 1, "seq_len": w.prompt_len, "parallelism": "none (1 GPU)",
            "kv_cache": args.kv_cache,
        },
        "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "gflop_per_step": round(flops / 1e9, 2),
        "attention_ms_per_chunk": [round(x, 4) for x in per_chunk_ms],
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": recorded_traffic() if args.kv_cache == "bf16" and not tp else None,
                     "kernel": "attn_kernel<bf16,128>",
                     "timing": ("HIP events taken by the attention kernel's dispatch "
                                "(hipExtLaunchKernel), every launch of the timed steps; the merge "
                                "launch of split rows follows them"
                                if args.event_timing == "dispatch" else
                                "HIP event records around every attention call of the timed steps")},
        "plan": [{"items": p["num_items"], "merge_rows": p["num_merge_rows"]} for p in bench.plan],
        "clock_warmup": {"steps": cw_steps, "seconds": round(cw_s, 3),
                         "why": "untimed steps before the warmup steps: an idle GPU's shader "
                                "clock ramps up over ~0.1 s of continuous work"},
    }
    if args.steady_warmup > 0:
        # the same measurement again after more untimed steps: the first
        # steps of a process run below the rate the GPU settles at
        _steps(torch, bench, args.steady_warmup)
        torch.cuda.synchronize()
        el2, attn2, chunks2 = _timed_steps(torch, args, bench)
        line["steady_state"] = {
            "untimed_steps_before": cw_steps + args.warmup + args.steps + args.steady_warmup,
            "value": round(flops * args.steps / el2 / 1e12, 2),
            "ms_per_step": round(el2 * 1e3 / args.steps, 4),
            "roofline_achieved": round(flops * args.steps / (attn2 / 1e3) / 1e12, 2),
            "attention_ms_per_chunk": [round(x, 4) for x in chunks2],
        }
    gc.enable()
    if not args.no_cpu_baseline and args.kv_cache == "bf16" and not tp:
        line["cpu_baseline"] = cpu_baseline(bench.w, bench.max_blocks)
    print(json.dumps(line), flush=True)


def run_prefix_batch(args):
    """Config 3: 16 requests share a 4096-token prefix held in 256 blocks
    (block size 16, reference counted); one varlen call computes their
    suffixes (16*U{16..32} tokens each) at cached_seq_len 4096: the cache
    write of the suffixes and the attention.  TFLOP/s over the algorithmic
    FLOPs of the call."""
    import torch
    from chunked_prefill_paged_amd import AttnCall, HostScheduler, cache_shapes
    from synth import config3_suffix_lengths, free_block_order, get_workload

    w = get_workload("c3")
    H, G, D, bs = w.num_heads, w.num_kv_heads, w.head_dim, w.block_size
    prefix = w.prompt_len
    suffix = [int(x) for x in config3_suffix_lengths(w)]
    nb = prefix // bs + sum(-(-x // bs) for x in suffix) + 64
    sched = HostScheduler(nb, bs, w.max_batched_tokens, -(-(prefix + 512) // bs),
                          free_order=free_block_order(nb, w.seed))
    sched.add_decode(999, prefix)                 # the request that computed the prefix
    shared = list(sched.request_blocks(999))
    for i, x in enumerate(suffix):
        sched.add_request(i, prefix + x, shared)
    sched.free_request(999)
    b = sched.step()
    T = int(b["num_tokens"])
    dev = "cuda"
    ks, vs = cache_shapes(nb, G, bs, D)
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed)
    k_cache = torch.randn(ks, generator=gen, device=dev).to(torch.bfloat16)
    v_cache = torch.randn(vs, generator=gen, device=dev).to(torch.bfloat16)
    q = torch.randn((T, H, D), generator=gen, device=dev).to(torch.bfloat16)
    kn = torch.randn((T, G, D), generator=gen, device=dev).to(torch.bfloat16)
    vn = torch.randn((T, G, D), generator=gen, device=dev).to(torch.bfloat16)
    out = torch.empty_like(q)
    d = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a, dtype=dt)).to(dev)   # noqa: E731
    call = AttnCall(q=q, k_new=kn, v_new=vn, k_cache=k_cache, v_cache=v_cache, out=out,
                    cu_seqlens_q=d(b["cu_seqlens_q"], np.int32),
                    cached_seq_len=d(b["cached_seq_len"], np.int32),
                    block_table=d(b["block_table"], np.int32), slot_mapping=None,
                    h_cu_seqlens_q=np.asarray(b["cu_seqlens_q"], np.int32),
                    h_cached_seq_len=np.asarray(b["cached_seq_len"], np.int32),
                    kv_segment_size=w.kv_segment_size, split_keys_prefill=args.split_keys_prefill)
    call.set_workspace(torch.empty(max(256, call.workspace_bytes()), dtype=torch.uint8, device=dev))
    flops = sum(4 * H * D * (x * prefix + x * (x + 1) // 2) for x in suffix)
    steps, warm = max(1, args.steps), max(1, args.warmup)
    t = _time_steps(torch, call, steps, warm)
    hip = HipEvents()
    evs = [(hip.create(), hip.create()) for _ in range(steps)]
    for a, e in evs:
        call.prepare()
        call.attention_timed(a, e)
    torch.cuda.synchronize()
    kern_ms = sum(hip.elapsed_ms(a, e) for a, e in evs) / steps
    for a, e in evs:
        hip.destroy(a)
        hip.destroy(e)
    value = flops / t / 1e12
    print(json.dumps({
        "metric": "prefix-cached batch: attention TFLOP/s over the suffixes (config 3)",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": steps, "warmup": warm,
        "ms_per_step": round(t * 1e3, 4), "higher_is_better": True, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"16 requests x suffix 16*U{{16..32}} ({T} tokens) over a shared "
                               f"4096-token prefix in 256 blocks, bs16, S{w.kv_segment_size}, "
                               f"H{H}/G{G}/D{D}"},
        "gflop_per_step": round(flops / 1e9, 2),
        "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(flops / (kern_ms / 1e3) / 1e12, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(flops / (kern_ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                     "traffic": None, "kernel": "attn_kernel<bf16,128>"},
    }), flush=True)


if __name__ == "__main__":
    main()

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

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline]
    python bench.py --copy-probe      # one plain 1 GiB device copy, for
                                      # calibrating HBM byte counters

The roofline's "traffic" is the attention kernel's HBM bytes per launch as
measured by hardware counters and recorded, with the hash of the kernel
sources it was measured on, in profiles/attn_kernel_10k_prompt_hbm_traffic.txt;
it is reported only while those sources are unchanged (null otherwise).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA (published)
PEAK_HBM_GBS = 8000.0
ROOT = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = ("chunked_prefill_paged_amd/csrc/cpa_attn.hip", "chunked_prefill_paged_amd/csrc/cpa_plan.h")
TRAFFIC_FILE = "profiles/attn_kernel_10k_prompt_hbm_traffic.txt"
COPY_PROBE_BYTES = 1 << 30


def _args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--kv-segment-size", type=int, default=1024)
    ap.add_argument("--split-keys-prefill", type=int, default=0,
                    help="0 automatic, -1 never, else keys per work item")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run a plain 1 GiB device-to-device copy 5 times and exit")
    return ap.parse_args()


def kernel_sources_sha256() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic():
    """HBM bytes per attention launch from the committed counter summary, or
    None when the kernel sources changed since it was measured."""
    path = os.path.join(ROOT, TRAFFIC_FILE)
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
    """The 10k-token prompt, its device buffers and the per-chunk calls."""

    def __init__(self, kv_segment_size, split_pre):
        import torch
        from chunked_prefill_paged_amd import AttnCall, HostScheduler, cache_shapes
        from synth import free_block_order, get_workload, prompt_qkv

        self.torch = torch
        w = get_workload("c2")
        self.w = w
        q32, k32, v32 = prompt_qkv(w)
        dev = "cuda"
        self.q = torch.from_numpy(q32).to(torch.bfloat16).to(dev)
        self.k = torch.from_numpy(k32).to(torch.bfloat16).to(dev)
        self.v = torch.from_numpy(v32).to(torch.bfloat16).to(dev)
        self.out = torch.empty_like(self.q)
        ks, vs = cache_shapes(w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim)
        self.k_cache = torch.zeros(ks, dtype=torch.bfloat16, device=dev)
        self.v_cache = torch.zeros(vs, dtype=torch.bfloat16, device=dev)
        self.max_blocks = -(-w.prompt_len // w.block_size)
        self.sched = HostScheduler(w.num_blocks, w.block_size, w.max_batched_tokens,
                                   self.max_blocks, free_order=free_block_order(w.num_blocks, w.seed))
        self.AttnCall = AttnCall
        self.S = kv_segment_size
        self.split_pre = split_pre
        self.rid = 0
        # chunk plan of the prompt (fixed): build one call per chunk index with
        # persistent device descriptor buffers and pinned host staging
        from chunked_prefill_paged_amd import schedule_prompt
        self.chunks = schedule_prompt(w.max_batched_tokens, 0, w.prompt_len)
        self.calls, self.dev_desc, self.pinned, self.copied = [], [], [], []
        pos = 0
        ws_bytes = 256
        for n in self.chunks:
            d_i32 = torch.zeros(2 + 1 + self.max_blocks, dtype=torch.int32, device=dev)
            d_i64 = torch.zeros(n, dtype=torch.int64, device=dev)
            p_i32 = torch.zeros(d_i32.shape, dtype=torch.int32, pin_memory=True)
            p_i64 = torch.zeros(d_i64.shape, dtype=torch.int64, pin_memory=True)
            call = AttnCall(q=self.q[pos:pos + n], k_new=self.k[pos:pos + n], v_new=self.v[pos:pos + n],
                            k_cache=self.k_cache, v_cache=self.v_cache, out=self.out[pos:pos + n],
                            cu_seqlens_q=d_i32[0:2], cached_seq_len=d_i32[2:3],
                            block_table=d_i32[3:].view(1, self.max_blocks), slot_mapping=d_i64,
                            h_cu_seqlens_q=np.array([0, n], np.int32),
                            h_cached_seq_len=np.array([pos], np.int32),
                            kv_segment_size=kv_segment_size, split_keys_prefill=split_pre)
            ws_bytes = max(ws_bytes, call.workspace_bytes())
            self.calls.append(call)
            self.dev_desc.append((d_i32, d_i64))
            self.pinned.append((p_i32, p_i64))
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
            p_i32, p_i64 = self.pinned[i]
            if self.copied[i] is not None:
                self.copied[i].synchronize()        # staging buffer of the previous step is free
            a32 = p_i32.numpy()
            a32[0:2] = b["cu_seqlens_q"]
            a32[2] = b["cached_seq_len"][0]
            a32[3:] = b["block_table"][0]
            p_i64.numpy()[:] = b["slot_mapping"]
            d_i32, d_i64 = self.dev_desc[i]
            d_i32.copy_(p_i32, non_blocking=True)
            d_i64.copy_(p_i64, non_blocking=True)
            ev = torch.cuda.Event()
            ev.record()
            self.copied[i] = ev
            call.args.h_cu_seqlens_q = b["cu_seqlens_q"].ctypes.data
            call.args.h_cached_seq_len = b["cached_seq_len"].ctypes.data
            call._keep_host = (b["cu_seqlens_q"], b["cached_seq_len"])
            call.prepare()
            if events is not None:
                events[i][0].record()
            call.attention()
            if events is not None:
                events[i][1].record()
            sched.commit()
        sched.free_request(self.rid)
        self.rid += 1


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
            "sample": f"{steps} whole steps: the 10k prompt's 5 chunks (2048x4 + 1808), all 32 "
                      "query heads, oracle scheduler + cache write + attention in numpy float64 "
                      f"({flops / 1e9:.2f} GFLOP)"}


def main():
    args = _args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_probe:
        copy_probe()
        return
    bench = PromptBench(args.kv_segment_size, args.split_keys_prefill)
    flops = bench.flops_per_step()
    for _ in range(args.warmup):
        bench.step()
    torch.cuda.synchronize()
    events = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in bench.chunks] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        ev = [list(p) for p in events[s]]
        bench.step(ev)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    attn_ms = sum(a.elapsed_time(b) for step in events for (a, b) in step)
    per_chunk_ms = [sum(events[s][i][0].elapsed_time(events[s][i][1]) for s in range(args.steps))
                    / args.steps for i in range(len(bench.chunks))]
    value = flops * args.steps / elapsed / 1e12
    achieved = flops * args.steps / (attn_ms / 1e3) / 1e12
    w = bench.w
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
            "workload": "10k-token GQA chunked prefill: chunks 2048x4+1808 (cached 0..8192), "
                        f"H32/G8/D128, block_size 128, kv_segment_size {args.kv_segment_size}",
            "global_batch": 1, "seq_len": w.prompt_len, "parallelism": "none (1 GPU)",
        },
        "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "gflop_per_step": round(flops / 1e9, 2),
        "attention_ms_per_chunk": [round(x, 4) for x in per_chunk_ms],
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": recorded_traffic(),
                     "kernel": "attn_kernel<bf16,128> (+ merge_kernel when rows are split)"},
        "plan": [{"items": p["num_items"], "merge_rows": p["num_merge_rows"]} for p in bench.plan],
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(bench.w, bench.max_blocks)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

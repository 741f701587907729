"""The five synthetic workloads and their seeded draws.

Shapes follow the chunked-prefill pages: a 10,000-token prompt chunked at
2048 (Neuron "Prefill Processing" page, section "Prefill Segmentation"), a
32k prompt chunked at 2048 with block_size 16 (vLLM chunked-prefill KV page,
section 2.1), GQA 32/8 with head_dim 128 (prefill-optimisation tutorial,
section 6).  No public dataset is involved; every value is drawn here.

Rules
-----
* Host draws use ``numpy.random.default_rng(seed)`` in float32, then the
  caller casts (torch ``.to(bfloat16)`` rounds to nearest even).
* Per-sequence substreams use ``seed * 100000 + index`` so one sequence can be
  regenerated without the others.
* Block ids are handed out from a seeded permutation of the pool
  (``free_block_order``), which scatters every table across the pool.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str              # "fp32" or "bf16"
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    kv_segment_size: int
    seed: int
    input_std: float        # standard deviation of Q, K, V draws
    prompt_len: int = 0     # single-prompt workloads (1, 2, 5)
    max_batched_tokens: int = 0
    num_blocks: int = 0     # pool size when fixed by the workload (0: derived)
    description: str = ""

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def group(self) -> int:
        return self.num_heads // self.num_kv_heads


WORKLOADS = {
    "c1": Workload(
        name="c1", dtype="fp32", num_heads=4, num_kv_heads=4, head_dim=64,
        block_size=16, kv_segment_size=512, seed=1001, input_std=1.0 / 8.0,
        prompt_len=1024, max_batched_tokens=256, num_blocks=128,
        description="fp32, H=G=4, D=64, 1024-token prompt in 4 chunks of 256, "
                    "bs16, S512, pool 128 blocks (seeded permutation)"),
    "c2": Workload(
        name="c2", dtype="bf16", num_heads=32, num_kv_heads=8, head_dim=128,
        block_size=128, kv_segment_size=1024, seed=1002, input_std=1.0,
        prompt_len=10000, max_batched_tokens=2048, num_blocks=96,
        description="bf16, 10,000-token prompt, budget 2048 (chunks 4x2048+1808), "
                    "bs128, S1024, GQA 32/8, D128"),
    "c3": Workload(
        name="c3", dtype="bf16", num_heads=32, num_kv_heads=8, head_dim=128,
        block_size=16, kv_segment_size=1024, seed=1003, input_std=1.0,
        prompt_len=4096, max_batched_tokens=16384,
        description="bf16, 16 requests sharing a 4096-token prefix (256 shared "
                    "blocks, bs16), suffix 16*U{16..32}, GQA 32/8, D128, S1024"),
    "c4": Workload(
        name="c4", dtype="bf16", num_heads=32, num_kv_heads=8, head_dim=128,
        block_size=16, kv_segment_size=2048, seed=1004, input_std=1.0,
        prompt_len=32768, max_batched_tokens=2048,
        description="bf16, 256 decodes (context 16*U{64..2048}) + 1792-token chunk "
                    "of a 32,768-token prompt at cached 30,720, budget 2048, bs16, "
                    "S2048, GQA 32/8, D128, pool ceil(1.2 x demand)"),
    "c5": Workload(
        name="c5", dtype="bf16", num_heads=64, num_kv_heads=8, head_dim=128,
        block_size=16, kv_segment_size=4096, seed=1005, input_std=1.0,
        prompt_len=32768, max_batched_tokens=2048, num_blocks=2048,
        description="bf16, 32,768-token prompt in 16 chunks of 2048, bs16, S4096, "
                    "GQA 64/8, D128"),
}


def get_workload(name: str) -> Workload:
    return WORKLOADS[name]


def draw_normal(seed: int, shape, std: float = 1.0) -> np.ndarray:
    """float32 draws N(0, std^2) from ``default_rng(seed)``."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def prompt_qkv(w: Workload, prompt_len: int | None = None, seed: int | None = None):
    """Q [P, H, D], K [P, G, D], V [P, G, D] float32 for a whole prompt.

    Drawn once and sliced per chunk, so chunked and monolithic runs see
    identical values.  Three substreams: seed*10+0 (Q), +1 (K), +2 (V).
    """
    p = w.prompt_len if prompt_len is None else prompt_len
    s = w.seed if seed is None else seed
    q = draw_normal(s * 10 + 0, (p, w.num_heads, w.head_dim), w.input_std)
    k = draw_normal(s * 10 + 1, (p, w.num_kv_heads, w.head_dim), w.input_std)
    v = draw_normal(s * 10 + 2, (p, w.num_kv_heads, w.head_dim), w.input_std)
    return q, k, v


def free_block_order(num_blocks: int, seed: int) -> np.ndarray:
    """Seeded permutation of block ids 0..num_blocks-1 (int32): the order in
    which a pool hands out its free blocks."""
    rng = np.random.default_rng(seed)
    return rng.permutation(num_blocks).astype(np.int32)


def config3_suffix_lengths(w: Workload, num_requests: int = 16) -> np.ndarray:
    """Suffix lengths 16*U{16..32}: uniform over the 17 multiples of 16 in
    [256, 512]."""
    rng = np.random.default_rng(w.seed * 100000 + 99999)
    return (16 * rng.integers(16, 33, size=num_requests)).astype(np.int64)


def config4_decode_contexts(w: Workload, num_decodes: int = 256) -> np.ndarray:
    """Decode context lengths 16*U{64..2048}: uniform in [1024, 32768] and
    block-aligned to 16."""
    rng = np.random.default_rng(w.seed * 100000 + 99999)
    return (16 * rng.integers(64, 2049, size=num_decodes)).astype(np.int64)

"""Python face of the host scheduler entry points (marshalling only)."""
from __future__ import annotations

import ctypes
import weakref

import numpy as np

from . import _lib


def _i32p(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _i64p(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))


def schedule_prompt(max_batched_tokens: int, active_decodes: int, total_prompt_tokens: int,
                    block_size: int = 0, align_to_block: bool = False, capacity: int = 1 << 16):
    """Chunk sizes of one prompt (see cpa_schedule_prompt)."""
    buf = np.zeros(capacity, dtype=np.int32)
    n = ctypes.c_int32()
    st = _lib.lib().cpa_schedule_prompt(max_batched_tokens, active_decodes, total_prompt_tokens,
                                        block_size, int(bool(align_to_block)), _i32p(buf), capacity,
                                        ctypes.byref(n))
    _lib.check(st, "cpa_schedule_prompt")
    return buf[:n.value].tolist()


class HostScheduler:
    """Decode-first token-budget scheduler with a paged block pool."""

    def __init__(self, num_blocks: int, block_size: int, max_batched_tokens: int,
                 max_blocks_per_seq: int, long_prefill_cap: int = 0, align_to_block: bool = False,
                 free_order=None, prefix_caching: bool = False,
                 max_long_partial_prefills: int = 0, preemption: bool = False):
        self.block_size = block_size
        self.max_blocks = max_blocks_per_seq
        self.budget = max_batched_tokens
        cfg = _lib.SchedConfig()
        cfg.num_blocks = num_blocks
        cfg.block_size = block_size
        cfg.max_batched_tokens = max_batched_tokens
        cfg.max_blocks_per_seq = max_blocks_per_seq
        cfg.long_prefill_cap = long_prefill_cap
        cfg.align_to_block = int(bool(align_to_block))
        cfg.prefix_caching = int(bool(prefix_caching))
        cfg.max_long_partial_prefills = max_long_partial_prefills
        cfg.preemption = int(bool(preemption))
        self._order = None
        if free_order is not None:
            self._order = np.ascontiguousarray(free_order, dtype=np.int32)
            cfg.free_order = _i32p(self._order)
        handle = ctypes.c_void_p()
        _lib.check(_lib.lib().cpa_sched_create(ctypes.byref(cfg), ctypes.byref(handle)),
                   "cpa_sched_create")
        self._h = handle
        self._max_seqs = 0
        # released when the object is collected or, at the latest, at
        # interpreter exit while the library is still loaded
        self._release = weakref.finalize(self, _lib.lib().cpa_sched_destroy, handle)

    def add_request(self, req_id: int, num_prompt_tokens: int, prefix_blocks=()):
        blocks = np.ascontiguousarray(prefix_blocks, dtype=np.int32)
        _lib.check(_lib.lib().cpa_sched_add_request(self._h, req_id, num_prompt_tokens,
                                                    _i32p(blocks), len(blocks)),
                   "cpa_sched_add_request")
        self._max_seqs += 1

    def add_request_tokens(self, req_id: int, tokens, namespace: str = "default"):
        """A prompt given by its token ids (prefix caching matches and
        registers its full blocks)."""
        t = np.ascontiguousarray(tokens, dtype=np.uint32)
        _lib.check(_lib.lib().cpa_sched_add_request_tokens(
            self._h, req_id, t.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32)), len(t),
            namespace.encode("utf-8")), "cpa_sched_add_request_tokens")
        self._max_seqs += 1

    def add_decode(self, req_id: int, context_len: int):
        _lib.check(_lib.lib().cpa_sched_add_decode(self._h, req_id, context_len),
                   "cpa_sched_add_decode")
        self._max_seqs += 1

    def add_partial(self, req_id: int, num_prompt_tokens: int, num_computed_tokens: int):
        _lib.check(_lib.lib().cpa_sched_add_partial(self._h, req_id, num_prompt_tokens,
                                                    num_computed_tokens), "cpa_sched_add_partial")
        self._max_seqs += 1

    def step(self) -> dict:
        """Next step's batch descriptor as numpy arrays."""
        ms = max(1, self._max_seqs)
        out = {
            "req_ids": np.zeros(ms, dtype=np.int64),
            "q_lens": np.zeros(ms, dtype=np.int32),
            "cu_seqlens_q": np.zeros(ms + 1, dtype=np.int32),
            "cached_seq_len": np.zeros(ms, dtype=np.int32),
            "block_table": np.zeros((ms, self.max_blocks), dtype=np.int32),
            "slot_mapping": np.zeros(self.budget, dtype=np.int64),
        }
        b = _lib.Batch()
        b.max_seqs, b.max_tokens = ms, self.budget
        b.req_ids, b.q_lens = _i64p(out["req_ids"]), _i32p(out["q_lens"])
        b.cu_seqlens_q, b.cached_seq_len = _i32p(out["cu_seqlens_q"]), _i32p(out["cached_seq_len"])
        b.block_table, b.slot_mapping = _i32p(out["block_table"]), _i64p(out["slot_mapping"])
        _lib.check(_lib.lib().cpa_sched_step(self._h, ctypes.byref(b)), "cpa_sched_step")
        s, t = b.num_seqs, b.num_tokens
        return {"req_ids": out["req_ids"][:s], "q_lens": out["q_lens"][:s],
                "cu_seqlens_q": out["cu_seqlens_q"][:s + 1],
                "cached_seq_len": out["cached_seq_len"][:s],
                "block_table": out["block_table"][:s], "slot_mapping": out["slot_mapping"][:t],
                "num_seqs": s, "num_tokens": t}

    def last_preempted(self) -> list:
        """Ids of the requests the last step preempted."""
        buf = np.zeros(max(1, self._max_seqs), dtype=np.int64)
        n = ctypes.c_int32()
        _lib.check(_lib.lib().cpa_sched_last_preempted(self._h, _i64p(buf), len(buf),
                                                       ctypes.byref(n)), "cpa_sched_last_preempted")
        return buf[:n.value].tolist()

    def commit(self):
        _lib.check(_lib.lib().cpa_sched_commit(self._h), "cpa_sched_commit")

    def free_request(self, req_id: int):
        _lib.check(_lib.lib().cpa_sched_free_request(self._h, req_id), "cpa_sched_free_request")

    def request_info(self, req_id: int) -> dict:
        v = [ctypes.c_int32() for _ in range(4)]
        _lib.check(_lib.lib().cpa_sched_request_info(self._h, req_id, *(ctypes.byref(x) for x in v)),
                   "cpa_sched_request_info")
        return {"num_tokens": v[0].value, "num_computed": v[1].value, "num_blocks": v[2].value,
                "is_decode": bool(v[3].value)}

    def request_blocks(self, req_id: int):
        nb = self.request_info(req_id)["num_blocks"]
        buf = np.zeros(max(1, nb), dtype=np.int32)
        n = ctypes.c_int32()
        _lib.check(_lib.lib().cpa_sched_request_blocks(self._h, req_id, _i32p(buf), len(buf),
                                                       ctypes.byref(n)), "cpa_sched_request_blocks")
        return buf[:n.value]

    def slots(self, req_id: int, pos0: int, n: int):
        buf = np.zeros(max(1, n), dtype=np.int64)
        _lib.check(_lib.lib().cpa_sched_slots(self._h, req_id, pos0, n, _i64p(buf)), "cpa_sched_slots")
        return buf[:n]

    def num_free_blocks(self) -> int:
        v = ctypes.c_int32()
        _lib.check(_lib.lib().cpa_sched_num_free_blocks(self._h, ctypes.byref(v)),
                   "cpa_sched_num_free_blocks")
        return v.value

    def pool_stats(self) -> dict:
        v = [ctypes.c_int32() for _ in range(3)]
        _lib.check(_lib.lib().cpa_sched_pool_stats(self._h, *(ctypes.byref(x) for x in v)),
                   "cpa_sched_pool_stats")
        return {"active": v[0].value, "reclaimable": v[1].value, "empty": v[2].value}

    def prefix_match(self, tokens, namespace: str = "default") -> int:
        """Cached tokens (whole blocks) a prompt would match now."""
        t = np.ascontiguousarray(tokens, dtype=np.uint32)
        n = ctypes.c_int32()
        _lib.check(_lib.lib().cpa_sched_prefix_match(
            self._h, t.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32)), len(t),
            namespace.encode("utf-8"), ctypes.byref(n)), "cpa_sched_prefix_match")
        return n.value

    def refcount(self, block: int) -> int:
        v = ctypes.c_int32()
        _lib.check(_lib.lib().cpa_sched_block_refcount(self._h, block, ctypes.byref(v)),
                   "cpa_sched_block_refcount")
        return v.value

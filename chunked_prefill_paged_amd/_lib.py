"""ctypes view of libchunked_prefill_attn (include/chunked_prefill_attn.h).

Argument marshalling only: every step of the path runs in the library.  The
library must have been built (``python -m chunked_prefill_paged_amd.build``);
there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libchunked_prefill_attn.so")

CPA_OK = 0
CPA_ERR_INVALID_ARG = 1
CPA_ERR_UNSUPPORTED = 2
CPA_ERR_BUDGET_EXHAUSTED = 3
CPA_ERR_OUT_OF_BLOCKS = 4
CPA_ERR_HIP = 5
CPA_ERR_WORKSPACE = 6
CPA_ERR_NOT_FOUND = 7
CPA_INLINE_DESC_INTS = 896      # largest batch descriptor the launches take inline (int32s)

CPA_BF16 = 0
CPA_FP32 = 1
CPA_FP8_E4M3 = 2

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_p_i32 = ctypes.POINTER(ctypes.c_int32)
_p_i64 = ctypes.POINTER(ctypes.c_int64)


class AttnArgs(ctypes.Structure):
    _fields_ = [
        ("dtype", _i32), ("num_seqs", _i32), ("total_q", _i32), ("num_heads", _i32),
        ("num_kv_heads", _i32), ("head_dim", _i32), ("block_size", _i32),
        ("kv_segment_size", _i32), ("max_blocks_per_seq", _i32), ("num_blocks", _i32),
        ("decode_token_threshold", _i32), ("split_keys_prefill", _i32),
        ("split_keys_decode", _i32), ("scale", ctypes.c_float),
        ("q", _vp), ("k_new", _vp), ("v_new", _vp), ("k_cache", _vp), ("v_cache", _vp),
        ("cu_seqlens_q", _vp), ("cached_seq_len", _vp), ("block_table", _vp),
        ("slot_mapping", _vp), ("out", _vp), ("lse", _vp), ("workspace", _vp),
        ("workspace_bytes", ctypes.c_size_t), ("h_cu_seqlens_q", _vp), ("h_cached_seq_len", _vp),
        ("kv_dtype", _i32), ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float),
        ("h_block_table", _vp),
    ]


class RopeArgs(ctypes.Structure):
    _fields_ = [("theta", ctypes.c_float), ("interleaved", _i32), ("q_out", _vp)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("num_items", _i32), ("num_merge_rows", _i32), ("num_partials", _i64),
                ("split_keys_prefill", _i32), ("split_keys_decode", _i32),
                ("workspace_bytes", ctypes.c_size_t)]


class SchedConfig(ctypes.Structure):
    _fields_ = [("num_blocks", _i32), ("block_size", _i32), ("max_batched_tokens", _i32),
                ("max_blocks_per_seq", _i32), ("long_prefill_cap", _i32),
                ("align_to_block", _i32), ("free_order", _p_i32), ("prefix_caching", _i32),
                ("max_long_partial_prefills", _i32), ("preemption", _i32)]


class Batch(ctypes.Structure):
    _fields_ = [("max_seqs", _i32), ("max_tokens", _i32), ("req_ids", _p_i64),
                ("q_lens", _p_i32), ("cu_seqlens_q", _p_i32), ("cached_seq_len", _p_i32),
                ("block_table", _p_i32), ("slot_mapping", _p_i64), ("num_seqs", _i32),
                ("num_tokens", _i32)]


# every function the header declares, with its ctypes signature
SIGNATURES = {
    "cpa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "cpa_abi_version": (ctypes.c_int, []),
    "cpa_check_args": (ctypes.c_int, [ctypes.POINTER(AttnArgs)]),
    "cpa_plan_counts": (ctypes.c_int, [ctypes.POINTER(AttnArgs), ctypes.POINTER(PlanInfo)]),
    "cpa_workspace_bytes": (ctypes.c_int, [ctypes.POINTER(AttnArgs), ctypes.POINTER(ctypes.c_size_t)]),
    "cpa_reshape_and_cache": (ctypes.c_int, [ctypes.POINTER(AttnArgs), _vp]),
    "cpa_prepare": (ctypes.c_int, [ctypes.POINTER(AttnArgs), _vp]),
    "cpa_attention": (ctypes.c_int, [ctypes.POINTER(AttnArgs), _vp]),
    "cpa_attention_timed": (ctypes.c_int, [ctypes.POINTER(AttnArgs), _vp, _vp, _vp]),
    "cpa_chunked_prefill_attn": (ctypes.c_int, [ctypes.POINTER(AttnArgs), _vp]),
    "cpa_chunked_prefill_attn_noalloc": (ctypes.c_int, [ctypes.POINTER(AttnArgs), _vp]),
    "cpa_rope_reshape_and_cache": (ctypes.c_int, [ctypes.POINTER(AttnArgs), ctypes.POINTER(RopeArgs), _vp]),
    "cpa_rope_prepare": (ctypes.c_int, [ctypes.POINTER(AttnArgs), ctypes.POINTER(RopeArgs), _vp]),
    "cpa_rope_chunked_prefill_attn": (ctypes.c_int, [ctypes.POINTER(AttnArgs), ctypes.POINTER(RopeArgs), _vp]),
    "cpa_schedule_prompt": (ctypes.c_int, [_i32, _i32, _i64, _i32, _i32, _p_i32, _i32, _p_i32]),
    "cpa_sched_create": (ctypes.c_int, [ctypes.POINTER(SchedConfig), ctypes.POINTER(_vp)]),
    "cpa_sched_destroy": (None, [_vp]),
    "cpa_sched_add_request": (ctypes.c_int, [_vp, _i64, _i32, _p_i32, _i32]),
    "cpa_sched_add_request_tokens": (ctypes.c_int, [_vp, _i64, ctypes.POINTER(ctypes.c_uint32), _i32,
                                                    ctypes.c_char_p]),
    "cpa_sched_add_decode": (ctypes.c_int, [_vp, _i64, _i32]),
    "cpa_sched_add_partial": (ctypes.c_int, [_vp, _i64, _i32, _i32]),
    "cpa_sched_step": (ctypes.c_int, [_vp, ctypes.POINTER(Batch)]),
    "cpa_sched_commit": (ctypes.c_int, [_vp]),
    "cpa_sched_last_preempted": (ctypes.c_int, [_vp, _p_i64, _i32, _p_i32]),
    "cpa_sched_free_request": (ctypes.c_int, [_vp, _i64]),
    "cpa_sched_request_info": (ctypes.c_int, [_vp, _i64, _p_i32, _p_i32, _p_i32, _p_i32]),
    "cpa_sched_request_blocks": (ctypes.c_int, [_vp, _i64, _p_i32, _i32, _p_i32]),
    "cpa_sched_slots": (ctypes.c_int, [_vp, _i64, _i32, _i32, _p_i64]),
    "cpa_sched_num_free_blocks": (ctypes.c_int, [_vp, _p_i32]),
    "cpa_sched_block_refcount": (ctypes.c_int, [_vp, _i32, _p_i32]),
    "cpa_sched_pool_stats": (ctypes.c_int, [_vp, _p_i32, _p_i32, _p_i32]),
    "cpa_sched_prefix_match": (ctypes.c_int, [_vp, ctypes.POINTER(ctypes.c_uint32), _i32,
                                              ctypes.c_char_p, _p_i32]),
}


class CpaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class BudgetExhausted(CpaError):
    pass


class OutOfBlocks(CpaError):
    pass


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it was not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m chunked_prefill_paged_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_string(status: int) -> str:
    return lib().cpa_status_string(status).decode()


def check(status: int, where: str) -> None:
    if status == CPA_OK:
        return
    if status == CPA_ERR_BUDGET_EXHAUSTED:
        raise BudgetExhausted(status, where)
    if status == CPA_ERR_OUT_OF_BLOCKS:
        raise OutOfBlocks(status, where)
    raise CpaError(status, where)

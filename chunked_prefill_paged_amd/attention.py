"""Python face of the attention entry points (marshalling only).

``AttnCall`` fills the C struct from torch tensors (device pointers) and
numpy host mirrors, keeps them alive, and forwards to the library on the
current torch stream.  It allocates nothing on the device itself: the caller
passes the workspace (``AttnCall.workspace_bytes()`` tells its size).
"""
from __future__ import annotations

import ctypes

import numpy as np

from . import _lib

_DTYPES = {"bfloat16": _lib.CPA_BF16, "float32": _lib.CPA_FP32}


_FP8_CACHE = ("uint8", "float8_e4m3fn")     # one-byte E4M3 codes


def _dtype_code(t) -> int:
    name = str(t.dtype).replace("torch.", "")
    if name not in _DTYPES:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return _DTYPES[name]


def _is_fp8_cache(t) -> bool:
    return str(t.dtype).replace("torch.", "") in _FP8_CACHE


def _ptr(t) -> int:
    if t is None:
        return 0
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is not None:
        return int(stream)
    import torch
    return int(torch.cuda.current_stream().cuda_stream)


def cache_shapes(num_blocks: int, num_kv_heads: int, block_size: int, head_dim: int):
    """Shapes of (k_cache, v_cache): K rows per block and head, V stored
    transposed per block and head."""
    return ((num_blocks, num_kv_heads, block_size, head_dim),
            (num_blocks, num_kv_heads, head_dim, block_size))


INLINE_DESC_INTS = _lib.CPA_INLINE_DESC_INTS


class AttnCall:
    """One batch's attention metadata bound to its tensors."""

    def __init__(self, *, q, k_new, v_new, k_cache, v_cache, out, cu_seqlens_q,
                 cached_seq_len, block_table, slot_mapping, h_cu_seqlens_q,
                 h_cached_seq_len, kv_segment_size, scale=None, lse=None, workspace=None,
                 decode_token_threshold=0, split_keys_prefill=0, split_keys_decode=0,
                 k_scale=1.0, v_scale=1.0, h_block_table=None):
        """A cache of one-byte elements (uint8 or float8_e4m3fn) holds E4M3
        codes under per-tensor scales ``k_scale`` / ``v_scale``; the other
        tensors are then bfloat16.  ``h_block_table`` (host int32 [num_seqs,
        max_blocks]) lets the launches carry the batch descriptor in their
        own arguments when it fits ``INLINE_DESC_INTS``; the device
        ``cu_seqlens_q``, ``cached_seq_len`` and ``block_table`` may then be
        None."""
        num_blocks, num_kv_heads, block_size, head_dim = k_cache.shape
        if tuple(v_cache.shape) != (num_blocks, num_kv_heads, head_dim, block_size):
            raise ValueError(f"v_cache must be {(num_blocks, num_kv_heads, head_dim, block_size)}")
        total_q = k_new.shape[0]
        num_heads = q.shape[1] if q is not None else num_kv_heads
        h_cu = np.ascontiguousarray(h_cu_seqlens_q, dtype=np.int32)
        h_cached = np.ascontiguousarray(h_cached_seq_len, dtype=np.int32)
        h_bt = None if h_block_table is None else np.ascontiguousarray(h_block_table, dtype=np.int32)
        if h_bt is not None and (h_bt.ndim != 2 or h_bt.shape[0] != len(h_cu) - 1):
            raise ValueError("h_block_table must be [num_seqs, max_blocks]")
        self._keep = [q, k_new, v_new, k_cache, v_cache, out, cu_seqlens_q, cached_seq_len,
                      block_table, slot_mapping, lse, h_cu, h_cached, h_bt]
        for t in (cu_seqlens_q, cached_seq_len, block_table):
            if t is not None and str(t.dtype) != "torch.int32":
                raise TypeError("cu_seqlens_q, cached_seq_len and block_table must be int32")
        if slot_mapping is not None and str(slot_mapping.dtype) != "torch.int64":
            raise TypeError("slot_mapping must be int64")
        a = _lib.AttnArgs()
        if _is_fp8_cache(k_cache):
            a.dtype = _dtype_code(k_new)
            a.kv_dtype = _lib.CPA_FP8_E4M3
            a.k_scale, a.v_scale = float(k_scale), float(v_scale)
        else:
            a.dtype = _dtype_code(k_cache)
        a.num_seqs = len(h_cu) - 1
        a.total_q = total_q
        a.num_heads = num_heads
        a.num_kv_heads = num_kv_heads
        a.head_dim = head_dim
        a.block_size = block_size
        a.kv_segment_size = kv_segment_size
        a.max_blocks_per_seq = (block_table.shape[1] if block_table is not None
                                else h_bt.shape[1] if h_bt is not None else 1)
        a.num_blocks = num_blocks
        a.decode_token_threshold = decode_token_threshold
        a.split_keys_prefill = split_keys_prefill
        a.split_keys_decode = split_keys_decode
        a.scale = float(scale if scale is not None else head_dim ** -0.5)
        a.q, a.k_new, a.v_new = _ptr(q), _ptr(k_new), _ptr(v_new)
        a.k_cache, a.v_cache = _ptr(k_cache), _ptr(v_cache)
        a.cu_seqlens_q, a.cached_seq_len = _ptr(cu_seqlens_q), _ptr(cached_seq_len)
        a.block_table, a.slot_mapping = _ptr(block_table), _ptr(slot_mapping)
        a.out, a.lse = _ptr(out), _ptr(lse)
        a.h_cu_seqlens_q = h_cu.ctypes.data
        a.h_cached_seq_len = h_cached.ctypes.data
        a.h_block_table = h_bt.ctypes.data if h_bt is not None else None
        self.args = a
        if workspace is not None:
            self.set_workspace(workspace)

    def set_workspace(self, workspace) -> None:
        self._workspace = workspace
        self.args.workspace = _ptr(workspace)
        self.args.workspace_bytes = workspace.numel() * workspace.element_size()

    def plan_info(self) -> dict:
        info = _lib.PlanInfo()
        _lib.check(_lib.lib().cpa_plan_counts(ctypes.byref(self.args), ctypes.byref(info)),
                   "cpa_plan_counts")
        return {f: getattr(info, f) for f, _ in info._fields_}

    def workspace_bytes(self) -> int:
        n = ctypes.c_size_t()
        _lib.check(_lib.lib().cpa_workspace_bytes(ctypes.byref(self.args), ctypes.byref(n)),
                   "cpa_workspace_bytes")
        return n.value

    def check(self) -> None:
        _lib.check(_lib.lib().cpa_check_args(ctypes.byref(self.args)), "cpa_check_args")

    def reshape_and_cache(self, stream=None) -> None:
        _lib.check(_lib.lib().cpa_reshape_and_cache(ctypes.byref(self.args), _stream(stream)),
                   "cpa_reshape_and_cache")

    def prepare(self, stream=None) -> None:
        _lib.check(_lib.lib().cpa_prepare(ctypes.byref(self.args), _stream(stream)), "cpa_prepare")

    def attention(self, stream=None) -> None:
        _lib.check(_lib.lib().cpa_attention(ctypes.byref(self.args), _stream(stream)),
                   "cpa_attention")

    def attention_timed(self, start_event, stop_event, stream=None) -> None:
        """attention() with the kernel's dispatch taking two raw hipEvent_t
        handles (ints): their elapsed time is the kernel's duration."""
        _lib.check(_lib.lib().cpa_attention_timed(ctypes.byref(self.args), _stream(stream),
                                                  start_event, stop_event), "cpa_attention_timed")

    def __call__(self, stream=None) -> None:
        _lib.check(_lib.lib().cpa_chunked_prefill_attn(ctypes.byref(self.args), _stream(stream)),
                   "cpa_chunked_prefill_attn")

    def call_noalloc(self, stream=None) -> None:
        """The whole chunk step on the library's own per-GPU scratch (the
        workspace set here is not used)."""
        _lib.check(_lib.lib().cpa_chunked_prefill_attn_noalloc(ctypes.byref(self.args),
                                                               _stream(stream)),
                   "cpa_chunked_prefill_attn_noalloc")

    # rotary position embedding fused into the cache write (``rope`` is a
    # ``Rope``); the rotated queries land in ``rope.q_out``
    def rope_reshape_and_cache(self, rope, stream=None) -> None:
        _lib.check(_lib.lib().cpa_rope_reshape_and_cache(ctypes.byref(self.args),
                                                         ctypes.byref(rope.args), _stream(stream)),
                   "cpa_rope_reshape_and_cache")

    def rope_prepare(self, rope, stream=None) -> None:
        _lib.check(_lib.lib().cpa_rope_prepare(ctypes.byref(self.args), ctypes.byref(rope.args),
                                               _stream(stream)), "cpa_rope_prepare")

    def rope_call(self, rope, stream=None) -> None:
        _lib.check(_lib.lib().cpa_rope_chunked_prefill_attn(ctypes.byref(self.args),
                                                            ctypes.byref(rope.args),
                                                            _stream(stream)),
                   "cpa_rope_chunked_prefill_attn")


class Rope:
    """Rotary-embedding parameters: base ``theta``, pairing (``interleaved``
    False: element i with i + D/2; True: 2i with 2i + 1) and the tensor that
    receives the rotated queries (may be the query tensor itself)."""

    def __init__(self, q_out, theta: float = 10000.0, interleaved: bool = False):
        self._keep = q_out
        self.args = _lib.RopeArgs()
        self.args.theta = float(theta)
        self.args.interleaved = 1 if interleaved else 0
        self.args.q_out = _ptr(q_out)

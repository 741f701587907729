"""The C-ABI library loads, exports every function include/*.h declares, and
refuses bad host-visible arguments before touching the device.  CPU only: no
call here launches a kernel."""
import ctypes
import glob
import os
import re

import numpy as np
import pytest

from chunked_prefill_paged_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for path in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(path).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"\b(cpa_[a-z0-9_]+)\s*\(", text):
            names.add(m.group(1))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    lib = _lib.lib()
    declared = _declared_functions()
    assert len(declared) >= 20
    for name in declared:
        assert hasattr(lib, name), f"{name} declared but not exported"
    assert set(declared) == set(_lib.SIGNATURES), "binding and header disagree"
    assert lib.cpa_abi_version() == 3


def test_status_strings():
    for code in range(8):
        assert _lib.status_string(code) != "unknown status"
    assert _lib.status_string(99) == "unknown status"


def _args(**over):
    a = _lib.AttnArgs()
    a.dtype, a.num_seqs, a.total_q, a.num_heads, a.num_kv_heads = 0, 2, 300, 32, 8
    a.head_dim, a.block_size, a.kv_segment_size = 128, 16, 1024
    a.max_blocks_per_seq, a.num_blocks, a.scale = 200, 1000, 128 ** -0.5
    cu = np.array([0, 100, 300], dtype=np.int32)
    cached = np.array([1000, 0], dtype=np.int32)
    keep = [cu, cached]
    fake = 0x1000   # never dereferenced: only host checks run here
    for f in ("q", "k_new", "v_new", "k_cache", "v_cache", "cu_seqlens_q", "cached_seq_len",
              "block_table", "slot_mapping", "out"):
        setattr(a, f, fake)
    for k, v in over.items():
        if k == "cu":
            cu = np.asarray(v, dtype=np.int32); keep.append(cu)
        elif k == "cached":
            cached = np.asarray(v, dtype=np.int32); keep.append(cached)
        else:
            setattr(a, k, v)
    a.h_cu_seqlens_q, a.h_cached_seq_len = cu.ctypes.data, cached.ctypes.data
    return a, keep


def _plan(a):
    info = _lib.PlanInfo()
    st = _lib.lib().cpa_plan_counts(ctypes.byref(a), ctypes.byref(info))
    return st, info


def test_plan_counts_for_a_valid_batch():
    a, _keep = _args()
    st, info = _plan(a)
    assert st == 0
    # seq 0: 100 tokens x 4 heads = 400 rows -> 4 tiles; seq 1: 200 x 4 = 800 -> 7 tiles.
    # 11 items x 8 KV heads = 88 workgroups leave the GPU idle, so the
    # automatic plan splits prefill rows at the smallest step tried, one
    # segment (1024 keys): seq 0 (kv 1100) -> 2 splits, seq 1 (kv 200) -> 1
    assert info.num_items == 4 * 2 + 7 and info.num_merge_rows == 100
    assert info.num_partials == 2 * 100 * 32 and info.split_keys_prefill == 1024
    a0, _k0 = _args(split_keys_prefill=-1)
    st, info = _plan(a0)
    assert st == 0 and info.num_items == 4 + 7 and info.num_merge_rows == 0 and info.num_partials == 0
    a2, _k2 = _args(split_keys_prefill=1024)
    st, info = _plan(a2)
    # seq 0 kv 1100 -> 2 splits; seq 1 kv 200 -> 1
    assert st == 0 and info.num_items == 4 * 2 + 7 and info.num_merge_rows == 100
    assert info.num_partials == 2 * 100 * 32


@pytest.mark.parametrize("field,value,code", [
    ("head_dim", 96, _lib.CPA_ERR_UNSUPPORTED),
    ("num_kv_heads", 5, _lib.CPA_ERR_INVALID_ARG),          # 32 % 5 != 0
    ("kv_segment_size", 768, _lib.CPA_ERR_INVALID_ARG),     # not in {512,...,4096}
    ("block_size", 12, _lib.CPA_ERR_UNSUPPORTED),
    ("max_blocks_per_seq", 60, _lib.CPA_ERR_INVALID_ARG),  # 1100 tokens need 69 blocks
    ("split_keys_prefill", 1000, _lib.CPA_ERR_INVALID_ARG),  # not a multiple of S
    ("num_seqs", 0, _lib.CPA_ERR_INVALID_ARG),
    ("dtype", 7, _lib.CPA_ERR_INVALID_ARG),
])
def test_bad_arguments_are_refused(field, value, code):
    a, _keep = _args(**{field: value})
    assert _plan(a)[0] == code
    assert _lib.lib().cpa_prepare(ctypes.byref(a), None) == code
    assert _lib.lib().cpa_attention(ctypes.byref(a), None) == code


def test_bad_host_mirrors_are_refused():
    a, _k = _args(cu=[0, 100, 299])                  # does not end at total_q
    assert _plan(a)[0] == _lib.CPA_ERR_INVALID_ARG
    a, _k = _args(cu=[0, 200, 100], total_q=100)    # decreasing
    assert _plan(a)[0] == _lib.CPA_ERR_INVALID_ARG
    a, _k = _args(cached=[-1, 0])
    assert _plan(a)[0] == _lib.CPA_ERR_INVALID_ARG
    a, _k = _args(kv_segment_size=0)                 # no segments but cached KV present
    assert _plan(a)[0] == _lib.CPA_ERR_INVALID_ARG


@pytest.mark.parametrize("over", [
    {"cu": [0, 100, 299]},                 # does not end at total_q
    {"cu": [1, 100, 300]},                 # does not start at 0
    {"cu": [0, 200, 100], "total_q": 100}, # decreasing
    {"cached": [-1, 0]},                   # negative cached length
    {"cached": [4000, 0]},                 # 4100 tokens need 257 blocks > 200 per row
])
def test_cache_write_refuses_bad_host_mirrors(over):
    # the cache-write entry points check the host mirrors they are given the
    # way attention calls do, before any launch
    a, _k = _args(slot_mapping=0, **over)
    assert _lib.lib().cpa_reshape_and_cache(ctypes.byref(a), None) == _lib.CPA_ERR_INVALID_ARG
    p = ctypes.byref(_rope())
    assert _lib.lib().cpa_rope_reshape_and_cache(ctypes.byref(a), p, None) == _lib.CPA_ERR_INVALID_ARG


def test_no_alloc_call_refuses_more_than_its_scratch():
    # 8 decode rows over a million cached tokens each, split per 512-key
    # segment: ~1954 partial states per (row, head), about 260 MB > 64 MiB.
    # Refused from the host-side plan alone, before any device call.
    cu = np.arange(9, dtype=np.int32)
    cached = np.full(8, 1_000_000, dtype=np.int32)
    a, _keep = _args(num_seqs=8, total_q=8, cu=cu, cached=cached, max_blocks_per_seq=62501,
                     num_blocks=600000, kv_segment_size=512, split_keys_decode=512)
    st, info = _plan(a)
    assert st == 0 and info.workspace_bytes > (64 << 20)
    assert _lib.lib().cpa_chunked_prefill_attn_noalloc(ctypes.byref(a), None) == _lib.CPA_ERR_WORKSPACE


def test_missing_workspace_is_refused_before_launch():
    a, _keep = _args()
    a.workspace, a.workspace_bytes = 0, 0
    assert _lib.lib().cpa_prepare(ctypes.byref(a), None) == _lib.CPA_ERR_WORKSPACE
    st, info = _plan(a)
    a.workspace, a.workspace_bytes = 0x1000, info.workspace_bytes - 1
    assert _lib.lib().cpa_attention(ctypes.byref(a), None) == _lib.CPA_ERR_WORKSPACE


def test_fp32_head_dim_128_is_unsupported():
    a, _keep = _args(dtype=1)
    assert _lib.lib().cpa_check_args(ctypes.byref(a)) == _lib.CPA_ERR_UNSUPPORTED


def test_missing_slot_mapping_needs_a_block_table():
    # without slot_mapping the cache write derives slots from the block table,
    # so that table (and the sequence descriptors) must be there
    a, _keep = _args(slot_mapping=0, block_table=0)
    st = _lib.lib().cpa_reshape_and_cache(ctypes.byref(a), None)
    assert st == _lib.CPA_ERR_INVALID_ARG
    a, _keep = _args(slot_mapping=0)
    assert _lib.lib().cpa_check_args(ctypes.byref(a)) == 0


def _rope(theta=10000.0, interleaved=0, q_out=0x2000):
    r = _lib.RopeArgs()
    r.theta, r.interleaved, r.q_out = theta, interleaved, q_out
    return r


@pytest.mark.parametrize("rope,over", [
    (None, {}),                                   # no rope parameters
    (_rope(theta=0.0), {}),
    (_rope(theta=float("nan")), {}),
    (_rope(interleaved=2), {}),
    (_rope(q_out=0), {}),                         # nowhere to put the rotated queries
    (_rope(), {"q": 0}),
    (_rope(), {"cached_seq_len": 0}),             # positions need the cached lengths
    (_rope(), {"num_heads": 12}),                 # not a multiple of 8 KV heads
])
def test_bad_rope_requests_are_refused(rope, over):
    a, _keep = _args(**over)
    p = ctypes.byref(rope) if rope is not None else None
    assert _lib.lib().cpa_rope_reshape_and_cache(ctypes.byref(a), p, None) == _lib.CPA_ERR_INVALID_ARG
    assert _lib.lib().cpa_rope_prepare(ctypes.byref(a), p, None) == _lib.CPA_ERR_INVALID_ARG
    assert _lib.lib().cpa_rope_chunked_prefill_attn(ctypes.byref(a), p, None) == _lib.CPA_ERR_INVALID_ARG


def test_rope_with_an_fp8_cache_is_unsupported():
    # the rotating cache write stores bf16 rows only
    a, _keep = _args()
    a.kv_dtype = 2                                # CPA_FP8_E4M3
    p = ctypes.byref(_rope())
    assert _lib.lib().cpa_rope_reshape_and_cache(ctypes.byref(a), p, None) == _lib.CPA_ERR_UNSUPPORTED
    assert _lib.lib().cpa_rope_prepare(ctypes.byref(a), p, None) == _lib.CPA_ERR_UNSUPPORTED
    assert _lib.lib().cpa_rope_chunked_prefill_attn(ctypes.byref(a), p, None) == _lib.CPA_ERR_UNSUPPORTED


def test_binding_struct_matches_the_header(tmp_path):
    """Size and field offsets of cpa_attn_args as the C compiler lays it out
    against the binding's ctypes mirror, and the inline-descriptor limit."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("no C compiler")
    fields = [f for f, _ in _lib.AttnArgs._fields_]
    src = tmp_path / "layout.c"
    src.write_text("#include <stdio.h>\n#include <stddef.h>\n#include \"chunked_prefill_attn.h\"\n"
                   "int main(void) {\n  printf(\"%zu %d\\n\", sizeof(cpa_attn_args), CPA_INLINE_DESC_INTS);\n"
                   + "".join('  printf("%%zu\\n", offsetof(cpa_attn_args, %s));\n' % f for f in fields)
                   + "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()
    assert int(out[0]) == ctypes.sizeof(_lib.AttnArgs)
    assert int(out[1]) == _lib.CPA_INLINE_DESC_INTS
    for f, off in zip(fields, out[2:]):
        assert int(off) == getattr(_lib.AttnArgs, f).offset, f


def test_inline_descriptor_replaces_the_device_arrays():
    """With host copies of the whole descriptor the device arrays may be
    absent; past the inline limit they are required again."""
    lib = _lib.lib()
    bt = np.zeros((2, 200), dtype=np.int32)
    a, _keep = _args(cu_seqlens_q=None, cached_seq_len=None, block_table=None)
    assert lib.cpa_check_args(ctypes.byref(a)) == _lib.CPA_ERR_INVALID_ARG
    a.h_block_table = bt.ctypes.data                      # 2*2 + 1 + 400 ints: inline
    assert lib.cpa_check_args(ctypes.byref(a)) == _lib.CPA_OK
    big = np.zeros((2, 500), dtype=np.int32)              # 1005 ints: too many
    a.max_blocks_per_seq, a.h_block_table = 500, big.ctypes.data
    assert 2 * 2 + 1 + 2 * 500 > _lib.CPA_INLINE_DESC_INTS
    assert lib.cpa_check_args(ctypes.byref(a)) == _lib.CPA_ERR_INVALID_ARG
    a.cu_seqlens_q = a.cached_seq_len = a.block_table = 0x1000
    assert lib.cpa_check_args(ctypes.byref(a)) == _lib.CPA_OK

"""Oracle for an FP8 (E4M3) KV cache: the code of each stored element and
its value.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"Prefill Optimisation: Prefix Caching, Chunked Prefill, and
Disaggregation", section 3, names the element type as part of what a cache
entry is (a cache holds a representation of K and V, FP8 among them); the
pages give no format details, so the reading here is the common one:
* E4M3 in the OCP "FN" layout: 1 sign bit, 4 exponent bits (bias 7), 3
  mantissa bits; no infinities; exponent 15 with mantissa 7 is NaN, so the
  largest finite magnitude is 1.75 * 2^8 = 448; subnormals are m/8 * 2^-6;
* a cache element is stored as the code of x * (1/scale), one scale per
  tensor (K and V each); the product is taken in float32, as the kernel
  takes it (the code is an integer decided by floating point, so both sides
  decide it in the same precision), then rounded to the nearest E4M3 value,
  ties to the even code, magnitudes above 448 saturating to 448;
* the value of a stored element is decode(code) * scale.
"""
from __future__ import annotations

import numpy as np


def _grid():
    """Values of the 127 non-negative finite codes 0x00 .. 0x7E, ascending."""
    vals = []
    for code in range(0x7F):
        e, m = code >> 3, code & 7
        vals.append(m / 8.0 * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7))
    return np.array(vals)


GRID = _grid()
MAX = float(GRID[-1])        # 448


def decode(codes) -> np.ndarray:
    """float64 values of E4M3 codes (uint8); NaN codes decode to NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    mag = c & 0x7F
    out = GRID[np.minimum(mag, 0x7E)].copy()
    out[mag == 0x7F] = np.nan
    return np.where(c & 0x80, -out, out)


def encode(x) -> np.ndarray:
    """E4M3 codes (uint8) of float values: nearest value, ties to the even
    code, saturating at 448 in magnitude; the sign bit is the input's (a
    negative value that rounds to zero is -0)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), MAX)
    hi = np.searchsorted(GRID, a, side="left")          # GRID[hi-1] < a <= GRID[hi]
    hi = np.minimum(hi, len(GRID) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = a - GRID[lo], GRID[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(a == GRID[lo], lo, code).astype(np.uint8)   # exact values
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)   # the sign is kept, also on 0


def quantize(x, scale: float) -> np.ndarray:
    """Codes of x stored under ``scale``: x * float32(1/scale) in float32."""
    inv = np.float32(1.0) / np.float32(scale)
    t = (np.asarray(x, dtype=np.float32) * inv).astype(np.float32)
    return encode(t.astype(np.float64))


def dequantize(codes, scale: float) -> np.ndarray:
    return decode(codes) * float(np.float32(scale))


def cache_write(k_pool, v_pool, k_new, v_new, block_tables, cu_seqlens_q, cached_seq_len,
                block_size: int, k_scale: float, v_scale: float):
    """The cache write into pools of E4M3 codes (uint8, the oracle's canonical
    ``[num_blocks, block_size, G, D]`` layout): every active token's K and V
    codes at its slot, every other slot unchanged."""
    from . import attention as _attn
    return _attn.cache_write(np.asarray(k_pool, dtype=np.uint8), np.asarray(v_pool, dtype=np.uint8),
                             quantize(k_new, k_scale), quantize(v_new, v_scale), block_tables,
                             cu_seqlens_q, cached_seq_len, block_size)

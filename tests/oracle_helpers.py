"""Small drivers that chain oracle calls the way an engine would (test-side)."""
import numpy as np

from oracle import attention as oa


def empty_pools(num_blocks, block_size, num_kv_heads, head_dim, fill=0.0):
    shape = (num_blocks, block_size, num_kv_heads, head_dim)
    return np.full(shape, fill, dtype=np.float64), np.full(shape, fill, dtype=np.float64)


def run_chunked(q, k, v, chunks, block_size, table, num_blocks, num_kv_heads, scale,
                segmented=None):
    """Process one prompt chunk by chunk through the oracle; returns the
    concatenated outputs ``[P, H, D]`` and the final pools.  ``segmented``
    (a kv_segment_size) switches to the segment-loop oracle."""
    k_pool, v_pool = empty_pools(num_blocks, block_size, num_kv_heads, q.shape[2])
    outs, c = [], 0
    for n in chunks:
        cu, cached = [0, n], [c]
        k_pool, v_pool = oa.cache_write(k_pool, v_pool, k[c:c + n], v[c:c + n], [table], cu,
                                        cached, block_size)
        if segmented:
            o = oa.segmented_attention(q[c:c + n], k_pool, v_pool, [table], cu, cached,
                                       block_size, scale, num_kv_heads, segmented)
        else:
            o = oa.attention(q[c:c + n], k_pool, v_pool, [table], cu, cached, block_size,
                             scale, num_kv_heads)
        outs.append(o)
        c += n
    return np.concatenate(outs), k_pool, v_pool


def chunks_of(total, size):
    out = []
    while total > 0:
        out.append(min(size, total))
        total -= out[-1]
    return out

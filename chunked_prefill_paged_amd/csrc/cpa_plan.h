// Work decomposition of one attention call, shared by the host (grid sizes,
// workspace size) and the device (the work list written into the workspace).
// The same inline functions run on both sides, so the two always agree.
//
// A work item is (sequence b, row tile rt, split s) for one KV head g (g is
// the other grid coordinate).  Rows of sequence b are its (token, query head
// of group g) pairs, token-major: row R -> token R / hpg, head g*hpg + R % hpg.
// A tile holds kRows rows.  Split s covers keys [s*P, (s+1)*P) of the row's
// causal range [0, c_b + t + 1), P a multiple of kv_segment_size: the
// pages' cached segments ("Prefill Processing", section "How Segmentation
// Works with KV Segments") grouped into work items; the item that reaches
// past c_b also holds the chunk's causal self part.  Splits of one row are
// merged by log-sum-exp; within an item consecutive segments are merged on
// the fly by the online softmax.
#pragma once

#include <cstddef>
#include <cstdint>

#ifdef __HIPCC__
#define CPA_HD __host__ __device__
#else
#define CPA_HD
#endif

namespace cpa {

constexpr int kRows = 128;            // rows per work item (4 waves x 32)
constexpr int kMaxSeqs = 4096;        // sequences per call (plan held in LDS)
constexpr int kNoSplit = 0x7fffffff;  // keys per item when a row is not split
constexpr int kInlineDescInts = 896;  // cu, cached and block table passed inline (int32s)

struct SeqPlan {
    int32_t tiles;    // row tiles
    int32_t nsplit;   // items per row tile
    int64_t items;    // tiles * nsplit
    int64_t parts;    // partial (split, token, head) states, 0 when nsplit == 1
    int32_t merge;    // tokens needing a merge pass
};

CPA_HD inline int32_t keys_per_item(int32_t n, int32_t dec_thresh, int32_t split_pre,
                                    int32_t split_dec) {
    return n <= dec_thresh ? split_dec : split_pre;
}

CPA_HD inline SeqPlan seq_plan(int32_t n, int32_t c, int32_t hpg, int32_t num_heads,
                               int32_t dec_thresh, int32_t split_pre, int32_t split_dec) {
    SeqPlan p{0, 1, 0, 0, 0};
    if (n <= 0) return p;
    p.tiles = (int32_t)(((int64_t)n * hpg + kRows - 1) / kRows);
    const int32_t P = keys_per_item(n, dec_thresh, split_pre, split_dec);
    const int64_t kv = (int64_t)c + n;
    p.nsplit = (kv <= P) ? 1 : (int32_t)((kv + P - 1) / P);
    p.items = (int64_t)p.tiles * p.nsplit;
    if (p.nsplit > 1) {
        p.parts = (int64_t)p.nsplit * n * num_heads;
        p.merge = n;
    }
    return p;
}

// Byte offsets of the workspace sections (256-byte aligned).
struct WsLayout {
    size_t seq_info;   // int4 [B]: item offset, nsplit, partial offset, merge offset
    size_t items;      // int4 [num_items]: b, rt, s, nsplit
    size_t merge;      // int2 [num_merge]: b, t
    size_t part_ml;    // float2 [num_parts]: m (log2 units), l
    size_t part_o;     // float [num_parts, D]: unnormalised output
    size_t desc;       // int32 [kInlineDescInts]: cu, cached, block table (inline uploads)
    size_t total;
};

CPA_HD inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

CPA_HD inline WsLayout ws_layout(int32_t num_seqs, int64_t items, int64_t merge, int64_t parts,
                                 int32_t head_dim) {
    WsLayout w;
    size_t off = 256;   // header
    w.seq_info = off;  off = align256(off + (size_t)num_seqs * 16);
    w.items = off;     off = align256(off + (size_t)items * 16);
    w.merge = off;     off = align256(off + (size_t)merge * 8);
    w.part_ml = off;   off = align256(off + (size_t)parts * 8);
    w.part_o = off;    off = align256(off + (size_t)parts * head_dim * 4);
    w.desc = off;      off = align256(off + (size_t)kInlineDescInts * 4);
    w.total = off;
    return w;
}

}  // namespace cpa

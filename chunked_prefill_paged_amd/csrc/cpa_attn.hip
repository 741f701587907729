// Device side of libchunked_prefill_attn: the paged-cache write, the
// segmented attention over a paged KV cache, and the log-sum-exp merge of
// split rows, written for MI355X (gfx950, CDNA4), plus the C entry points
// that validate host-visible arguments and launch them.
//
// Method (all citations are to the pages this library implements):
//   * a chunk of active tokens first writes its K/V into the paged cache
//     ("Prefill Processing", section "How Segmentation Works with KV
//     Segments"), then attends to its sequence's cached KV, visited in
//     kv_segment_size segments with the last one partial ("Prefill
//     Processing", sections "Kernel Interface", "Partial KV Segment
//     Handling"), and causally to itself ("Prefill Optimisation: Prefix
//     Caching, Chunked Prefill, and Disaggregation", section 2, "Causal
//     equivalence");
//   * partial softmax states are rescaled and merged (same page, section 2:
//     online softmax rescales running normalisers across blocks).
//
// Kernel design (gfx950):
//   * A work item is 128 query rows = (token, query head) pairs of one KV
//     head group, so one K/V tile in LDS serves all H/G heads of the group.
//     4 waves x 32 rows; each wave owns 32 rows.
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16 (fp32: v_mfma_f32_32x32x2_f32): a lane then
//     holds 16 keys of one query row per 32-key block, so the row max and
//     row sum are in-lane reductions plus one exchange with the lane 32 away.
//   * The K rows fed to the A operand are permuted (bits 2 and 3 of the row
//     index swapped) so that each lane's probabilities for one PV k-step are
//     8 consecutive keys; with V stored transposed in the cache
//     ([block, head, D, block_size]) the PV A operand is then a plain 16-byte
//     LDS read.  O^T = V^T P^T accumulates in 4 (D=128) 32x32 fp32 tiles.
//   * K and V^T tiles of 64 keys are gathered through the block table and
//     double-buffered in LDS (XOR-swizzled 16-byte chunks against bank
//     conflicts), one barrier per tile.  A bf16 cache's full tiles go
//     straight into LDS (global_load_lds_dwordx4); an fp8 cache's codes go
//     through registers and become bf16 on the way into LDS; decode items
//     over an fp8 cache stream their codes three tiles ahead through two
//     loader waves.
//   * Masking is a select to -inf before exp2; keys at or past the
//     sequence's end reach LDS as zeros (not loaded, or loaded from the
//     sequence's last block and zeroed), so stale or NaN slots cannot reach
//     the MFMA.
//   * Workgroup ids are remapped so that each of the 8 XCDs runs a
//     contiguous range of (KV head, item) pairs: one KV head per XCD L2 when
//     G = 8.  Items are ordered longest-first within a sequence; a mixed
//     batch over a bf16 cache spreads its prefill items among the decode
//     items.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "chunked_prefill_attn.h"
#include "cpa_plan.h"

namespace cpa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kKeys = 64;   // keys per LDS tile
constexpr int kXcds = 8;
// Attention workgroups resident on one XCD at a time (32 CUs x 2).  The
// dispatcher hands an XCD's first such workgroups out across its CUs, CU j
// taking the j-th and the (j + 32)-th.
constexpr int kPairSlots = 64;
// Prefill items that a mixed batch's plan keeps together when it spreads
// them among the decode items.
constexpr long long kPrefillRun = 8;
constexpr float kLn2 = 0.69314718055994530942f;

// ---------------------------------------------------------------------------
// Global -> LDS gathers (global_load_lds_dwordx4: each lane's 16 bytes land
// at M0 + 16 * lane).  They are issued from inline asm so that their
// completion is awaited only where the kernel says so (s_waitcnt vmcnt
// before the barrier that publishes a tile): the compiler cannot tell the
// buffer being filled from the one being read and would otherwise wait for
// the gather before every LDS read that follows it.
// ---------------------------------------------------------------------------
__device__ inline uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// wave-uniform 64-bit base, per-lane 32-bit byte offset
__device__ inline void gather16(const void* base, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(voff), "s"(base), "s"(lds) : "memory", "m0");
}
// the same with the LDS slab address formed in M0 itself (lds0 + a constant)
template <int OFF>
__device__ inline void gather16_at(const void* base, uint32_t voff, uint32_t lds0) {
    asm volatile("s_add_u32 m0, %2, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(voff), "s"(base), "s"(lds0), "i"(OFF) : "memory", "m0");
}
// per-lane 64-bit address
__device__ inline void gather16(const void* addr, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(addr), "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop
// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maxima) through the
// builtin, so that the compiler's own wait insertion knows every vector
// memory load has completed here and adds none for its loads further on.
__device__ inline void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <typename T> struct Elem;
template <> struct Elem<__bf16> {
    static constexpr int kPerChunk = 8;  // elements per 16-byte chunk
    static constexpr int kPerFrag = 8;   // MFMA k elements per lane
    typedef bf16x8 Frag;
    __device__ static inline f32x16 mma(Frag a, Frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};
template <> struct Elem<float> {
    static constexpr int kPerChunk = 4;
    static constexpr int kPerFrag = 1;
    typedef float Frag;
    __device__ static inline f32x16 mma(Frag a, Frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
};

__device__ __forceinline__ int swap_bits23(int x) {
    return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1);
}

// Physical workgroup ids go round-robin over the XCDs; give XCD x the
// contiguous logical range [start_x, start_x + count_x).
__device__ __forceinline__ int xcd_remap(int pid, int n) {
    const int q = n / kXcds, r = n % kXcds;
    const int x = pid % kXcds, k = pid / kXcds;
    return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + k;
}

// Zero the elements of a 16-byte chunk from index `keep` on.
template <typename T>
__device__ __forceinline__ u32x4 keep_first(u32x4 v, int keep) {
    constexpr int kPerWord = 4 / sizeof(T);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        uint32_t mask = 0;
#pragma unroll
        for (int e = 0; e < kPerWord; ++e) {
            if (w * kPerWord + e < keep) mask |= (sizeof(T) == 2 ? 0xffffu : 0xffffffffu) << (16 * e);
        }
        v[w] &= mask;
    }
    return v;
}

// ---------------------------------------------------------------------------
// Attention kernel
// ---------------------------------------------------------------------------
struct AttnParams {
    const void* q;
    const void* k_cache;
    const void* v_cache;
    void* out;
    float* lse;
    const int32_t* cu;
    const int32_t* cached;
    const int32_t* block_table;
    const int4* seq_info;
    const int4* items;
    float2* part_ml;
    float* part_o;
    int32_t num_items;
    int32_t num_heads;
    int32_t num_kv_heads;
    int32_t hpg;
    int32_t block_size;
    int32_t log2_bs;
    int32_t max_blocks;
    int32_t num_blocks;
    int32_t total_q;
    int32_t dec_thresh;
    int32_t split_pre;
    int32_t split_dec;
    float scale_log2;   // softmax scale * log2(e) (* the K scale of an fp8 cache)
    float v_scale;      // V scale of an fp8 cache (1 otherwise)
};

// FP8: the cache holds E4M3 codes (K [nb, G, bs, D], V^T [nb, G, D, bs], one
// byte each); tiles are gathered through registers one tile ahead, turned
// into bf16 exactly (every E4M3 value is a bf16 value) and stored into the
// same LDS tiles as a bf16 cache, so the products do not change.  The K
// scale is folded into the softmax scale and the V scale into the output.
template <typename T, int D, bool FP8>
__global__ __launch_bounds__(kThreads, 2) void attn_kernel(const AttnParams p) {
    using E = Elem<T>;
    using Frag = typename E::Frag;
    constexpr int EPC = E::kPerChunk;
    constexpr int KPL = E::kPerFrag;
    constexpr int NCK = D / EPC;                    // 16-B chunks per K row
    constexpr int NCV = kKeys / EPC;                // 16-B chunks per V^T row
    constexpr int SWK = (NCK < 16 ? NCK : 16) - 1;  // K swizzle mask
    constexpr int SWV = 7;                          // V^T swizzle mask
    constexpr int NLD = kKeys * NCK / kThreads;     // 16-B loads per thread per tile (each of K, V)
    constexpr int NQF = D / (2 * KPL);              // Q fragments (k-steps over D)
    constexpr int NKS = kKeys / (2 * KPL);          // PV k-steps per tile
    constexpr int NDT = D / 32;                     // 32-row tiles of O^T
    static_assert(NLD * kThreads == kKeys * NCK, "tile must split evenly over threads");

    __shared__ __attribute__((aligned(16))) T lds_k[2][kKeys * D];
    __shared__ __attribute__((aligned(16))) T lds_v[2][D * kKeys];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: slab indices stay scalar
    const int half = lane >> 5;
    const int lrow = lane & 31;
    const int G = p.num_kv_heads;

    const int logical = xcd_remap(blockIdx.x, p.num_items * G);
    const int g = logical / p.num_items;
    const int4 item = p.items[logical - g * p.num_items];
    const int b = item.x, rt = item.y, split = item.z, nsplit = item.w;

    const int q0 = p.cu[b];
    const int n = p.cu[b + 1] - q0;
    const int c = p.cached[b];
    const int kv_len = c + n;
    const int hpg = p.hpg;
    const int rows_total = n * hpg;
    const int row0 = rt * kRows;
    const int t_last = (min(row0 + kRows, rows_total) - 1) / hpg;
    const int P = keys_per_item(n, p.dec_thresh, p.split_pre, p.split_dec);
    const int k0 = (nsplit == 1) ? 0 : split * P;
    const int k1 = (nsplit == 1) ? kv_len : min(k0 + P, kv_len);
    const int kend = min(k1, c + t_last + 1);

    // this lane's query row
    const int R = row0 + wave * 32 + lrow;
    const bool row_ok = R < rows_total;
    const int t = row_ok ? R / hpg : 0;
    const int head = g * hpg + (row_ok ? R - (R / hpg) * hpg : 0);
    const int lim = row_ok ? c + t : -1;          // last key position the row may see
    const int wrow0 = row0 + wave * 32;
    const bool wave_on = wrow0 < rows_total;
    const int wt_min = wrow0 / hpg;
    const int wt_max = (min(wrow0 + 32, rows_total) - 1) / hpg;

    const int32_t* bt = p.block_table + (size_t)b * p.max_blocks;
    const T* kc = (const T*)p.k_cache;
    const T* vc = (const T*)p.v_cache;
    const int bs = p.block_size;
    const int lbs = p.log2_bs;

    // Q: lane holds elements [half*D/2, half*D/2 + D/2) of its row, as the
    // B-operand fragments of the NQF k-steps over D (fragment f covers
    // elements half*D/2 + f*KPL .. + KPL-1)
    Frag qf[NQF];
    {
        const T* qp = (const T*)p.q + ((size_t)(q0 + t) * p.num_heads + head) * D + half * (D / 2);
#pragma unroll
        for (int f = 0; f < NQF; ++f) {
            if constexpr (KPL == 8) {
                qf[f] = row_ok ? *(const Frag*)(qp + f * KPL) : Frag{};
            } else {
                qf[f] = row_ok ? qp[f] : 0.f;
            }
        }
    }

    float m_run = -INFINITY;
    float m2 = -INFINITY;        // the hand-ordered path's reference, in log2 units
    float l_run = 0.f;
    f32x16 oacc[NDT];
#pragma unroll
    for (int i = 0; i < NDT; ++i) oacc[i] = f32x16{};

    u32x4 kreg[NLD], vreg[NLD];
    const uint32_t nb_max = (uint32_t)p.num_blocks - 1;
    // Guarded gather for the tile that reaches the end of the sequence: keys
    // at or past kv_len are zero-filled, V^T chunks straddling it are masked.
    auto load_tile_edge = [&](int ts) {
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int cidx = i * kThreads + tid;
            const int key = cidx / NCK, ch = cidx % NCK;
            const int j = ts + key;
            u32x4 val = {0u, 0u, 0u, 0u};
            if (j < kv_len) {
                const uint32_t blk = min((uint32_t)bt[j >> lbs], nb_max);
                val = *(const u32x4*)(kc + (((size_t)blk * G + g) * bs + (j & (bs - 1))) * D + ch * EPC);
            }
            kreg[i] = val;
        }
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int cidx = i * kThreads + tid;
            const int d = cidx / NCV, kcn = cidx % NCV;
            const int j = ts + kcn * EPC;
            u32x4 val = {0u, 0u, 0u, 0u};
            if (j < kv_len) {
                const uint32_t blk = min((uint32_t)bt[j >> lbs], nb_max);
                val = *(const u32x4*)(vc + (((size_t)blk * G + g) * D + d) * bs + (j & (bs - 1)));
                if (kv_len - j < EPC) val = keep_first<T>(val, kv_len - j);
            }
            vreg[i] = val;
        }
    };
    // Full tiles (all 64 keys exist) are gathered straight into LDS with
    // global_load_lds_dwordx4: one instruction fills a 1 KiB slab, lane L's
    // 16 bytes landing at slab + 16*L.  Each lane therefore fetches the
    // global chunk that belongs at its (swizzled) slot.  K slab s holds rows
    // s*RK.., V^T slab s holds rows d = s*RV..; wave w fills slabs
    // w*NLD .. w*NLD+NLD-1 of both.  The RK rows of a K slab always share a
    // block (block_size >= 8 >= RK), so its block id is wave-uniform.
    constexpr int RK = 64 / NCK;
    constexpr int RV = 64 / NCV;
    static_assert(RK <= 8, "K slab rows must fit the smallest block");
    // Per-lane DMA source offsets: K slab i (row offset within the block-run
    // and swizzled chunk) and V^T slab i (d row v_d0 + i*RV, key chunk whose
    // swizzle depends only on the parity of the slab's 8-row group).
    int k_dma_off[NLD];
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
        const int rk = (wave * NLD + i) * RK + lane / NCK;
        k_dma_off[i] = (lane / NCK) * D + ((lane % NCK) ^ (swap_bits23(rk & 31) & SWK)) * EPC;
    }
    // When a wave's NLD slabs (NLD * RK consecutive keys) lie in one block
    // (block_size >= NLD * RK), one scalar base per tile serves all of them:
    // slab i is then i * RK rows further, folded into its lane offset.
    constexpr int KRUN = NLD * RK;
    uint32_t k_run_off[NLD];
#pragma unroll
    for (int i = 0; i < NLD; ++i) k_run_off[i] = (uint32_t)((k_dma_off[i] + i * RK * D) * (int)sizeof(T));
    const int v_d0 = wave * NLD * RV + lane / NCV;
    auto v_dma_key = [&](int i) {
        const int d = v_d0 + i * RV;
        return ((lane % NCV) ^ (((d & 7) ^ ((d >> 3) & 1)) & SWV)) * EPC;
    };
    // Block ids of a tile's keys: lane L holds entry L of the (at most
    // kKeys / 8) table entries the tile spans.  They are loaded one tile
    // ahead, so issuing the gathers never waits on a table read.
    const int nbt = bs >= kKeys ? 1 : (kKeys >> lbs);
    // (Entries are clamped to the cache where they are used: a clamp here
    // would wait for the load, and with it for every gather issued before.)
    auto load_bt = [&](int ts) -> int {
        return bt[(ts >> lbs) + min(lane, nbt - 1)];
    };
    const char* kc_g = (const char*)(kc + (size_t)g * bs * D);
    const char* vc_g = (const char*)(vc + (size_t)g * D * bs);
    const uint32_t blk_bytes = (uint32_t)(G * bs * D * (int)sizeof(T));
    auto dma_k = [&](int ts, int buf, int btv) {
        const uint32_t lds0 = lds_addr(&lds_k[buf][0]);
        if (bs >= KRUN) {
            const int kr = wave * KRUN;                    // first key of the wave's run
            const uint32_t blk = min((uint32_t)__builtin_amdgcn_readlane(btv, bs >= kKeys ? 0 : (kr >> lbs)), nb_max);
            const char* base = kc_g + (size_t)blk * blk_bytes + ((ts + kr) & (bs - 1)) * (D * (int)sizeof(T));
            const uint32_t l0 = lds0 + wave * NLD * 1024;
            gather16_at<0>(base, k_run_off[0], l0);
            if constexpr (NLD > 1) gather16_at<1024>(base, k_run_off[1], l0);
            if constexpr (NLD > 2) gather16_at<2048>(base, k_run_off[2], l0);
            if constexpr (NLD > 3) gather16_at<3072>(base, k_run_off[3], l0);
            static_assert(NLD <= 4, "at most four slabs per wave");
            return;
        }
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int sl = wave * NLD + i;
            const int kt = sl * RK;                        // first key of the slab within the tile
            const uint32_t blk = min((uint32_t)__builtin_amdgcn_readlane(btv, bs >= kKeys ? 0 : (kt >> lbs)), nb_max);
            const char* base = kc_g + (size_t)blk * blk_bytes + ((ts + kt) & (bs - 1)) * (D * (int)sizeof(T));
            gather16(base, (uint32_t)(k_dma_off[i] * (int)sizeof(T)), lds0 + sl * 1024);
        }
    };
    auto dma_v = [&](int ts, int buf, int btv) {
        const uint32_t lds0 = lds_addr(&lds_v[buf][0]);
        if (bs >= kKeys) {
            // the 64 keys of the tile share one block: scalar base, 32-bit lane offsets
            const uint32_t blk = min((uint32_t)__builtin_amdgcn_readlane(btv, 0), nb_max);
            const char* base = vc_g + (size_t)blk * blk_bytes + (ts & (bs - 1)) * (int)sizeof(T);
            const uint32_t l0 = lds0 + wave * NLD * 1024;
            auto off = [&](int i) { return (uint32_t)(((v_d0 + i * RV) * bs + v_dma_key(i)) * (int)sizeof(T)); };
            gather16_at<0>(base, off(0), l0);
            if constexpr (NLD > 1) gather16_at<1024>(base, off(1), l0);
            if constexpr (NLD > 2) gather16_at<2048>(base, off(2), l0);
            if constexpr (NLD > 3) gather16_at<3072>(base, off(3), l0);
        } else {
#pragma unroll
            for (int i = 0; i < NLD; ++i) {
                const int sl = wave * NLD + i;
                const int kk = v_dma_key(i);                // key offset within the tile (per lane)
                const uint32_t blk = min((uint32_t)__shfl(btv, kk >> lbs), nb_max);
                const char* base = vc_g + (size_t)blk * blk_bytes;
                const uint32_t off = (uint32_t)(((v_d0 + i * RV) * bs + ((ts + kk) & (bs - 1))) * (int)sizeof(T));
                gather16(base + off, lds0 + sl * 1024);
            }
        }
    };
    // FP8 gathers: per thread NL8 16-byte chunks of K (16 consecutive d of one
    // key) and of V^T (16 consecutive keys of one d), zero past the sequence
    constexpr int NC8K = D / 16;                    // fp8 chunks per K row
    constexpr int NC8V = kKeys / 16;                // fp8 chunks per V^T row
    constexpr int NL8 = kKeys * NC8K / kThreads;
    static_assert(!FP8 || (NL8 * kThreads == kKeys * NC8K && NL8 * kThreads == D * NC8V),
                  "fp8 tile must split evenly over threads");
    u32x4 f8k[FP8 ? NL8 : 1], f8v[FP8 ? NL8 : 1];
    auto load_tile_fp8 = [&](int ts, int btv) {
        if constexpr (FP8) {
            const uint8_t* k8 = (const uint8_t*)p.k_cache;
            const uint8_t* v8 = (const uint8_t*)p.v_cache;
            if (ts + kKeys <= kv_len) {
                // A full tile: no guards.  The 8 keys of a wave's K chunks of
                // one slot lie in one block (block_size >= 16), so its id is
                // wave-uniform and the block base scalar; a thread's offsets
                // within the blocks do not change from tile to tile.
                const size_t blk8 = (size_t)G * bs * D;        // bytes of one block
                const uint32_t tsb = ts & (bs - 1);             // the tile's start within its block
                // (the thread's offsets are formed here, per tile, in 32 bits
                // from an unsigned thread index: kept across the loop they
                // would cost registers the tile needs)
                uint32_t t = tid;
                asm volatile("" : "+v"(t));
#pragma unroll
                for (int i = 0; i < NL8; ++i) {
                    const uint32_t cidx = i * kThreads + t;
                    const uint32_t key = cidx / NC8K, c8 = cidx % NC8K;
                    const int key0 = (i * kThreads + wave * 64) / NC8K;
                    const uint32_t blk = min((uint32_t)__builtin_amdgcn_readlane(btv, key0 >> lbs), nb_max);
                    const uint8_t* kb = k8 + blk * blk8 + ((size_t)g * bs + tsb) * D;   // wave-uniform
                    f8k[i] = *(const u32x4*)(kb + ((key & (bs - 1)) * D + c8 * 16));
                }
#pragma unroll
                for (int i = 0; i < NL8; ++i) {
                    const uint32_t cidx = i * kThreads + t;
                    const uint32_t d = cidx / NC8V, kc = cidx % NC8V;
                    const uint32_t off = (g * D + d) * bs + tsb + ((kc * 16) & (bs - 1));
                    if (bs >= kKeys) {
                        const uint32_t blk = min((uint32_t)__builtin_amdgcn_readlane(btv, 0), nb_max);
                        f8v[i] = *(const u32x4*)(v8 + blk * blk8 + off);
                    } else {
                        const uint32_t blk = min((uint32_t)__shfl(btv, (kc * 16) >> lbs), nb_max);
                        f8v[i] = *(const u32x4*)(v8 + blk * blk8 + off);
                    }
                }
                return;
            }
#pragma unroll
            for (int i = 0; i < NL8; ++i) {
                const int cidx = i * kThreads + tid;
                const int key = cidx / NC8K, c8 = cidx % NC8K;
                const int j = ts + key;
                const uint32_t bi = bs >= kKeys ? (uint32_t)__builtin_amdgcn_readlane(btv, 0)
                                                : (uint32_t)__shfl(btv, key >> lbs);
                const uint32_t blk = min(bi, nb_max);
                u32x4 val = {0u, 0u, 0u, 0u};
                if (j < kv_len)
                    val = *(const u32x4*)(k8 + (((size_t)blk * G + g) * bs + (j & (bs - 1))) * D + c8 * 16);
                f8k[i] = val;
            }
#pragma unroll
            for (int i = 0; i < NL8; ++i) {
                const int cidx = i * kThreads + tid;
                const int d = cidx / NC8V, kc = cidx % NC8V;
                const int j = ts + kc * 16;              // 16 keys of one block (bs >= 16)
                const uint32_t bi = bs >= kKeys ? (uint32_t)__builtin_amdgcn_readlane(btv, 0)
                                                : (uint32_t)__shfl(btv, (kc * 16) >> lbs);
                const uint32_t blk = min(bi, nb_max);
                u32x4 val = {0u, 0u, 0u, 0u};
                if (j < kv_len) {
                    val = *(const u32x4*)(v8 + (((size_t)blk * G + g) * D + d) * bs + (j & (bs - 1)));
                    if (kv_len - j < 16) {
#pragma unroll
                        for (int w = 0; w < 4; ++w) {
                            const int keep = min(max(kv_len - j - 4 * w, 0), 4);
                            val[w] &= keep >= 4 ? 0xffffffffu : ((1u << (8 * keep)) - 1u);
                        }
                    }
                }
                f8v[i] = val;
            }
        }
    };
    // 16 E4M3 codes -> 16 bf16 (two 16-byte chunks)
    auto fp8_to_bf16 = [&](u32x4 x, u32x4& lo, u32x4& hi) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const uint32_t a = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[w], 1.0f, false));
            const uint32_t c = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[w], 1.0f, true));
            if (w < 2) { lo[2 * w] = a; lo[2 * w + 1] = c; }
            else { hi[2 * w - 4] = a; hi[2 * w - 3] = c; }
        }
    };
    auto store_tile_fp8 = [&](int buf) {
        if constexpr (FP8) {
#pragma unroll
            for (int i = 0; i < NL8; ++i) {
                const int cidx = i * kThreads + tid;
                const int key = cidx / NC8K, c8 = cidx % NC8K;
                const int sw = swap_bits23(key & 31) & SWK;
                u32x4 lo, hi;
                fp8_to_bf16(f8k[i], lo, hi);
                *(u32x4*)&lds_k[buf][key * D + ((2 * c8) ^ sw) * EPC] = lo;
                *(u32x4*)&lds_k[buf][key * D + ((2 * c8 + 1) ^ sw) * EPC] = hi;
            }
#pragma unroll
            for (int i = 0; i < NL8; ++i) {
                const int cidx = i * kThreads + tid;
                const int d = cidx / NC8V, kc = cidx % NC8V;
                const int sw = ((d & 7) ^ ((d >> 3) & 1)) & SWV;
                u32x4 lo, hi;
                fp8_to_bf16(f8v[i], lo, hi);
                *(u32x4*)&lds_v[buf][d * kKeys + ((2 * kc) ^ sw) * EPC] = lo;
                *(u32x4*)&lds_v[buf][d * kKeys + ((2 * kc + 1) ^ sw) * EPC] = hi;
            }
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int cidx = i * kThreads + tid;
            const int key = cidx / NCK, ch = cidx % NCK;
            const int sw = swap_bits23(key & 31) & SWK;
            *(u32x4*)&lds_k[buf][key * D + (ch ^ sw) * EPC] = kreg[i];
        }
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int cidx = i * kThreads + tid;
            const int d = cidx / NCV, kcn = cidx % NCV;
            const int sw = ((d & 7) ^ ((d >> 3) & 1)) & SWV;
            *(u32x4*)&lds_v[buf][d * kKeys + (kcn ^ sw) * EPC] = vreg[i];
        }
    };

    const float sl2e = p.scale_log2;
    typedef f32x16 Scores[2];   // S^T of one 64-key tile: two 32-key blocks

    // S^T = K Q^T (raw, unscaled scores) from K buffer kbuf
    auto qk = [&](int kbuf, Scores& S) {
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            S[sub] = f32x16{};
            const T* kb = &lds_k[kbuf][(sub * 32 + swap_bits23(lrow)) * D];
            const int sw = lane & SWK;
#pragma unroll
            for (int f = 0; f < NQF; ++f) {
                const int e = half * (D / 2) + f * KPL;
                const int ch = e / EPC, within = e % EPC;
                const Frag a = *(const Frag*)(kb + (ch ^ sw) * EPC + within);
                S[sub] = E::mma(a, qf[f], S[sub]);
            }
        }
    };
    // Causal / split-end mask (boundary tiles only), then the row maximum.
    // Register r of block sub holds key ts + sub*32 + 16*(r/8) + 8*half + r%8.
    auto mask_max = [&](int ts, Scores& S) -> float {
        if ((ts + kKeys - 1 > c + wt_min) || (ts + kKeys > k1)) {
#pragma unroll
            for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int j = ts + sub * 32 + ((r >> 3) << 4) + (half << 3) + (r & 7);
                    if (j > lim || j >= k1) S[sub][r] = -INFINITY;
                }
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[sub][r]);
        }
        return fmaxf(mx, __shfl_xor(mx, 32));
    };
    // Lazy rescaling: the row's reference maximum moves only when a tile's
    // maximum exceeds it by more than 8 (log2 units), so most tiles skip the
    // O rescale and exp2 arguments stay <= 8.  (-inf - -inf is NaN, which
    // compares false: an all-masked row keeps its -inf reference.)
    auto update_ref = [&](float mx) {
        const bool grow = (mx - m_run) * sl2e > 8.f;
        if (__builtin_amdgcn_ballot_w64(grow)) {
            const float m_new = grow ? mx : m_run;
            const float alpha = grow ? __builtin_amdgcn_exp2f((m_run - m_new) * sl2e) : 1.f;
            l_run *= alpha;
#pragma unroll
            for (int i = 0; i < NDT; ++i) oacc[i] *= alpha;
            m_run = m_new;
        }
    };
    // P = exp2(S*scale*log2e - m), row sums, and the P^T fragments of PV
    auto probs = [&](Scores& S, Frag (&pf)[NKS]) {
        const float nm = (m_run == -INFINITY) ? 0.f : -m_run * sl2e;
        float rs = 0.f;
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(S[sub][r], sl2e, nm));
                S[sub][r] = pv;
                if constexpr (KPL != 8) rs += pv;
            }
        }
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            if constexpr (KPL == 8) {
                // bf16 weights: the row sum adds the rounded values the PV
                // product uses
                const int sub = ks >> 1, r0 = (ks & 1) * 8;
                bf16x8 v;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    v[i] = (__bf16)S[sub][r0 + i];
                    rs += (float)v[i];
                }
                pf[ks] = v;
            } else {
                pf[ks] = S[ks >> 4][ks & 15];
            }
        }
        l_run += rs;
    };
    // O^T += V^T P^T from V buffer vbuf
    auto pv = [&](int vbuf, const Frag (&pf)[NKS]) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            const int drow = dt * 32 + lrow;
            const T* vb = &lds_v[vbuf][drow * kKeys];
            const int sw = ((drow & 7) ^ ((drow >> 3) & 1)) & SWV;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                int key0;
                if constexpr (KPL == 8) {
                    key0 = ks * 16 + half * 8;
                } else {
                    const int sub = ks >> 4, r = ks & 15;
                    key0 = sub * 32 + ((r >> 3) << 4) + (half << 3) + (r & 7);
                }
                const int ch = key0 / EPC, within = key0 % EPC;
                const Frag a = *(const Frag*)(vb + (ch ^ sw) * EPC + within);
                oacc[dt] = E::mma(a, pf[ks], oacc[dt]);
            }
        }
    };
    auto active = [&](int ts) { return wave_on && ts <= c + wt_max; };

    // In bf16 with D = 128 every tile runs a hand-ordered sequence in half
    // tiles of 32 keys (tiles on the causal diagonal, at a split end or at
    // the sequence end first mask their scores to -inf).  LDS fragments are prefetched three MFMAs ahead through four
    // rotating registers; sched_barrier fences pin the order:
    //   P1  S0 = K[0:32] Q^T        (8 MFMAs)
    //   P2  S1 = K[32:64] Q^T       (8 MFMAs)  || exp, sum, convert of S0, then S0's check
    //   P3  O += V[0:32] P0         (8 MFMAs)  || exp, sum, convert of S1, then S1's check
    //   P4  O += V[32:64] P1        (8 MFMAs)
    // The reference maximum of a row moves only when the 16 exps of some
    // lane's share of a 32-key block sum past 2^12, so that one of them
    // exceeds 2^8: the common path takes no maximum and needs no exchange
    // between the two lanes of a row, and keeps every exp2 argument <= 12;
    // the rare path takes the row maximum, raises the reference to it and
    // rescales O and l.  Each block is checked before its PV is issued and
    // after every PV formed under the old reference, so a rescale covers
    // exactly those products.
    constexpr bool kHandOrdered = (KPL == 8 && D == 128);
    // LDS byte offsets of this lane's fragments: K fragment (k-step s8,
    // 32-key block sb) at k_base + ((s8*16) ^ k_x) + sb*32*D*2; V fragment
    // (k-step ks, d tile dt) at v_base + ((ks*32) ^ v_x) + dt*32*64*2.
    uint32_t k_base = 0, k_x = 0, v_base = 0, v_x = 0;
    // The same offsets summed once per fragment column: K k-step f at
    // kad[f] (+ 8 KiB for the second 32-key block), V k-step ks at vad[ks]
    // (+ 4 KiB per d tile).  The empty asm keeps the sums whole: otherwise
    // the compiler re-adds the two parts before every LDS read, one VALU
    // instruction each on the issue port the softmax needs.
    uint32_t kad[8] = {}, vad[4] = {};
    if constexpr (kHandOrdered) {
        k_base = (uint32_t)(swap_bits23(lrow) * D * 2 + ((half * 8) ^ (lane & 8)) * 16);
        k_x = (uint32_t)((lane & 7) * 16);
        const int swl = ((lrow & 7) ^ ((lrow >> 3) & 1)) & SWV;
        v_base = (uint32_t)(lrow * kKeys * 2 + (half ^ (swl & 1)) * 16);
        v_x = (uint32_t)((swl & 6) * 16);
#pragma unroll
        for (int f = 0; f < 8; ++f) {
            kad[f] = k_base + ((f * 16) ^ k_x);
            asm volatile("" : "+v"(kad[f]));
        }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            vad[ks] = v_base + ((ks * 32) ^ v_x);
            asm volatile("" : "+v"(vad[ks]));
        }
    }
    // The hand-ordered path's raw score accumulators (each QK chain starts
    // from zero).  The softmax scale is applied in float to every score, in
    // the FMA that forms its exp2 argument t = S * scale * log2(e) - m2:
    // folding it into bf16 queries instead would round q * scale once more,
    // a logit error of about 2^-9 * scale * |q| |k| that peaked softmaxes
    // (large logits) turn into output errors beyond the bf16 tolerance.
    f32x16 S0 = {}, S1 = {};
    auto compute_tile = [&](int buf, int ts, bool masked) __attribute__((always_inline)) {
        if constexpr (kHandOrdered) {
            typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
            const char* kb = (const char*)&lds_k[buf][0];
            const char* vb = (const char*)&lds_v[buf][0];
            auto kfrag = [&](int f) {
                return *(const bf16x8*)(kb + kad[f & 7] + (f >> 3) * (32 * D * 2));
            };
            auto vfrag = [&](int i) {
                return *(const bf16x8*)(vb + vad[i >> 2] + (i & 3) * (32 * kKeys * 2));
            };
            // fragment j of the tile's 32 LDS reads: K fragments 0..15, then V 0..15
            auto frag = [&](int j) { return j < 16 ? kfrag(j) : vfrag(j - 16); };
            bf16x8 fr[4];
            u32x4 pw[4];
            float rs = 0.f;
            const bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};
            // causal / split-end mask of one 32-key block (register r holds
            // key ts + blk*32 + 16*(r/8) + 8*half + r%8)
            auto apply_mask = [&](f32x16& S, int blk) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int j = ts + blk * 32 + ((r >> 3) << 4) + (half << 3) + (r & 7);
                    if (j > lim || j >= k1) S[r] = -INFINITY;
                }
            };
            // S0 and S1 hold raw scores; their exp2 arguments are t = S *
            // scale * log2(e) - m2 (m2: the row's reference maximum in log2
            // units, taken as 0 while unset).  The rare path's maximum is taken
            // on S: MFMA results need no NaN quieting here, so one v_max3
            // folds two scores.
            auto ref_nm = [&]() { return (m2 == -INFINITY) ? 0.f : -m2; };
            float nm = ref_nm();
            // one v_max3 per score pair, chained (the compiler otherwise
            // builds a tree of two-input maxima)
            auto max3 = [](float a, float b, float c) {
                float d;
                asm("v_max3_f32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
                return d;
            };
            // exp/sum/convert of registers r, r+1 of t into pw (the empty
            // asm consumes the results where they are computed: a
            // speculative exp that a rescale recomputes would otherwise be
            // sunk by the compiler past the decision, out of its MFMA phase)
            auto ex2 = [&](const f32x16& S, int ks, int r) {
                const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[r], sl2e, nm));
                const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[r + 1], sl2e, nm));
                const bf16x2 pk = {(__bf16)e0, (__bf16)e1};
                // the row sum adds the rounded weights the PV product uses,
                // so that a dominant key's rounding cancels in O / l
                rs = __builtin_amdgcn_fdot2_f32_bf16(pk, kOnes2, rs, false);
                const uint32_t w = __builtin_bit_cast(uint32_t, pk);
                asm volatile("" :: "v"(w), "v"(rs));
                pw[ks][(r & 7) >> 1] = w;
            };
            // some lane's n exps of one share sum past cap = n * 2^8 (so one
            // of them has t > 8), or some row of the wave has no reference
            auto over = [&](float sum, float cap) {
                return __builtin_amdgcn_ballot_w64(m2 == -INFINITY || sum > cap) != 0;
            };
            // the lane's maximum raw score over registers [r0, 16) of a block
            auto tmax = [&](const f32x16& S, int r0) {
                float ht = -INFINITY;
#pragma unroll
                for (int r = r0; r < 16; r += 2) ht = max3(ht, S[r], S[r + 1]);
                return ht;
            };
            // raise those references to the row maximum (t of the largest
            // score), rescaling O and l; nm follows the new reference
            auto decide = [&](float hs) {
                const float ps = fmaxf(hs, __shfl_xor(hs, 32));
                const float pt = __builtin_fmaf(ps, sl2e, nm);   // -inf stays -inf
                const bool g = (m2 == -INFINITY) ? pt > -INFINITY : pt > 8.f;
                const float m_new = g ? ((m2 == -INFINITY) ? 0.f : m2) + pt : m2;
                const float alpha = g ? __builtin_amdgcn_exp2f(m2 - m_new) : 1.f;
                l_run *= alpha;
#pragma unroll
                for (int i = 0; i < NDT; ++i) oacc[i] *= alpha;
                m2 = m_new;
                nm = ref_nm();
            };
            fr[0] = frag(0);
            fr[1] = frag(1);
            fr[2] = frag(2);
            S0 = f32x16{};
            S1 = f32x16{};
            __builtin_amdgcn_sched_barrier(0);
            // P1
#pragma unroll
            for (int f = 0; f < 8; ++f) {
                fr[(f + 3) & 3] = frag(f + 3);
                S0 = E::mma(fr[f & 3], qf[f], S0);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (masked) apply_mask(S0, 0);
            __builtin_amdgcn_sched_barrier(0);
            // Speculative exps: a block's exps use the current reference
            // before the block is checked; when the check fails (rare; always
            // while some row of the wave has no reference, as on an item's
            // first tile), the block's exps are redone under the new
            // reference.
            // P2: S1 MFMAs; exps of S0
#pragma unroll
            for (int f = 8; f < 16; ++f) {
                fr[(f + 3) & 3] = frag(f + 3);
                S1 = E::mma(fr[f & 3], qf[f & 7], S1);
                const int r = 2 * (f - 8);
                ex2(S0, r >> 3, r);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (over(rs, 4096.f)) {
                decide(tmax(S0, 0));
                rs = 0.f;
#pragma unroll
                for (int r = 0; r < 16; r += 2) ex2(S0, r >> 3, r);
            }
            l_run += rs;                 // before S1's decision may rescale l
            rs = 0.f;
            if (masked) apply_mask(S1, 1);
            __builtin_amdgcn_sched_barrier(0);
            // P3: PV of the first half under the exps of S1
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                fr[(i + 3) & 3] = frag(16 + i + 3);
                oacc[i & 3] = E::mma(fr[i & 3], __builtin_bit_cast(bf16x8, pw[i >> 2]), oacc[i & 3]);
                ex2(S1, 2 + (i >> 2), 2 * i);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (over(rs, 4096.f)) {
                decide(tmax(S1, 0));
                rs = 0.f;
#pragma unroll
                for (int r = 0; r < 16; r += 2) ex2(S1, 2 + (r >> 3), r);
            }
            l_run += rs;
            __builtin_amdgcn_sched_barrier(0);
            // P4: PV of the second half
#pragma unroll
            for (int i = 8; i < 16; ++i) {
                if (i + 3 < 16) fr[(i + 3) & 3] = frag(16 + i + 3);
                oacc[i & 3] = E::mma(fr[i & 3], __builtin_bit_cast(bf16x8, pw[i >> 2]), oacc[i & 3]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    // Tiles [tile0, tile0 + ntiles) cover keys [k0, kend).  The first nfull
    // have all 64 keys in the sequence and are gathered straight into LDS,
    // one tile ahead (double buffer, one barrier per tile); a last tile that
    // reaches past the sequence end goes through guarded register loads.
    if (kend > k0) {
        const int tile0 = k0 / kKeys;
        const int ntiles = (kend - k0 + kKeys - 1) / kKeys;
        const int nfull = min(ntiles, max(0, kv_len / kKeys - tile0));
        Scores S;
        Frag pf[NKS];
        auto tstart = [&](int u) { return (tile0 + u) * kKeys; };
        int btn = 0;                     // block ids of tile u + 1
        // (an fp8 cache reads the table for every tile, the last included:
        // columns stay within the sequence's blocks)
        const int last_col = (kv_len - 1) >> lbs;
        auto load_bt8 = [&](int ts) -> int {
            return bt[min((ts >> lbs) + min(lane, nbt - 1), last_col)];
        };
        // Decode items over an fp8 cache (all rows in wave 0: n * hpg <=
        // 32) are bound by the tile bytes in flight: with every wave loading
        // codes for the next tile and converting them after this one, one
        // 16 KiB tile is in flight.  For them waves 1 and 2 stream the codes
        // three tiles ahead through registers instead, converting and storing
        // tile u + 1 into the other buffer after the barrier of tile u while
        // wave 0 computes tile u; wave 3 only keeps the barriers.  (The same
        // for a bf16 cache was not faster: its gathers straight into LDS
        // already keep the decode rows at the rate HBM gives them.)
        const bool stream8 = FP8 && kHandOrdered && rows_total <= 32 && ntiles >= 2;
        if (stream8 && wave == 3) {
            for (int u = 0; u < ntiles; ++u) __syncthreads();
        } else if (stream8 && wave > 0) {
            if constexpr (FP8) {
                // A tile's K and V^T codes form 2 * NG groups of 64 16-byte
                // chunks; loader wave w (1, 2) holds groups w - 1 + 2 i in its
                // slot i, lane L chunk L of each: slots below NG / 2 hold K,
                // the others V^T.  Every slot is one load on every path, so the
                // compiler's wait counts stay exact across the loop.  A K group
                // is KG consecutive keys of one block (block_size >= 16), 1 KiB
                // contiguous from a wave-uniform base; a V^T group is DG rows d,
                // lane L reading the 16 keys at chunk L % NC8V of row L / NC8V,
                // whose block does not depend on the slot.
                const uint8_t* k8 = (const uint8_t*)p.k_cache;
                const uint8_t* v8 = (const uint8_t*)p.v_cache;
                const int w1 = wave - 1;
                constexpr int NG = kKeys * NC8K / 64;
                constexpr int KG = 64 / NC8K, DG = 64 / NC8V;
                constexpr int NSL = NG;                       // slots per loader lane (2 * NG groups, 2 waves)
                static_assert(kKeys * NC8K == D * NC8V && NG * 64 == kKeys * NC8K && KG <= 16 && NG % 2 == 0,
                              "whole groups; a K group inside the smallest block");
                const int v_lane_key = (lane % NC8V) * 16;    // first key of this lane's V^T chunk
                const int v_lane_off = (lane / NC8V) * bs + (v_lane_key & (bs - 1));
                const int v_sel = v_lane_key >> lbs;          // its table entry, relative to the tile
                auto v_base = [&](int ts, int btv) -> const uint8_t* {
                    const uint32_t blk = min((uint32_t)__shfl(btv, v_sel), nb_max);
                    return v8 + ((size_t)blk * G + g) * D * bs + (ts & (bs - 1)) + v_lane_off;
                };
                auto load_slot = [&](int ts, int btv, const uint8_t* vb, int i) -> u32x4 {
                    if (i < NG / 2) {
                        const int key0 = (w1 + 2 * i) * KG;
                        const uint32_t blk = min((uint32_t)__builtin_amdgcn_readlane(btv, key0 >> lbs), nb_max);
                        const uint8_t* kb = k8 + (((size_t)blk * G + g) * bs + (ts & (bs - 1)) + (key0 & (bs - 1))) * D;
                        return *(const u32x4*)(kb + lane * 16);
                    }
                    return *(const u32x4*)(vb + (w1 + 2 * (i - NG / 2)) * DG * bs);
                };
                // slot i into LDS buffer buf as bf16, in store_tile_fp8's layout;
                // the keys of a sequence's last tile past its end are zeroed
                auto store_slot = [&](int buf, int ts, int i, u32x4 val) {
                    const bool tail = ts + kKeys > kv_len;
                    if (i < NG / 2) {
                        const int key = (w1 + 2 * i) * KG + lane / NC8K, c8 = lane % NC8K;
                        if (tail && ts + key >= kv_len) val = u32x4{0u, 0u, 0u, 0u};
                        const int sw = swap_bits23(key & 31) & SWK;
                        u32x4 lo, hi;
                        fp8_to_bf16(val, lo, hi);
                        *(u32x4*)&lds_k[buf][key * D + ((2 * c8) ^ sw) * EPC] = lo;
                        *(u32x4*)&lds_k[buf][key * D + ((2 * c8 + 1) ^ sw) * EPC] = hi;
                    } else {
                        const int d = (w1 + 2 * (i - NG / 2)) * DG + lane / NC8V, kc = lane % NC8V;
                        if (tail) {
                            const int j = ts + v_lane_key;
#pragma unroll
                            for (int w = 0; w < 4; ++w) {
                                const int keep = min(max(kv_len - j - 4 * w, 0), 4);
                                val[w] &= keep >= 4 ? 0xffffffffu : ((1u << (8 * keep)) - 1u);
                            }
                        }
                        const int sw = ((d & 7) ^ ((d >> 3) & 1)) & SWV;
                        u32x4 lo, hi;
                        fp8_to_bf16(val, lo, hi);
                        *(u32x4*)&lds_v[buf][d * kKeys + ((2 * kc) ^ sw) * EPC] = lo;
                        *(u32x4*)&lds_v[buf][d * kKeys + ((2 * kc + 1) ^ sw) * EPC] = hi;
                    }
                };
                auto load_tile = [&](u32x4 (&st)[NSL], int u, int btv) __attribute__((always_inline)) {
                    const int ts = tstart(u);
                    const uint8_t* vb = v_base(ts, btv);
#pragma unroll
                    for (int i = 0; i < NSL; ++i) st[i] = load_slot(ts, btv, vb, i);
                };
                auto store_stage = [&](const u32x4 (&st)[NSL], int buf, int u) __attribute__((always_inline)) {
                    const int ts = tstart(u);
#pragma unroll
                    for (int i = 0; i < NSL; ++i) store_slot(buf, ts, i, st[i]);
                };
                u32x4 sa[NSL], sb[NSL], sc[NSL];
                auto last = [&](int u) { return min(u, ntiles - 1); };
                // (the prologue issues its last loads in the loop's order:
                // a stage, its ids register, the next stage, ... so the
                // wait counts the compiler carries into the loop are the
                // loop's own)
                const int id0 = load_bt8(tstart(0)), id1 = load_bt8(tstart(1));
                const int id2 = load_bt8(tstart(last(2))), id3 = load_bt8(tstart(last(3)));
                load_tile(sa, 0, id0);
                load_tile(sb, 1, id1);
                int ida = load_bt8(tstart(last(4)));
                load_tile(sc, last(2), id2);
                int idb = load_bt8(tstart(last(5)));
                store_stage(sa, 0, 0);
                load_tile(sa, last(3), id3);
                int idc = load_bt8(tstart(last(6)));
                // Before the barrier of tile u (u a multiple of 3): tile u is
                // in buffer u & 1, tiles u + 1, u + 2, u + 3 in sb, sc, sa,
                // and ida, idb, idc hold the ids of tiles u + 4, u + 5, u + 6.
                // Each step stores one stage, reloads it three tiles ahead
                // and then reloads its ids register three tiles ahead: no
                // register changes hands, every load is issued on every path
                // (tiles past the item's last repeat it, from L2), so the
                // wait before a store drains just that stage and leaves the
                // other two in flight.  (The steady loop has no branch; the
                // last one to three tiles follow it.)
                auto step = [&](u32x4 (&st)[NSL], int& id, int t) __attribute__((always_inline)) {
                    __builtin_amdgcn_sched_barrier(0);
                    store_stage(st, t & 1, t);
                    load_tile(st, last(t + 3), id);
                    id = load_bt8(tstart(last(t + 6)));
                    __builtin_amdgcn_sched_barrier(0);
                };
                int u = 0;
                for (; u + 3 < ntiles; u += 3) {
                    __syncthreads();                 // tile u stored; tile u - 1 computed
                    step(sb, ida, u + 1);
                    __syncthreads();
                    step(sc, idb, u + 2);
                    __syncthreads();
                    step(sa, idc, u + 3);
                }
                __syncthreads();
                if (u + 1 < ntiles) {
                    step(sb, ida, u + 1);
                    __syncthreads();
                    if (u + 2 < ntiles) {
                        step(sc, idb, u + 2);
                        __syncthreads();
                    }
                }
            }
        } else {
            if constexpr (FP8) {
                if (!stream8) {
                    load_tile_fp8(tstart(0), load_bt8(tstart(0)));
                    store_tile_fp8(0);
                    if (ntiles > 1) btn = load_bt8(tstart(1));
                }
            } else {
                if (nfull > 0) {
                    const int bt0 = load_bt(tstart(0));
                    dma_k(tstart(0), 0, bt0);
                    dma_v(tstart(0), 0, bt0);
                }
                if (nfull > 1) btn = load_bt(tstart(1));
            }
            wait_vmem();                     // Q and the first block ids
            // One tile.  With blocks of 64 keys or more the loop below calls it
            // twice per iteration with buf a constant, so every LDS fragment read
            // is a fixed register plus an immediate offset, with no address
            // arithmetic in the tile.
            auto tile = [&](const int u, const int buf) __attribute__((always_inline)) {
                const int ts = tstart(u);
                if (!FP8 && u >= nfull) {    // the sequence's last tile
                    load_tile_edge(ts);
                    store_tile(buf);
                }
                // this tile's gathers have landed (each wave waits for its own,
                // the barrier for everyone's); all waves are done with buf ^ 1
                wait_vmem();
                __syncthreads();
                if constexpr (FP8) {
                    if (!stream8) {
                        if (u + 1 < ntiles) load_tile_fp8(tstart(u + 1), btn);
                        if (u + 2 < ntiles) btn = load_bt8(tstart(u + 2));
                    }
                } else {
                    if (u + 1 < nfull) {
                        dma_k(tstart(u + 1), buf ^ 1, btn);
                        dma_v(tstart(u + 1), buf ^ 1, btn);
                    }
                    if (u + 2 < nfull) btn = load_bt(tstart(u + 2));
                }
                if (active(ts)) {
                    const bool masked = (ts + kKeys - 1 > c + wt_min) || (ts + kKeys > k1);
                    if constexpr (kHandOrdered) {
                        compute_tile(buf, ts, masked);
                    } else {
                        qk(buf, S);
                        update_ref(mask_max(ts, S));
                        probs(S, pf);
                        pv(buf, pf);
                    }
                }
                // the next tile of an fp8 cache goes into the other buffer, which
                // every wave finished reading before this tile's barrier
                if constexpr (FP8) {
                    if (!stream8 && u + 1 < ntiles) store_tile_fp8(buf ^ 1);
                }
            };
            if (bs >= kKeys) {
                for (int u = 0; u < ntiles; u += 2) {
                    tile(u, 0);
                    if (u + 1 < ntiles) tile(u + 1, 1);
                }
            } else {
                // (small blocks: one tile body, the buffer chosen at run time;
                // two bodies measured slower here)
                for (int u = 0; u < ntiles; ++u) tile(u, u & 1);
            }
        }
    }

    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float mlog2 = kHandOrdered ? m2 : m_run * sl2e;   // reference in log2 units
    if (!row_ok) return;
    if (nsplit == 1) {
        const float inv = p.v_scale / l_tot;
        T* op = (T*)p.out + ((size_t)(q0 + t) * p.num_heads + head) * D;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                const int d = dt * 32 + rq * 8 + half * 4;
                if constexpr (sizeof(T) == 2) {
                    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
                    bf16x4 v;
#pragma unroll
                    for (int i = 0; i < 4; ++i) v[i] = (__bf16)(oacc[dt][rq * 4 + i] * inv);
                    *(bf16x4*)(op + d) = v;
                } else {
                    f32x4 v;
#pragma unroll
                    for (int i = 0; i < 4; ++i) v[i] = oacc[dt][rq * 4 + i] * inv;
                    *(f32x4*)(op + d) = v;
                }
            }
        }
        if (p.lse && half == 0)
            p.lse[(size_t)head * p.total_q + q0 + t] = (mlog2 + __log2f(l_tot)) * kLn2;
    } else {
        const size_t pidx = (size_t)p.seq_info[b].z + ((size_t)split * n + t) * p.num_heads + head;
        float* po = p.part_o + pidx * D;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                const int d = dt * 32 + rq * 8 + half * 4;
                f32x4 v;
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] = oacc[dt][rq * 4 + i] * p.v_scale;
                *(f32x4*)(po + d) = v;
            }
        }
        if (half == 0) p.part_ml[pidx] = make_float2(mlog2, l_tot);
    }
}

// ---------------------------------------------------------------------------
// Merge of split rows: m = max m_s, l = sum l_s 2^(m_s - m),
// O = sum O~_s 2^(m_s - m) / l  (states kept in log2 units).
// ---------------------------------------------------------------------------
struct MergeParams {
    const int32_t* cu;
    const int4* seq_info;
    const int2* merge;
    const float2* part_ml;
    const float* part_o;
    void* out;
    float* lse;
    int32_t num_heads;
    int32_t total_q;
    int32_t num_merge;
};

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void merge_kernel(const MergeParams p) {
    // one thread per (merge row, head, 4-element chunk of D)
    constexpr int NC = D / 4;
    const int H = p.num_heads;
    const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (gid >= (int64_t)p.num_merge * H * NC) return;
    const int row = (int)(gid / (H * NC));
    const int h = (int)(gid / NC % H), dc = (int)(gid % NC);
    const int2 e = p.merge[row];
    const int b = e.x, t = e.y;
    const int q0 = p.cu[b];
    const int n = p.cu[b + 1] - q0;
    const int4 si = p.seq_info[b];
    const int nsplit = si.y;
    const size_t base = (size_t)si.z + (size_t)t * H + h;   // partial of split s at base + s*n*H
    const size_t sstride = (size_t)n * H;
    float m = -INFINITY;
    for (int s = 0; s < nsplit; ++s) m = fmaxf(m, p.part_ml[base + s * sstride].x);
    float l = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int s = 0; s < nsplit; ++s) {
        const size_t pi = base + s * sstride;
        const float2 ml = p.part_ml[pi];
        const f32x4 o = *(const f32x4*)(p.part_o + pi * D + dc * 4);
        // a split with no visible key has m = -inf, l = 0 and O = 0
        const float w = ml.x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml.x - m);
        l += w * ml.y;
        acc += w * o;
    }
    const float inv = 1.f / l;
    T* op = (T*)p.out + ((size_t)(q0 + t) * H + h) * D + dc * 4;
    if constexpr (sizeof(T) == 2) {
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        bf16x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = (__bf16)(acc[i] * inv);
        *(bf16x4*)op = v;
    } else {
        *(f32x4*)op = acc * inv;
    }
    if (p.lse && dc == 0) p.lse[(size_t)h * p.total_q + q0 + t] = (m + __log2f(l)) * kLn2;
}

// ---------------------------------------------------------------------------
// Prep kernel: cache write (all but the last workgroup) and the work plan
// (last workgroup).
// ---------------------------------------------------------------------------
struct PrepParams {
    const void* k_new;
    const void* v_new;
    void* k_cache;
    void* v_cache;
    const int64_t* slots;             // NULL: derived from block_table
    const int32_t* block_table;
    int32_t max_blocks;
    int32_t total_q;
    int32_t num_kv_heads;
    int32_t block_size;
    int32_t log2_bs;
    int32_t num_blocks;
    int32_t cache_wgs;
    // rotary embedding (rope != 0): 1 pairs element i with i + D/2, 2 pairs
    // 2i with 2i + 1; q rows of the workgroup's KV-head group are rotated
    // into q_out, keys on their way into the cache
    int32_t rope;
    int32_t rope_wgs;
    float rope_theta;
    // fp8 cache: codes of x * inv_k (K) and x * inv_v (V)
    float inv_k, inv_v;
    const void* q;
    void* q_out;
    // plan (only when plan != 0)
    int32_t plan;
    const int32_t* cu;
    const int32_t* cached;
    int32_t num_seqs;
    int32_t hpg;
    int32_t num_heads;
    int32_t dec_thresh;
    int32_t split_pre;
    int32_t split_dec;
    int4* seq_info;
    int4* items;
    int2* merge;
    int32_t* header;
    // inline descriptor: its length, and (with a plan) where the workspace
    // copy for the attention launch goes
    int32_t desc_len;
    int32_t* desc_out;
};

// cu_seqlens_q [B + 1], cached_seq_len [B] and the block table [B, max_blocks],
// passed by value as a kernel argument
struct InlineDesc {
    int32_t v[kInlineDescInts];
};

constexpr int kPlanSmem = (3 * kMaxSeqs + 2) * 4 + kMaxSeqs * 2;
constexpr int kPrepSmem = kPlanSmem > 64 * (128 + 1) * 4 ? kPlanSmem : 64 * (128 + 1) * 4;   // >= V tile
static_assert(kMaxSeqs <= 65536, "sequence ids are held as 16-bit values in the plan builder");

// Rows of kCacheTok new tokens of KV head g go to their slots.  K rows are
// copied with 16-byte stores; V is staged in LDS and written as columns of
// the transposed layout, lanes over tokens so that neighbouring slots
// coalesce.
//
// With ROPE, keys are rotated before they are stored, and separate
// workgroups rotate the queries (kRopeQTok tokens, all heads, each) into
// q_out; every token turns at its absolute position cached_seq_len[b] +
// (offset in its chunk) ("Prefill Optimisation ...", section 2, "Causal
// equivalence": positional encodings use absolute positions; "Chunked
// Prefill", "From scratch": the cached length is the position offset).  The
// pages name rotary embedding without writing it out; this is the standard
// form: pair i of a head turns by p * theta^(-2i/D) radians, (x, y) ->
// (x cos - y sin, x sin + y cos).  The angle, up to tens of thousands of
// radians, is formed and reduced to [-pi, pi] in double precision; cos and
// sin of the reduced angle are then taken in float (error below 2^-22).  A
// query workgroup shares one cos/sin table among all heads; a cache-write
// workgroup (one KV head) evaluates each angle where it uses it.
constexpr int kCacheTok = 64;   // tokens per cache-write workgroup
constexpr int kRopeQTok = 8;    // tokens per query-rotation workgroup

// cos/sin of angle pos * freq: reduced to [-pi, pi] in double, then float
__device__ inline float2 rope_cos_sin(int pos, double freq) {
    const double a = (double)pos * freq;
    const double r = a - 6.283185307179586477 * rint(a * 0.159154943091895335769);
    float sn, cn;
    sincosf((float)r, &sn, &cn);
    return make_float2(cn, sn);
}

// Rotation of one unit of a row: pairs ch*EPC .. ch*EPC + EPC - 1, whose
// two source chunks ua, ub come from rope_load; cs(i) gives cos/sin of pair
// i.  The rotated chunks go to the same places of the row at dst.
template <typename T, int D, typename CS>
__device__ inline void rope_rotate_store(u32x4 ua, u32x4 ub, T* dst, int ch, CS cs, bool interleaved) {
    constexpr int EPC = 16 / sizeof(T);
    constexpr int NCK = D / EPC;
    // unit ch covers pairs ch*EPC .. ch*EPC + EPC - 1 of the row: chunks ch
    // and ch + NCK/2 (rotate-half) or chunks 2ch and 2ch + 1 (interleaved)
    const int ca = interleaved ? 2 * ch : ch;
    const int cb = interleaved ? 2 * ch + 1 : ch + NCK / 2;
    T va[EPC], vb[EPC];
    __builtin_memcpy(va, &ua, 16);
    __builtin_memcpy(vb, &ub, 16);
    float x[2 * EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
        x[e] = (float)va[e];
        x[EPC + e] = (float)vb[e];
    }
    float y[2 * EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
        const int i0 = interleaved ? 2 * e : e;
        const int i1 = interleaved ? 2 * e + 1 : EPC + e;
        const float2 c = cs(ch * EPC + e);
        y[i0] = __builtin_fmaf(x[i0], c.x, -x[i1] * c.y);
        y[i1] = __builtin_fmaf(x[i0], c.y, x[i1] * c.x);
    }
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
        va[e] = (T)y[e];
        vb[e] = (T)y[EPC + e];
    }
    __builtin_memcpy(&ua, va, 16);
    __builtin_memcpy(&ub, vb, 16);
    *(u32x4*)(dst + ca * EPC) = ua;
    *(u32x4*)(dst + cb * EPC) = ub;
}

// The two source chunks of a rotation unit (see rope_rotate_store).
template <typename T, int D>
__device__ inline void rope_load(const T* src, int ch, bool interleaved, u32x4& ua, u32x4& ub) {
    constexpr int EPC = 16 / sizeof(T);
    constexpr int NCK = D / EPC;
    ua = *(const u32x4*)(src + (interleaved ? 2 * ch : ch) * EPC);
    ub = *(const u32x4*)(src + (interleaved ? 2 * ch + 1 : ch + NCK / 2) * EPC);
}


// Absolute position of token tok: its sequence b by binary search over
// cu_seqlens_q, then cached_seq_len[b] + (tok - cu[b]).  *seq receives b.
__device__ inline int token_position(const PrepParams& p, int tok, int* seq) {
    int lo = 0, hi = p.num_seqs;                  // cu[lo] <= tok < cu[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (p.cu[mid] <= tok) lo = mid; else hi = mid;
    }
    *seq = lo;
    return p.cached[lo] + (tok - p.cu[lo]);
}

// theta^(-2i/D) of the D/2 pairs, in double
template <int D>
__device__ void rope_freqs(const PrepParams& p, double* s_freq) {
    if (threadIdx.x < D / 2) s_freq[threadIdx.x] = pow((double)p.rope_theta, -2.0 * threadIdx.x / D);
}

// E4M3 codes of scaled values: clamped to the largest finite magnitude (448),
// then rounded to nearest, ties to even, by the conversion instruction.
__device__ inline float sat448(float x) { return fminf(fmaxf(x, -448.f), 448.f); }
__device__ inline uint32_t fp8_pack4(float a, float b, float c, float d) {
    const uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sat448(a), sat448(b), 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sat448(c), sat448(d), (int)w, true);
}

template <typename T, int D, bool ROPE, bool FP8>
__device__ void cache_write(const PrepParams& p, char* smem) {
    constexpr int EPC = 16 / sizeof(T);
    constexpr int NCK = D / EPC;
    constexpr int LD = D + 4 / (int)sizeof(T);   // LDS pitch: one extra 32-bit word
    T* tile = (T*)smem;
    const int G = p.num_kv_heads;
    const int grp = blockIdx.x / G, g = blockIdx.x - grp * G;
    const int tok0 = grp * kCacheTok;
    const int ntok = min(kCacheTok, p.total_q - tok0);
    const int tid = threadIdx.x;
    const T* kn = (const T*)p.k_new;
    const T* vn = (const T*)p.v_new;
    T* kc = (T*)p.k_cache;
    T* vc = (T*)p.v_cache;
    const int bs = p.block_size;
    const int64_t nslots = (int64_t)p.num_blocks * bs;
    // this thread's chunks of V, and of K unless rotated, loaded before
    // anything else (they depend on no slot): the LDS and cache stores come
    // after the slots, one round trip per workgroup
    constexpr int NIT = kCacheTok * NCK / kThreads;
    static_assert(NIT * kThreads == kCacheTok * NCK, "chunks split evenly over the threads");
    u32x4 vv[NIT], kv[NIT];
#pragma unroll
    for (int i = 0; i < NIT; ++i) {
        const int cidx = tid + i * kThreads;
        const int tk = cidx / NCK, ch = cidx - tk * NCK;
        const size_t src = ((size_t)(tok0 + min(tk, ntok - 1)) * G + g) * D + ch * EPC;
        vv[i] = *(const u32x4*)(vn + src);
        if constexpr (!ROPE) kv[i] = *(const u32x4*)(kn + src);
    }
    // (with RoPE: the two source chunks of each of this thread's K rotation
    // units, rotated once the positions are known)
    constexpr int NKU = ROPE ? kCacheTok * (NCK / 2) / kThreads : 1;   // rotation units per thread
    static_assert(!ROPE || NKU * kThreads == kCacheTok * (NCK / 2), "units split evenly over the threads");
    u32x4 ka[NKU], kb[NKU];
    if constexpr (ROPE) {
        const bool inter = p.rope == 2;
#pragma unroll
        for (int i = 0; i < NKU; ++i) {
            const int u = tid + i * kThreads;
            const int tk = u / (NCK / 2), ch = u - tk * (NCK / 2);
            rope_load<T, D>(kn + ((size_t)(tok0 + min(tk, ntok - 1)) * G + g) * D, ch, inter, ka[i], kb[i]);
        }
    }
    // slots of the tokens: given, or derived from the block table at the
    // token's position
    __shared__ int64_t s_slot[kCacheTok];
    __shared__ int s_pos[kCacheTok];
    if (tid < ntok) {
        const int tok = tok0 + tid;
        int64_t slot = 0;
        int seq = 0, pos = 0;
        if (ROPE || !p.slots) pos = token_position(p, tok, &seq);
        if (p.slots) {
            slot = p.slots[tok];
        } else {
            const int col = pos >> p.log2_bs;
            slot = (col >= 0 && col < p.max_blocks)
                       ? (int64_t)p.block_table[(size_t)seq * p.max_blocks + col] * bs + (pos & (bs - 1))
                       : -1;
        }
        s_slot[tid] = slot;
        s_pos[tid] = pos;
    }
    __shared__ double s_freq[ROPE ? D / 2 : 1];
    if constexpr (ROPE) rope_freqs<D>(p, s_freq);
    __syncthreads();
    if constexpr (ROPE) {
        // keys: rotate, then store at the slot (one KV head per workgroup,
        // so each (token, pair) angle is used once: no table)
        const bool inter = p.rope == 2;
#pragma unroll
        for (int i = 0; i < NKU; ++i) {
            const int u = tid + i * kThreads;
            const int tk = u / (NCK / 2), ch = u - tk * (NCK / 2);
            if (tk >= ntok) continue;
            const int64_t slot = s_slot[tk];
            if (slot >= 0 && slot < nslots) {
                const int64_t blk = slot >> p.log2_bs;
                const int off = (int)(slot & (bs - 1));
                const int pos = s_pos[tk];
                rope_rotate_store<T, D>(ka[i], kb[i], kc + ((blk * G + g) * bs + off) * D, ch,
                                        [&](int i) { return rope_cos_sin(pos, s_freq[i]); }, inter);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < NIT; ++i) {
        const int cidx = tid + i * kThreads;
        const int tk = cidx / NCK, ch = cidx - tk * NCK;
        if (tk >= ntok) continue;
        uint32_t* dst = (uint32_t*)(tile + tk * LD + ch * EPC);
        dst[0] = vv[i].x;
        dst[1] = vv[i].y;
        dst[2] = vv[i].z;
        dst[3] = vv[i].w;
        if constexpr (FP8) {
            // 8 bf16 of K -> 8 codes at the slot's row (D bytes)
            const int64_t slot = s_slot[tk];
            if (slot >= 0 && slot < nslots) {
                const int64_t blk = slot >> p.log2_bs;
                const int off = (int)(slot & (bs - 1));
                T e[8];
                __builtin_memcpy(e, &kv[i], 16);
                uint2 q8;
                q8.x = fp8_pack4((float)e[0] * p.inv_k, (float)e[1] * p.inv_k, (float)e[2] * p.inv_k,
                                 (float)e[3] * p.inv_k);
                q8.y = fp8_pack4((float)e[4] * p.inv_k, (float)e[5] * p.inv_k, (float)e[6] * p.inv_k,
                                 (float)e[7] * p.inv_k);
                *(uint2*)((uint8_t*)p.k_cache + ((blk * G + g) * bs + off) * D + ch * 8) = q8;
            }
        } else if constexpr (!ROPE) {
            const int64_t slot = s_slot[tk];
            if (slot >= 0 && slot < nslots) {
                const int64_t blk = slot >> p.log2_bs;
                const int off = (int)(slot & (bs - 1));
                *(u32x4*)(kc + ((blk * G + g) * bs + off) * D + ch * EPC) = kv[i];
            }
        }
    }
    __syncthreads();
    // V columns: kCacheTok lanes over tokens, the rest of the wave over d
    // (a 16-byte store of 8 consecutive tokens per lane measured no faster)
    constexpr int kLanesD = 64 / kCacheTok;
    const int lane = tid & 63, wave = tid >> 6;
    const int tk = lane % kCacheTok;
    if (tk < ntok) {
        const int64_t slot = s_slot[tk];
        if (slot >= 0 && slot < nslots) {
            const int64_t blk = slot >> p.log2_bs;
            const int off = (int)(slot & (bs - 1));
            if constexpr (FP8) {
                uint8_t* col = (uint8_t*)p.v_cache + (blk * G + g) * D * (int64_t)bs + off;
                for (int d = wave * kLanesD + lane / kCacheTok; d < D; d += 4 * kLanesD)
                    col[(size_t)d * bs] = (uint8_t)__builtin_amdgcn_cvt_pk_fp8_f32(
                        sat448((float)tile[tk * LD + d] * p.inv_v), 0.f, 0, false);
            } else {
                T* col = vc + (blk * G + g) * D * (int64_t)bs + off;
                for (int d = wave * kLanesD + lane / kCacheTok; d < D; d += 4 * kLanesD)
                    col[(size_t)d * bs] = tile[tk * LD + d];
            }
        }
    }
}

// Rotation of the queries of kRopeQTok tokens (all heads) into q_out, from
// a cos/sin table of the tokens x D/2 pairs shared by the heads.
template <typename T, int D>
__device__ void rope_queries(const PrepParams& p, int qgrp) {
    constexpr int EPC = 16 / sizeof(T);
    constexpr int NCK = D / EPC;
    __shared__ int s_pos[kRopeQTok];
    __shared__ double s_freq[D / 2];
    __shared__ float2 s_cs[kRopeQTok * (D / 2)];
    const int tid = threadIdx.x;
    const int tok0 = qgrp * kRopeQTok;
    const int ntok = min(kRopeQTok, p.total_q - tok0);
    if (tid < ntok) {
        int seq;
        s_pos[tid] = token_position(p, tok0 + tid, &seq);
    }
    rope_freqs<D>(p, s_freq);
    __syncthreads();
    for (int idx = tid; idx < ntok * (D / 2); idx += kThreads) {
        const int tk = idx / (D / 2), i = idx - tk * (D / 2);
        s_cs[idx] = rope_cos_sin(s_pos[tk], s_freq[i]);
    }
    __syncthreads();
    const bool inter = p.rope == 2;
    const int H = p.num_heads;
    const T* qs = (const T*)p.q;
    T* qd = (T*)p.q_out;
    // kQB units per thread at a time, their loads first
    constexpr int kQB = 4;
    const int nunits = ntok * H * (NCK / 2);
    for (int u0 = tid; u0 < nunits; u0 += kQB * kThreads) {
        u32x4 qa[kQB], qb[kQB];
#pragma unroll
        for (int k = 0; k < kQB; ++k) {
            const int u = min(u0 + k * kThreads, nunits - 1);
            const int row = u / (NCK / 2), ch = u - row * (NCK / 2);
            rope_load<T, D>(qs + ((size_t)tok0 * H + row) * D, ch, inter, qa[k], qb[k]);
        }
#pragma unroll
        for (int k = 0; k < kQB; ++k) {
            const int u = u0 + k * kThreads;
            if (u >= nunits) break;
            const int row = u / (NCK / 2), ch = u - row * (NCK / 2);
            const int tk = row / H;
            const float2* cs = s_cs + tk * (D / 2);
            rope_rotate_store<T, D>(qa[k], qb[k], qd + ((size_t)tok0 * H + row) * D, ch,
                                    [&](int i) { return cs[i]; }, inter);
        }
    }
}

// The plan's per-thread counters, scanned together.
struct PlanCounts {
    long long it_pre, it_dec, parts;
    int merge, n_pre;
};

// Inclusive scan of the counters over the workgroup: within each wave by
// shuffles, then the totals of the waves before it through LDS (two
// barriers; a barrier per step of a shared-memory scan made the plan
// builder the longest part of the prepare launch).
__device__ PlanCounts block_scan_incl(PlanCounts x, PlanCounts* wtot) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const long long a = __shfl_up(x.it_pre, off), b = __shfl_up(x.it_dec, off),
                        c = __shfl_up(x.parts, off);
        const int d = __shfl_up(x.merge, off), e = __shfl_up(x.n_pre, off);
        if (lane >= off) {
            x.it_pre += a;
            x.it_dec += b;
            x.parts += c;
            x.merge += d;
            x.n_pre += e;
        }
    }
    if (lane == 63) wtot[w] = x;
    __syncthreads();
    for (int i = 0; i < w; ++i) {
        x.it_pre += wtot[i].it_pre;
        x.it_dec += wtot[i].it_dec;
        x.parts += wtot[i].parts;
        x.merge += wtot[i].merge;
        x.n_pre += wtot[i].n_pre;
    }
    __syncthreads();
    return x;
}

// Work plan.  Items of prefill sequences (n > decode threshold) come first,
// in sequence order, each sequence's longest row tiles first; items of
// decode rows follow.  Long causal items thus start before the short ones.
// Within the first kPairSlots row tiles of a sequence (the F longest), the
// lighter half runs in ascending order, so that a CU's two first workgroups
// are the j-th longest and the j-th shortest of them: the causal triangle's
// long and short rows share a CU, and the long one has the CU to itself
// once the short one ends.
//
// With a bf16 cache and both kinds present (a mixed batch), the prefill
// items are spread over the first three quarters of the decode items
// instead (interleave), in runs of kPrefillRun consecutive items: taken all
// at once they hold most of an XCD's slots and the decode items, whose rate
// follows the slots they get, wait; spread, a prefill item shares its CU
// with decode workgroups, which use the matrix cores little.  A run's items
// (neighbouring row tiles) start together and read the same K/V tiles at
// about the same time, so L2 serves their re-reads; single items spread
// apart each fetched the sequence's K/V from HBM.  An fp8 cache keeps the
// prefill items first: its decode workgroups convert codes with vector
// instructions and slow a prefill workgroup beside them.
__device__ void build_plan(const PrepParams& p, char* smem, bool interleave) {
    int* s_item = (int*)smem;                 // [kMaxSeqs + 1] first item of the k-th issued sequence
    int* s_merge = s_item + (kMaxSeqs + 1);   // [kMaxSeqs + 1] first merge row of sequence b
    int* s_nsplit = s_merge + (kMaxSeqs + 1); // [kMaxSeqs]     splits of the k-th issued sequence
    uint16_t* s_seq = (uint16_t*)(s_nsplit + kMaxSeqs);   // [kMaxSeqs] sequence issued k-th
    __shared__ PlanCounts sc_w[kThreads / 64];
    const int B = p.num_seqs, tid = threadIdx.x;
    const int per = (B + kThreads - 1) / kThreads;
    const int b_lo = min(B, tid * per), b_hi = min(B, b_lo + per);
    auto plan_of = [&](int b) {
        return seq_plan(p.cu[b + 1] - p.cu[b], p.cached[b], p.hpg, p.num_heads, p.dec_thresh,
                        p.split_pre, p.split_dec);
    };
    auto is_prefill = [&](int b) { return p.cu[b + 1] - p.cu[b] > p.dec_thresh; };
    long long it_pre = 0, it_dec = 0, parts = 0;
    int merge = 0, n_pre = 0;
    for (int b = b_lo; b < b_hi; ++b) {
        const SeqPlan sp = plan_of(b);
        if (is_prefill(b)) {
            it_pre += sp.items;
            ++n_pre;
        } else {
            it_dec += sp.items;
        }
        parts += sp.parts;
        merge += sp.merge;
    }
    const PlanCounts sc = block_scan_incl(PlanCounts{it_pre, it_dec, parts, merge, n_pre}, sc_w);
    const long long sc_pre = sc.it_pre, sc_dec = sc.it_dec, sc_parts = sc.parts;
    const int sc_merge = sc.merge, sc_npre = sc.n_pre;
    __shared__ long long tot[3];
    __shared__ int tot_i[2];
    if (tid == kThreads - 1) {
        tot[0] = sc_pre;
        tot[1] = sc_dec;
        tot[2] = sc_parts;
        tot_i[0] = sc_merge;
        tot_i[1] = sc_npre;
    }
    __syncthreads();
    const long long items_pre = tot[0], items_all = tot[0] + tot[1];
    const int npre_all = tot_i[1];
    if (tid == 0) {
        s_item[B] = (int)items_all;
        s_merge[B] = tot_i[0];
        p.header[0] = (int)items_all;
        p.header[1] = tot_i[0];
        p.header[2] = (int)tot[2];
    }
    // exclusive prefixes of this thread's range
    long long io_pre = sc_pre - it_pre, io_dec = items_pre + sc_dec - it_dec, po = sc_parts - parts;
    int mo = sc_merge - merge;
    int k_pre = sc_npre - n_pre;                          // issue slot of the next prefill sequence
    int k_dec = npre_all + (b_lo - (sc_npre - n_pre));    // decode sequences before b_lo: b_lo - prefill ones
    for (int b = b_lo; b < b_hi; ++b) {
        const SeqPlan sp = plan_of(b);
        const bool pre = is_prefill(b);
        const long long io = pre ? io_pre : io_dec;
        const int k = pre ? k_pre++ : k_dec++;
        p.seq_info[b] = make_int4((int)io, sp.nsplit, (int)po, mo);
        s_item[k] = (int)io;
        s_seq[k] = (uint16_t)b;
        s_nsplit[k] = sp.nsplit;
        s_merge[b] = mo;
        if (pre) io_pre += sp.items; else io_dec += sp.items;
        po += sp.parts;
        mo += sp.merge;
    }
    __syncthreads();
    // Items and merge rows.  A sequence with few of them (a decode row: one
    // per key range) is written by one thread, all such sequences at once; a
    // longer one by one wave, lanes over its entries.  (One wave per
    // sequence for all of them made a batch of 256 decodes spend ~20 us
    // here.)
    const int wv = tid >> 6, ln = tid & 63;
    constexpr int kWaves = kThreads / 64;
    constexpr int kFew = 32;
    // Position of the item issued i-th.  With interleave, prefill run m
    // (items m * kPrefillRun ..) goes right before decode item
    // floor(m * W / runs), W being three quarters of the decode items;
    // decode item j then has the runs m with m * W < (j + 1) * runs, and
    // their items, before it.
    const long long W = interleave ? (items_all - items_pre) * 3 / 4 : 0;
    const long long runs = (items_pre + kPrefillRun - 1) / kPrefillRun;
    auto place = [&](long long i) -> long long {
        if (items_pre == 0 || W == 0) return i;
        if (i < items_pre) return i + ((i / kPrefillRun) * W) / runs;
        const long long j = i - items_pre;
        return j + min(items_pre, kPrefillRun * min(runs, ((j + 1) * runs + W - 1) / W));
    };
    auto write_items = [&](int k, int first, int step) {   // k-th issued sequence
        const int bq = s_seq[k];
        const int i0 = s_item[k], ni = s_item[k + 1] - i0;
        const int nsplit = s_nsplit[k];
        const int tiles = ni / nsplit;
        const int F = min(tiles, kPairSlots);
        for (int local = first; local < ni; local += step) {
            const int li = local / nsplit;
            int rt = tiles - 1 - li;                     // longest row tiles first
            if (li < F && li >= F - F / 2) rt = tiles - F + (li - (F - F / 2));
            p.items[place(i0 + local)] = make_int4(bq, rt, local % nsplit, nsplit);
        }
    };
    // (issued sequences own contiguous item ranges: prefill ones, then decode ones)
    for (int k = tid; k < B; k += kThreads) {
        if (s_item[k + 1] - s_item[k] <= kFew) write_items(k, 0, 1);
    }
    for (int k = wv; k < B; k += kWaves) {
        if (s_item[k + 1] - s_item[k] > kFew) write_items(k, ln, 64);
    }
    for (int b = tid; b < B; b += kThreads) {
        const int m0 = s_merge[b], m1 = s_merge[b + 1];
        if (m1 - m0 <= kFew) {
            for (int i = m0; i < m1; ++i) p.merge[i] = make_int2(b, i - m0);
        }
    }
    for (int b = wv; b < B; b += kWaves) {
        const int m0 = s_merge[b], m1 = s_merge[b + 1];
        if (m1 - m0 > kFew) {
            for (int i = m0 + ln; i < m1; i += 64) p.merge[i] = make_int2(b, i - m0);
        }
    }
}

// Grid: cache_wgs cache-write workgroups, then (with ROPE) rope_wgs
// query-rotation workgroups, then (with a plan) one plan builder.
template <typename T, int D, bool ROPE, bool FP8>
__device__ void prep_body(const PrepParams& p, char* smem) {
    const int wg = blockIdx.x;
    if (wg < p.cache_wgs) {
        cache_write<T, D, ROPE, FP8>(p, smem);
        return;
    }
    if constexpr (ROPE) {
        if (wg < p.cache_wgs + p.rope_wgs) {
            rope_queries<T, D>(p, wg - p.cache_wgs);
            return;
        }
    }
    build_plan(p, smem, !FP8);
}

template <typename T, int D, bool ROPE, bool FP8>
__global__ __launch_bounds__(kThreads) void prep_kernel(const PrepParams p) {
    __shared__ __attribute__((aligned(16))) char smem[kPrepSmem];
    prep_body<T, D, ROPE, FP8>(p, smem);
}

// The same with the batch descriptor in the kernel arguments: every
// workgroup reads it there, and the plan builder also leaves a copy in the
// workspace for the attention launch.
template <typename T, int D, bool ROPE, bool FP8>
__global__ __launch_bounds__(kThreads) void prep_kernel_inline(const PrepParams p0, const InlineDesc d) {
    __shared__ __attribute__((aligned(16))) char smem[kPrepSmem];
    PrepParams p = p0;
    p.cu = d.v;
    p.cached = d.v + p.num_seqs + 1;
    p.block_table = d.v + 2 * p.num_seqs + 1;
    if (p.plan && blockIdx.x == gridDim.x - 1) {
        for (int i = threadIdx.x; i < p.desc_len; i += kThreads) p.desc_out[i] = d.v[i];
    }
    prep_body<T, D, ROPE, FP8>(p, smem);
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
struct Resolved {
    int32_t hpg, dec_thresh, split_pre, split_dec, log2_bs, seg;
    int64_t items, parts;
    int64_t merge;
    WsLayout ws;
};

inline bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }
inline int ilog2(int x) {
    int r = 0;
    while ((1 << r) < x) ++r;
    return r;
}

cpa_status check_common(const cpa_attn_args* a) {
    if (!a) return CPA_ERR_INVALID_ARG;
    if (a->dtype != CPA_BF16 && a->dtype != CPA_FP32) return CPA_ERR_INVALID_ARG;
    if (a->num_kv_heads <= 0 || a->total_q < 0) return CPA_ERR_INVALID_ARG;
    if (a->head_dim <= 0 || a->block_size <= 0 || a->num_blocks <= 0) return CPA_ERR_INVALID_ARG;
    if (a->head_dim != 64 && a->head_dim != 128) return CPA_ERR_UNSUPPORTED;
    if (!is_pow2(a->block_size) || a->block_size < 8 || a->block_size > 512) return CPA_ERR_UNSUPPORTED;
    // cache element type: that of dtype, or E4M3 codes under bf16 q/k/v/out
    if (a->kv_dtype != 0 && a->kv_dtype != a->dtype && a->kv_dtype != CPA_FP8_E4M3)
        return CPA_ERR_INVALID_ARG;
    if (a->kv_dtype == CPA_FP8_E4M3) {
        if (a->dtype != CPA_BF16 || a->block_size < 16) return CPA_ERR_UNSUPPORTED;
        for (float sc : {a->k_scale, a->v_scale})
            if (!std::isfinite(sc) || sc < 0.f) return CPA_ERR_INVALID_ARG;
    }
    if ((int64_t)a->num_blocks * a->block_size > (int64_t)1 << 40) return CPA_ERR_INVALID_ARG;
    return CPA_OK;
}

// Workgroups that fill MI355X in one pass: 256 CUs x 2 resident workgroups.
constexpr int64_t kFillWgs = 512;

cpa_status resolve(const cpa_attn_args* a, Resolved* r) {
    cpa_status st = check_common(a);
    if (st != CPA_OK) return st;
    if (a->num_seqs <= 0 || a->num_heads <= 0 || a->max_blocks_per_seq <= 0) return CPA_ERR_INVALID_ARG;
    if (a->num_seqs > kMaxSeqs) return CPA_ERR_UNSUPPORTED;
    if (a->num_heads % a->num_kv_heads != 0) return CPA_ERR_INVALID_ARG;
    if (!std::isfinite(a->scale) || !(a->scale > 0.f)) return CPA_ERR_INVALID_ARG;
    const int S = a->kv_segment_size;
    if (S != 0 && S != 512 && S != 1024 && S != 2048 && S != 4096) return CPA_ERR_INVALID_ARG;
    if (S != 0 && S % a->block_size != 0) return CPA_ERR_INVALID_ARG;
    if (a->decode_token_threshold < 0) return CPA_ERR_INVALID_ARG;
    const int seg = S ? S : 1024;
    auto resolve_split = [&](int32_t v, int32_t auto_value, int32_t* outv) -> cpa_status {
        if (v == 0) *outv = auto_value;
        else if (v < 0) *outv = kNoSplit;
        else if (v % seg != 0) return CPA_ERR_INVALID_ARG;
        else *outv = v;
        return CPA_OK;
    };
    r->seg = seg;
    r->hpg = a->num_heads / a->num_kv_heads;
    r->dec_thresh = a->decode_token_threshold ? a->decode_token_threshold : 1;
    r->log2_bs = ilog2(a->block_size);
    if ((st = resolve_split(a->split_keys_prefill, kNoSplit, &r->split_pre)) != CPA_OK) return st;
    if ((st = resolve_split(a->split_keys_decode, seg, &r->split_dec)) != CPA_OK) return st;
    if (!a->h_cu_seqlens_q || !a->h_cached_seq_len) return CPA_ERR_INVALID_ARG;
    const int32_t* cu = a->h_cu_seqlens_q;
    const int32_t* cc = a->h_cached_seq_len;
    if (cu[0] != 0 || cu[a->num_seqs] != a->total_q) return CPA_ERR_INVALID_ARG;
    for (int b = 0; b < a->num_seqs; ++b) {
        const int64_t n = (int64_t)cu[b + 1] - cu[b];
        if (n < 0 || cc[b] < 0) return CPA_ERR_INVALID_ARG;
        if (S == 0 && cc[b] != 0) return CPA_ERR_INVALID_ARG;
        const int64_t kv = cc[b] + n;
        if (kv >= ((int64_t)1 << 30)) return CPA_ERR_INVALID_ARG;
        if ((kv + a->block_size - 1) / a->block_size > a->max_blocks_per_seq) return CPA_ERR_INVALID_ARG;
    }
    int64_t items = 0, parts = 0, merge = 0;
    auto count = [&](int32_t split_pre) {
        items = parts = merge = 0;
        for (int b = 0; b < a->num_seqs; ++b) {
            const SeqPlan sp = seq_plan(cu[b + 1] - cu[b], cc[b], r->hpg, a->num_heads, r->dec_thresh,
                                        split_pre, r->split_dec);
            items += sp.items;
            parts += sp.parts;
            merge += sp.merge;
        }
    };
    count(r->split_pre);
    // Automatic prefill splits: when the call's work items leave most of the
    // GPU idle (fewer workgroups than half of kFillWgs, one per CU; e.g. one
    // KV-head group's share of a prompt), prefill rows are split into key
    // ranges of 8, 4, 2 or 1 segments, the longest that fills the GPU, their
    // partial states merged afterwards.  (A grid close to kFillWgs is left
    // alone: splitting it only adds a second pass and the merge.)
    if (a->split_keys_prefill == 0 && 2 * items * a->num_kv_heads < kFillWgs) {
        for (int mult : {8, 4, 2, 1}) {
            count(seg * mult);
            r->split_pre = seg * mult;
            if (items * a->num_kv_heads >= kFillWgs) break;
        }
    }
    if (items * a->num_kv_heads >= ((int64_t)1 << 31) || parts >= ((int64_t)1 << 31)) return CPA_ERR_UNSUPPORTED;
    r->items = items;
    r->parts = parts;
    r->merge = merge;
    r->ws = ws_layout(a->num_seqs, items, merge, parts, a->head_dim);
    return CPA_OK;
}

static_assert(kInlineDescInts == CPA_INLINE_DESC_INTS, "inline descriptor size");

// int32 values of the batch descriptor: cu_seqlens_q, cached_seq_len, block table
inline int64_t desc_ints(const cpa_attn_args* a) {
    return 2 * (int64_t)a->num_seqs + 1 + (int64_t)a->num_seqs * a->max_blocks_per_seq;
}
// the descriptor travels in the launches' arguments (host copies given, small enough)
inline bool inline_desc(const cpa_attn_args* a) {
    return a->h_block_table && a->h_cu_seqlens_q && a->h_cached_seq_len && a->num_seqs > 0 &&
           a->max_blocks_per_seq > 0 && desc_ints(a) <= kInlineDescInts;
}
// device copies of the descriptor, or NULL where they may be absent
inline bool have_desc(const cpa_attn_args* a) {
    return inline_desc(a) || (a->cu_seqlens_q && a->cached_seq_len && a->block_table);
}

cpa_status check_pointers(const cpa_attn_args* a, bool attention) {
    if (a->total_q > 0 && (!a->k_new || !a->v_new)) return CPA_ERR_INVALID_ARG;
    // without a slot mapping, slots come from the block table
    if (a->total_q > 0 && !a->slot_mapping &&
        (!have_desc(a) || a->num_seqs <= 0 || a->max_blocks_per_seq <= 0))
        return CPA_ERR_INVALID_ARG;
    if (!a->k_cache || !a->v_cache) return CPA_ERR_INVALID_ARG;
    if (attention) {
        if (a->total_q > 0 && (!a->q || !a->out)) return CPA_ERR_INVALID_ARG;
        if (!have_desc(a)) return CPA_ERR_INVALID_ARG;
    }
    return CPA_OK;
}

// Host mirrors of the descriptor, when a cache-write entry point is given
// them: cu_seqlens_q starts at 0, ends at total_q and never decreases, no
// cached length is negative, and without a slot mapping every sequence's
// positions fit a block-table row (the checks resolve() makes for attention).
cpa_status check_host_mirrors(const cpa_attn_args* a) {
    if (!a->h_cu_seqlens_q || !a->h_cached_seq_len) return CPA_OK;
    if (a->num_seqs <= 0) return CPA_ERR_INVALID_ARG;
    const int32_t* cu = a->h_cu_seqlens_q;
    if (cu[0] != 0 || cu[a->num_seqs] != a->total_q) return CPA_ERR_INVALID_ARG;
    for (int b = 0; b < a->num_seqs; ++b) {
        if (cu[b + 1] < cu[b] || a->h_cached_seq_len[b] < 0) return CPA_ERR_INVALID_ARG;
        // slots derived from the table: the positions must fit a table row
        if (!a->slot_mapping &&
            ((int64_t)a->h_cached_seq_len[b] + cu[b + 1] - cu[b] + a->block_size - 1) / a->block_size >
                a->max_blocks_per_seq)
            return CPA_ERR_INVALID_ARG;
    }
    return CPA_OK;
}

inline bool kv_fp8(const cpa_attn_args* a) { return a->kv_dtype == CPA_FP8_E4M3; }

inline float scale_or_one(float s) { return s == 0.f ? 1.f : s; }

template <typename T, int D, bool FP8>
cpa_status launch_prep(const cpa_attn_args* a, const Resolved* r, bool plan, const cpa_rope_args* rope,
                       hipStream_t stream) {
    PrepParams p{};
    if constexpr (FP8) {
        p.inv_k = 1.f / scale_or_one(a->k_scale);
        p.inv_v = 1.f / scale_or_one(a->v_scale);
    }
    p.k_new = a->k_new;
    p.v_new = a->v_new;
    p.k_cache = a->k_cache;
    p.v_cache = a->v_cache;
    p.slots = a->slot_mapping;
    p.block_table = a->block_table;
    p.max_blocks = a->max_blocks_per_seq;
    p.cu = a->cu_seqlens_q;
    p.cached = a->cached_seq_len;
    p.num_seqs = a->num_seqs;
    p.total_q = a->total_q;
    p.num_kv_heads = a->num_kv_heads;
    p.block_size = a->block_size;
    p.log2_bs = ilog2(a->block_size);
    p.num_blocks = a->num_blocks;
    p.cache_wgs = ((a->total_q + kCacheTok - 1) / kCacheTok) * a->num_kv_heads;
    p.plan = plan ? 1 : 0;
    if (plan) {
        char* ws = (char*)a->workspace;
        p.cu = a->cu_seqlens_q;
        p.cached = a->cached_seq_len;
        p.num_seqs = a->num_seqs;
        p.hpg = r->hpg;
        p.num_heads = a->num_heads;
        p.dec_thresh = r->dec_thresh;
        p.split_pre = r->split_pre;
        p.split_dec = r->split_dec;
        p.header = (int32_t*)ws;
        p.seq_info = (int4*)(ws + r->ws.seq_info);
        p.items = (int4*)(ws + r->ws.items);
        p.merge = (int2*)(ws + r->ws.merge);
    }
    p.num_heads = a->num_heads;
    if (rope) {
        p.rope = rope->interleaved ? 2 : 1;
        p.rope_wgs = (a->total_q + kRopeQTok - 1) / kRopeQTok;
        p.rope_theta = rope->theta;
        p.q = a->q;
        p.q_out = rope->q_out;
    }
    const int grid = p.cache_wgs + p.rope_wgs + (plan ? 1 : 0);
    if (grid == 0) return CPA_OK;
    if constexpr (FP8) {
        if (rope) return CPA_ERR_UNSUPPORTED;   // (refused earlier by check_rope)
    }
    if (inline_desc(a)) {
        // the host copies go into the launch's own arguments
        InlineDesc d;
        const int B = a->num_seqs;
        const int64_t nbt = (int64_t)B * a->max_blocks_per_seq;
        std::memcpy(d.v, a->h_cu_seqlens_q, (size_t)(B + 1) * 4);
        std::memcpy(d.v + B + 1, a->h_cached_seq_len, (size_t)B * 4);
        std::memcpy(d.v + 2 * B + 1, a->h_block_table, (size_t)nbt * 4);
        p.desc_len = (int32_t)desc_ints(a);
        p.desc_out = plan ? (int32_t*)((char*)a->workspace + r->ws.desc) : nullptr;
        if constexpr (FP8)
            hipLaunchKernelGGL((prep_kernel_inline<T, D, false, true>), dim3(grid), dim3(kThreads), 0, stream,
                               p, d);
        else if (rope)
            hipLaunchKernelGGL((prep_kernel_inline<T, D, true, false>), dim3(grid), dim3(kThreads), 0, stream,
                               p, d);
        else
            hipLaunchKernelGGL((prep_kernel_inline<T, D, false, false>), dim3(grid), dim3(kThreads), 0,
                               stream, p, d);
    } else {
        if constexpr (FP8)
            hipLaunchKernelGGL((prep_kernel<T, D, false, true>), dim3(grid), dim3(kThreads), 0, stream, p);
        else if (rope)
            hipLaunchKernelGGL((prep_kernel<T, D, true, false>), dim3(grid), dim3(kThreads), 0, stream, p);
        else
            hipLaunchKernelGGL((prep_kernel<T, D, false, false>), dim3(grid), dim3(kThreads), 0, stream, p);
    }
    return hipGetLastError() == hipSuccess ? CPA_OK : CPA_ERR_HIP;
}

template <typename T, int D, bool FP8>
cpa_status launch_attention(const cpa_attn_args* a, const Resolved* r, hipStream_t stream,
                            hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr) {
    char* ws = (char*)a->workspace;
    if (r->items > 0) {
        AttnParams p{};
        p.q = a->q;
        p.k_cache = a->k_cache;
        p.v_cache = a->v_cache;
        p.out = a->out;
        p.lse = a->lse;
        p.cu = a->cu_seqlens_q;
        p.cached = a->cached_seq_len;
        p.block_table = a->block_table;
        if (inline_desc(a)) {           // the copy the prepare launch left
            const int32_t* dw = (const int32_t*)(ws + r->ws.desc);
            p.cu = dw;
            p.cached = dw + a->num_seqs + 1;
            p.block_table = dw + 2 * a->num_seqs + 1;
        }
        p.seq_info = (const int4*)(ws + r->ws.seq_info);
        p.items = (const int4*)(ws + r->ws.items);
        p.part_ml = (float2*)(ws + r->ws.part_ml);
        p.part_o = (float*)(ws + r->ws.part_o);
        p.num_items = (int32_t)r->items;
        p.num_heads = a->num_heads;
        p.num_kv_heads = a->num_kv_heads;
        p.hpg = r->hpg;
        p.block_size = a->block_size;
        p.log2_bs = r->log2_bs;
        p.max_blocks = a->max_blocks_per_seq;
        p.num_blocks = a->num_blocks;
        p.total_q = a->total_q;
        p.dec_thresh = r->dec_thresh;
        p.split_pre = r->split_pre;
        p.split_dec = r->split_dec;
        p.scale_log2 = a->scale * 1.44269504088896340736f * (FP8 ? scale_or_one(a->k_scale) : 1.f);
        p.v_scale = FP8 ? scale_or_one(a->v_scale) : 1.f;
        const int grid = (int)(r->items * a->num_kv_heads);
        if (ev0 || ev1)   // events taken by the dispatch itself
            hipExtLaunchKernelGGL((attn_kernel<T, D, FP8>), dim3(grid), dim3(kThreads), 0, stream, ev0, ev1, 0,
                                  p);
        else
            hipLaunchKernelGGL((attn_kernel<T, D, FP8>), dim3(grid), dim3(kThreads), 0, stream, p);
        if (hipGetLastError() != hipSuccess) return CPA_ERR_HIP;
    }
    if (r->merge > 0) {
        MergeParams m{};
        m.cu = inline_desc(a) ? (const int32_t*)(ws + r->ws.desc) : a->cu_seqlens_q;
        m.seq_info = (const int4*)(ws + r->ws.seq_info);
        m.merge = (const int2*)(ws + r->ws.merge);
        m.part_ml = (const float2*)(ws + r->ws.part_ml);
        m.part_o = (const float*)(ws + r->ws.part_o);
        m.out = a->out;
        m.lse = a->lse;
        m.num_heads = a->num_heads;
        m.total_q = a->total_q;
        m.num_merge = (int32_t)r->merge;
        const int64_t threads = r->merge * a->num_heads * (D / 4);
        hipLaunchKernelGGL((merge_kernel<T, D>), dim3((int)((threads + kThreads - 1) / kThreads)),
                           dim3(kThreads), 0, stream, m);
        if (hipGetLastError() != hipSuccess) return CPA_ERR_HIP;
    }
    return CPA_OK;
}

// Scratch of the entry point that allocates nothing: one array per GPU,
// held from the code object's load to the end of the process.  In host code
// `scratch` names a host-side stand-in; the device address of each GPU's
// copy comes from hipGetSymbolAddress, taken once per device with that
// device current, and only that address is ever handed to a launch.
constexpr size_t kNoAllocScratch = CPA_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) char scratch[kNoAllocScratch];

}  // namespace cpa

using namespace cpa;

namespace {

cpa_status prep_dispatch(const cpa_attn_args* a, const Resolved* r, bool plan, const cpa_rope_args* rope,
                         hipStream_t s) {
    if (kv_fp8(a))
        return a->head_dim == 128 ? launch_prep<__bf16, 128, true>(a, r, plan, rope, s)
                                  : launch_prep<__bf16, 64, true>(a, r, plan, rope, s);
    if (a->dtype == CPA_BF16)
        return a->head_dim == 128 ? launch_prep<__bf16, 128, false>(a, r, plan, rope, s)
                                  : launch_prep<__bf16, 64, false>(a, r, plan, rope, s);
    return a->head_dim == 128 ? launch_prep<float, 128, false>(a, r, plan, rope, s)
                              : launch_prep<float, 64, false>(a, r, plan, rope, s);
}

// Host-visible checks of a rotary-embedding request: positions come from
// cu_seqlens_q and cached_seq_len, so those are needed even with slots.
cpa_status check_rope(const cpa_attn_args* a, const cpa_rope_args* rope) {
    if (!rope) return CPA_ERR_INVALID_ARG;
    if (!std::isfinite(rope->theta) || !(rope->theta > 0.f)) return CPA_ERR_INVALID_ARG;
    if (rope->interleaved != 0 && rope->interleaved != 1) return CPA_ERR_INVALID_ARG;
    if (a->num_heads <= 0 || a->num_heads % a->num_kv_heads != 0) return CPA_ERR_INVALID_ARG;
    if (a->total_q > 0 && (!a->q || !rope->q_out || a->num_seqs <= 0 ||
                           (!inline_desc(a) && (!a->cu_seqlens_q || !a->cached_seq_len))))
        return CPA_ERR_INVALID_ARG;
    if (kv_fp8(a)) return CPA_ERR_UNSUPPORTED;   // the rotating cache write stores bf16 rows
    return CPA_OK;
}

cpa_status attn_dispatch(const cpa_attn_args* a, const Resolved* r, hipStream_t s, hipEvent_t e0 = nullptr,
                         hipEvent_t e1 = nullptr) {
    if (kv_fp8(a))
        return a->head_dim == 128 ? launch_attention<__bf16, 128, true>(a, r, s, e0, e1)
                                  : launch_attention<__bf16, 64, true>(a, r, s, e0, e1);
    if (a->dtype == CPA_BF16)
        return a->head_dim == 128 ? launch_attention<__bf16, 128, false>(a, r, s, e0, e1)
                                  : launch_attention<__bf16, 64, false>(a, r, s, e0, e1);
    if (a->head_dim == 128) return CPA_ERR_UNSUPPORTED;   // fp32 D=128 needs 128 KiB of LDS tiles
    return launch_attention<float, 64, false>(a, r, s, e0, e1);
}

cpa_status check_workspace(const cpa_attn_args* a, const Resolved* r) {
    if (!a->workspace || a->workspace_bytes < r->ws.total) return CPA_ERR_WORKSPACE;
    return CPA_OK;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

cpa_status scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return CPA_ERR_HIP;
    if (dev >= kMaxDevices) return CPA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return CPA_ERR_HIP;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return CPA_OK;
}

}  // namespace

extern "C" {

const char* cpa_status_string(int status) {
    switch (status) {
        case CPA_OK: return "ok";
        case CPA_ERR_INVALID_ARG: return "invalid argument";
        case CPA_ERR_UNSUPPORTED: return "unsupported configuration";
        case CPA_ERR_BUDGET_EXHAUSTED: return "token budget exhausted";
        case CPA_ERR_OUT_OF_BLOCKS: return "out of KV-cache blocks";
        case CPA_ERR_HIP: return "HIP error";
        case CPA_ERR_WORKSPACE: return "workspace missing or too small";
        case CPA_ERR_NOT_FOUND: return "unknown request";
        default: return "unknown status";
    }
}

int cpa_abi_version(void) { return CPA_ABI_VERSION; }

cpa_status cpa_check_args(const cpa_attn_args* a) {
    Resolved r;
    cpa_status st = resolve(a, &r);
    if (st != CPA_OK) return st;
    if (a->dtype == CPA_FP32 && a->head_dim == 128) return CPA_ERR_UNSUPPORTED;
    return check_pointers(a, true);
}

cpa_status cpa_plan_counts(const cpa_attn_args* a, cpa_plan_info* info) {
    if (!info) return CPA_ERR_INVALID_ARG;
    Resolved r;
    cpa_status st = resolve(a, &r);
    if (st != CPA_OK) return st;
    info->num_items = (int32_t)r.items;
    info->num_merge_rows = (int32_t)r.merge;
    info->num_partials = r.parts;
    info->split_keys_prefill = r.split_pre == kNoSplit ? 0 : r.split_pre;
    info->split_keys_decode = r.split_dec == kNoSplit ? 0 : r.split_dec;
    info->workspace_bytes = r.ws.total;
    return CPA_OK;
}

cpa_status cpa_workspace_bytes(const cpa_attn_args* a, size_t* bytes) {
    if (!bytes) return CPA_ERR_INVALID_ARG;
    Resolved r;
    cpa_status st = resolve(a, &r);
    if (st != CPA_OK) return st;
    *bytes = r.ws.total;
    return CPA_OK;
}

cpa_status cpa_reshape_and_cache(const cpa_attn_args* a, void* stream) {
    cpa_status st = check_common(a);
    if (st != CPA_OK) return st;
    if ((st = check_pointers(a, false)) != CPA_OK) return st;
    if ((st = check_host_mirrors(a)) != CPA_OK) return st;
    Resolved r{};
    return prep_dispatch(a, &r, false, nullptr, (hipStream_t)stream);
}

cpa_status cpa_prepare(const cpa_attn_args* a, void* stream) {
    Resolved r;
    cpa_status st = resolve(a, &r);
    if (st != CPA_OK) return st;
    if (a->dtype == CPA_FP32 && a->head_dim == 128) return CPA_ERR_UNSUPPORTED;
    if ((st = check_pointers(a, true)) != CPA_OK) return st;
    if ((st = check_workspace(a, &r)) != CPA_OK) return st;
    return prep_dispatch(a, &r, true, nullptr, (hipStream_t)stream);
}

cpa_status cpa_attention(const cpa_attn_args* a, void* stream) {
    Resolved r;
    cpa_status st = resolve(a, &r);
    if (st != CPA_OK) return st;
    if ((st = check_pointers(a, true)) != CPA_OK) return st;
    if ((st = check_workspace(a, &r)) != CPA_OK) return st;
    return attn_dispatch(a, &r, (hipStream_t)stream);
}

cpa_status cpa_attention_timed(const cpa_attn_args* a, void* stream, void* start_event, void* stop_event) {
    if (!start_event || !stop_event) return CPA_ERR_INVALID_ARG;
    Resolved r;
    cpa_status st = resolve(a, &r);
    if (st != CPA_OK) return st;
    if ((st = check_pointers(a, true)) != CPA_OK) return st;
    if ((st = check_workspace(a, &r)) != CPA_OK) return st;
    return attn_dispatch(a, &r, (hipStream_t)stream, (hipEvent_t)start_event, (hipEvent_t)stop_event);
}

cpa_status cpa_chunked_prefill_attn(const cpa_attn_args* a, void* stream) {
    cpa_status st = cpa_prepare(a, stream);
    if (st != CPA_OK) return st;
    return cpa_attention(a, stream);
}

cpa_status cpa_chunked_prefill_attn_noalloc(const cpa_attn_args* a, void* stream) {
    Resolved r;
    cpa_status st = resolve(a, &r);
    if (st != CPA_OK) return st;
    if (r.ws.total > kNoAllocScratch) return CPA_ERR_WORKSPACE;
    void* ptr = nullptr;
    if ((st = scratch_address(&ptr)) != CPA_OK) return st;
    // the prepare launch writes every scratch byte the attention launch
    // reads (plan, descriptor copy; partials before their merge), so
    // nothing needs clearing
    cpa_attn_args local = *a;
    local.workspace = ptr;
    local.workspace_bytes = kNoAllocScratch;
    return cpa_chunked_prefill_attn(&local, stream);
}

cpa_status cpa_rope_reshape_and_cache(const cpa_attn_args* a, const cpa_rope_args* rope, void* stream) {
    cpa_status st = check_common(a);
    if (st != CPA_OK) return st;
    if ((st = check_pointers(a, false)) != CPA_OK) return st;
    if ((st = check_host_mirrors(a)) != CPA_OK) return st;
    if ((st = check_rope(a, rope)) != CPA_OK) return st;
    Resolved r{};
    return prep_dispatch(a, &r, false, rope, (hipStream_t)stream);
}

cpa_status cpa_rope_prepare(const cpa_attn_args* a, const cpa_rope_args* rope, void* stream) {
    Resolved r;
    cpa_status st = resolve(a, &r);
    if (st != CPA_OK) return st;
    if (a->dtype == CPA_FP32 && a->head_dim == 128) return CPA_ERR_UNSUPPORTED;
    if ((st = check_pointers(a, true)) != CPA_OK) return st;
    if ((st = check_rope(a, rope)) != CPA_OK) return st;
    if ((st = check_workspace(a, &r)) != CPA_OK) return st;
    return prep_dispatch(a, &r, true, rope, (hipStream_t)stream);
}

cpa_status cpa_rope_chunked_prefill_attn(const cpa_attn_args* a, const cpa_rope_args* rope, void* stream) {
    cpa_status st = cpa_rope_prepare(a, rope, stream);
    if (st != CPA_OK) return st;
    cpa_attn_args rotated = *a;
    rotated.q = rope->q_out;
    return cpa_attention(&rotated, stream);
}

}  // extern "C"

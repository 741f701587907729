/*
 * chunked_prefill_attn.h -- C ABI of libchunked_prefill_attn, chunked-prefill /
 * prefix-cached attention over a paged KV cache for AMD MI355X (gfx950).
 *
 * What one call computes ("Prefill Processing", sections "How Segmentation
 * Works with KV Segments", "Kernel Interface" and "Partial KV Segment
 * Handling"; "Prefill Optimisation: Prefix Caching, Chunked Prefill, and
 * Disaggregation", section 2, "Causal equivalence"):
 *   for every sequence b of a packed batch, its n_b active tokens (absolute
 *   positions c_b .. c_b+n_b-1, c_b = cached_seq_len[b]) are written into the
 *   paged KV cache, then each active token attends to the cached KV of its
 *   own sequence (positions < c_b, visited in kv_segment_size segments, the
 *   last one partial) and causally to the chunk itself (positions <= its own).
 *   out[t,h] = sum_j softmax_j(scale * <q[t,h], K_j>) V_j,  j <= c_b + t.
 *   Query head h reads KV head h / (num_heads / num_kv_heads).
 *
 * Conventions
 *   - Every pointer in cpa_attn_args is owned by the caller.  Pointers marked
 *     "device" are HIP device memory; "host" ones are ordinary host memory.
 *   - The library never allocates, frees or synchronises.  Device work is
 *     enqueued on the given stream (a hipStream_t passed as void*; NULL is the
 *     null stream) and the call returns at once.
 *   - Errors are returned as cpa_status codes.  Only host-visible arguments
 *     are validated (dimensions, host mirrors of the lengths); device-resident
 *     values (block ids, slots) are preconditions.  The attention kernel
 *     clamps a block id outside [0, num_blocks) to num_blocks - 1 (it reads
 *     that block instead), and the cache write skips a slot outside
 *     [0, num_blocks*block_size) and a block-table column outside the row, so
 *     a bad table gives wrong results, never an out-of-bounds access.
 *
 * Device layouts (dtype = element type; row-major, innermost last)
 *   q        [total_q, num_heads,    head_dim]
 *   k_new    [total_q, num_kv_heads, head_dim]   this call's new keys
 *   v_new    [total_q, num_kv_heads, head_dim]   this call's new values
 *   k_cache  [num_blocks, num_kv_heads, block_size, head_dim]
 *   v_cache  [num_blocks, num_kv_heads, head_dim, block_size]
 *            (values of one block and head are stored transposed: for a
 *            fixed dimension d the block_size tokens are contiguous)
 *   out      [total_q, num_heads, head_dim]
 *   lse      [num_heads, total_q] float32, optional (natural-log
 *            log-sum-exp of each row's scaled logits)
 *   cu_seqlens_q   int32 [num_seqs + 1], cu[0] = 0, cu[num_seqs] = total_q
 *   cached_seq_len int32 [num_seqs]      (the pages' prior_tokens, one per
 *                                         sequence)
 *   block_table    int32 [num_seqs, max_blocks_per_seq]; position p of
 *                  sequence b lives in block block_table[b][p / block_size]
 *                  at offset p % block_size; only the first
 *                  cdiv(c_b + n_b, block_size) columns are read
 *   slot_mapping   int64 [total_q]; slot = block * block_size + offset of
 *                  each active token ("Prefill Processing", section
 *                  "Attention Metadata")
 */
#ifndef CHUNKED_PREFILL_ATTN_H
#define CHUNKED_PREFILL_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CPA_ABI_VERSION 3

/* Largest batch descriptor (2 * num_seqs + 1 + num_seqs * max_blocks_per_seq
 * int32 values) that cpa_prepare can take inline from host copies. */
#define CPA_INLINE_DESC_INTS 896

typedef enum cpa_status {
    CPA_OK = 0,
    CPA_ERR_INVALID_ARG = 1,      /* a host-visible argument is out of range   */
    CPA_ERR_UNSUPPORTED = 2,      /* valid, but not built (e.g. head_dim 96)   */
    CPA_ERR_BUDGET_EXHAUSTED = 3, /* no prefill progress possible              */
    CPA_ERR_OUT_OF_BLOCKS = 4,    /* the pool cannot hold the step's blocks    */
    CPA_ERR_HIP = 5,              /* a HIP launch or runtime call failed       */
    CPA_ERR_WORKSPACE = 6,        /* workspace missing or smaller than needed  */
    CPA_ERR_NOT_FOUND = 7         /* unknown request id                        */
} cpa_status;

typedef enum cpa_dtype {
    CPA_BF16 = 0,                 /* bfloat16 in/out, float32 accumulation     */
    CPA_FP32 = 1,                 /* float32 throughout                        */
    CPA_FP8_E4M3 = 2              /* KV cache only (kv_dtype): OCP E4M3 codes  */
} cpa_dtype;

/* Per-call attention metadata: the pages' metadata dict ("Prefill
 * Processing", section "Attention Metadata") as a plain struct. */
typedef struct cpa_attn_args {
    int32_t dtype;                  /* cpa_dtype                                */
    int32_t num_seqs;               /* B, 1 .. 4096                             */
    int32_t total_q;                /* T = sum of chunk lengths                 */
    int32_t num_heads;              /* H (query heads)                          */
    int32_t num_kv_heads;           /* G, divides H                             */
    int32_t head_dim;               /* D: 64 or 128                             */
    int32_t block_size;             /* power of two, 8 .. 512                   */
    int32_t kv_segment_size;        /* 512, 1024, 2048 or 4096 (multiple of
                                       block_size); 0 = no cached KV: every
                                       cached_seq_len must then be 0            */
    int32_t max_blocks_per_seq;     /* block_table row width                    */
    int32_t num_blocks;             /* pool size                                */
    int32_t decode_token_threshold; /* rows with n_b <= this are decode rows;
                                       0 means 1 ("1 + max_num_draft_tokens")   */
    int32_t split_keys_prefill;     /* keys per work item for prefill rows:
                                       0 automatic, -1 never split, else a
                                       multiple of kv_segment_size.  Automatic
                                       leaves rows unsplit unless the call's
                                       work items times num_kv_heads number
                                       under 256 (one per CU of MI355X); then
                                       it takes the longest of 8, 4, 2, 1
                                       segments per item that reaches 512 (one
                                       full pass), or 1 segment                 */
    int32_t split_keys_decode;      /* same for decode rows (0: one segment)    */
    float   scale;                  /* softmax scale > 0, usually 1/sqrt(D)     */
    const void* q;                  /* device                                   */
    const void* k_new;              /* device                                   */
    const void* v_new;              /* device                                   */
    void* k_cache;                  /* device, written in place                 */
    void* v_cache;                  /* device, written in place                 */
    const int32_t* cu_seqlens_q;    /* device                                   */
    const int32_t* cached_seq_len;  /* device                                   */
    const int32_t* block_table;     /* device                                   */
    const int64_t* slot_mapping;    /* device, or NULL: each active token's slot
                                       is then block_table[b][p / block_size] *
                                       block_size + p % block_size, p =
                                       cached_seq_len[b] + its offset in the
                                       chunk, the same formula                 */
    void* out;                      /* device                                   */
    float* lse;                     /* device, may be NULL                      */
    void* workspace;                /* device scratch, >= cpa_workspace_bytes() */
    size_t workspace_bytes;
    const int32_t* h_cu_seqlens_q;  /* host copy of cu_seqlens_q (grid sizing)  */
    const int32_t* h_cached_seq_len;/* host copy of cached_seq_len             */
    /* Cache element type ("Prefill Optimisation ...", section 3 counts the
     * element type among what makes a cache entry): 0 (or dtype) keeps
     * dtype; CPA_FP8_E4M3 stores one-byte OCP E4M3 codes, with dtype
     * CPA_BF16 and block_size >= 16 (else CPA_ERR_UNSUPPORTED).  A stored
     * code is that of x * (1/scale), the product in float, clamped to
     * +-448, rounded to nearest even; its value is code * scale.  k_cache
     * and v_cache keep their layouts with one byte per element. */
    int32_t kv_dtype;
    float   k_scale;                /* fp8 cache: K scale, > 0 (0 means 1)     */
    float   v_scale;                /* fp8 cache: V scale, > 0 (0 means 1)     */
    /* Host copy of block_table (num_seqs rows of max_blocks_per_seq), or
     * NULL.  When it is given and the descriptor fits CPA_INLINE_DESC_INTS,
     * the launches take cu_seqlens_q, cached_seq_len and the block table
     * from the host copies, read at the call (no separate upload): the
     * prepare launch carries them as kernel arguments and leaves a copy in
     * the workspace, which cpa_attention then reads.  The device arrays are
     * not read and may be NULL; cpa_prepare and cpa_attention of one batch
     * must then both be given the host copies.  A larger descriptor needs
     * the device arrays, as does a NULL h_block_table. */
    const int32_t* h_block_table;
} cpa_attn_args;

/* Work decomposition the library derives from the host mirrors. */
typedef struct cpa_plan_info {
    int32_t num_items;          /* work items per KV head (grid = items * G)  */
    int32_t num_merge_rows;     /* tokens whose partials need a merge pass    */
    int64_t num_partials;       /* (split, token, head) partial states        */
    int32_t split_keys_prefill; /* resolved keys per item, 0 = unsplit        */
    int32_t split_keys_decode;
    size_t  workspace_bytes;
} cpa_plan_info;

/* Name of a status code (static string). */
const char* cpa_status_string(int status);

/* CPA_ABI_VERSION of the built library. */
int cpa_abi_version(void);

/* Validate every host-visible field of *args (no device access). */
cpa_status cpa_check_args(const cpa_attn_args* args);

/* Work plan and workspace size for *args (host only).  The workspace holds
 * the device-side work list and, when rows are split across work items,
 * their partial softmax states. */
cpa_status cpa_plan_counts(const cpa_attn_args* args, cpa_plan_info* info);
cpa_status cpa_workspace_bytes(const cpa_attn_args* args, size_t* bytes);

/* Cache write alone: k_new/v_new row t goes to slot slot_mapping[t] of
 * k_cache/v_cache, bit for bit ("Prefill Processing", section "How
 * Segmentation Works with KV Segments": each iteration writes the KV of its
 * active tokens).  Reads dtype, num_kv_heads, head_dim, block_size,
 * num_blocks, total_q and the five pointers it needs; with slot_mapping NULL
 * also num_seqs, max_blocks_per_seq, cu_seqlens_q, cached_seq_len and
 * block_table, from which the slots are derived. */
cpa_status cpa_reshape_and_cache(const cpa_attn_args* args, void* stream);

/* Cache write plus the device work plan (written into the workspace). */
cpa_status cpa_prepare(const cpa_attn_args* args, void* stream);

/* Attention over the cache (segments of cached KV + causal self part) and
 * the log-sum-exp merge of split rows.  Reads the plan that cpa_prepare
 * wrote into the same workspace for the same batch; may be called again
 * (e.g. once per layer with other q/cache/out pointers of the same shapes). */
cpa_status cpa_attention(const cpa_attn_args* args, void* stream);

/* cpa_attention with the attention kernel's own dispatch taking two events
 * (hipEvent_t, created by the caller on the device of `stream`): start_event
 * when the kernel starts, stop_event when it ends, so that their elapsed
 * time is the kernel's duration with no event records of their own in the
 * stream.  The merge launch of split rows, if any, follows stop_event.  For
 * callers that time the kernel inside a measured loop.  CPA_ERR_INVALID_ARG
 * for a NULL event; otherwise as cpa_attention. */
cpa_status cpa_attention_timed(const cpa_attn_args* args, void* stream, void* start_event,
                               void* stop_event);

/* cpa_prepare followed by cpa_attention: the whole chunk step. */
cpa_status cpa_chunked_prefill_attn(const cpa_attn_args* args, void* stream);

/* Bytes of the library's own per-GPU scratch (below). */
#define CPA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* cpa_chunked_prefill_attn for callers that cannot allocate (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * plan and any partial states go to a scratch array of
 * CPA_NOALLOC_SCRATCH_BYTES that the library holds on each GPU from its
 * first use there until the process ends; args->workspace and
 * args->workspace_bytes are ignored.  No allocation or free of any kind
 * happens in the call.  Every call on one GPU shares that GPU's scratch, so
 * calls that overlap on one GPU (other streams, other threads) race: the
 * caller serialises them.  CPA_ERR_WORKSPACE when the call needs more than
 * CPA_NOALLOC_SCRATCH_BYTES (cpa_workspace_bytes tells); otherwise as
 * cpa_chunked_prefill_attn. */
cpa_status cpa_chunked_prefill_attn_noalloc(const cpa_attn_args* args, void* stream);

/* ---------------------------------------------------------------------
 * Rotary position embedding fused into the cache write.
 *
 * Every active token is rotated at its absolute position p = cached_seq_len[b]
 * + (its offset in the chunk) ("Prefill Optimisation: Prefix Caching, Chunked
 * Prefill, and Disaggregation", section 2, "Causal equivalence": positional
 * encodings take the token's absolute position in the whole sequence;
 * "Chunked Prefill" blog note, section "From scratch": the cached length is
 * the position offset of a step's tokens).  The pages name the rotary
 * embedding without writing it out; the form here is the standard one: pair
 * i of a head (i = 0 .. head_dim/2 - 1) turns by p * theta^(-2i/head_dim)
 * radians, (x, y) -> (x cos - y sin, x sin + y cos), computed in float from
 * cos/sin evaluated in double and rounded to float; results are rounded to
 * the element type.  Values are not rotated.
 * ------------------------------------------------------------------- */
typedef struct cpa_rope_args {
    float   theta;        /* rotary base, finite and > 0 (10000 is common)    */
    int32_t interleaved;  /* 0: element i pairs with i + head_dim/2
                             ("rotate half"); 1: element 2i with 2i + 1      */
    void*   q_out;        /* device [total_q, num_heads, head_dim], element
                             type of q: the rotated queries.  May equal
                             args->q (rotation in place); otherwise the two
                             must not overlap.                               */
} cpa_rope_args;

/* Cache write of rotated keys (values unchanged), and the rotated queries
 * into rope->q_out.  Reads what cpa_reshape_and_cache reads plus q,
 * num_heads, num_seqs, cu_seqlens_q and cached_seq_len (positions are
 * needed even when slot_mapping is given).  CPA_ERR_INVALID_ARG for a NULL
 * rope, a bad theta or interleaved flag, num_heads not a multiple of
 * num_kv_heads, or a missing pointer; CPA_ERR_UNSUPPORTED with an FP8
 * cache (kv_dtype CPA_FP8_E4M3): the rotation is written into bf16 rows
 * only. */
cpa_status cpa_rope_reshape_and_cache(const cpa_attn_args* args, const cpa_rope_args* rope,
                                      void* stream);

/* cpa_prepare with the rotation above in its cache write. */
cpa_status cpa_rope_prepare(const cpa_attn_args* args, const cpa_rope_args* rope, void* stream);

/* cpa_rope_prepare, then cpa_attention on the rotated queries (rope->q_out
 * in place of args->q): the whole chunk step of a rotary model. */
cpa_status cpa_rope_chunked_prefill_attn(const cpa_attn_args* args, const cpa_rope_args* rope,
                                         void* stream);

/* ---------------------------------------------------------------------
 * Host scheduler (no device memory).
 * ------------------------------------------------------------------- */

/* Chunk sizes of one prompt under a token budget with active_decodes
 * decodes holding one token each ("Prefill Optimisation ...", section 7,
 * schedule_prompt).  align_to_block != 0 cuts every chunk that does not
 * finish the prompt to whole blocks ("vLLM Chunked Prefill 如何改变 KV Cache
 * 管理", section 2.3).  Writes at most `capacity` sizes to chunks and their
 * number to *num_chunks.  CPA_ERR_BUDGET_EXHAUSTED when no token (or no
 * whole block) fits; CPA_ERR_INVALID_ARG for non-positive budget, negative
 * counts, or capacity too small. */
cpa_status cpa_schedule_prompt(int32_t max_batched_tokens, int32_t active_decodes,
                               int64_t total_prompt_tokens, int32_t block_size,
                               int32_t align_to_block, int32_t* chunks,
                               int32_t capacity, int32_t* num_chunks);

/* Decode-first token-budget scheduler with a paged block pool.
 * Decodes take one token each, then prefills in arrival order take
 * min(remaining, budget left, long_prefill_cap) tokens, cut to whole blocks
 * when align_to_block is set and the prompt does not finish ("Chunked
 * Prefill" blog note, section "From scratch"; "Prefill Optimisation ...",
 * section 2).  Blocks are allocated incrementally: cdiv(computed + new,
 * block_size) minus those held ("Prefill Processing", section "Block
 * Allocation").  Shared prefix blocks are reference counted. */
typedef struct cpa_sched cpa_sched;

typedef struct cpa_sched_config {
    int32_t num_blocks;          /* pool size                                 */
    int32_t block_size;
    int32_t max_batched_tokens;  /* token budget per step                     */
    int32_t max_blocks_per_seq;  /* block-table row width                     */
    int32_t long_prefill_cap;    /* per-prefill cap per step, 0 = none        */
    int32_t align_to_block;      /* prefix caching on: block-aligned chunks   */
    const int32_t* free_order;   /* host [num_blocks]: order in which free
                                    blocks are handed out (a permutation of
                                    0..num_blocks-1), NULL = 0,1,2,...         */
    int32_t prefix_caching;      /* 1: match and register full prompt blocks
                                    of requests given by token ids (below)    */
    int32_t max_long_partial_prefills; /* prompts longer than long_prefill_cap
                                    scheduled per step at most (0: no limit);
                                    later long prompts wait while shorter ones
                                    behind them run ("vLLM Chunked Prefill
                                    ...", section 3.3)                         */
    int32_t preemption;          /* 1: a step whose blocks do not fit preempts
                                    requests instead of failing (see
                                    cpa_sched_step)                            */
} cpa_sched_config;

/* Batch descriptor of one step, written into caller-owned host arrays. */
typedef struct cpa_batch {
    int32_t max_seqs;            /* in: capacity of the per-sequence arrays   */
    int32_t max_tokens;          /* in: capacity of slot_mapping              */
    int64_t* req_ids;            /* [max_seqs]                                */
    int32_t* q_lens;             /* [max_seqs]                                */
    int32_t* cu_seqlens_q;       /* [max_seqs + 1]                            */
    int32_t* cached_seq_len;     /* [max_seqs]                                */
    int32_t* block_table;        /* [max_seqs * max_blocks_per_seq], rows
                                    padded with 0 past the held blocks        */
    int64_t* slot_mapping;       /* [max_tokens]                              */
    int32_t num_seqs;            /* out                                       */
    int32_t num_tokens;          /* out                                       */
} cpa_batch;

cpa_status cpa_sched_create(const cpa_sched_config* config, cpa_sched** out);
void       cpa_sched_destroy(cpa_sched* sched);

/* New prompt; prefix_blocks (may be NULL) are the shared blocks of a prefix
 * hit, so num_prefix_blocks * block_size tokens start out computed (the
 * lookup happens only before the first chunk: "vLLM Chunked Prefill ...",
 * section 2.2).  Every prefix block must be active (held by someone). */
cpa_status cpa_sched_add_request(cpa_sched* sched, int64_t req_id, int32_t num_prompt_tokens,
                                 const int32_t* prefix_blocks, int32_t num_prefix_blocks);

/* New prompt given by its token ids under a scope (name_space; NULL means
 * "default").  With prefix_caching on ("Prefill Optimisation ...", section
 * 3, "vLLM block hash chain"; "vLLM Chunked Prefill ...", sections 2.2 and
 * 3.1):
 *   - when the request is first scheduled, its prompt's full blocks are
 *     looked up along the parent-chained digest of (parent, scope, token
 *     ids), over the blocks of that first chunk only and leaving at least the
 *     prompt's last token to compute; the matched blocks join its table with
 *     their reference counts raised and count as computed;
 *   - each full prompt block it computes is registered under its digest
 *     (the first block holding a digest keeps it);
 *   - blocks it releases that hold a registered digest become reclaimable
 *     (its last block first) and are evicted, least recently freed first,
 *     only when no empty block is left.
 * Without prefix caching it behaves as cpa_sched_add_request with no
 * prefix.  CPA_ERR_INVALID_ARG for an empty prompt, a duplicate id or a
 * prompt longer than a table row maps. */
cpa_status cpa_sched_add_request_tokens(cpa_sched* sched, int64_t req_id, const uint32_t* tokens,
                                        int32_t num_tokens, const char* name_space);

/* Running sequence with context_len cached tokens and one token to decode;
 * its cdiv(context_len, block_size) cache blocks are taken from the pool. */
cpa_status cpa_sched_add_decode(cpa_sched* sched, int64_t req_id, int32_t context_len);

/* Prompt of num_prompt_tokens whose first num_computed_tokens are already in
 * the cache (an earlier chunk, a resumed request): it takes
 * cdiv(num_computed_tokens, block_size) blocks from the pool now and continues
 * from position num_computed_tokens ("vLLM Chunked Prefill ...", section 2.1:
 * num_computed_tokens is the resume pointer). */
cpa_status cpa_sched_add_partial(cpa_sched* sched, int64_t req_id, int32_t num_prompt_tokens,
                                 int32_t num_computed_tokens);

/* Build the next step (tokens, block growth, descriptor).  When the pool
 * cannot hold the step: without preemption, CPA_ERR_OUT_OF_BLOCKS and
 * nothing changes; with it ("vLLM Chunked Prefill ...", section 4), the most
 * recently arrived request holding blocks is preempted (all its blocks
 * released, its progress reset to position 0, so it recomputes every known
 * token later) and the step is planned again without it, until it fits;
 * CPA_ERR_OUT_OF_BLOCKS only when nothing is left to preempt (preemptions
 * made so far stay made). */
cpa_status cpa_sched_step(cpa_sched* sched, cpa_batch* batch);

/* Ids of the requests the last cpa_sched_step preempted, in order. */
cpa_status cpa_sched_last_preempted(const cpa_sched* sched, int64_t* ids, int32_t capacity,
                                    int32_t* num);

/* Advance every request of the last step; a finished prompt becomes a decode. */
cpa_status cpa_sched_commit(cpa_sched* sched);

/* Release a request's block references. */
cpa_status cpa_sched_free_request(cpa_sched* sched, int64_t req_id);

cpa_status cpa_sched_request_info(const cpa_sched* sched, int64_t req_id, int32_t* num_tokens,
                                  int32_t* num_computed, int32_t* num_blocks, int32_t* is_decode);
cpa_status cpa_sched_request_blocks(const cpa_sched* sched, int64_t req_id, int32_t* blocks,
                                    int32_t capacity, int32_t* num_blocks);
/* Slots of positions pos0 .. pos0+n-1 of a request (positions must lie in
 * held blocks). */
cpa_status cpa_sched_slots(const cpa_sched* sched, int64_t req_id, int32_t pos0, int32_t n,
                           int64_t* slots);
/* Blocks allocation can hand out: empty plus reclaimable cached ones
 * ("Prefill Optimisation ...", section 3, "Accounting considerations"). */
cpa_status cpa_sched_num_free_blocks(const cpa_sched* sched, int32_t* num_free);
/* The pool's three disjoint buckets: active (reference count > 0),
 * reclaimable cached (count 0, registered digest) and empty (any may be
 * NULL). */
cpa_status cpa_sched_pool_stats(const cpa_sched* sched, int32_t* num_active,
                                int32_t* num_reclaimable, int32_t* num_empty);
/* Tokens of `tokens` (full blocks from the first) that are registered now
 * under name_space; no state changes. */
cpa_status cpa_sched_prefix_match(const cpa_sched* sched, const uint32_t* tokens, int32_t num_tokens,
                                  const char* name_space, int32_t* num_cached_tokens);
cpa_status cpa_sched_block_refcount(const cpa_sched* sched, int32_t block, int32_t* refcount);

#ifdef __cplusplus
}
#endif

#endif /* CHUNKED_PREFILL_ATTN_H */

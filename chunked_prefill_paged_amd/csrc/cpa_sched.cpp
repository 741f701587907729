// Host side of the path: token-budget scheduling, the paged block pool and
// the batch descriptor.  Pure host C++; no device memory is touched here.
//
// Sources: "Prefill Optimisation: Prefix Caching, Chunked Prefill, and
// Disaggregation", section 2 (decode-first budget) and section 7
// (schedule_prompt); "Chunked Prefill" blog note, section "From scratch"
// (per-prefill cap, skip instead of raise); "vLLM Chunked Prefill 如何改变 KV
// Cache 管理", sections 2.1-2.3 (incremental allocation, first-chunk-only
// prefix hits, block-aligned budget); "Prefill Processing", sections
// "Scheduler Integration" and "Block Allocation".

#include <cstdint>
#include <cstring>
#include <deque>
#include <new>
#include <vector>

#include "chunked_prefill_attn.h"

namespace {

inline int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Request {
    int64_t id;
    int32_t num_tokens;    // tokens known (prompt, then + generated)
    int32_t num_computed;  // tokens whose KV is cached
    bool is_decode;
    std::vector<int32_t> blocks;
};

}  // namespace

struct cpa_sched {
    int32_t block_size = 0;
    int32_t budget = 0;
    int32_t max_blocks = 0;
    int32_t cap = 0;
    bool align = false;
    std::deque<int32_t> free_list;      // FIFO: hand out from the front
    std::vector<int32_t> ref;           // reference count per block
    std::vector<Request> reqs;          // arrival order
    std::vector<std::pair<size_t, int32_t>> last;  // (request index, tokens) of the last step

    Request* find(int64_t id) {
        for (auto& r : reqs)
            if (r.id == id) return &r;
        return nullptr;
    }
    const Request* find(int64_t id) const {
        for (auto& r : reqs)
            if (r.id == id) return &r;
        return nullptr;
    }
    void take(int32_t n, std::vector<int32_t>& dst) {
        for (int32_t i = 0; i < n; ++i) {
            int32_t b = free_list.front();
            free_list.pop_front();
            ref[b] = 1;
            dst.push_back(b);
        }
    }
    void release(const std::vector<int32_t>& blocks) {
        for (int32_t b : blocks) {
            if (--ref[b] == 0) free_list.push_back(b);
        }
    }
};

extern "C" {

cpa_status cpa_schedule_prompt(int32_t max_batched_tokens, int32_t active_decodes,
                               int64_t total_prompt_tokens, int32_t block_size,
                               int32_t align_to_block, int32_t* chunks, int32_t capacity,
                               int32_t* num_chunks) {
    if (!num_chunks || max_batched_tokens <= 0 || active_decodes < 0 || total_prompt_tokens < 0)
        return CPA_ERR_INVALID_ARG;
    if (align_to_block && block_size <= 0) return CPA_ERR_INVALID_ARG;
    *num_chunks = 0;
    const int64_t budget = (int64_t)max_batched_tokens - active_decodes;
    if (budget <= 0) return CPA_ERR_BUDGET_EXHAUSTED;
    int64_t remaining = total_prompt_tokens;
    int32_t count = 0;
    while (remaining > 0) {
        int64_t take = remaining < budget ? remaining : budget;
        if (align_to_block && take < remaining) {
            take = (take / block_size) * block_size;
            if (take == 0) return CPA_ERR_BUDGET_EXHAUSTED;
        }
        if (count >= capacity || !chunks) return CPA_ERR_INVALID_ARG;
        chunks[count++] = (int32_t)take;
        remaining -= take;
    }
    *num_chunks = count;
    return CPA_OK;
}

cpa_status cpa_sched_create(const cpa_sched_config* cfg, cpa_sched** out) {
    if (!cfg || !out) return CPA_ERR_INVALID_ARG;
    *out = nullptr;
    if (cfg->num_blocks <= 0 || cfg->block_size <= 0 || cfg->max_batched_tokens <= 0 ||
        cfg->max_blocks_per_seq <= 0 || cfg->long_prefill_cap < 0)
        return CPA_ERR_INVALID_ARG;
    cpa_sched* s = new (std::nothrow) cpa_sched();
    if (!s) return CPA_ERR_INVALID_ARG;
    s->block_size = cfg->block_size;
    s->budget = cfg->max_batched_tokens;
    s->max_blocks = cfg->max_blocks_per_seq;
    s->cap = cfg->long_prefill_cap;
    s->align = cfg->align_to_block != 0;
    s->ref.assign(cfg->num_blocks, 0);
    if (cfg->free_order) {
        std::vector<char> seen(cfg->num_blocks, 0);
        for (int32_t i = 0; i < cfg->num_blocks; ++i) {
            int32_t b = cfg->free_order[i];
            if (b < 0 || b >= cfg->num_blocks || seen[b]) {
                delete s;
                return CPA_ERR_INVALID_ARG;   // not a permutation
            }
            seen[b] = 1;
            s->free_list.push_back(b);
        }
    } else {
        for (int32_t i = 0; i < cfg->num_blocks; ++i) s->free_list.push_back(i);
    }
    *out = s;
    return CPA_OK;
}

void cpa_sched_destroy(cpa_sched* s) { delete s; }

cpa_status cpa_sched_add_request(cpa_sched* s, int64_t req_id, int32_t num_prompt_tokens,
                                 const int32_t* prefix_blocks, int32_t num_prefix_blocks) {
    if (!s || num_prompt_tokens <= 0 || num_prefix_blocks < 0) return CPA_ERR_INVALID_ARG;
    if (num_prefix_blocks > 0 && !prefix_blocks) return CPA_ERR_INVALID_ARG;
    if (s->find(req_id)) return CPA_ERR_INVALID_ARG;
    const int64_t computed = (int64_t)num_prefix_blocks * s->block_size;
    if (computed >= num_prompt_tokens) return CPA_ERR_INVALID_ARG;
    if (cdiv64(num_prompt_tokens, s->block_size) > s->max_blocks) return CPA_ERR_INVALID_ARG;
    for (int32_t i = 0; i < num_prefix_blocks; ++i) {
        int32_t b = prefix_blocks[i];
        if (b < 0 || b >= (int32_t)s->ref.size() || s->ref[b] <= 0) return CPA_ERR_INVALID_ARG;
    }
    Request r;
    r.id = req_id;
    r.num_tokens = num_prompt_tokens;
    r.num_computed = (int32_t)computed;
    r.is_decode = false;
    for (int32_t i = 0; i < num_prefix_blocks; ++i) {
        s->ref[prefix_blocks[i]] += 1;
        r.blocks.push_back(prefix_blocks[i]);
    }
    s->reqs.push_back(std::move(r));
    return CPA_OK;
}

cpa_status cpa_sched_add_decode(cpa_sched* s, int64_t req_id, int32_t context_len) {
    if (!s || context_len <= 0) return CPA_ERR_INVALID_ARG;
    if (s->find(req_id)) return CPA_ERR_INVALID_ARG;
    const int64_t need = cdiv64(context_len, s->block_size);
    if (cdiv64((int64_t)context_len + 1, s->block_size) > s->max_blocks) return CPA_ERR_INVALID_ARG;
    if (need > (int64_t)s->free_list.size()) return CPA_ERR_OUT_OF_BLOCKS;
    Request r;
    r.id = req_id;
    r.num_tokens = context_len + 1;
    r.num_computed = context_len;
    r.is_decode = true;
    s->take((int32_t)need, r.blocks);
    s->reqs.push_back(std::move(r));
    return CPA_OK;
}

cpa_status cpa_sched_add_partial(cpa_sched* s, int64_t req_id, int32_t num_prompt_tokens,
                                 int32_t num_computed_tokens) {
    if (!s || num_computed_tokens < 0 || num_prompt_tokens <= num_computed_tokens)
        return CPA_ERR_INVALID_ARG;
    if (s->find(req_id)) return CPA_ERR_INVALID_ARG;
    if (cdiv64(num_prompt_tokens, s->block_size) > s->max_blocks) return CPA_ERR_INVALID_ARG;
    const int64_t need = cdiv64(num_computed_tokens, s->block_size);
    if (need > (int64_t)s->free_list.size()) return CPA_ERR_OUT_OF_BLOCKS;
    Request r;
    r.id = req_id;
    r.num_tokens = num_prompt_tokens;
    r.num_computed = num_computed_tokens;
    r.is_decode = false;
    s->take((int32_t)need, r.blocks);
    s->reqs.push_back(std::move(r));
    return CPA_OK;
}

cpa_status cpa_sched_step(cpa_sched* s, cpa_batch* out) {
    if (!s || !out) return CPA_ERR_INVALID_ARG;
    std::vector<std::pair<size_t, int32_t>> picked;
    int64_t used = 0;
    // decodes first, one token each
    for (size_t i = 0; i < s->reqs.size(); ++i) {
        if (s->reqs[i].is_decode && used < s->budget) {
            picked.emplace_back(i, 1);
            used += 1;
        }
    }
    // then prefills in arrival order with what is left
    for (size_t i = 0; i < s->reqs.size(); ++i) {
        const Request& r = s->reqs[i];
        if (r.is_decode) continue;
        if (used >= s->budget) break;
        const int64_t remaining = (int64_t)r.num_tokens - r.num_computed;
        int64_t take = remaining < s->budget - used ? remaining : s->budget - used;
        if (s->cap > 0 && take > s->cap) take = s->cap;
        if (s->align && take < remaining) take = (take / s->block_size) * s->block_size;
        if (take <= 0) continue;
        picked.emplace_back(i, (int32_t)take);
        used += take;
    }
    // capacity of the caller's arrays
    if ((int64_t)picked.size() > out->max_seqs || used > out->max_tokens) return CPA_ERR_INVALID_ARG;
    if (!out->req_ids || !out->q_lens || !out->cu_seqlens_q || !out->cached_seq_len ||
        !out->block_table || !out->slot_mapping)
        return CPA_ERR_INVALID_ARG;
    // block growth: all or nothing
    int64_t need_total = 0;
    std::vector<int32_t> need_new(picked.size());
    for (size_t k = 0; k < picked.size(); ++k) {
        const Request& r = s->reqs[picked[k].first];
        const int64_t need = cdiv64((int64_t)r.num_computed + picked[k].second, s->block_size);
        if (need > s->max_blocks) return CPA_ERR_INVALID_ARG;
        need_new[k] = (int32_t)(need - (int64_t)r.blocks.size());
        need_total += need_new[k];
    }
    if (need_total > (int64_t)s->free_list.size()) return CPA_ERR_OUT_OF_BLOCKS;
    for (size_t k = 0; k < picked.size(); ++k) {
        Request& r = s->reqs[picked[k].first];
        if (need_new[k] > 0) s->take(need_new[k], r.blocks);
    }
    // descriptor
    out->cu_seqlens_q[0] = 0;
    int64_t tok = 0;
    for (size_t k = 0; k < picked.size(); ++k) {
        const Request& r = s->reqs[picked[k].first];
        const int32_t n = picked[k].second;
        out->req_ids[k] = r.id;
        out->q_lens[k] = n;
        out->cached_seq_len[k] = r.num_computed;
        out->cu_seqlens_q[k + 1] = out->cu_seqlens_q[k] + n;
        int32_t* row = out->block_table + (size_t)k * s->max_blocks;
        const size_t held = r.blocks.size();
        for (int32_t j = 0; j < s->max_blocks; ++j) row[j] = (size_t)j < held ? r.blocks[j] : 0;
        for (int32_t t = 0; t < n; ++t) {
            const int64_t p = (int64_t)r.num_computed + t;
            out->slot_mapping[tok++] =
                (int64_t)r.blocks[p / s->block_size] * s->block_size + p % s->block_size;
        }
    }
    out->num_seqs = (int32_t)picked.size();
    out->num_tokens = (int32_t)used;
    s->last = std::move(picked);
    return CPA_OK;
}

cpa_status cpa_sched_commit(cpa_sched* s) {
    if (!s) return CPA_ERR_INVALID_ARG;
    for (auto& pk : s->last) {
        Request& r = s->reqs[pk.first];
        r.num_computed += pk.second;
        if (r.is_decode) {
            r.num_tokens += 1;
        } else if (r.num_computed == r.num_tokens) {
            r.is_decode = true;
            r.num_tokens += 1;
        }
    }
    s->last.clear();
    return CPA_OK;
}

cpa_status cpa_sched_free_request(cpa_sched* s, int64_t req_id) {
    if (!s) return CPA_ERR_INVALID_ARG;
    for (size_t i = 0; i < s->reqs.size(); ++i) {
        if (s->reqs[i].id == req_id) {
            s->release(s->reqs[i].blocks);
            s->reqs.erase(s->reqs.begin() + (ptrdiff_t)i);
            s->last.clear();   // indices of an uncommitted step are no longer valid
            return CPA_OK;
        }
    }
    return CPA_ERR_NOT_FOUND;
}

cpa_status cpa_sched_request_info(const cpa_sched* s, int64_t req_id, int32_t* num_tokens,
                                  int32_t* num_computed, int32_t* num_blocks, int32_t* is_decode) {
    if (!s) return CPA_ERR_INVALID_ARG;
    const Request* r = s->find(req_id);
    if (!r) return CPA_ERR_NOT_FOUND;
    if (num_tokens) *num_tokens = r->num_tokens;
    if (num_computed) *num_computed = r->num_computed;
    if (num_blocks) *num_blocks = (int32_t)r->blocks.size();
    if (is_decode) *is_decode = r->is_decode ? 1 : 0;
    return CPA_OK;
}

cpa_status cpa_sched_request_blocks(const cpa_sched* s, int64_t req_id, int32_t* blocks,
                                    int32_t capacity, int32_t* num_blocks) {
    if (!s || !num_blocks) return CPA_ERR_INVALID_ARG;
    const Request* r = s->find(req_id);
    if (!r) return CPA_ERR_NOT_FOUND;
    if ((int64_t)r->blocks.size() > capacity || (!blocks && !r->blocks.empty()))
        return CPA_ERR_INVALID_ARG;
    for (size_t i = 0; i < r->blocks.size(); ++i) blocks[i] = r->blocks[i];
    *num_blocks = (int32_t)r->blocks.size();
    return CPA_OK;
}

cpa_status cpa_sched_slots(const cpa_sched* s, int64_t req_id, int32_t pos0, int32_t n,
                           int64_t* slots) {
    if (!s || pos0 < 0 || n < 0 || (n > 0 && !slots)) return CPA_ERR_INVALID_ARG;
    const Request* r = s->find(req_id);
    if (!r) return CPA_ERR_NOT_FOUND;
    if (cdiv64((int64_t)pos0 + n, s->block_size) > (int64_t)r->blocks.size()) return CPA_ERR_INVALID_ARG;
    for (int32_t t = 0; t < n; ++t) {
        const int64_t p = (int64_t)pos0 + t;
        slots[t] = (int64_t)r->blocks[p / s->block_size] * s->block_size + p % s->block_size;
    }
    return CPA_OK;
}

cpa_status cpa_sched_num_free_blocks(const cpa_sched* s, int32_t* num_free) {
    if (!s || !num_free) return CPA_ERR_INVALID_ARG;
    *num_free = (int32_t)s->free_list.size();
    return CPA_OK;
}

cpa_status cpa_sched_block_refcount(const cpa_sched* s, int32_t block, int32_t* refcount) {
    if (!s || !refcount || block < 0 || block >= (int32_t)s->ref.size()) return CPA_ERR_INVALID_ARG;
    *refcount = s->ref[block];
    return CPA_OK;
}

}  // extern "C"

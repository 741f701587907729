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

//
// Prefix caching (optional): "Prefill Optimisation ...", section 3 ("vLLM
// block hash chain": a full block is identified by its parent's digest, the
// scope and its ordered token ids; full-block-only reuse; "Cache granularity
// and eviction in preallocated pools": active, reclaimable cached and empty
// blocks, the free count including reclaimable ones, eviction as host
// metadata) and "vLLM Chunked Prefill ...", sections 2.2 and 3.1 (the
// lookup happens once, at a request's first scheduling, over its first
// chunk).  Digests here are 64-bit; every hit is verified against the
// block's stored parent digest, scope and tokens, so a digest collision can
// only cost a miss, never a wrong reuse.

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <deque>
#include <list>
#include <new>
#include <unordered_map>
#include <vector>

#include "chunked_prefill_attn.h"

namespace {

inline int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline uint64_t mix64(uint64_t x) {
    x ^= x >> 30;
    x *= 0xbf58476d1ce4e5b9ULL;
    x ^= x >> 27;
    x *= 0x94d049bb133111ebULL;
    x ^= x >> 31;
    return x;
}

// digest of a full block from its parent's digest (0 for the first block),
// the scope digest and its token ids
uint64_t block_digest(uint64_t parent, uint64_t scope, const uint32_t* tok, int32_t n) {
    uint64_t h = mix64(parent + 0x9e3779b97f4a7c15ULL);
    h = mix64(h ^ scope);
    for (int32_t i = 0; i < n; ++i) h = mix64(h ^ ((uint64_t)tok[i] | ((uint64_t)(i + 1) << 32)));
    return h | 1;   // never 0, the "no parent" value
}

// FNV-1a over the scope name
uint64_t scope_digest(const char* name) {
    uint64_t h = 0xcbf29ce484222325ULL;
    for (const char* c = name ? name : "default"; *c; ++c) {
        h ^= (unsigned char)*c;
        h *= 0x100000001b3ULL;
    }
    return h;
}

struct Request {
    int64_t id;
    int32_t num_tokens;    // tokens known (prompt, then + generated)
    int32_t num_computed;  // tokens whose KV is cached
    bool is_decode;
    std::vector<int32_t> blocks;
    // prefix caching
    std::vector<uint32_t> tokens;    // prompt token ids (empty: not given)
    uint64_t scope = 0;
    std::vector<uint64_t> digests;   // chained digests of its first full blocks
    bool looked_up = false;
};

// identity of a registered block, for verifying a digest hit
struct BlockKey {
    uint64_t parent = 0, scope = 0;
    std::vector<uint32_t> tokens;
};

}  // namespace

struct cpa_sched {
    int32_t block_size = 0;
    int32_t budget = 0;
    int32_t max_blocks = 0;
    int32_t cap = 0;
    bool align = false;
    bool caching = false;
    std::deque<int32_t> free_list;      // empty blocks, FIFO: hand out from the front
    std::vector<int32_t> ref;           // reference count per block
    std::vector<Request> reqs;          // arrival order
    std::vector<std::pair<size_t, int32_t>> last;  // (request index, tokens) of the last step
    // prefix caching: digest held by each block (0: none), the digest table,
    // reclaimable cached blocks oldest first
    std::vector<uint64_t> digest;
    std::vector<BlockKey> key;
    std::unordered_map<uint64_t, int32_t> table;
    std::list<int32_t> lru;
    std::vector<std::list<int32_t>::iterator> lru_pos;
    // long prompts per step and preemption
    int32_t max_long = 0;
    bool preemption = false;
    std::vector<int64_t> preempted;     // ids preempted by the last step

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
    int64_t num_free() const { return (int64_t)free_list.size() + (int64_t)lru.size(); }
    // empty blocks first, then the least recently freed cached block
    void take(int32_t n, std::vector<int32_t>& dst) {
        for (int32_t i = 0; i < n; ++i) {
            int32_t b;
            if (!free_list.empty()) {
                b = free_list.front();
                free_list.pop_front();
            } else {
                b = lru.front();
                lru.pop_front();
                table.erase(digest[b]);
                digest[b] = 0;
                key[b] = BlockKey();
            }
            ref[b] = 1;
            dst.push_back(b);
        }
    }
    // blocks left unused go back empty in order; cached ones become
    // reclaimable, the sequence's last block first
    void release(const std::vector<int32_t>& blocks) {
        std::vector<int32_t> unused;
        for (int32_t b : blocks)
            if (--ref[b] == 0) unused.push_back(b);
        for (int32_t b : unused)
            if (!digest[b]) free_list.push_back(b);
        for (auto it = unused.rbegin(); it != unused.rend(); ++it)
            if (digest[*it]) lru_pos[*it] = lru.insert(lru.end(), *it);
    }
    // release every block of r and send it back to position 0: it recomputes
    // all its known tokens (and looks its prefix up again)
    void preempt(Request& r) {
        release(r.blocks);
        r.blocks.clear();
        r.num_computed = 0;
        r.is_decode = false;
        r.looked_up = false;
        r.digests.clear();
    }
    void claim(int32_t b) {
        if (ref[b] == 0) lru.erase(lru_pos[b]);
        ref[b] += 1;
    }
    // blocks of the longest run of the first nblk full blocks of `tok` that
    // are registered (digests in `dig`)
    void lookup(const std::vector<uint32_t>& tok, uint64_t scope, int32_t nblk,
                std::vector<int32_t>& hit, std::vector<uint64_t>& dig) const {
        uint64_t parent = 0;
        for (int32_t j = 0; j < nblk; ++j) {
            const uint32_t* t = tok.data() + (size_t)j * block_size;
            const uint64_t d = block_digest(parent, scope, t, block_size);
            auto f = table.find(d);
            if (f == table.end()) break;
            const BlockKey& k = key[f->second];
            if (k.parent != parent || k.scope != scope ||
                std::memcmp(k.tokens.data(), t, sizeof(uint32_t) * block_size) != 0)
                break;
            hit.push_back(f->second);
            dig.push_back(d);
            parent = d;
        }
    }
    // register the request's newly full prompt blocks (first holder wins)
    void register_blocks(Request& r) {
        const int64_t known = (int64_t)r.tokens.size();
        const int64_t full = (r.num_computed < known ? r.num_computed : known) / block_size;
        for (int64_t j = (int64_t)r.digests.size(); j < full; ++j) {
            const uint64_t parent = r.digests.empty() ? 0 : r.digests.back();
            const uint32_t* t = r.tokens.data() + (size_t)j * block_size;
            const uint64_t d = block_digest(parent, r.scope, t, block_size);
            const int32_t b = r.blocks[(size_t)j];
            if (!table.count(d)) {
                table[d] = b;
                digest[b] = d;
                key[b].parent = parent;
                key[b].scope = r.scope;
                key[b].tokens.assign(t, t + block_size);
            }
            r.digests.push_back(d);
        }
    }
    // tokens a prefill with `remaining` left gets when `used` of the budget is taken
    int64_t take_for(int64_t remaining, int64_t used) const {
        int64_t t = remaining < budget - used ? remaining : budget - used;
        if (cap > 0 && t > cap) t = cap;
        if (align && t < remaining) t = (t / block_size) * block_size;
        return t;
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
    s->caching = cfg->prefix_caching != 0;
    if (cfg->max_long_partial_prefills < 0) {
        delete s;
        return CPA_ERR_INVALID_ARG;
    }
    s->max_long = cfg->max_long_partial_prefills;
    s->preemption = cfg->preemption != 0;
    s->ref.assign(cfg->num_blocks, 0);
    s->digest.assign(cfg->num_blocks, 0);
    s->key.resize(cfg->num_blocks);
    s->lru_pos.resize(cfg->num_blocks);
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

cpa_status cpa_sched_add_request_tokens(cpa_sched* s, int64_t req_id, const uint32_t* tokens,
                                        int32_t num_tokens, const char* name_space) {
    if (!s || num_tokens <= 0 || !tokens) return CPA_ERR_INVALID_ARG;
    if (s->find(req_id)) return CPA_ERR_INVALID_ARG;
    if (cdiv64(num_tokens, s->block_size) > s->max_blocks) return CPA_ERR_INVALID_ARG;
    Request r;
    r.id = req_id;
    r.num_tokens = num_tokens;
    r.num_computed = 0;
    r.is_decode = false;
    r.tokens.assign(tokens, tokens + num_tokens);
    r.scope = scope_digest(name_space);
    s->reqs.push_back(std::move(r));
    return CPA_OK;
}

cpa_status cpa_sched_add_decode(cpa_sched* s, int64_t req_id, int32_t context_len) {
    if (!s || context_len <= 0) return CPA_ERR_INVALID_ARG;
    if (s->find(req_id)) return CPA_ERR_INVALID_ARG;
    const int64_t need = cdiv64(context_len, s->block_size);
    if (cdiv64((int64_t)context_len + 1, s->block_size) > s->max_blocks) return CPA_ERR_INVALID_ARG;
    if (need > s->num_free()) return CPA_ERR_OUT_OF_BLOCKS;
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
    if (need > s->num_free()) return CPA_ERR_OUT_OF_BLOCKS;
    Request r;
    r.id = req_id;
    r.num_tokens = num_prompt_tokens;
    r.num_computed = num_computed_tokens;
    r.is_decode = false;
    s->take((int32_t)need, r.blocks);
    s->reqs.push_back(std::move(r));
    return CPA_OK;
}

}  // extern "C"

namespace {

// One step's picks before anything changes: (request index, tokens), the
// prefix hits of requests seen for the first time, and the new blocks each
// pick needs.
struct StepPlan {
    struct Hit {
        std::vector<int32_t> blocks;
        std::vector<uint64_t> digests;
    };
    std::vector<std::pair<size_t, int32_t>> picked;
    std::vector<int32_t> hit_of;   // per request: index into hits, -1 none
    std::vector<Hit> hits;
    std::vector<int32_t> need_new;
    int64_t used = 0, need_total = 0, claimed = 0;
    bool too_wide = false;         // a table row cannot map a pick
};

// Decodes first, one token each; then prefills in arrival order with what is
// left.  A prefill seen for the first time looks its prefix up over its first
// chunk (leaving at least the prompt's last token to compute).  Prompts longer
// than the per-prefill cap beyond max_long in a step wait; shorter ones behind
// them go on.  Requests marked in `skip` (preempted this step) wait.
void plan_step(const cpa_sched* s, const std::vector<char>& skip, StepPlan& p) {
    p.hit_of.assign(s->reqs.size(), -1);
    for (size_t i = 0; i < s->reqs.size(); ++i) {
        if (s->reqs[i].is_decode && !skip[i] && p.used < s->budget) {
            p.picked.emplace_back(i, 1);
            p.used += 1;
        }
    }
    int32_t longs = 0;
    for (size_t i = 0; i < s->reqs.size(); ++i) {
        const Request& q = s->reqs[i];
        if (q.is_decode || skip[i]) continue;
        if (p.used >= s->budget) break;
        const bool is_long = s->cap > 0 && q.num_tokens > s->cap;
        if (is_long && s->max_long > 0 && longs >= s->max_long) continue;
        int64_t computed = q.num_computed;
        bool look = false;
        StepPlan::Hit h;
        if (s->caching && !q.tokens.empty() && !q.looked_up && q.num_computed == 0) {
            const int64_t first = s->take_for(q.num_tokens, p.used);
            const int64_t lim = first < q.num_tokens - 1 ? first : q.num_tokens - 1;
            s->lookup(q.tokens, q.scope, (int32_t)(lim > 0 ? lim / s->block_size : 0), h.blocks,
                      h.digests);
            computed = (int64_t)h.blocks.size() * s->block_size;
            look = true;
        }
        const int64_t take = s->take_for((int64_t)q.num_tokens - computed, p.used);
        if (take <= 0) continue;
        if (look) {
            p.hit_of[i] = (int32_t)p.hits.size();
            p.hits.push_back(std::move(h));
        }
        p.picked.emplace_back(i, (int32_t)take);
        p.used += take;
        longs += is_long;
    }
    // block growth (prefix hits on reclaimable blocks take them out of the
    // free count)
    std::vector<int32_t> claimed;
    p.need_new.resize(p.picked.size());
    for (size_t k = 0; k < p.picked.size(); ++k) {
        const Request& q = s->reqs[p.picked[k].first];
        const int32_t hi = p.hit_of[p.picked[k].first];
        const int64_t computed = hi < 0 ? q.num_computed : (int64_t)p.hits[hi].blocks.size() * s->block_size;
        const int64_t held = hi < 0 ? (int64_t)q.blocks.size() : (int64_t)p.hits[hi].blocks.size();
        const int64_t need = cdiv64(computed + p.picked[k].second, s->block_size);
        if (need > s->max_blocks) p.too_wide = true;
        p.need_new[k] = (int32_t)(need - held);
        p.need_total += p.need_new[k];
        if (hi >= 0)
            for (int32_t b : p.hits[hi].blocks)
                if (s->ref[b] == 0) claimed.push_back(b);
    }
    std::sort(claimed.begin(), claimed.end());
    claimed.erase(std::unique(claimed.begin(), claimed.end()), claimed.end());
    p.claimed = (int64_t)claimed.size();
}

}  // namespace

extern "C" {

cpa_status cpa_sched_step(cpa_sched* s, cpa_batch* out) {
    if (!s || !out) return CPA_ERR_INVALID_ARG;
    if (!out->req_ids || !out->q_lens || !out->cu_seqlens_q || !out->cached_seq_len ||
        !out->block_table || !out->slot_mapping)
        return CPA_ERR_INVALID_ARG;
    // plan; when the pool cannot hold it, preempt the most recently arrived
    // request holding blocks (first come, first served: "vLLM Chunked
    // Prefill ...", section 4) and plan again
    std::vector<char> skip(s->reqs.size(), 0);
    s->preempted.clear();
    StepPlan plan;
    for (;;) {
        plan = StepPlan();
        plan_step(s, skip, plan);
        if (plan.too_wide) return CPA_ERR_INVALID_ARG;
        if (plan.need_total <= s->num_free() - plan.claimed) break;
        if (!s->preemption) return CPA_ERR_OUT_OF_BLOCKS;
        int64_t victim = -1;
        for (size_t i = s->reqs.size(); i-- > 0;)
            if (!skip[i] && !s->reqs[i].blocks.empty()) {
                victim = (int64_t)i;
                break;
            }
        if (victim < 0) return CPA_ERR_OUT_OF_BLOCKS;
        s->preempt(s->reqs[(size_t)victim]);
        skip[(size_t)victim] = 1;
        s->preempted.push_back(s->reqs[(size_t)victim].id);
    }
    auto& picked = plan.picked;
    const int64_t used = plan.used;
    // capacity of the caller's arrays
    if ((int64_t)picked.size() > out->max_seqs || used > out->max_tokens) return CPA_ERR_INVALID_ARG;
    for (size_t k = 0; k < picked.size(); ++k) {
        const int32_t hi = plan.hit_of[picked[k].first];
        if (hi < 0) continue;
        Request& r = s->reqs[picked[k].first];
        r.looked_up = true;
        for (int32_t b : plan.hits[hi].blocks) s->claim(b);
        r.blocks = plan.hits[hi].blocks;
        r.num_computed = (int32_t)(r.blocks.size() * (size_t)s->block_size);
        r.digests = plan.hits[hi].digests;
    }
    for (size_t k = 0; k < picked.size(); ++k) {
        Request& r = s->reqs[picked[k].first];
        if (plan.need_new[k] > 0) s->take(plan.need_new[k], r.blocks);
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
        if (s->caching && !r.tokens.empty()) s->register_blocks(r);
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
    *num_free = (int32_t)s->num_free();
    return CPA_OK;
}

cpa_status cpa_sched_last_preempted(const cpa_sched* s, int64_t* ids, int32_t capacity,
                                    int32_t* num) {
    if (!s || !num) return CPA_ERR_INVALID_ARG;
    if ((int64_t)s->preempted.size() > capacity || (!ids && !s->preempted.empty()))
        return CPA_ERR_INVALID_ARG;
    for (size_t i = 0; i < s->preempted.size(); ++i) ids[i] = s->preempted[i];
    *num = (int32_t)s->preempted.size();
    return CPA_OK;
}

cpa_status cpa_sched_pool_stats(const cpa_sched* s, int32_t* num_active, int32_t* num_reclaimable,
                                int32_t* num_empty) {
    if (!s) return CPA_ERR_INVALID_ARG;
    int32_t active = 0;
    for (int32_t r : s->ref) active += r > 0;
    if (num_active) *num_active = active;
    if (num_reclaimable) *num_reclaimable = (int32_t)s->lru.size();
    if (num_empty) *num_empty = (int32_t)s->free_list.size();
    return CPA_OK;
}

cpa_status cpa_sched_prefix_match(const cpa_sched* s, const uint32_t* tokens, int32_t num_tokens,
                                  const char* name_space, int32_t* num_cached_tokens) {
    if (!s || num_tokens < 0 || (num_tokens > 0 && !tokens) || !num_cached_tokens)
        return CPA_ERR_INVALID_ARG;
    std::vector<uint32_t> tok(tokens, tokens + num_tokens);
    std::vector<int32_t> hit;
    std::vector<uint64_t> dig;
    s->lookup(tok, scope_digest(name_space), num_tokens / s->block_size, hit, dig);
    *num_cached_tokens = (int32_t)(hit.size() * (size_t)s->block_size);
    return CPA_OK;
}

cpa_status cpa_sched_block_refcount(const cpa_sched* s, int32_t block, int32_t* refcount) {
    if (!s || !refcount || block < 0 || block >= (int32_t)s->ref.size()) return CPA_ERR_INVALID_ARG;
    *refcount = s->ref[block];
    return CPA_OK;
}

}  // extern "C"

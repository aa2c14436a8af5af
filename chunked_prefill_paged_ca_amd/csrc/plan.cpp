// plan.cpp -- ca_plan_batch: decode-first token-budget packing of one mixed step (host only).
//
// Follows pinghaoyang.com.cn "Sarathi-Serve 完全拆解", section "一个 512-token 预算的例子" (decodes
// first, then the left-over budget to prefills, several chunks allowed in one step, total never
// above the budget), blog.vllbc.top "Chunked Prefill 与 PD 分离", section "3.1 Algorithm 3 的顺序"
// (running decodes, then in-progress chunks, then new requests -- the caller lists them in that
// order) and section "7.3" (a per-request chunk cap, max_chunk here), and magicnetworld.com
// "分块预填充与 Stall-free 调度", section "六·补二" (a chunk is the smaller of the budget left and
// the prompt left).  The output is the ragged metadata named in "Sarathi-Serve 完全拆解", section
// "混合批不是把两类注意力强行做成同一个形状".  Optional tile alignment of chunks that do not end
// their prompt: "Sarathi-Serve 完全拆解", section "257 为什么可能比 256 慢 32%" (chunk sizes one past
// a tile multiple waste a row of tiles; candidate sizes are aligned to multiples such as 32).

#include <atomic>
#include <cstdint>
#include <string>
#include <vector>

#include "internal.h"

namespace {

std::atomic<uint64_t> g_generation{0};

struct Pick {
    int32_t req;
    int32_t q;
};

}  // namespace

extern "C" ca_status ca_plan_batch(const ca_request* reqs, int32_t n, const ca_plan_params* prm,
                                   ca_plan* plan) {
    ca::clear_error();
    if (!prm || !plan) { ca::set_error("ca_plan_batch: null params or plan"); return CA_ERR_INVALID_ARG; }
    if (n < 0 || (n > 0 && !reqs)) { ca::set_error("ca_plan_batch: bad request array"); return CA_ERR_INVALID_ARG; }
    const int64_t P = prm->page_size;
    if (prm->token_budget <= 0 || P <= 0 || prm->max_chunk < 0 || prm->num_pool_pages <= 0 ||
        prm->chunk_align < 0) {
        ca::set_error("ca_plan_batch: token_budget, page_size and num_pool_pages must be > 0, "
                      "max_chunk and chunk_align >= 0");
        return CA_ERR_INVALID_ARG;
    }
    for (int32_t i = 0; i < n; ++i) {
        const ca_request& r = reqs[i];
        if (r.num_computed < 0 || r.num_prompt_left < 0 || r.num_pages < 0 ||
            (r.num_pages > 0 && !r.block_table)) {
            ca::set_error("ca_plan_batch: request " + std::to_string(i) + " has a negative field or no block table");
            return CA_ERR_INVALID_ARG;
        }
    }

    std::vector<Pick> picks;
    picks.reserve(static_cast<size_t>(n));
    int64_t budget = prm->token_budget;
    int32_t deferred = 0;
    int32_t decodes = 0;

    // Decodes: one token each, caller order; once the budget is gone the rest wait.
    for (int32_t i = 0; i < n; ++i) {
        const ca_request& r = reqs[i];
        if (r.num_prompt_left != 0) continue;
        if (budget == 0) { ++deferred; continue; }
        if (static_cast<int64_t>(r.num_pages) * P < static_cast<int64_t>(r.num_computed) + 1) {
            ca::set_error("ca_plan_batch: decode request " + std::to_string(i) + " has no free slot for its token");
            return CA_ERR_NO_PAGES;
        }
        picks.push_back({i, 1});
        ++decodes;
        --budget;
    }
    // Prefill chunks from the budget the decodes left, caller order.
    for (int32_t i = 0; i < n && budget > 0; ++i) {
        const ca_request& r = reqs[i];
        if (r.num_prompt_left == 0) continue;
        int64_t take = r.num_prompt_left;
        if (take > budget) take = budget;
        if (prm->max_chunk > 0 && take > prm->max_chunk) take = prm->max_chunk;
        const int64_t room = static_cast<int64_t>(r.num_pages) * P - r.num_computed;
        if (take > room) take = room;
        // a chunk that leaves part of the prompt for later steps is cut to a tile multiple
        if (prm->chunk_align > 1 && take < r.num_prompt_left) take -= take % prm->chunk_align;
        if (take <= 0) continue;
        picks.push_back({i, static_cast<int32_t>(take)});
        budget -= take;
    }

    // Sizes and page-id validation over exactly the pages the step will touch.
    int64_t tokens = 0, pages = 0;
    for (const Pick& pk : picks) {
        const ca_request& r = reqs[pk.req];
        const int64_t kv_len = static_cast<int64_t>(r.num_computed) + pk.q;
        const int64_t np = (kv_len + P - 1) / P;
        for (int64_t j = 0; j < np; ++j) {
            const int32_t id = r.block_table[j];
            if (id < 0 || id >= prm->num_pool_pages) {
                ca::set_error("ca_plan_batch: request " + std::to_string(pk.req) + " uses page id " +
                              std::to_string(id) + " outside the pool");
                return CA_ERR_INVALID_ARG;
            }
        }
        tokens += pk.q;
        pages += np;
    }
    const int32_t ns = static_cast<int32_t>(picks.size());
    plan->num_seqs = ns;
    plan->num_decodes = decodes;
    plan->num_tokens = static_cast<int32_t>(tokens);
    plan->num_pages = static_cast<int32_t>(pages);
    plan->num_deferred_decodes = deferred;
    plan->page_size = static_cast<int32_t>(P);
    if (ns > plan->cap_seqs || pages > plan->cap_pages) {
        ca::set_error("ca_plan_batch: plan arrays too small (need " + std::to_string(ns) + " sequences, " +
                      std::to_string(pages) + " pages)");
        return CA_ERR_CAPACITY;
    }
    if (!plan->req_ids || !plan->qo_indptr || !plan->kv_page_indptr || !plan->kv_last_page_len ||
        (pages > 0 && !plan->kv_page_indices)) {
        ca::set_error("ca_plan_batch: null plan array");
        return CA_ERR_INVALID_ARG;
    }

    int32_t row = 0, pg = 0;
    plan->qo_indptr[0] = 0;
    plan->kv_page_indptr[0] = 0;
    for (int32_t s = 0; s < ns; ++s) {
        const ca_request& r = reqs[picks[s].req];
        const int32_t kv_len = r.num_computed + picks[s].q;
        const int32_t np = static_cast<int32_t>((kv_len + P - 1) / P);
        plan->req_ids[s] = picks[s].req;
        for (int32_t j = 0; j < np; ++j) plan->kv_page_indices[pg + j] = r.block_table[j];
        row += picks[s].q;
        pg += np;
        plan->qo_indptr[s + 1] = row;
        plan->kv_page_indptr[s + 1] = pg;
        plan->kv_last_page_len[s] = kv_len - (np - 1) * static_cast<int32_t>(P);
    }
    plan->generation = ++g_generation;
    return CA_OK;
}

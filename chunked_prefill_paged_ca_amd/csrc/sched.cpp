// sched.cpp -- ca_sched: the multi-step driver around ca_plan_batch (host only).
//
// magicnetworld.com "分块预填充与 Stall-free 调度", section "六·补二、调度器每一轮在做什么": each round
// first lets every running decode take one token -- a decode that needs KV space when none is
// left is preempted and later recomputed from its first token -- then spends the budget left on
// prefill chunks (the smaller of the budget left and the prompt left), and puts an unfinished
// prompt back for the next round.  pinghaoyang.com.cn "Sarathi-Serve 完全拆解", section
// "一个 512-token 预算的例子", step 4: a prefill that finishes its prompt is a decode from the next
// round on.  The packing itself is ca_plan_batch (same parameters); this file keeps the request
// state across rounds and the page pool's free list, and gives each request the pages its
// scheduled tokens need before the plan is made.
//
// Free list: first in, first out.  The pool starts as pages 0, 1, ..., N-1 in that order; a page
// is taken from the front and returned to the back (a finished or preempted request returns its
// pages in block-table order).

#include <cstdint>
#include <deque>
#include <string>
#include <vector>

#include "internal.h"

namespace {

struct Req {
    int32_t prompt_len = 0;
    int32_t max_new = 0;
    int32_t state = CA_REQ_WAITING;
    int32_t nc = 0;         // tokens in the cache
    int32_t left = 0;       // prompt tokens (or, after a preemption, tokens to recompute) left
    int32_t generated = 0;  // decode steps run
    int32_t preemptions = 0;
    std::vector<int32_t> pages;
};

}  // namespace

struct ca_sched {
    ca_plan_params prm{};
    std::vector<Req> reqs;
    std::deque<int32_t> free_list;
    std::vector<uint8_t> is_free;
    // the step waiting for ca_sched_commit: (request id, tokens)
    std::vector<std::pair<int32_t, int32_t>> pending;
    bool has_pending = false;
    std::vector<ca_request> creqs;
    std::vector<int32_t> active;
};

namespace {

void release(ca_sched* s, Req& r) {
    for (int32_t p : r.pages) {
        s->free_list.push_back(p);
        s->is_free[static_cast<size_t>(p)] = 1;
    }
    r.pages.clear();
}

int32_t take_page(ca_sched* s) {
    const int32_t p = s->free_list.front();
    s->free_list.pop_front();
    s->is_free[static_cast<size_t>(p)] = 0;
    return p;
}

int64_t align_chunk(int64_t q, int64_t left, int32_t align) {
    if (align > 1 && q < left) q -= q % align;
    return q;
}

}  // namespace

extern "C" ca_status ca_sched_create(const ca_plan_params* params, ca_sched** out) {
    ca::clear_error();
    if (!params || !out) { ca::set_error("ca_sched_create: null argument"); return CA_ERR_INVALID_ARG; }
    *out = nullptr;
    if (params->token_budget <= 0 || params->page_size <= 0 || params->max_chunk < 0 ||
        params->chunk_align < 0 || params->num_pool_pages <= 0 || params->num_pool_pages > INT32_MAX) {
        ca::set_error("ca_sched_create: token_budget, page_size and num_pool_pages must be > 0 "
                      "(pool below 2^31 pages), max_chunk and chunk_align >= 0");
        return CA_ERR_INVALID_ARG;
    }
    ca_sched* s = new ca_sched();
    s->prm = *params;
    s->is_free.assign(static_cast<size_t>(params->num_pool_pages), 1);
    for (int64_t p = 0; p < params->num_pool_pages; ++p) s->free_list.push_back(static_cast<int32_t>(p));
    *out = s;
    return CA_OK;
}

extern "C" ca_status ca_sched_destroy(ca_sched* s) {
    ca::clear_error();
    delete s;
    return CA_OK;
}

extern "C" ca_status ca_sched_add(ca_sched* s, int32_t prompt_len, int32_t max_new_tokens,
                                  int32_t num_cached, const int32_t* cached_pages, int32_t* id) {
    ca::clear_error();
    if (!s || !id) { ca::set_error("ca_sched_add: null argument"); return CA_ERR_INVALID_ARG; }
    if (s->has_pending) { ca::set_error("ca_sched_add: commit the planned step first"); return CA_ERR_INVALID_ARG; }
    if (prompt_len < 1 || max_new_tokens < 0 || num_cached < 0 || num_cached >= prompt_len) {
        ca::set_error("ca_sched_add: need prompt_len >= 1, max_new_tokens >= 0, 0 <= num_cached < prompt_len");
        return CA_ERR_INVALID_ARG;
    }
    const int64_t P = s->prm.page_size;
    const int64_t npg = (num_cached + P - 1) / P;
    Req r;
    r.prompt_len = prompt_len;
    r.max_new = max_new_tokens;
    r.nc = num_cached;
    r.left = prompt_len - num_cached;
    if (cached_pages) {
        // the caller's pages already hold the prefix: they must be distinct pages of the free list
        std::vector<int32_t> seen;
        for (int64_t j = 0; j < npg; ++j) {
            const int32_t p = cached_pages[j];
            if (p < 0 || p >= s->prm.num_pool_pages || !s->is_free[static_cast<size_t>(p)]) {
                ca::set_error("ca_sched_add: cached page " + std::to_string(p) + " is outside the pool or not free");
                for (int32_t q : seen) s->is_free[static_cast<size_t>(q)] = 1;
                return CA_ERR_INVALID_ARG;
            }
            s->is_free[static_cast<size_t>(p)] = 0;
            seen.push_back(p);
        }
        std::deque<int32_t> rest;
        for (int32_t p : s->free_list)
            if (s->is_free[static_cast<size_t>(p)]) rest.push_back(p);
        s->free_list.swap(rest);
        r.pages.assign(cached_pages, cached_pages + npg);
    } else {
        // the prefix goes into pages taken from the free list; the caller fills them
        if (static_cast<int64_t>(s->free_list.size()) < npg) {
            ca::set_error("ca_sched_add: not enough free pages for the cached prefix");
            return CA_ERR_NO_PAGES;
        }
        for (int64_t j = 0; j < npg; ++j) r.pages.push_back(take_page(s));
    }
    *id = static_cast<int32_t>(s->reqs.size());
    s->reqs.push_back(std::move(r));
    return CA_OK;
}

extern "C" ca_status ca_sched_step(ca_sched* s, ca_plan* plan) {
    ca::clear_error();
    if (!s || !plan) { ca::set_error("ca_sched_step: null argument"); return CA_ERR_INVALID_ARG; }
    if (s->has_pending) { ca::set_error("ca_sched_step: commit the planned step first"); return CA_ERR_INVALID_ARG; }
    const int64_t P = s->prm.page_size;
    const int32_t mc = s->prm.max_chunk, align = s->prm.chunk_align;
    int64_t budget = s->prm.token_budget;
    std::vector<uint8_t> preempted(s->reqs.size(), 0);
    std::vector<int32_t> want(s->reqs.size(), 0);

    // 1. decodes, in admission order: one token each while the budget lasts; a decode whose next
    //    token needs a page when none is free gives all its pages back and waits to be recomputed
    for (size_t i = 0; i < s->reqs.size(); ++i) {
        Req& r = s->reqs[i];
        if (r.state != CA_REQ_RUNNING || budget == 0) continue;
        if (static_cast<int64_t>(r.nc) + 1 > static_cast<int64_t>(r.pages.size()) * P) {
            if (s->free_list.empty()) {
                release(s, r);
                r.left = r.nc;
                r.nc = 0;
                r.state = CA_REQ_WAITING;
                ++r.preemptions;
                preempted[i] = 1;
                continue;
            }
            r.pages.push_back(take_page(s));
        }
        want[i] = 1;
        --budget;
    }
    // 2. prefill chunks, in admission order, from the budget left; a chunk is also cut to the
    //    slots its pages and the free list can hold (then aligned again)
    for (size_t i = 0; i < s->reqs.size() && budget > 0; ++i) {
        Req& r = s->reqs[i];
        if (r.state != CA_REQ_WAITING || preempted[i]) continue;
        int64_t q = r.left < budget ? r.left : budget;
        if (mc > 0 && q > mc) q = mc;
        q = align_chunk(q, r.left, align);
        const int64_t slots = static_cast<int64_t>(r.pages.size() + s->free_list.size()) * P - r.nc;
        if (q > slots) q = align_chunk(slots, r.left, align);
        if (q <= 0) continue;
        const int64_t need = (r.nc + q + P - 1) / P - static_cast<int64_t>(r.pages.size());
        for (int64_t j = 0; j < need; ++j) r.pages.push_back(take_page(s));
        want[i] = static_cast<int32_t>(q);
        budget -= q;
    }

    // 3. the plan over the requests still in play (not finished, not preempted this round)
    s->active.clear();
    s->creqs.clear();
    for (size_t i = 0; i < s->reqs.size(); ++i) {
        const Req& r = s->reqs[i];
        if (r.state == CA_REQ_FINISHED || preempted[i]) continue;
        ca_request c{};
        c.num_computed = r.nc;
        c.num_prompt_left = r.state == CA_REQ_WAITING ? r.left : 0;
        c.num_pages = static_cast<int32_t>(r.pages.size());
        c.block_table = r.pages.empty() ? nullptr : r.pages.data();
        s->creqs.push_back(c);
        s->active.push_back(static_cast<int32_t>(i));
    }
    const ca_status st = ca_plan_batch(s->creqs.data(), static_cast<int32_t>(s->creqs.size()), &s->prm, plan);
    if (st != CA_OK) return st;
    // request ids instead of positions in the active list; the plan must be what step 1-2 chose
    s->pending.clear();
    int32_t total = 0;
    for (int32_t k = 0; k < plan->num_seqs; ++k) {
        const int32_t id = s->active[static_cast<size_t>(plan->req_ids[k])];
        plan->req_ids[k] = id;
        const int32_t q = plan->qo_indptr[k + 1] - plan->qo_indptr[k];
        if (q != want[static_cast<size_t>(id)]) {
            ca::set_error("ca_sched_step: internal mismatch between page allocation and plan for request " +
                          std::to_string(id));
            return CA_ERR_INTERNAL;
        }
        s->pending.emplace_back(id, q);
        ++total;
    }
    for (size_t i = 0; i < want.size(); ++i)
        if (want[i] > 0) --total;
    if (total != 0) {
        ca::set_error("ca_sched_step: internal mismatch between page allocation and plan");
        return CA_ERR_INTERNAL;
    }
    s->has_pending = true;
    return CA_OK;
}

extern "C" ca_status ca_sched_commit(ca_sched* s) {
    ca::clear_error();
    if (!s) { ca::set_error("ca_sched_commit: null argument"); return CA_ERR_INVALID_ARG; }
    if (!s->has_pending) { ca::set_error("ca_sched_commit: no planned step"); return CA_ERR_INVALID_ARG; }
    for (const auto& pk : s->pending) {
        Req& r = s->reqs[static_cast<size_t>(pk.first)];
        r.nc += pk.second;
        if (r.state == CA_REQ_WAITING) {
            r.left -= pk.second;
            if (r.left == 0) r.state = r.generated >= r.max_new ? CA_REQ_FINISHED : CA_REQ_RUNNING;
        } else {
            ++r.generated;
            if (r.generated >= r.max_new) r.state = CA_REQ_FINISHED;
        }
        if (r.state == CA_REQ_FINISHED) release(s, r);
    }
    s->pending.clear();
    s->has_pending = false;
    return CA_OK;
}

extern "C" ca_status ca_sched_get(const ca_sched* s, int32_t id, ca_sched_request* out) {
    ca::clear_error();
    if (!s || !out) { ca::set_error("ca_sched_get: null argument"); return CA_ERR_INVALID_ARG; }
    if (id < 0 || id >= static_cast<int32_t>(s->reqs.size())) {
        ca::set_error("ca_sched_get: no request " + std::to_string(id));
        return CA_ERR_INVALID_ARG;
    }
    const Req& r = s->reqs[static_cast<size_t>(id)];
    out->state = r.state;
    out->num_computed = r.nc;
    out->num_prompt_left = r.state == CA_REQ_WAITING ? r.left : 0;
    out->num_generated = r.generated;
    out->num_pages = static_cast<int32_t>(r.pages.size());
    out->num_preemptions = r.preemptions;
    out->block_table = r.pages.empty() ? nullptr : r.pages.data();
    return CA_OK;
}

extern "C" int64_t ca_sched_free_pages(const ca_sched* s) {
    return s ? static_cast<int64_t>(s->free_list.size()) : -1;
}

/*
 * oracle.c -- plain, slow, fp64 CPU oracle for one mixed chunked-prefill + decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call this file;
 * only the test suite, the smoke check and the benchmark's CPU-baseline leg use it.  It shares
 * no header, helper, table or constant with the HIP library: it has its own header
 * (oracle.h) and its own build (oracle/build.py, plain gcc).
 *
 * Sources (the pages this follows; section names are the pages' own headings):
 *   [SS]  pinghaoyang.com.cn/aigc/posts/sarathi-serve/  "Sarathi-Serve 完全拆解"
 *   [SA]  bowenzhou.top/papers/2023/Sarathi              "Sarathi：让解码搭上 prefill 的顺风车"
 *   [CP]  blog.vllbc.top/visual-reading/chunked-prefill-pd-disaggregation/
 *                                                        "Chunked Prefill 与 PD 分离"
 *   [SF]  magicnetworld.com/.../chunked-prefill-stall-free-scheduling/
 *                                                        "分块预填充与 Stall-free 调度"
 *
 * What is computed, in the pages' order:
 *   1. oracle_plan       -- decode-first token-budget packing of one step
 *                           ([SS] "一个 512-token 预算的例子"; [CP] "3.1 Algorithm 3 的顺序";
 *                            [SF] "六·补二、调度器每一轮在做什么") and the ragged metadata
 *                           (qo_indptr / kv_page_indptr / kv_page_indices / kv_last_page_len,
 *                            [SS] "混合批不是把两类注意力强行做成同一个形状").
 *   2. oracle_rope       -- rotary position embedding at ABSOLUTE positions ([SS] "分块不等于
 *                           截断上下文", last paragraph; [SS] "先验证数值与状态正确性").
 *   3. oracle_attention  -- causal softmax attention of a request's rows over all keys 0..p
 *                           of that request, scaled by 1/sqrt(d_h) ([SS] "分块不等于截断上下文").
 *   4. rounding helpers  -- one rounding of an fp64 value to the storage type (bf16 nearest-even
 *                           or fp32); the pages fix no precision, this is the stated reading.
 *
 * Every floating-point step is fp64, with no fused multiply-add (the build passes
 * -ffp-contract=off) and keys reduced in ascending order.  The attention keeps its own dense,
 * per-request K/V arrays: it never sees a page table, so a paging mistake elsewhere shows up
 * as a mismatch.
 */
#include "oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------------------------ */
/* 1. Plan                                                                                     */
/* ------------------------------------------------------------------------------------------ */

/*
 * Decode-first packing under a token budget tau:
 *   - every running decode contributes exactly one token and is placed first, in caller order
 *     ([SS] "一个 512-token 预算的例子" step 1; [CP] "3.1 Algorithm 3 的顺序");
 *   - the budget left after the decodes goes to prefills, in caller order (the caller lists
 *     in-progress chunks before new requests, which is Algorithm 3's order), each receiving
 *     min(prompt tokens left, budget left) -- optionally also capped by max_chunk, the per-request
 *     cap of [CP] "7.3 vLLM 默认值不是通用答案" -- and several chunks may share one step
 *     ([SS] same section, closing paragraph);
 *   - the total never exceeds tau.  If there are more decodes than tau, the first tau decodes
 *     run and the rest are deferred and counted ([SS] "Decode 数增大时，Prefill 余量会自动缩小"
 *     leaves this open; keeping the cap is the reading taken).
 * A prefill is also capped by the free slots of its block table (num_pages*page_size minus the
 * tokens already cached); a decode without a free slot is an error (CA-style status 2).
 * With chunk_align > 1, a prefill chunk that does not reach the end of its prompt is rounded
 * down to a multiple of chunk_align, and skipped if that leaves nothing ([SS] "257 为什么可能比
 * 256 慢 32%": chunk sizes are snapped to tile multiples such as 32 because one token past a
 * multiple costs a whole extra row of tiles; the final chunk of a prompt is whatever is left).
 *
 * Output metadata for scheduled sequence s (decodes first), with kv_len = num_computed + q:
 *   qo_indptr[s+1]   = qo_indptr[s] + q
 *   npages           = ceil(kv_len / page_size)
 *   kv_page_indptr[s+1] = kv_page_indptr[s] + npages
 *   kv_page_indices  gets block_table[0 .. npages)
 *   kv_last_page_len = kv_len - (npages-1)*page_size        (always in [1, page_size])
 */
int oracle_plan(int32_t n, const int32_t* num_computed, const int32_t* num_prompt_left,
                const int32_t* num_pages, const int64_t* bt_offset, const int32_t* bt,
                int32_t token_budget, int32_t max_chunk, int32_t chunk_align, int32_t page_size,
                int64_t num_pool_pages, int32_t cap_seqs, int32_t cap_pages,
                int32_t* req_ids, int32_t* qo_indptr, int32_t* kv_page_indptr,
                int32_t* kv_page_indices, int32_t* kv_last_page_len, int32_t* counts) {
    if (n < 0 || token_budget <= 0 || page_size <= 0 || max_chunk < 0 || chunk_align < 0 ||
        num_pool_pages <= 0)
        return ORACLE_INVALID_ARG;
    if (n > 0 && (num_computed == NULL || num_prompt_left == NULL || num_pages == NULL ||
                  bt_offset == NULL))
        return ORACLE_INVALID_ARG;
    for (int32_t i = 0; i < n; i++) {
        if (num_computed[i] < 0 || num_prompt_left[i] < 0 || num_pages[i] < 0)
            return ORACLE_INVALID_ARG;
        if (num_pages[i] > 0 && bt == NULL) return ORACLE_INVALID_ARG;
    }

    /* Scheduling decisions, kept in scheduling order. */
    int32_t* sched_req = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
    int32_t* sched_q = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
    int32_t ns = 0, nd = 0, deferred = 0;
    int64_t left = token_budget;

    /* Pass 1: decodes, one token each, in caller order. */
    for (int32_t i = 0; i < n; i++) {
        if (num_prompt_left[i] != 0) continue;
        if (left == 0) { deferred++; continue; }
        int64_t slots = (int64_t)num_pages[i] * page_size;
        if (slots < (int64_t)num_computed[i] + 1) {
            free(sched_req); free(sched_q);
            return ORACLE_NO_PAGES;
        }
        sched_req[ns] = i; sched_q[ns] = 1; ns++; nd++;
        left -= 1;
    }
    /* Pass 2: prefill chunks, in caller order, from what the decodes left. */
    for (int32_t i = 0; i < n && left > 0; i++) {
        if (num_prompt_left[i] == 0) continue;
        int64_t q = num_prompt_left[i];
        if (left < q) q = left;
        if (max_chunk > 0 && max_chunk < q) q = max_chunk;
        int64_t room = (int64_t)num_pages[i] * page_size - num_computed[i];
        if (room < q) q = room;
        /* Tile alignment: a chunk after which prompt tokens remain is rounded down to a
         * multiple of chunk_align; the last chunk of a prompt keeps its length. */
        if (chunk_align > 1 && q < num_prompt_left[i]) q = (q / chunk_align) * chunk_align;
        if (q <= 0) continue;
        sched_req[ns] = i; sched_q[ns] = (int32_t)q; ns++;
        left -= q;
    }

    /* Sizes, then the page ids that will be read or written must lie inside the pool. */
    int64_t total_tokens = 0, total_pages = 0;
    for (int32_t s = 0; s < ns; s++) {
        int32_t r = sched_req[s];
        int64_t kv_len = (int64_t)num_computed[r] + sched_q[s];
        int64_t np = (kv_len + page_size - 1) / page_size;
        for (int64_t j = 0; j < np; j++) {
            int32_t pid = bt[bt_offset[r] + j];
            if (pid < 0 || (int64_t)pid >= num_pool_pages) {
                free(sched_req); free(sched_q);
                return ORACLE_INVALID_ARG;
            }
        }
        total_tokens += sched_q[s];
        total_pages += np;
    }
    if (counts) {
        counts[0] = ns; counts[1] = nd; counts[2] = (int32_t)total_tokens;
        counts[3] = (int32_t)total_pages; counts[4] = deferred;
    }
    if (ns > cap_seqs || total_pages > cap_pages) {
        free(sched_req); free(sched_q);
        return ORACLE_CAPACITY;
    }

    qo_indptr[0] = 0;
    kv_page_indptr[0] = 0;
    for (int32_t s = 0; s < ns; s++) {
        int32_t r = sched_req[s];
        int64_t kv_len = (int64_t)num_computed[r] + sched_q[s];
        int64_t np = (kv_len + page_size - 1) / page_size;
        req_ids[s] = r;
        qo_indptr[s + 1] = qo_indptr[s] + sched_q[s];
        kv_page_indptr[s + 1] = kv_page_indptr[s] + (int32_t)np;
        for (int64_t j = 0; j < np; j++)
            kv_page_indices[kv_page_indptr[s] + j] = bt[bt_offset[r] + j];
        kv_last_page_len[s] = (int32_t)(kv_len - (np - 1) * page_size);
    }
    free(sched_req); free(sched_q);
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------------------------ */
/* 2. Rotary position embedding at absolute positions                                          */
/* ------------------------------------------------------------------------------------------ */

/*
 * For a token at absolute position p (never restarted per chunk -- [SS] "分块不等于截断上下文"
 * and the RoPE item of "先验证数值与状态正确性") each head vector x of size d is rotated pairwise:
 * pair i (0 <= i < d/2) is (x[i], x[i + d/2]) and turns by the angle p * theta^(-2i/d):
 *     x'[i]       = x[i] cos(a) - x[i+d/2] sin(a)
 *     x'[i+d/2]   = x[i+d/2] cos(a) + x[i] sin(a)
 * The pages do not name the pairing or the base; split-half pairing and base theta (10000 by
 * default) is the reading taken.  V is never rotated.
 */
void oracle_rope(int32_t ntok, int32_t nheads, int32_t head_dim, const int32_t* pos,
                 double theta, const double* x, double* out) {
    int32_t half = head_dim / 2;
    for (int32_t t = 0; t < ntok; t++) {
        for (int32_t h = 0; h < nheads; h++) {
            const double* xi = x + ((int64_t)t * nheads + h) * head_dim;
            double* yo = out + ((int64_t)t * nheads + h) * head_dim;
            for (int32_t i = 0; i < half; i++) {
                double inv_freq = pow(theta, -2.0 * (double)i / (double)head_dim);
                double angle = (double)pos[t] * inv_freq;
                double c = cos(angle), s = sin(angle);
                double a = xi[i], b = xi[i + half];
                yo[i] = a * c - b * s;
                yo[i + half] = b * c + a * s;
            }
        }
    }
}

/* ------------------------------------------------------------------------------------------ */
/* 3. Causal attention of one request's rows                                                   */
/* ------------------------------------------------------------------------------------------ */

/*
 * Row t sits at absolute position pos[t] and sees keys 0..pos[t] of its own request -- the
 * whole history plus the current chunk up to itself, never a later position
 * ([SS] "分块不等于截断上下文"; [SA] "Chunked-prefills：把 prefill 切成饱和的等分").  A decode row is
 * the case pos = kv_len - 1.  Query head h reads kv head h / (Hq/Hkv) (contiguous GQA groups:
 * the pages only name GQA, this grouping is the reading taken).
 *     s_j = (q . k_j) * scale,  m = max_j s_j,  w_j = exp(s_j - m),
 *     out = sum_j w_j v_j / sum_j w_j,  lse = m + log(sum_j w_j).
 */
typedef struct {
    int32_t nrows, hq, hkv, d, kv_len;
    const double *q, *k, *v;
    const int32_t* pos;
    double scale;
    double *out, *lse;
    int64_t item_begin, item_end;  /* items are (row, q head) pairs */
} attn_job;

static void attend_one(const attn_job* J, int32_t t, int32_t h, double* scores) {
    int32_t group = J->hq / J->hkv;
    int32_t g = h / group;
    int32_t p = J->pos[t];
    const double* qv = J->q + ((int64_t)t * J->hq + h) * J->d;
    double m = -INFINITY;
    for (int32_t j = 0; j <= p; j++) {
        const double* kv = J->k + ((int64_t)j * J->hkv + g) * J->d;
        double dot = 0.0;
        for (int32_t e = 0; e < J->d; e++) dot += qv[e] * kv[e];
        scores[j] = dot * J->scale;
        if (scores[j] > m) m = scores[j];
    }
    double l = 0.0;
    for (int32_t j = 0; j <= p; j++) {
        scores[j] = exp(scores[j] - m);
        l += scores[j];
    }
    double* o = J->out + ((int64_t)t * J->hq + h) * J->d;
    for (int32_t e = 0; e < J->d; e++) o[e] = 0.0;
    for (int32_t j = 0; j <= p; j++) {
        const double* vv = J->v + ((int64_t)j * J->hkv + g) * J->d;
        for (int32_t e = 0; e < J->d; e++) o[e] += scores[j] * vv[e];
    }
    for (int32_t e = 0; e < J->d; e++) o[e] /= l;
    if (J->lse) J->lse[(int64_t)t * J->hq + h] = m + log(l);
}

static void* attn_worker(void* arg) {
    attn_job* J = (attn_job*)arg;
    double* scores = (double*)malloc(sizeof(double) * (size_t)(J->kv_len > 0 ? J->kv_len : 1));
    for (int64_t it = J->item_begin; it < J->item_end; it++)
        attend_one(J, (int32_t)(it / J->hq), (int32_t)(it % J->hq), scores);
    free(scores);
    return NULL;
}

int oracle_attention(int32_t nrows, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                     int32_t kv_len, const double* q, const int32_t* pos, const double* k,
                     const double* v, double scale, double* out, double* lse, int32_t nthreads) {
    if (nrows < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || kv_len < 0 ||
        num_q_heads % num_kv_heads != 0)
        return ORACLE_INVALID_ARG;
    for (int32_t t = 0; t < nrows; t++)
        if (pos[t] < 0 || pos[t] >= kv_len) return ORACLE_INVALID_ARG;
    int64_t items = (int64_t)nrows * num_q_heads;
    if (nthreads < 1) nthreads = 1;
    if (items < nthreads) nthreads = (int32_t)(items > 0 ? items : 1);

    attn_job* jobs = (attn_job*)calloc((size_t)nthreads, sizeof(attn_job));
    pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
    for (int32_t w = 0; w < nthreads; w++) {
        attn_job* J = &jobs[w];
        J->nrows = nrows; J->hq = num_q_heads; J->hkv = num_kv_heads; J->d = head_dim;
        J->kv_len = kv_len; J->q = q; J->k = k; J->v = v; J->pos = pos; J->scale = scale;
        J->out = out; J->lse = lse;
        J->item_begin = items * w / nthreads;
        J->item_end = items * (w + 1) / nthreads;
    }
    for (int32_t w = 1; w < nthreads; w++) pthread_create(&th[w], NULL, attn_worker, &jobs[w]);
    attn_worker(&jobs[0]);
    for (int32_t w = 1; w < nthreads; w++) pthread_join(th[w], NULL);
    free(jobs); free(th);
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------------------------ */
/* 4. One rounding to the storage type                                                         */
/* ------------------------------------------------------------------------------------------ */

/*
 * bfloat16 has 8 significant bits and fp32's exponent range.  With x = f * 2^e, 0.5 <= |f| < 1
 * (frexp), the spacing of bf16 values around x is 2^(e-8) for normal numbers and 2^-133 below
 * the normal range, so x rounds to rint(x / q) * q with q the larger of the two (rint rounds
 * half to even in the default rounding mode).  Scaling by a power of two is exact.  Results
 * beyond the largest finite bf16 become infinities.
 */
double oracle_bf16_value(double x) {
    if (isnan(x) || isinf(x) || x == 0.0) return x;
    int e;
    (void)frexp(x, &e);
    int qexp = e - 8;
    if (qexp < -133) qexp = -133;
    double r = ldexp(rint(ldexp(x, -qexp)), qexp);
    const double bf16_max = 3.3895313892515355e38; /* (2 - 2^-7) * 2^127 */
    if (fabs(r) > bf16_max) return x > 0 ? INFINITY : -INFINITY;
    return r;
}

void oracle_round(int64_t n, int32_t to_bf16, const double* x, double* out) {
    for (int64_t i = 0; i < n; i++)
        out[i] = to_bf16 ? oracle_bf16_value(x[i]) : (double)(float)x[i];
}

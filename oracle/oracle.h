/*
 * oracle.h -- the CPU oracle's own interface (test infrastructure only; see oracle.c).
 * Deliberately independent of the library's include/ca.h: the two share no declarations.
 */
#ifndef CA_ORACLE_H
#define CA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_OK = 0, ORACLE_INVALID_ARG = 1, ORACLE_NO_PAGES = 2, ORACLE_CAPACITY = 3 };

/* Decode-first token-budget plan.  Block tables are flattened: request i's table is
 * bt[bt_offset[i] .. bt_offset[i] + num_pages[i]).  counts = {num_seqs, num_decodes,
 * num_tokens, num_pages, num_deferred_decodes}, written on OK and on CAPACITY. */
int oracle_plan(int32_t n, const int32_t* num_computed, const int32_t* num_prompt_left,
                const int32_t* num_pages, const int64_t* bt_offset, const int32_t* bt,
                int32_t token_budget, int32_t max_chunk, int32_t chunk_align, int32_t page_size,
                int64_t num_pool_pages, int32_t cap_seqs, int32_t cap_pages,
                int32_t* req_ids, int32_t* qo_indptr, int32_t* kv_page_indptr,
                int32_t* kv_page_indices, int32_t* kv_last_page_len, int32_t* counts);

/* x, out: [ntok, nheads, head_dim] fp64; pos: [ntok] absolute positions. */
void oracle_rope(int32_t ntok, int32_t nheads, int32_t head_dim, const int32_t* pos,
                 double theta, const double* x, double* out);

/* q: [nrows, Hq, d], k, v: [kv_len, Hkv, d] (one request, dense), out: [nrows, Hq, d],
 * lse: [nrows, Hq] or NULL.  Row t attends keys 0..pos[t]. */
int oracle_attention(int32_t nrows, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                     int32_t kv_len, const double* q, const int32_t* pos, const double* k,
                     const double* v, double scale, double* out, double* lse, int32_t nthreads);

double oracle_bf16_value(double x);
/* out[i] = x[i] rounded once to bf16 (to_bf16 != 0) or to fp32, as an fp64 value. */
void oracle_round(int64_t n, int32_t to_bf16, const double* x, double* out);

#ifdef __cplusplus
}
#endif
#endif

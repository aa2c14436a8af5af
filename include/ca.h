/*
 * ca.h -- C ABI of the MI355X (gfx950) mixed chunked-prefill + decode paged-attention library.
 *
 * One call of ca_plan_batch + ca_append_kv_rope + ca_mixed_attention is one step of the
 * Sarathi-Serve style mixed batch: running decodes contribute one query each, prefill prompts
 * contribute a chunk of queries at absolute positions [s_{k-1}, s_k), and every query attends
 * causally to all keys of its own request up to and including itself, read from a paged KV
 * cache (history pages plus the pages the current chunk was just appended to).
 *
 * Sources (page title, then the section the call follows):
 *   [SS] pinghaoyang.com.cn/aigc/posts/sarathi-serve/  "Sarathi-Serve 完全拆解"
 *   [CP] blog.vllbc.top/visual-reading/chunked-prefill-pd-disaggregation/  "Chunked Prefill 与 PD 分离"
 *   [SF] magicnetworld.com/tech/articles/2026-10-02-chunked-prefill-stall-free-scheduling/
 *        "分块预填充与 Stall-free 调度"
 *   [SA] bowenzhou.top/papers/2023/Sarathi  "Sarathi：让解码搭上 prefill 的顺风车"
 *
 * Conventions shared by every entry point:
 *   - The caller owns every buffer.  Host arrays are plain pointers; device buffers are device
 *     pointers (e.g. from hipMalloc or a framework allocator).  No pointer is retained after a
 *     call returns.  A ca_ctx owns only its internal workspace (pinned staging memory, device
 *     metadata and split-KV partials), grown on demand and freed by ca_destroy.
 *   - Device work is enqueued asynchronously on the given hipStream_t (passed as void*; NULL is
 *     the null stream).  The host waits only when the ctx's ring of 8 pinned staging slots comes
 *     back to a slot an earlier launch may still be reading: until the attention launch that
 *     followed that reader on its stream has started (it stores a completion word into pinned
 *     memory as it starts), or, when no attention launch followed it on that stream, for the
 *     whole device (hipDeviceSynchronize).  One ctx must not be used from two streams
 *     concurrently unless the caller orders those streams.
 *   - Errors: every call returns a ca_status; ca_last_error() gives a detail message for the
 *     calling thread.  Arguments are validated before anything is enqueued; on an error
 *     nothing is launched.
 *   - Device buffers of q, k, v, the caches and o must be 16-byte aligned (the kernels move
 *     16-byte vectors); lse 4-byte aligned.  A misaligned pointer is CA_ERR_INVALID_ARG.
 *
 * Paged KV cache layout (element type per ca_dtype, page size P, head dim d, Hkv kv heads):
 *   k_cache: [num_pool_pages][Hkv][d/8][P][8]
 *       slot s, dim e of a page at ((e/8)*P + s)*8 + e%8: for each block of 8 dims, the P slots'
 *       8-element runs one after another
 *   v_cache: [num_pool_pages][Hkv][d/16][P/4][16][4]
 *       slot s, dim e of a page at (((e/16)*(P/4) + s/4)*16 + e%16)*4 + s%4: for each block of
 *       16 dims and each group of 4 slots, the 16 dims' 4-slot runs one after another
 * Each (page, kv head) block is one contiguous P*d run in both caches.  Token at absolute
 * position p of a request lives in logical page p / P, slot p % P.  (Both layouts put the
 * elements one matrix-core operand fragment needs from a page in a single run per wavefront
 * load: 16 bytes per lane for K, 8 for V.)
 */
#ifndef CA_H
#define CA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CA_OK = 0,
    CA_ERR_INVALID_ARG = 1, /* null pointer, bad size, page id outside the pool, ... */
    CA_ERR_NO_PAGES = 2,    /* a decode's block table has no free slot for its new token */
    CA_ERR_CAPACITY = 3,    /* caller arrays too small; required sizes are in the counts */
    CA_ERR_UNSUPPORTED = 4, /* a valid but unimplemented shape (e.g. head_dim not 64/128) */
    CA_ERR_DEVICE = 5,      /* a HIP runtime error */
    CA_ERR_INTERNAL = 6     /* a consistency check inside the library failed (a library bug) */
} ca_status;

typedef enum { CA_BF16 = 0, CA_FP32 = 1 } ca_dtype;

/* One request as the scheduler sees it at the start of a step ([SS] "分块不等于截断上下文", last
 * paragraph: processed length, chunk length, absolute positions, block table, last-page length). */
typedef struct {
    int32_t num_computed;       /* tokens already in the KV cache (prefix hits included) */
    int32_t num_prompt_left;    /* prompt tokens not yet computed; 0 marks a decode */
    int32_t num_pages;          /* entries in block_table */
    int32_t reserved;
    const int32_t* block_table; /* host memory: physical page id of logical page i */
} ca_request;

typedef struct {
    int32_t token_budget;   /* tau: total query tokens of the step, decodes included (> 0) */
    int32_t max_chunk;      /* per-request cap on a prefill chunk; 0 = no cap */
    int32_t page_size;      /* P (> 0) */
    int32_t chunk_align;    /* tile multiple A for chunks that do not end their prompt; 0 or 1 =
                               none ([SS] "257 为什么可能比 256 慢 32%": a chunk one token past a
                               tile multiple costs a whole extra row of tiles, and candidate chunk
                               sizes are aligned to tile multiples such as 32) */
    int64_t num_pool_pages; /* page ids must lie in [0, num_pool_pages) */
} ca_plan_params;

/* Plan output.  The caller allocates the arrays (host memory) and sets the capacities; the
 * library fills the arrays and the counts.  Scheduled sequence s (s < num_seqs) is request
 * req_ids[s]; sequences [0, num_decodes) are decodes ([SS] "混合批不是把两类注意力强行做成同一个形状"
 * names the four metadata arrays). */
typedef struct {
    int32_t cap_seqs;          /* capacity of req_ids, kv_last_page_len; indptrs hold cap_seqs+1 */
    int32_t cap_pages;         /* capacity of kv_page_indices */
    int32_t* req_ids;          /* [num_seqs] index into the request array */
    int32_t* qo_indptr;        /* [num_seqs+1] rows of sequence s in the flat token arrays */
    int32_t* kv_page_indptr;   /* [num_seqs+1] */
    int32_t* kv_page_indices;  /* [num_pages] physical pages of each sequence after the append */
    int32_t* kv_last_page_len; /* [num_seqs] valid slots of the last page, in [1, P] */
    int32_t num_seqs;          /* out */
    int32_t num_decodes;       /* out */
    int32_t num_tokens;        /* out: T = qo_indptr[num_seqs] */
    int32_t num_pages;         /* out: kv_page_indptr[num_seqs] */
    int32_t num_deferred_decodes; /* out: decodes left out because the budget ran out */
    int32_t page_size;         /* out: P the plan was made for */
    uint64_t generation;       /* out: unique per successful plan; keys the device-side copy */
} ca_plan;

typedef struct {
    int32_t num_q_heads;  /* Hq */
    int32_t num_kv_heads; /* Hkv; Hq % Hkv == 0, q head h reads kv head h / (Hq / Hkv) */
    int32_t head_dim;     /* d: 64 or 128 */
    int32_t page_size;    /* P: must equal the plan's */
    ca_dtype dtype;       /* storage type of q, k, v, caches and o; accumulation is fp32 */
    float sm_scale;       /* 0 => 1 / sqrt(d) */
    float rope_theta;     /* 0 => 10000 */
} ca_attn_desc;

typedef struct ca_ctx ca_ctx;

/*
 * Create a context bound to HIP device `device`.  *out receives the handle.
 * The launch shape is chosen per call from the plan and the device's CU count.  For measurement,
 * ca_create reads these overrides from the environment (unset = the default choice):
 *   CA_DECODE_WGS=n         decode workgroups of an attention launch (fused, or decode rows alone);
 *   CA_DECODE_WAVES=n       waves per decode workgroup, 1..8 (default 4);
 *   CA_CHUNK_SPLIT=n        keys per prefill-chunk split (rounded up to 32 and to at least
 *                           1/64 of the longest chunk row's keys);
 *   CA_SPLIT_ATTENTION=1    decode and prefill-chunk rows as two launches instead of one;
 *   CA_PROJECTION_LIBRARY=1 ca_qkv_projection always through hipBLASLt;
 *   CA_PROJECTION_TILE=bm,bn,s  tile shape of ca_qkv_projection's tiled kernel (bm x bn one of
 *                           32/64/96/128 x 64/96/128, 128 x 192, 128 x 256, 256 x 96,
 *                           256 x 128; K split over s workgroups, 1 <= s <= min(64, K / 64));
 *                           a shape that is not built or does not fit the product is
 *                           CA_ERR_INVALID_ARG;
 *   CA_DEBUG_VALIDATE=1     ca_append_kv_rope(_packed) also checks that no two scheduled tokens
 *                           append to the same (page, slot) (ca_plan_validate with
 *                           CA_VALIDATE_WRITE_TARGETS; a host-side sort of the step's targets).
 * The context's pinned staging ring (8 slots of 2 MiB) is allocated here; device workspace is
 * allocated by the first call that needs it and grows only for a larger step.
 * Errors: CA_ERR_INVALID_ARG (null out, no such device), CA_ERR_DEVICE (a HIP error).
 */
ca_status ca_create(int device, ca_ctx** out);
/* Free the context's workspace.  The caller must have synchronised the streams it used with
 * this context; the library itself only waits for the device when a staging slot may still be
 * read by a launch (before its pinned memory is freed). */
ca_status ca_destroy(ca_ctx* ctx);

/*
 * ca_plan_batch -- decode-first token-budget packing of one step (host only, no device work).
 * Follows [SS] "一个 512-token 预算的例子", [CP] "3.1 Algorithm 3 的顺序" and [SF] "六·补二":
 *   1. decodes (num_prompt_left == 0), in caller order, one token each, while budget remains;
 *      the rest are deferred and counted in num_deferred_decodes;
 *   2. prefills, in caller order (list in-progress chunks before new requests), each getting
 *      min(num_prompt_left, budget left, max_chunk if > 0, free slots of its block table);
 *      the scan stops when the budget is used up.  Several chunks may share a step.
 *   3. with chunk_align = A > 1, a chunk that does not finish its prompt is cut down to a
 *      multiple of A; one cut to 0 is not scheduled (the budget stays for the requests after
 *      it), and the chunk that finishes a prompt is never cut.
 * For each scheduled sequence: kv_len = num_computed + q, pages = ceil(kv_len / P) taken from
 * the front of its block table, kv_last_page_len = kv_len - (pages - 1) * P.
 * Errors: CA_ERR_INVALID_ARG (n < 0, budget/page size <= 0, negative fields or chunk_align,
 * missing table,
 * a scheduled page id outside the pool), CA_ERR_NO_PAGES (a decode whose table has fewer than
 * num_computed + 1 slots), CA_ERR_CAPACITY (num_seqs > cap_seqs or num_pages > cap_pages; the
 * counts then hold the required sizes).
 */
ca_status ca_plan_batch(const ca_request* reqs, int32_t n, const ca_plan_params* params,
                        ca_plan* plan);

/*
 * ca_plan_validate -- host-only consistency check of a plan against a pool of num_pool_pages
 * pages (no device work; the device calls run the same check on every new plan generation).
 * Checks: indptr arrays start at 0 and agree with num_tokens / num_pages; every sequence has
 * >= 1 row, >= 1 page, kv_last_page_len in [1, P] and no more rows than keys; decodes have one
 * row; every page id lies in [0, num_pool_pages).  With CA_VALIDATE_WRITE_TARGETS it also checks
 * that the (page, slot) each scheduled token is appended to -- position p of a sequence goes to
 * slot p % P of its logical page p / P -- is unique over the step: the block tables must stay
 * consistent across appends ([SS] "先验证数值与状态正确性"), and two sequences whose tables share
 * a page they both write would race inside the append.
 * Errors: CA_ERR_INVALID_ARG (null plan or arrays, an inconsistency above; ca_last_error names
 * the sequences and the slot of a collision, unknown flags).
 */
enum { CA_VALIDATE_WRITE_TARGETS = 1 };
ca_status ca_plan_validate(const ca_plan* plan, int64_t num_pool_pages, int32_t flags);

/*
 * ca_append_kv_rope -- rotary embedding at absolute positions, then append the step's K/V.
 * ([SS] "分块不等于截断上下文": positions continue across chunks, and a chunk's K/V is in the paged
 * cache before its queries read the history pages together with the chunk's own pages.)
 * Row t of sequence s sits at absolute position p = kv_len_s - q_s + (t - qo_indptr[s]).
 *   q_in, q_out : [T, Hq, d]  (q_out may equal q_in)   q_out = RoPE_p(q_in)
 *   k_new, v_new: [T, Hkv, d]                           k_cache <- RoPE_p(k_new), v_cache <- v_new
 * RoPE pairs element i with i + d/2 and turns the pair by p * theta^(-2i/d); angles are formed
 * in fp64 and each result is rounded once to the storage type.  V is not rotated.
 * The slots written are those of positions [kv_len - q, kv_len) of every scheduled sequence.
 */
ca_status ca_append_kv_rope(ca_ctx* ctx, const ca_attn_desc* desc, const ca_plan* plan,
                            const void* q_in, void* q_out, const void* k_new, const void* v_new,
                            void* k_cache, void* v_cache, int64_t num_pool_pages,
                            void* hip_stream);

/*
 * ca_mixed_attention -- causal attention of every row of the step over the paged cache.
 * For row t at position p of sequence s and q head h (kv head g = h / (Hq/Hkv)):
 *   s_j      = scale * (q[t,h,:] . k_j[g,:])  for keys j = 0..p of sequence s
 *   o[t,h,:] = sum_{j<=p} softmax_j(s) v_j[g,:]     (scale = desc->sm_scale)
 *   lse[t,h] = log sum_{j<=p} exp(s_j)  (natural log; pass NULL to skip)
 * ([SS] "分块不等于截断上下文"; decodes are the case p = kv_len - 1.)
 *   q: [T, Hq, d] (already rotated), o: [T, Hq, d], lse: [T, Hq] fp32 or NULL.
 * bf16 with Hq/Hkv <= 16: one launch runs decode rows (split-KV, partials merged by log-sum-exp
 * weights) beside chunk rows (LDS-staged bf16 MFMA); fp32 storage uses a plain fp32 kernel.
 * When the chunk work outnumbers the workgroup slots, persistent workers take it from work
 * queues whose counters live in ctx (two sets, used by turns: each attention launch zeroes the
 * set the next one claims from): the calls on one ctx must run in the order they are enqueued,
 * which one stream (or events between streams) guarantees.
 */
ca_status ca_mixed_attention(ca_ctx* ctx, const ca_attn_desc* desc, const ca_plan* plan,
                             const void* q, const void* k_cache, const void* v_cache,
                             int64_t num_pool_pages, void* o, float* lse, void* hip_stream);

/*
 * ca_mixed_attention_noalloc -- ca_mixed_attention for callers that cannot allocate memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same arguments,
 * same results (within the bf16 / fp32 tolerance of ca_mixed_attention; the chunk rows may be cut
 * into fewer key splits), and it calls no hipMalloc, hipFree, hipHostMalloc or other allocating
 * routine:
 *   - its workspace (the step's metadata and the split-KV partials) is a static device array of
 *     64 MiB in this library, one per device, held from ca_create on that device until the
 *     process ends; when the chunk partials would not fit, the chunk rows' key splits are made
 *     longer until they do;
 *   - the metadata reaches the device through the pinned staging slots ca_create allocated.
 * The caller still owns q, the caches, o and lse.  Every no-alloc call on a device shares that
 * device's array and leaves the last call's contents in it: calls that overlap on one device
 * (two streams, two contexts, two threads) race; calls on one stream are ordered.  No part of
 * the array needs to start at zero.  It never reuses or updates the device metadata that
 * ca_append_kv_rope / ca_mixed_attention keep for a plan (it uploads its own copy every call).
 * Errors: those of ca_mixed_attention, and CA_ERR_CAPACITY when the step's metadata exceeds a
 * staging slot (2 MiB) or its metadata and decode partials exceed the 64 MiB array (ca_last_error
 * gives the size needed).
 */
ca_status ca_mixed_attention_noalloc(ca_ctx* ctx, const ca_attn_desc* desc, const ca_plan* plan,
                                     const void* q, const void* k_cache, const void* v_cache,
                                     int64_t num_pool_pages, void* o, float* lse, void* hip_stream);

/*
 * Kernel timing (the tracing layer).  When enabled, every launch the library makes carries a
 * start/stop HIP event pair attached to the dispatch itself (hipExtLaunchKernel), so the
 * figures are device time of that launch alone and timing adds no packet to the stream.
 * ca_profile_read waits for the recorded events, copies up to `cap` records (oldest first),
 * sets *count to the number copied and forgets every record read or not.
 * Names are static strings: "upload" (the step's metadata, host staging -> device, when an
 * attention call is the first to see a plan; after ca_append_kv_rope the append launch has
 * copied it, inside "append_rope"), "append_rope",
 * "attention" (decode and prefill-chunk rows in one launch; with CA_SPLIT_ATTENTION=1 in the
 * environment at ca_create they are two launches named "chunk" and "decode"), "merge" (both
 * kinds of split merge in one launch) and "generic" (the plain fp32 kernel with its merge).
 * At most 65536 launches are kept between reads; later ones are not recorded.
 */
typedef struct {
    const char* kernel;
    float ms;
} ca_profile_record;

/* ca_profile_enable's `enable`: 0 = off, CA_PROFILE_ALL = every launch, or an OR of the
 * single-kind flags to time only those launches (each timed launch costs a few microseconds of
 * device time, so a throughput run times only what it reports).  ATTENTION covers "attention",
 * "chunk", "decode" and "generic". */
enum {
    CA_PROFILE_ALL = 1,
    CA_PROFILE_UPLOAD = 2,
    CA_PROFILE_APPEND = 4,
    CA_PROFILE_ATTENTION = 8,
    CA_PROFILE_MERGE = 16,
    CA_PROFILE_PROJECTION = 32 /* "qkv_projection" */
};

ca_status ca_profile_enable(ca_ctx* ctx, int enable);
ca_status ca_profile_read(ca_ctx* ctx, ca_profile_record* out, int32_t cap, int32_t* count);

/*
 * ca_qkv_projection -- the step's q, k and v from its hidden states, as one matrix product over
 * the whole mixed token array ([SA] "Decode-maximal batching：顺车的账本": the linear layers of the
 * decode tokens and of the prefill chunk run as one GEMM, so each weight is read once for all of
 * them; attention stays separate).
 *   qkv[T][Hq + 2 Hkv][d] = x[T][hidden] . w^T, where w is [(Hq + 2 Hkv) d][hidden] (one row per
 *   output feature, rows ordered q heads, then k heads, then v heads) and T = num_tokens (the
 *   plan's row order: decode rows, then chunk rows).  bf16 operands and result, fp32
 *   accumulation.  Up to 16 tokens (hidden a multiple of 2048) a kernel of this library streams
 *   the weights once through the matrix cores; otherwise, or with CA_PROJECTION_LIBRARY=1 in the
 *   environment at ca_create, a library GEMM (hipBLASLt), planned once per token count and cached
 *   in ctx.
 * Device buffers x, w, qkv (16-byte aligned).  Errors: CA_ERR_INVALID_ARG (null pointer, sizes,
 * hidden not a multiple of 8), CA_ERR_UNSUPPORTED (dtype not bf16), CA_ERR_DEVICE (a hipBLASLt or
 * HIP error).
 */
ca_status ca_qkv_projection(ca_ctx* ctx, const ca_attn_desc* desc, int32_t num_tokens,
                            int32_t hidden, const void* x, const void* w, void* qkv,
                            void* hip_stream);

/*
 * ca_append_kv_rope_packed -- ca_append_kv_rope reading q, k_new and v_new in place from the
 * packed projection output qkv[T][Hq + 2 Hkv][d] (q heads, k heads, v heads of each row), with
 * no copy in between.  q_out [T][Hq][d] receives the rotated q and must not overlap qkv; the
 * caches, plan and errors are those of ca_append_kv_rope.
 */
ca_status ca_append_kv_rope_packed(ca_ctx* ctx, const ca_attn_desc* desc, const ca_plan* plan,
                                   const void* qkv, void* q_out, void* k_cache, void* v_cache,
                                   int64_t num_pool_pages, void* hip_stream);

/*
 * ---- Multi-step driver: ca_sched (host only, no device work) ----
 * The serving loop around ca_plan_batch, following [SF] "六·补二、调度器每一轮在做什么" (each round:
 * running decodes first, one token each; a decode that needs KV space when none is left is
 * preempted and later recomputed from its first token; the budget left goes to prefill chunks;
 * an unfinished prompt is taken up again next round) and [SS] "一个 512-token 预算的例子" step 4 (a
 * prefill that finishes its prompt is a decode from the next round on).
 *   - The scheduler owns the page pool [0, num_pool_pages) as a first-in first-out free list
 *     (initially 0, 1, ..., N-1; pages are taken from the front and returned to the back).
 *   - ca_sched_step plans one round over the unfinished requests in admission order, with the
 *     rules and parameters of ca_plan_batch, after giving each scheduled request the pages its
 *     new tokens need: a decode whose token needs a page when the free list is empty is
 *     preempted instead (its pages go back to the free list; it waits, not scheduled this round,
 *     to recompute all the tokens it had cached), and a chunk is also cut to the slots its pages
 *     plus the free list can hold (then aligned again).  plan->req_ids holds request ids.  The
 *     plan arrays need cap_seqs >= unfinished requests and cap_pages >= their pages.
 *   - The caller then runs the round (ca_append_kv_rope + ca_mixed_attention with the plan) and
 *     calls ca_sched_commit: every scheduled request advances by its tokens; a prefill that
 *     reaches the end of its prompt starts decoding (or finishes, when it has already run
 *     max_new_tokens decode steps); a decode step counts towards max_new_tokens, and a request
 *     that reaches it finishes and returns its pages.
 * Not thread-safe: one caller at a time per ca_sched.
 */
typedef struct ca_sched ca_sched;

enum { CA_REQ_WAITING = 0, CA_REQ_RUNNING = 1, CA_REQ_FINISHED = 2 };

typedef struct {
    int32_t state;              /* CA_REQ_WAITING (prompt or recompute left), _RUNNING (decoding), _FINISHED */
    int32_t num_computed;       /* tokens in the cache */
    int32_t num_prompt_left;    /* tokens left to prefill (0 unless waiting) */
    int32_t num_generated;      /* decode steps run */
    int32_t num_pages;          /* entries of block_table */
    int32_t num_preemptions;
    const int32_t* block_table; /* host memory owned by the scheduler; valid until its next call */
} ca_sched_request;

/* Errors: CA_ERR_INVALID_ARG for null pointers or parameters ca_plan_batch would reject. */
ca_status ca_sched_create(const ca_plan_params* params, ca_sched** out);
ca_status ca_sched_destroy(ca_sched* s);
/* Admit a request of prompt_len tokens whose first num_cached (< prompt_len) are already in the
 * cache (a prefix hit; [CP] "7.1 chunked prefill 与 prefix caching 的相互影响": the rounds then
 * chunk only the tokens after the cached prefix): in cached_pages (ceil(num_cached / P) distinct free pages, which leave
 * the free list), or, with cached_pages NULL, in pages taken from the free list for the caller
 * to fill (read them with ca_sched_get).  It decodes max_new_tokens steps after its prompt.
 * *id receives the request id (0, 1, ... in admission order).  Errors: CA_ERR_INVALID_ARG (bad
 * sizes, a cached page outside the pool or not free, a step awaiting commit), CA_ERR_NO_PAGES
 * (not enough free pages for the prefix). */
ca_status ca_sched_add(ca_sched* s, int32_t prompt_len, int32_t max_new_tokens, int32_t num_cached,
                       const int32_t* cached_pages, int32_t* id);
/* Plan the next round into `plan` (see above).  Errors: those of ca_plan_batch, and
 * CA_ERR_INVALID_ARG when the previous round is not committed. */
ca_status ca_sched_step(ca_sched* s, ca_plan* plan);
/* Advance the requests of the planned round.  CA_ERR_INVALID_ARG when no round is planned. */
ca_status ca_sched_commit(ca_sched* s);
ca_status ca_sched_get(const ca_sched* s, int32_t id, ca_sched_request* out);
/* Pages on the free list (-1 for a null scheduler). */
int64_t ca_sched_free_pages(const ca_sched* s);

const char* ca_status_string(ca_status s);
/* Detail message of the calling thread's last failed call ("" if none). */
const char* ca_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* CA_H */

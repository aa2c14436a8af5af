// internal.h -- declarations shared by the library's translation units (not part of the ABI).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <string>

#include "ca.h"

namespace ca {

// Thread-local detail message behind ca_last_error().
void set_error(const std::string& msg);
void clear_error();

// Device view of a plan (the four ragged metadata arrays plus counts).  Kernels derive
//   kv_len(s) = (kv_page_indptr[s+1] - kv_page_indptr[s] - 1) * P + kv_last_page_len[s]
//   q_len(s)  = qo_indptr[s+1] - qo_indptr[s]
//   position of row t of s = kv_len(s) - q_len(s) + (t - qo_indptr[s]).
struct DevPlan {
    const int32_t* qo_indptr;
    const int32_t* kv_page_indptr;
    const int32_t* kv_page_indices;
    const int32_t* kv_last_page_len;
    const int32_t* row_seq;   // [num_tokens] sequence of each flat row (qo_indptr expanded)
    const int32_t* row_pos;   // [num_tokens] absolute position of each row
    const int32_t* row_page;  // [num_tokens] pool page that receives the row's K/V (slot pos % P)
    int32_t num_seqs;
    int32_t num_decodes;
    int32_t num_tokens;
    int32_t num_pages;
    int32_t page_size;
    // When set, the attention launch's first thread stores done_value here (pinned host memory)
    // as it starts: by stream order every earlier launch has finished by then, so the host learns
    // that the staging slot an earlier launch read may be refilled (no event in the stream).
    uint32_t* done_flag;
    uint32_t done_value;
};

// The store of DevPlan::done_flag (a system-scope store: the host polls the location).
__device__ __forceinline__ void report_done(const DevPlan& p) {
    if (p.done_flag) __hip_atomic_store(p.done_flag, p.done_value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Read-only plan metadata seen through the constant address space.  The attention kernel only
// reads the plan arrays (they are written by earlier launches), and saying so lets the compiler
// serve wave-uniform reads of them with scalar loads.  Through a generic pointer it cannot prove
// that the kernel's own stores (outputs, partials) leave them alone, and falls back to vector
// loads, which share the in-order vector-memory counter with the K/V loads: waiting for a page
// id would then also wait for every K/V load issued before it.
template <typename T>
using ConstPtr = const __attribute__((address_space(4))) T*;

template <typename T>
__device__ __forceinline__ ConstPtr<T> as_const(const T* p) {
    return (ConstPtr<T>)(p);
}

// Record i of an int4 array read through the constant address space.
__device__ __forceinline__ int4 load_rec(ConstPtr<int32_t> p, int i) {
    return make_int4(p[4 * i], p[4 * i + 1], p[4 * i + 2], p[4 * i + 3]);
}

struct Shape {
    int32_t hq, hkv, d, P;
    float scale;
    double theta;
    ca_dtype dtype;
};

// Optional timing events of one library call, attached to its launches with hipExtLaunchKernel
// (start with the first kernel of the call, stop with the last), so timing puts no extra packet
// in the stream.  Null events: no timing.
struct LaunchEvents {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};

// ---- launchers (each enqueues on `stream`; returns hipSuccess or the launch error) ----
// inv_freq: [d / 2] fp64 table theta^(-2i/d) in device memory.
// The QKV projection (linear.cpp): out[T][N] = x[T][K] . w[N][K]^T, bf16 with fp32
// accumulation, through hipBLASLt.  *L is created on first use and cached per shape.
struct Linear;
void linear_release(Linear* L);
bool linear_bf16(Linear*& L, int64_t T, int64_t K, int64_t N, const void* x, const void* w,
                 void* out, hipStream_t stream, std::string* err);
// The same product for few tokens (linear_skinny.hip): a kernel that streams the weights once
// through the matrix cores.  It takes T in [1, kSkinnyMaxTokens], K a multiple of 2048 and N a
// multiple of 32 (skinny_projection_fits); x [T][K], w [N][K], out [T][N], 16-byte aligned.
constexpr int64_t kSkinnyMaxTokens = 16;
bool skinny_projection_fits(int64_t T, int64_t K, int64_t N);
hipError_t launch_skinny_projection(int64_t T, int64_t K, int64_t N, const void* x, const void* w,
                                    void* out, hipStream_t stream, const LaunchEvents& ev);

// The same product beyond 16 tokens (linear_tiled.hip): an LDS-tiled MFMA GEMM over BM x BN
// output tiles, with K split over `nsplit` workgroups (fp32 partials, then a fixed-order sum)
// when the tiles alone would not fill the device.  It takes K a multiple of 64 and N a multiple
// of 64 (plan.ok false otherwise); partials need tiled_partial_bytes of device memory.
struct TiledPlan {
    int bm = 0, bn = 0, nsplit = 0;
    bool ok = false;
};
TiledPlan plan_tiled_projection(int64_t T, int64_t K, int64_t N, int num_cus);
size_t tiled_partial_bytes(const TiledPlan& pl, int64_t T, int64_t N);
bool tiled_shape_fits(const TiledPlan& pl, int64_t T, int64_t K, int64_t N);
hipError_t launch_tiled_projection(const TiledPlan& pl, int64_t T, int64_t K, int64_t N, const void* x,
                                   const void* w, void* out, float* part, hipStream_t stream,
                                   const LaunchEvents& ev);

// q_row, kv_row: elements between consecutive token rows of q_in and of k_new / v_new.
// row_pos, row_page: [num_tokens] per-row position and destination page (device memory or the
// device-mapped host staging).  meta_n16 > 0: the same launch also copies meta_n16 16-byte units
// from meta_src (device-mapped host staging) to meta_dst (device memory).  num_cus: the device's
// CU count (sizes the token workgroups so that they are all resident at once where they can be).
hipError_t launch_append_rope(const DevPlan& p, const Shape& sh, const int32_t* row_pos,
                              const int32_t* row_page, const double* inv_freq, const void* q_in,
                              void* q_out, const void* k_new, const void* v_new, void* k_cache,
                              void* v_cache, int64_t q_row, int64_t kv_row, const void* meta_src,
                              void* meta_dst, int64_t meta_n16, int num_cus, hipStream_t stream,
                              const LaunchEvents& ev);

// Generic split-KV attention for every row (one wave per (row, q head, split)), then merge.
// partial: fp32 workspace of num_tokens * hq * nsplit * (d + 2) floats.
// Rows [row0, num_tokens) only; partial indices are relative to row 0 of the step.
hipError_t launch_attention_generic(const DevPlan& p, const Shape& sh, int row0, const void* q,
                                    const void* k_cache, const void* v_cache, void* o,
                                    float* lse, float* partial, int nsplit,
                                    hipStream_t stream, const LaunchEvents& ev);

size_t generic_partial_floats(int32_t num_tokens, const Shape& sh, int nsplit);

}  // namespace ca

namespace ca {
// MFMA attention for a whole mixed step (bf16, G <= 16), one launch: the grid is dec_wgs decode
// workgroups followed by num_workers chunk workers (attn_mixed.hip).
//   decode: dec_items holds two int4 per item, {kv head, key begin, key end, partial slot or -1
//     (the item covers the whole row: output written directly)}, {row, offset of the row's page
//     ids in kv_page_indices, page count, 0}.  Decode workgroups run dec_wpg
//     wavefronts each (1 .. attention_decode_waves_per_wg()), and decode wave w (of dec_wgs *
//     dec_wpg) runs items [wave_items[w], wave_items[w + 1]) for w < num_waves.  Partials:
//     dec_acc [slots][G][d] fp32, dec_ml [slots][G] (max in log2 units, sum).
//   chunk: a query column is one (row, q head) pair of a kv head's group, numbered row * G +
//     head.  chunk_items: two int4 per workgroup, {seq, kv head, first column, partial slot or
//     -1}, {key begin, key end, 0, 0} (seq -1: padding).  Partials: chunk_acc
//     [slot][chunk_cols_per_block()][d] fp32 and chunk_ml [slot][cols].
//   chunk workers: direct mode (queue_mode false) needs num_workers == num_chunk_items, worker
//     w running item w; queue mode: num_workers persistent workers, the first num_static of
//     them starting with the launch, taking items through the counters in `queue`
//     (kQueueInts ints, zero on entry).  Every launch zeroes the other counter set
//     `queue_other` (kQueueInts ints), which the caller gives to the next queue-mode launch on
//     the stream: two sets used alternately need no clearing launch.
hipError_t launch_attention(const DevPlan& p, const Shape& sh, int dec_wgs, int dec_wpg,
                            const int4* dec_items, const int32_t* wave_items, int num_waves,
                            const int4* chunk_items,
                            int num_chunk_items, int num_workers, int num_static,
                            bool queue_mode, int* queue, int* queue_other,
                            const void* q, const void* k_cache,
                            const void* v_cache, float* dec_acc, float2* dec_ml,
                            float* chunk_acc, float2* chunk_ml, void* o, float* lse, hipStream_t stream,
                            const LaunchEvents& ev);
// Work-queue counters: eight, each alone in a 128-byte line (kQueueStride ints apart) so that
// the atomics of the eight queues do not contend for one line.
constexpr int kQueueStride = 32;
constexpr int kQueueInts = 8 * kQueueStride;  // ints of one work-queue counter set
int chunk_cols_per_block();
int attention_decode_waves_per_wg();
// Attention workgroups one CU holds at once.
int attention_wgs_per_cu(int d);

// One launch combining every split: decode merges[j] = {row, kv head, first slot, count}
// (partials [slot][G][d]); chunk groups: two int4 {seq, kv head, first column, first slot},
// {splits, first row of the sequence, rows of the sequence, 0} (partials
// [slot][chunk_cols_per_block()][d]).  Running maxima are in log2 units.  16 lanes per output
// (row, q head).
hipError_t launch_merge(const DevPlan& p, const Shape& sh, const int4* dec_merges, int num_dec,
                        const float* dec_acc, const float2* dec_ml, const int4* chunk_groups,
                        int num_chunk, const float* chunk_acc, const float2* chunk_ml, void* o,
                        float* lse, hipStream_t stream, const LaunchEvents& ev);
// Longest key range one chunk workgroup may cover (its page ids are staged in LDS).
int chunk_max_split_keys();
}  // namespace ca

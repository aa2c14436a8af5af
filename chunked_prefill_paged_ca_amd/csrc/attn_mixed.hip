// attn_mixed.hip -- one attention launch for a whole mixed step: decode rows and prefill-chunk
// rows side by side.
//
// bowenzhou.top "Sarathi：让解码搭上 prefill 的顺风车", section "Decode-maximal batching", and
// magicnetworld.com "分块预填充与 Stall-free 调度", section 一: a mixed batch pairs work that
// is bound by memory traffic (decodes read their whole K/V history once) with work bound by
// arithmetic (a prefill chunk reuses every K/V block for all its query rows), so the two kinds
// of work can run on the chip at the same time instead of one after the other.
//
// The grid is [dec_wgs decode workgroups][chunk workers].  Workgroups are dispatched in index
// order, so the decode workgroups (dec_wpg wavefronts each, every wave streaming its equal share
// of the decode K/V blocks, attn_decode.h) start first and stay resident on dec_wgs CUs until their
// shares are done; the chunk workers (attn_chunk.h) run on the remaining CUs from the start and
// take over the decode CUs as those drain.  Decode reaches the HBM bandwidth on a fraction of
// the CUs, so the chunk work fills CUs the decode stream does not need.  Either part may be
// empty.
//
// Chunk workers run in one of two modes.  Direct: worker w runs chunk item w (every item fits
// on the CUs free at the start).  Queue: one persistent worker per workgroup slot of the device;
// the items form eight queues, queue x (items [x per, x per + size(x)), per = ceil(n / 8)) for
// the workers on XCD x (workgroups are dealt to the XCDs round robin, so the workgroups that run
// side by side on one XCD share their K/V pages in its L2).  The first items of each queue go
// one each to the workers that start with the launch, without atomics; after that a worker
// claims items through the queue's counter (a device-scope atomic add in `queue[x]`), its own
// XCD's queue first, then the others, and leaves when all are empty.  No worker ever waits for
// another, so every worker ends.  Two counter sets are used by turns: a launch claims from one
// and its first thread zeroes the other, which the next queue-mode launch on the stream claims
// from (a count of finished workers for the last one to clear them would cost every worker
// another round trip at its end).

#include <hip/hip_runtime.h>

#include "attn_chunk.h"
#include "attn_decode.h"
#include "internal.h"

namespace ca {
namespace {

constexpr int kThreads = 64 * chunk::kWaves;  // both kinds of workgroup: 8 wavefronts
constexpr int kDecodeWaves = kThreads / 64;

template <int D>
__global__ void __launch_bounds__(kThreads, 1) mixed_kernel(
    DevPlan p, int dec_wgs, int dec_wpg, const int4* __restrict__ dec_items,
    const int32_t* __restrict__ wave_items, int num_waves, const int4* __restrict__ chunk_items,
    int num_chunk_items, int num_workers, int num_static, bool queue_mode,
    int* __restrict__ queue, int* __restrict__ queue_other,
    const uint16_t* __restrict__ qg,
    const uint16_t* __restrict__ k_cache, const uint16_t* __restrict__ v_cache, int hq, int hkv,
    float scale_log2, float* __restrict__ dec_acc, float2* __restrict__ dec_ml,
    float* __restrict__ chunk_acc, float2* __restrict__ chunk_ml, uint16_t* __restrict__ o,
    float* __restrict__ lse) {
    if (blockIdx.x == 0 && threadIdx.x == 0) report_done(p);
    // the other work-queue counter set, for the next queue-mode launch (see the top of the file)
    if (blockIdx.x == 0 && threadIdx.x < 8)
        __hip_atomic_store(queue_other + threadIdx.x * kQueueStride, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (static_cast<int>(blockIdx.x) < dec_wgs) {
        // wave-uniform indices: everything derived from them (item records, page ids) lives in
        // scalar registers and is read with scalar loads, which do not share the vector-load
        // counter the K/V prefetch relies on
        const int lane = threadIdx.x & 63;
        const int wi = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        if (wi >= dec_wpg) return;
        const int w = __builtin_amdgcn_readfirstlane(blockIdx.x * dec_wpg + wi);
        if (w >= num_waves) return;
        const ConstPtr<int32_t> bounds = as_const(wave_items);
        const ConstPtr<int32_t> recs = as_const(reinterpret_cast<const int32_t*>(dec_items));
        const int i_end = bounds[w + 1];
        for (int i = bounds[w]; i < i_end; ++i)
            decode::decode_item<D>(load_rec(recs, 2 * i), load_rec(recs, 2 * i + 1), as_const(p.kv_page_indices), qg,
                                   k_cache, v_cache, hq, hkv, scale_log2, dec_acc, dec_ml, o, lse,
                                   lane);
        return;
    }
    // Chunk worker (direct or queue mode, see the top of this file)
    __shared__ int s_item;
    const int w = blockIdx.x - dec_wgs;
    const int x = w & 7;  // this worker's XCD: workgroups are dealt to the XCDs round robin
    const int per = (num_chunk_items + 7) >> 3;
    auto qsize = [&](int qx) { return max(0, min(per, num_chunk_items - qx * per)); };
    auto qstatic = [&](int qx) { return min(max(0, (num_static - qx + 7) >> 3), qsize(qx)); };
    auto take = [&](int qx, int i) {
        const int k = qstatic(qx) + i;
        return k < qsize(qx) ? qx * per + k : -1;
    };
    auto claim = [&]() -> int {  // thread 0
        // the state of every queue is read along with the claim on this XCD's own queue (one
        // round trip between them), so that a worker whose queue is empty learns at once which
        // others still hold items, and one that finds all empty leaves after that one trip
        int seen[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) seen[k] = __hip_atomic_load(queue + k * kQueueStride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int it = take(x, atomicAdd(queue + x * kQueueStride, 1));
        if (it >= 0) return it;
        for (int k = 1; k < 8; ++k) {
            const int qx = (x + k) & 7;
            if (qstatic(qx) + seen[qx] >= qsize(qx)) continue;
            const int st = take(qx, atomicAdd(queue + qx * kQueueStride, 1));
            if (st >= 0) return st;
        }
        return -1;
    };
    auto next = [&]() {  // the whole workgroup: thread 0 claims, the others wait for its result
        if (threadIdx.x == 0) s_item = claim();
        __syncthreads();
        const int it = s_item;
        __syncthreads();
        return it;
    };
    int item;
    if (!queue_mode) item = w;
    else if (w < num_static && (w >> 3) < qstatic(x)) item = x * per + (w >> 3);
    else item = next();
    while (item >= 0) {
        chunk::chunk_item<D>(item, p, chunk_items, qg, k_cache, v_cache, hq, hkv, scale_log2,
                             chunk_acc, chunk_ml, o, lse);
        if (!queue_mode) break;
        // the next item is claimed only now: an item claimed ahead would be held behind this
        // one while idle workers find the queues empty
        item = next();
    }
}

}  // namespace

int chunk_cols_per_block() { return chunk::kCols; }
int chunk_max_split_keys() { return 16 * (chunk::kMaxItemPages - 2); }
int attention_decode_waves_per_wg() { return kDecodeWaves; }

hipError_t launch_attention(const DevPlan& p, const Shape& sh, int dec_wgs, int dec_wpg,
                            const int4* dec_items, const int32_t* wave_items, int num_waves,
                            const int4* chunk_items,
                            int num_chunk_items, int num_workers, int num_static,
                            bool queue_mode, int* queue, int* queue_other,
                            const void* q, const void* k_cache,
                            const void* v_cache, float* dec_acc, float2* dec_ml, float* chunk_acc,
                            float2* chunk_ml, void* o, float* lse, hipStream_t stream,
                            const LaunchEvents& ev) {
    if (num_waves <= 0) dec_wgs = 0;
    if (dec_wgs > 0 && (dec_wpg < 1 || dec_wpg > kDecodeWaves || dec_wgs * dec_wpg < num_waves))
        return hipErrorInvalidValue;
    if (num_chunk_items <= 0) num_workers = 0;
    if (num_workers > 0 && ((queue_mode && !queue) || (!queue_mode && num_workers != num_chunk_items)))
        return hipErrorInvalidValue;
    if (!queue_other) return hipErrorInvalidValue;
    const int grid = dec_wgs + num_workers;
    if (grid <= 0) return hipSuccess;
    const float scale_log2 = sh.scale * 1.4426950408889634f;
    auto qq = static_cast<const uint16_t*>(q);
    auto kc = static_cast<const uint16_t*>(k_cache);
    auto vc = static_cast<const uint16_t*>(v_cache);
    auto oo = static_cast<uint16_t*>(o);
    if (sh.d == 128)
        hipExtLaunchKernelGGL(mixed_kernel<128>, dim3(grid), dim3(kThreads), 0, stream, ev.start,
                              ev.stop, 0, p, dec_wgs, dec_wpg, dec_items, wave_items, num_waves,
                              chunk_items, num_chunk_items, num_workers, num_static, queue_mode,
                              queue, queue_other, qq, kc, vc, sh.hq, sh.hkv, scale_log2, dec_acc, dec_ml,
                              chunk_acc, chunk_ml, oo, lse);
    else
        hipExtLaunchKernelGGL(mixed_kernel<64>, dim3(grid), dim3(kThreads), 0, stream, ev.start,
                              ev.stop, 0, p, dec_wgs, dec_wpg, dec_items, wave_items, num_waves,
                              chunk_items, num_chunk_items, num_workers, num_static, queue_mode,
                              queue, queue_other, qq, kc, vc, sh.hq, sh.hkv, scale_log2, dec_acc, dec_ml,
                              chunk_acc, chunk_ml, oo, lse);
    return hipGetLastError();
}

// Attention workgroups one CU holds at once (register-limited).
int attention_wgs_per_cu(int d) {
    int blocks = 0;
    const hipError_t e = d == 128
        ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, mixed_kernel<128>, kThreads, 0)
        : hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, mixed_kernel<64>, kThreads, 0);
    if (e != hipSuccess || blocks <= 0) return 1;
    return blocks;
}

}  // namespace ca

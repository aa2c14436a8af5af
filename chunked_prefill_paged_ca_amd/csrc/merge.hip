// merge.hip -- log-sum-exp combination of split-KV partial results (decode splits and prefill-
// chunk key splits) in one launch.
//
// A split s of a query column holds m_s (running max, log2 units), l_s (sum of 2^(score - m_s))
// and acc_s (sum of 2^(score - m_s) v).  With M = max_s m_s over splits that saw a key,
//   o = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s,   lse = (M + log2 sum_s 2^(m_s - M) l_s) ln 2,
// which is the softmax over the union of the splits' keys.  (Not a step of the pages: it is how
// the library parallelises one row over many keys; see the causal attention of
// pinghaoyang.com.cn "Sarathi-Serve 完全拆解", section "分块不等于截断上下文", for what is merged.)
//
// Sixteen lanes per output column (row, q head), four columns per wavefront; a lane owns d / 16
// consecutive output dimensions.  Every lane walks the column's splits itself (the (m, l) pairs
// are the same few bytes for the 16 lanes), so there is no cross-lane traffic at all, and the
// partial rows are read with 16-byte loads, eight splits in flight at once.

#include <hip/hip_runtime.h>

#include <cmath>

#include "internal.h"
#include "mfma.h"

namespace ca {
namespace {

constexpr int kLanes = 16;  // lanes per column

template <int D>
__device__ __forceinline__ void combine(const float2* __restrict__ ml, int64_t ml_stride,
                                        const float* __restrict__ acc, int64_t acc_stride,
                                        int nsplit, int sub, uint16_t* __restrict__ out,
                                        float* __restrict__ lse_out) {
    constexpr int E = D / kLanes;  // dims per lane: 8 or 4
    constexpr int C = 8;           // splits whose loads are in flight together
    // One pass over the splits in chunks of C: every load of a chunk is issued before any of its
    // values is used (indices past the end are clamped and weighted 0), so a chunk costs one
    // memory round trip; the running max and sums are rescaled when a chunk raises the max.
    float M = -INFINITY, L = 0.0f;
    float a[E] = {};
    const float* base = acc + sub * E;
    for (int k0 = 0; k0 < nsplit; k0 += C) {
        float2 v[C];
        float4 x[C][E / 4];
#pragma unroll
        for (int j = 0; j < C; ++j) {
            const int k = k0 + j < nsplit ? k0 + j : nsplit - 1;
            v[j] = ml[k * ml_stride];
            if (k0 + j >= nsplit) v[j].y = 0.0f;
#pragma unroll
            for (int e = 0; e < E; e += 4) x[j][e / 4] = *reinterpret_cast<const float4*>(base + k * acc_stride + e);
        }
        float cm = M;
#pragma unroll
        for (int j = 0; j < C; ++j)
            if (v[j].y > 0.0f) cm = fmaxf(cm, v[j].x);
        if (cm == -INFINITY) continue;  // no split of this chunk saw a key
        const float r = exp2_fast(M - cm);  // 0 while M is still -inf
        L *= r;
#pragma unroll
        for (int e = 0; e < E; ++e) a[e] *= r;
        M = cm;
#pragma unroll
        for (int j = 0; j < C; ++j) {
            const float w = v[j].y > 0.0f ? exp2_fast(v[j].x - M) : 0.0f;
            L += w * v[j].y;
#pragma unroll
            for (int e = 0; e < E; e += 4) {
                a[e] += w * x[j][e / 4].x;
                a[e + 1] += w * x[j][e / 4].y;
                a[e + 2] += w * x[j][e / 4].z;
                a[e + 3] += w * x[j][e / 4].w;
            }
        }
    }
    const float inv = 1.0f / L;
    uint32_t packed[E / 2];
#pragma unroll
    for (int e = 0; e < E; e += 2)
        packed[e / 2] = f2bf(a[e] * inv) | (static_cast<uint32_t>(f2bf(a[e + 1] * inv)) << 16);
    if constexpr (E == 8) {
        *reinterpret_cast<uint4*>(out + sub * E) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    } else {
        *reinterpret_cast<uint2*>(out + sub * E) = make_uint2(packed[0], packed[1]);
    }
    if (lse_out && sub == 0) *lse_out = (M + __log2f(L)) * 0.69314718055994531f;
}

template <int D>
__global__ void __launch_bounds__(256) merge_kernel(
    int hq, int hkv, int cols, const int4* __restrict__ dec_merges, int num_dec,
    const float* __restrict__ dec_acc, const float2* __restrict__ dec_ml,
    const int4* __restrict__ chunk_groups, int num_chunk, const float* __restrict__ chunk_acc,
    const float2* __restrict__ chunk_ml, uint16_t* __restrict__ o, float* __restrict__ lse) {
    const int G = hq / hkv;
    const int sub = threadIdx.x & (kLanes - 1);
    int col = (blockIdx.x * 256 + threadIdx.x) / kLanes;
    const int dec_cols = num_dec * G;
    if (col < dec_cols) {
        // decode: column = (merge, q head c of the group); partials [slot][G][D]
        const int4 mg = dec_merges[col / G];
        const int c = col - (col / G) * G;
        const int64_t orow = static_cast<int64_t>(mg.x) * hq + mg.y * G + c;
        combine<D>(dec_ml + static_cast<int64_t>(mg.z) * G + c, G,
                   dec_acc + (static_cast<int64_t>(mg.z) * G + c) * D, static_cast<int64_t>(G) * D,
                   mg.w, sub, o + orow * D, lse ? lse + orow : nullptr);
        return;
    }
    col -= dec_cols;
    if (col >= num_chunk * cols) return;
    // chunk: column = (column block, column); partials [slot][cols][D]
    const int grp = col / cols, wc = col - grp * cols;
    const int4 g0 = chunk_groups[2 * grp];
    const int4 g1 = chunk_groups[2 * grp + 1];
    const int g = g0.y, cb = g0.z, first = g0.w;
    const int nsplit = g1.x, q0 = g1.y, q_len = g1.z;
    const int qc = cb + wc;  // (row, head) column inside the sequence's chunk
    if (qc >= q_len * G) return;
    const int row = qc / G, j = qc - (qc / G) * G;
    const int64_t orow = static_cast<int64_t>(q0 + row) * hq + g * G + j;
    combine<D>(chunk_ml + static_cast<int64_t>(first) * cols + wc, cols,
               chunk_acc + (static_cast<int64_t>(first) * cols + wc) * D, static_cast<int64_t>(cols) * D,
               nsplit, sub, o + orow * D, lse ? lse + orow : nullptr);
}

}  // namespace

hipError_t launch_merge(const DevPlan& p, const Shape& sh, const int4* dec_merges, int num_dec,
                        const float* dec_acc, const float2* dec_ml, const int4* chunk_groups,
                        int num_chunk, const float* chunk_acc, const float2* chunk_ml, void* o,
                        float* lse, hipStream_t stream, const LaunchEvents& ev) {
    (void)p;
    const int G = sh.hq / sh.hkv;
    const int cols = chunk_cols_per_block();
    const int64_t columns = static_cast<int64_t>(num_dec) * G + static_cast<int64_t>(num_chunk) * cols;
    if (columns <= 0) return hipSuccess;
    const int64_t per_block = 256 / kLanes;
    const dim3 grid(static_cast<unsigned>((columns + per_block - 1) / per_block)), block(256);
    auto oo = static_cast<uint16_t*>(o);
    if (sh.d == 128)
        hipExtLaunchKernelGGL(merge_kernel<128>, grid, block, 0, stream, ev.start, ev.stop, 0, sh.hq, sh.hkv, cols, dec_merges,
                           num_dec, dec_acc, dec_ml, chunk_groups, num_chunk, chunk_acc, chunk_ml, oo, lse);
    else
        hipExtLaunchKernelGGL(merge_kernel<64>, grid, block, 0, stream, ev.start, ev.stop, 0, sh.hq, sh.hkv, cols, dec_merges,
                           num_dec, dec_acc, dec_ml, chunk_groups, num_chunk, chunk_acc, chunk_ml, oo, lse);
    return hipGetLastError();
}

}  // namespace ca

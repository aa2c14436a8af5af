// merge.hip -- log-sum-exp combination of split-KV partial results (decode splits and prefill-
// chunk key splits) in one launch.
//
// A split s of a query column holds m_s (running max, log2 units), l_s (sum of 2^(score - m_s))
// and acc_s (sum of 2^(score - m_s) v).  With M = max_s m_s over splits that saw a key,
//   o = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s,   lse = (M + log2 sum_s 2^(m_s - M) l_s) ln 2,
// which is the softmax over the union of the splits' keys.  (Not a step of the pages: it is how
// this build parallelises one row over many keys; see the causal attention of
// pinghaoyang.com.cn "Sarathi-Serve 完全拆解", section "分块不等于截断上下文", for what is merged.)
//
// One wavefront per output (row, q head): lane k reads split k's (m, l) (at most 64 splits per
// wave step), the wave reduces M and the weighted sum, then each lane accumulates its output
// dimensions over the splits with independent, unrolled loads.

#include <hip/hip_runtime.h>

#include <cmath>

#include "internal.h"
#include "mfma.h"

namespace ca {
namespace {

template <int D>
__device__ __forceinline__ void combine(const float2* __restrict__ ml_base, int64_t ml_stride,
                                        const float* __restrict__ acc_base, int64_t acc_stride,
                                        int nsplit, int lane, uint16_t* __restrict__ out,
                                        float* __restrict__ lse_out) {
    float mx = -INFINITY;
    for (int k = lane; k < nsplit; k += 64) {
        const float2 ml = ml_base[k * ml_stride];
        if (ml.y > 0.0f) mx = fmaxf(mx, ml.x);
    }
#pragma unroll
    for (int o_ = 32; o_ >= 1; o_ >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o_, 64));
    float L = 0.0f;
    float a[D / 64] = {};
    for (int k0 = 0; k0 < nsplit; k0 += 64) {
        float wk = 0.0f;
        if (k0 + lane < nsplit) {
            const float2 ml = ml_base[(k0 + lane) * ml_stride];
            if (ml.y > 0.0f) {
                wk = exp2_fast(ml.x - mx);
                L += wk * ml.y;
            }
        }
        const int n = nsplit - k0 < 64 ? nsplit - k0 : 64;
        const float* base = acc_base + k0 * acc_stride + lane;
#pragma unroll 8
        for (int k = 0; k < n; ++k) {
            const float wgt = __shfl(wk, k, 64);
#pragma unroll
            for (int e = 0; e < D / 64; ++e) a[e] += wgt * base[k * acc_stride + 64 * e];
        }
    }
#pragma unroll
    for (int o_ = 32; o_ >= 1; o_ >>= 1) L += __shfl_xor(L, o_, 64);
    const float inv = 1.0f / L;
#pragma unroll
    for (int e = 0; e < D / 64; ++e) out[lane + 64 * e] = f2bf(a[e] * inv);
    if (lse_out && lane == 0) *lse_out = (mx + __log2f(L)) * 0.69314718055994531f;
}

template <int D>
__global__ void __launch_bounds__(256) merge_kernel(
    DevPlan p, int hq, int hkv, int cols, const int4* __restrict__ dec_merges, int num_dec,
    const float* __restrict__ dec_acc, const float2* __restrict__ dec_ml,
    const int4* __restrict__ chunk_groups, int num_chunk, const float* __restrict__ chunk_acc,
    const float2* __restrict__ chunk_ml, uint16_t* __restrict__ o, float* __restrict__ lse) {
    const int G = hq / hkv;
    const int lane = threadIdx.x & 63;
    int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int dec_waves = num_dec * G;
    if (wid < dec_waves) {
        // decode: wave = (merge, q head c of the group); partials [slot][G][D]
        const int4 mg = dec_merges[wid / G];
        const int c = wid - (wid / G) * G;
        const int row = p.qo_indptr[mg.x];
        const int64_t orow = static_cast<int64_t>(row) * hq + mg.y * G + c;
        combine<D>(dec_ml + static_cast<int64_t>(mg.z) * G + c, G,
                   dec_acc + (static_cast<int64_t>(mg.z) * G + c) * D, static_cast<int64_t>(G) * D,
                   mg.w, lane, o + orow * D, lse ? lse + orow : nullptr);
        return;
    }
    wid -= dec_waves;
    if (wid >= num_chunk * cols) return;
    // chunk: wave = (column block, column); partials [slot][cols][D]
    const int grp = wid / cols, wc = wid - grp * cols;
    const int4 g0 = chunk_groups[2 * grp];
    const int nsplit = chunk_groups[2 * grp + 1].x;
    const int s = g0.x, g = g0.y, cb = g0.z, first = g0.w;
    const int q0 = p.qo_indptr[s];
    const int q_len = p.qo_indptr[s + 1] - q0;
    const int col = cb + wc;
    if (col >= q_len * G) return;
    const int row = col / G, j = col - (col / G) * G;
    const int64_t orow = static_cast<int64_t>(q0 + row) * hq + g * G + j;
    combine<D>(chunk_ml + static_cast<int64_t>(first) * cols + wc, cols,
               chunk_acc + (static_cast<int64_t>(first) * cols + wc) * D, static_cast<int64_t>(cols) * D,
               nsplit, lane, o + orow * D, lse ? lse + orow : nullptr);
}

}  // namespace

hipError_t launch_merge(const DevPlan& p, const Shape& sh, const int4* dec_merges, int num_dec,
                        const float* dec_acc, const float2* dec_ml, const int4* chunk_groups,
                        int num_chunk, const float* chunk_acc, const float2* chunk_ml, void* o,
                        float* lse, hipStream_t stream) {
    const int G = sh.hq / sh.hkv;
    const int cols = chunk_cols_per_block();
    const int64_t waves = static_cast<int64_t>(num_dec) * G + static_cast<int64_t>(num_chunk) * cols;
    if (waves <= 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>((waves + 3) / 4)), block(256);
    auto oo = static_cast<uint16_t*>(o);
    if (sh.d == 128)
        hipLaunchKernelGGL(merge_kernel<128>, grid, block, 0, stream, p, sh.hq, sh.hkv, cols, dec_merges,
                           num_dec, dec_acc, dec_ml, chunk_groups, num_chunk, chunk_acc, chunk_ml, oo, lse);
    else
        hipLaunchKernelGGL(merge_kernel<64>, grid, block, 0, stream, p, sh.hq, sh.hkv, cols, dec_merges,
                           num_dec, dec_acc, dec_ml, chunk_groups, num_chunk, chunk_acc, chunk_ml, oo, lse);
    return hipGetLastError();
}

}  // namespace ca

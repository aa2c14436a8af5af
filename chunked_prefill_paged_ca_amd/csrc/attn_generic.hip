// attn_generic.hip -- plain split-KV paged attention for every row of a mixed step, plus the
// log-sum-exp merge of the splits.  This is the fp32 storage path; it handles any row (decode or
// chunk) the same way and favours simplicity over speed.
//
// What it computes: pinghaoyang.com.cn "Sarathi-Serve 完全拆解", section "分块不等于截断上下文" --
// the query at absolute position p attends to every key 0..p of its own request (history pages
// and the current chunk's pages alike) with softmax weights of q.k / sqrt(d_h).
//
// Work item = one wavefront per (row, q head, split).  The split cuts the row's visible keys
// 0..p into nsplit near-equal ranges.  Each wave keeps a running max m, running sum l and an
// accumulator (online softmax) over 64-key blocks: lane j scores key j of the block, the wave
// reduces max and sum, and every lane then accumulates its own output dimensions over the
// block's keys.  The merge combines the splits with weights exp(m_s - max m).

#include <hip/hip_runtime.h>

#include <cmath>

#include "dtype.h"
#include "internal.h"

namespace ca {
namespace {

constexpr int kWave = 64;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// partial layout: [row][q head][split][d + 2] with (acc[0..d), m, l)
template <typename T>
__global__ void __launch_bounds__(kWave) attn_generic_kernel(
    DevPlan p, const T* __restrict__ q, const T* __restrict__ k_cache,
    const T* __restrict__ v_cache, int hq, int hkv, int d, float scale, int nsplit, int row0,
    float* __restrict__ partial) {
    __shared__ float s_q[128];
    __shared__ float s_w[kWave];
    if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x == 0) report_done(p);

    const int t = row0 + blockIdx.x;
    const int h = blockIdx.y;
    const int split = blockIdx.z;
    const int lane = threadIdx.x;
    const int P = p.page_size;
    const int g = h / (hq / hkv);

    const int s = p.row_seq[t];
    const int page0 = p.kv_page_indptr[s];
    const int np = p.kv_page_indptr[s + 1] - page0;
    const int kv_len = (np - 1) * P + p.kv_last_page_len[s];
    const int q_len = p.qo_indptr[s + 1] - p.qo_indptr[s];
    const int pos = kv_len - q_len + (t - p.qo_indptr[s]);
    const int n_keys = pos + 1;
    const int per = (n_keys + nsplit - 1) / nsplit;
    const int k0 = min(split * per, n_keys);
    const int k1 = min(k0 + per, n_keys);

    for (int e = lane; e < d; e += kWave)
        s_q[e] = Storage<T>::load(q + (static_cast<int64_t>(t) * hq + h) * d + e);
    __syncthreads();

    float m = -INFINITY, l = 0.0f;
    float acc0 = 0.0f, acc1 = 0.0f;  // dims lane and lane + 64
    for (int kb = k0; kb < k1; kb += kWave) {
        const int j = kb + lane;
        float sc = -INFINITY;
        if (j < k1) {
            const int page = p.kv_page_indices[page0 + j / P];
            const int64_t run = (static_cast<int64_t>(page) * hkv + g) * P * d;
            const T* kr = k_cache + run + (j % P) * 8;  // slot's run in 8-dim block 0
            float dot = 0.0f;
            for (int e = 0; e < d; ++e) dot += s_q[e] * Storage<T>::load(kr + (e >> 3) * P * 8 + (e & 7));
            sc = dot * scale;
        }
        const float mb = wave_max(sc);
        const float m_new = fmaxf(m, mb);
        const float w = (j < k1) ? expf(sc - m_new) : 0.0f;
        const float alpha = (m == -INFINITY) ? 0.0f : expf(m - m_new);
        l = l * alpha + wave_sum(w);
        acc0 *= alpha;
        acc1 *= alpha;
        m = m_new;
        s_w[lane] = w;
        __syncthreads();
        const int nb = min(kWave, k1 - kb);
        for (int jj = 0; jj < nb; ++jj) {
            const int key = kb + jj;
            const int page = p.kv_page_indices[page0 + key / P];
            const int slot = key % P;
            const T* vr = v_cache + (static_cast<int64_t>(page) * hkv + g) * d * P + (slot >> 2) * 64 + (slot & 3);
            const float wj = s_w[jj];
            // dim e of the slot: 16-dim block e / 16 (P * 16 elements each), then (e % 16) * 4
            const int e0 = lane, e1 = lane + kWave;
            if (e0 < d) acc0 += wj * Storage<T>::load(vr + (e0 >> 4) * P * 16 + (e0 & 15) * 4);
            if (e1 < d) acc1 += wj * Storage<T>::load(vr + (e1 >> 4) * P * 16 + (e1 & 15) * 4);
        }
        __syncthreads();
    }

    float* out = partial + ((static_cast<int64_t>(t) * hq + h) * nsplit + split) * (d + 2);
    if (lane < d) out[lane] = acc0;
    if (lane + kWave < d) out[lane + kWave] = acc1;
    if (lane == 0) {
        out[d] = m;
        out[d + 1] = l;
    }
}

template <typename T>
__global__ void __launch_bounds__(128) merge_kernel(const float* __restrict__ partial, int hq,
                                                    int d, int nsplit, int row0, T* __restrict__ o,
                                                    float* __restrict__ lse) {
    const int t = row0 + blockIdx.x;
    const int h = blockIdx.y;
    const int e = threadIdx.x;
    const float* base = partial + (static_cast<int64_t>(t) * hq + h) * nsplit * (d + 2);
    float mx = -INFINITY;
    for (int sp = 0; sp < nsplit; ++sp) {
        const float* ps = base + sp * (d + 2);
        if (ps[d + 1] > 0.0f) mx = fmaxf(mx, ps[d]);
    }
    float L = 0.0f, acc = 0.0f;
    for (int sp = 0; sp < nsplit; ++sp) {
        const float* ps = base + sp * (d + 2);
        if (ps[d + 1] > 0.0f) {
            const float wgt = expf(ps[d] - mx);
            L += wgt * ps[d + 1];
            if (e < d) acc += wgt * ps[e];
        }
    }
    if (e < d) Storage<T>::store(o + (static_cast<int64_t>(t) * hq + h) * d + e, acc / L);
    if (lse && e == 0) lse[static_cast<int64_t>(t) * hq + h] = mx + logf(L);
}

}  // namespace

size_t generic_partial_floats(int32_t num_tokens, const Shape& sh, int nsplit) {
    return static_cast<size_t>(num_tokens) * sh.hq * nsplit * (sh.d + 2);
}

hipError_t launch_attention_generic(const DevPlan& p, const Shape& sh, int row0, const void* q,
                                    const void* k_cache, const void* v_cache, void* o,
                                    float* lse, float* partial, int nsplit,
                                    hipStream_t stream, const LaunchEvents& ev) {
    if (p.num_tokens - row0 <= 0) return hipSuccess;
    dim3 grid(p.num_tokens - row0, sh.hq, nsplit);
    dim3 mgrid(p.num_tokens - row0, sh.hq);
    if (sh.dtype == CA_FP32) {
        hipExtLaunchKernelGGL(attn_generic_kernel<float>, grid, dim3(kWave), 0, stream, ev.start, nullptr, 0, p,
                           static_cast<const float*>(q), static_cast<const float*>(k_cache),
                           static_cast<const float*>(v_cache), sh.hq, sh.hkv, sh.d, sh.scale,
                           nsplit, row0, partial);
        hipExtLaunchKernelGGL(merge_kernel<float>, mgrid, dim3(sh.d), 0, stream, nullptr, ev.stop, 0, partial, sh.hq, sh.d,
                           nsplit, row0, static_cast<float*>(o), lse);
    } else {
        hipExtLaunchKernelGGL(attn_generic_kernel<uint16_t>, grid, dim3(kWave), 0, stream, ev.start, nullptr, 0, p,
                           static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_cache),
                           static_cast<const uint16_t*>(v_cache), sh.hq, sh.hkv, sh.d, sh.scale,
                           nsplit, row0, partial);
        hipExtLaunchKernelGGL(merge_kernel<uint16_t>, mgrid, dim3(sh.d), 0, stream, nullptr, ev.stop, 0, partial, sh.hq,
                           sh.d, nsplit, row0, static_cast<uint16_t*>(o), lse);
    }
    return hipGetLastError();
}

}  // namespace ca

// append_rope.hip -- rotary embedding at absolute positions, then append K/V into the pages.
//
// pinghaoyang.com.cn "Sarathi-Serve 完全拆解", section "分块不等于截断上下文": each new token
// carries its absolute position (positions are never restarted per chunk) and its K/V goes into
// the paged cache, in its request's logical page p / P, slot p % P, before attention reads it.
//
// One workgroup per token.  The pair angles p * theta^(-2i/d) are formed in fp64 once per token
// (d/2 of them, shared by every head) and kept in LDS; each rotated element is computed in fp64
// and rounded once to the storage type.  Work per token is tiny and the kernel is bound by the
// bytes it moves (read q, k, v; write q', the K row and the V column of one slot).

#include <hip/hip_runtime.h>

#include "dtype.h"
#include "internal.h"

namespace ca {
namespace {

template <typename T>
__global__ void __launch_bounds__(256) append_rope_kernel(
    DevPlan p, const T* q_in, T* q_out, const T* __restrict__ k_new,
    const T* __restrict__ v_new, T* __restrict__ k_cache, T* __restrict__ v_cache, int hq, int hkv,
    int d, double theta) {
#pragma clang fp contract(off)
    __shared__ double s_cos[64];
    __shared__ double s_sin[64];
    const int t = blockIdx.x;
    const int P = p.page_size;
    const int s = p.row_seq[t];
    const int np = p.kv_page_indptr[s + 1] - p.kv_page_indptr[s];
    const int kv_len = (np - 1) * P + p.kv_last_page_len[s];
    const int q_len = p.qo_indptr[s + 1] - p.qo_indptr[s];
    const int pos = kv_len - q_len + (t - p.qo_indptr[s]);
    const int page = p.kv_page_indices[p.kv_page_indptr[s] + pos / P];
    const int slot = pos % P;
    const int half = d >> 1;

    for (int i = threadIdx.x; i < half; i += blockDim.x) {
        const double inv_freq = pow(theta, -2.0 * static_cast<double>(i) / static_cast<double>(d));
        const double angle = static_cast<double>(pos) * inv_freq;
        double sn, cs;
        sincos(angle, &sn, &cs);
        s_cos[i] = cs;
        s_sin[i] = sn;
    }
    __syncthreads();

    // Rotate every (head, pair) of q and k.  Each thread reads both members of its pair before
    // writing them, so q_out may alias q_in.
    const int pairs = (hq + hkv) * half;
    for (int idx = threadIdx.x; idx < pairs; idx += blockDim.x) {
        const int h = idx / half;
        const int i = idx - h * half;
        const T* src;
        T* dst;
        if (h < hq) {
            src = q_in + (static_cast<int64_t>(t) * hq + h) * d;
            dst = q_out + (static_cast<int64_t>(t) * hq + h) * d;
        } else {
            const int g = h - hq;
            src = k_new + (static_cast<int64_t>(t) * hkv + g) * d;
            dst = k_cache + ((static_cast<int64_t>(page) * hkv + g) * P + slot) * d;
        }
        const double a = static_cast<double>(Storage<T>::load(src + i));
        const double b = static_cast<double>(Storage<T>::load(src + i + half));
        const double c = s_cos[i], sn = s_sin[i];
        Storage<T>::store_from_double(dst + i, a * c - b * sn);
        Storage<T>::store_from_double(dst + i + half, b * c + a * sn);
    }

    // V is copied unrotated into the dimension-major page: element e of slot goes to [e][slot].
    const int vn = hkv * d;
    for (int idx = threadIdx.x; idx < vn; idx += blockDim.x) {
        const int g = idx / d;
        const int e = idx - g * d;
        v_cache[((static_cast<int64_t>(page) * hkv + g) * d + e) * P + slot] =
            v_new[(static_cast<int64_t>(t) * hkv + g) * d + e];
    }
}

}  // namespace

hipError_t launch_append_rope(const DevPlan& p, const Shape& sh, const void* q_in, void* q_out,
                              const void* k_new, const void* v_new, void* k_cache,
                              void* v_cache, hipStream_t stream) {
    if (p.num_tokens <= 0) return hipSuccess;
    dim3 grid(p.num_tokens), block(256);
    if (sh.dtype == CA_FP32) {
        hipLaunchKernelGGL(append_rope_kernel<float>, grid, block, 0, stream, p,
                           static_cast<const float*>(q_in), static_cast<float*>(q_out),
                           static_cast<const float*>(k_new), static_cast<const float*>(v_new),
                           static_cast<float*>(k_cache), static_cast<float*>(v_cache), sh.hq,
                           sh.hkv, sh.d, sh.theta);
    } else {
        hipLaunchKernelGGL(append_rope_kernel<uint16_t>, grid, block, 0, stream, p,
                           static_cast<const uint16_t*>(q_in), static_cast<uint16_t*>(q_out),
                           static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
                           static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache),
                           sh.hq, sh.hkv, sh.d, sh.theta);
    }
    return hipGetLastError();
}

}  // namespace ca

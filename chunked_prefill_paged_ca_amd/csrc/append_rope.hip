// append_rope.hip -- rotary embedding at absolute positions, then append K/V into the pages.
//
// pinghaoyang.com.cn "Sarathi-Serve 完全拆解", section "分块不等于截断上下文": each new token
// carries its absolute position (positions are never restarted per chunk) and its K/V goes into
// the paged cache, in its request's logical page p / P, slot p % P, before attention reads it.
//
// One workgroup per token.  The work per token is a few KB, so the kernel is bound by latency,
// and it is laid out to pay one memory round trip, not a chain of them:
//   * the token's position and destination page come from per-row arrays the host fills with
//     the plan (no sequence -> indptr -> page-id chain), and the inverse frequencies
//     theta^(-2i/d) are a host-computed fp64 table;
//   * when the step's metadata has not reached device memory yet, extra workgroups after the
//     token workgroups copy it there from the pinned host staging (for the attention launch that
//     follows in stream order), and the token workgroups read their two per-row values straight
//     from that staging: the copy overlaps the append instead of running before it;
//   * every q/k/v load is a 16-byte vector load, all issued before the first store (a thread
//     writes back exactly the elements it read, so q_out may alias q_in), and unconditional so
//     that they are in flight together; q, k and v rows are read with their own row strides, so
//     they may be the column ranges of one packed projection output;
//   * the d/2 pair angles are formed in fp64 once per token, shared through LDS, and each
//     rotated element is computed in fp64 and rounded once to the storage type.

#include <hip/hip_runtime.h>

#include "dtype.h"
#include "internal.h"

namespace ca {
namespace {

constexpr int kThreads = 256;
constexpr int kUnits = 4;  // q/k vector units per thread per pass

template <typename T>
struct Vec {
    static constexpr int N = 16 / sizeof(T);
    T e[N];
};

template <typename T>
__device__ __forceinline__ Vec<T> load16(const T* p) {
    const uint4 raw = *reinterpret_cast<const uint4*>(p);
    Vec<T> v;
    __builtin_memcpy(&v, &raw, sizeof(v));
    return v;
}

template <typename T>
__device__ __forceinline__ void store16(T* p, const Vec<T>& v) {
    uint4 raw;
    __builtin_memcpy(&raw, &v, sizeof(raw));
    *reinterpret_cast<uint4*>(p) = raw;
}

template <typename T>
__device__ __forceinline__ double widen(T x);
template <>
__device__ __forceinline__ double widen<float>(float x) { return static_cast<double>(x); }
template <>
__device__ __forceinline__ double widen<uint16_t>(uint16_t x) { return static_cast<double>(bf16_bits_to_float(x)); }

template <typename T>
__device__ __forceinline__ T narrow(double x);
template <>
__device__ __forceinline__ float narrow<float>(double x) { return static_cast<float>(x); }
template <>
__device__ __forceinline__ uint16_t narrow<uint16_t>(double x) { return double_to_bf16_bits(x); }

// Workgroups [num_tokens, gridDim.x) copy meta_n16 16-byte units from meta_src to meta_dst.
template <typename T>
__global__ void __launch_bounds__(kThreads) append_rope_kernel(
    const int32_t* __restrict__ row_pos, const int32_t* __restrict__ row_page,
    const double* __restrict__ inv_freq, const T* q_in, T* q_out, const T* __restrict__ k_new,
    const T* __restrict__ v_new, T* __restrict__ k_cache, T* __restrict__ v_cache, int hq,
    int hkv, int d, int P, int64_t q_row, int64_t kv_row, int num_tokens,
    const uint4* __restrict__ meta_src, uint4* __restrict__ meta_dst, int64_t meta_n16) {
#pragma clang fp contract(off)
    constexpr int N = Vec<T>::N;
    __shared__ double s_cos[64];
    __shared__ double s_sin[64];
    const int t = blockIdx.x;
    const int tid = threadIdx.x;
    if (t >= num_tokens) {  // metadata copy workgroup (uniform branch)
        const int64_t stride = static_cast<int64_t>(gridDim.x - num_tokens) * kThreads;
        for (int64_t i = static_cast<int64_t>(t - num_tokens) * kThreads + tid; i < meta_n16; i += stride)
            meta_dst[i] = meta_src[i];
        return;
    }
    const int half = d >> 1;
    const int per_head = half / N;  // vector units per head (each covers N pairs)
    const int units = (hq + hkv) * per_head;
    const int v_units = hkv * d / N;
    const int pos = row_pos[t];
    const int page = row_page[t];
    const int slot = pos % P;

    // Loads are unconditional (indices clamped into range; only the stores are predicated), so
    // they are all in flight together instead of each waiting at the end of its own branch.
    // The frequency load is issued first: waiting for it does not wait for the q/k/v loads.
    const double freq = inv_freq[tid < half ? tid : half - 1];
    Vec<T> vv = load16(v_new + t * kv_row + (tid < v_units ? tid : v_units - 1) * N);

    Vec<T> a[kUnits], b[kUnits];
    int i0[kUnits];
    auto load_pass = [&](int base) {
#pragma unroll
        for (int j = 0; j < kUnits; ++j) {
            const int u0 = base + tid + j * kThreads;
            const int u = u0 < units ? u0 : units - 1;
            const int h = u / per_head;
            i0[j] = (u - h * per_head) * N;
            const T* src = h < hq ? q_in + t * q_row + static_cast<int64_t>(h) * d
                                  : k_new + t * kv_row + static_cast<int64_t>(h - hq) * d;
            a[j] = load16(src + i0[j]);
            b[j] = load16(src + i0[j] + half);
        }
    };
    auto rotate_pass = [&](int base) {
#pragma unroll
        for (int j = 0; j < kUnits; ++j) {
            const int u = base + tid + j * kThreads;
            // skip a unit slot no lane of this wave uses (wave-uniform test)
            if (__builtin_amdgcn_readfirstlane(base + j * kThreads + (tid & ~63)) >= units) continue;
            Vec<T> ra, rb;
#pragma unroll
            for (int e = 0; e < N; ++e) {
                const double x = widen<T>(a[j].e[e]), y = widen<T>(b[j].e[e]);
                const double c = s_cos[i0[j] + e], s = s_sin[i0[j] + e];
                ra.e[e] = narrow<T>(x * c - y * s);
                rb.e[e] = narrow<T>(y * c + x * s);
            }
            if (u < units) {
                const int h = u / per_head;
                if (h < hq) {
                    T* dst = q_out + (static_cast<int64_t>(t) * hq + h) * d;
                    store16(dst + i0[j], ra);
                    store16(dst + i0[j] + half, rb);
                } else {
                    // K page: the slot's 8-dim runs, one per 8-dim block (a vector unit never
                    // straddles two blocks: it starts at a multiple of its length, which divides 8)
                    T* dst = k_cache + (static_cast<int64_t>(page) * hkv + (h - hq)) * P * d;
                    const int e0 = i0[j], e1 = i0[j] + half;
                    store16(dst + ((e0 >> 3) * P + slot) * 8 + (e0 & 7), ra);
                    store16(dst + ((e1 >> 3) * P + slot) * 8 + (e1 & 7), rb);
                }
            }
        }
    };

    load_pass(0);
    if (tid < half) {
        double sn, cs;
        sincos(static_cast<double>(pos) * freq, &sn, &cs);
        s_cos[tid] = cs;
        s_sin[tid] = sn;
    }
    __syncthreads();
    rotate_pass(0);
    for (int base = kThreads * kUnits; base < units; base += kThreads * kUnits) {
        load_pass(base);
        rotate_pass(base);
    }

    // V goes unrotated into its page: dim e of the slot lands in the run of 16-dim block e / 16
    // and 4-slot group slot / 4, at (e % 16) * 4 + slot % 4 (a vector unit stays in one block)
    for (int vu = tid; vu < v_units; vu += kThreads) {
        if (vu != tid) vv = load16(v_new + t * kv_row + vu * N);
        const int g = (vu * N) / d;
        const int e0 = vu * N - g * d;
        T* vp = v_cache + (static_cast<int64_t>(page) * hkv + g) * P * d +
                (((e0 >> 4) * (P >> 2) + (slot >> 2)) * 16 + (e0 & 15)) * 4 + (slot & 3);
#pragma unroll
        for (int e = 0; e < N; ++e) vp[4 * e] = vv.e[e];
    }
}

}  // namespace

hipError_t launch_append_rope(const DevPlan& p, const Shape& sh, const int32_t* row_pos,
                              const int32_t* row_page, const double* inv_freq, const void* q_in,
                              void* q_out, const void* k_new, const void* v_new, void* k_cache,
                              void* v_cache, int64_t q_row, int64_t kv_row, const void* meta_src,
                              void* meta_dst, int64_t meta_n16, hipStream_t stream,
                              const LaunchEvents& ev) {
    if (p.num_tokens <= 0) return hipSuccess;
    // one 16-byte unit per copy thread: the staging is read over PCIe, where many small reads in
    // flight at once are what keeps the copy short
    const int64_t copy_wgs64 = meta_n16 > 0 ? (meta_n16 + kThreads - 1) / kThreads : 0;
    const int copy_wgs = static_cast<int>(copy_wgs64 < 256 ? copy_wgs64 : 256);
    const dim3 grid(p.num_tokens + copy_wgs), block(kThreads);
    const uint4* msrc = static_cast<const uint4*>(meta_src);
    uint4* mdst = static_cast<uint4*>(meta_dst);
    if (sh.dtype == CA_FP32) {
        hipExtLaunchKernelGGL(append_rope_kernel<float>, grid, block, 0, stream, ev.start, ev.stop, 0, row_pos, row_page,
                           inv_freq, static_cast<const float*>(q_in), static_cast<float*>(q_out),
                           static_cast<const float*>(k_new), static_cast<const float*>(v_new),
                           static_cast<float*>(k_cache), static_cast<float*>(v_cache), sh.hq,
                           sh.hkv, sh.d, p.page_size, q_row, kv_row, p.num_tokens, msrc, mdst, meta_n16);
    } else {
        hipExtLaunchKernelGGL(append_rope_kernel<uint16_t>, grid, block, 0, stream, ev.start, ev.stop, 0, row_pos,
                           row_page, inv_freq, static_cast<const uint16_t*>(q_in),
                           static_cast<uint16_t*>(q_out), static_cast<const uint16_t*>(k_new),
                           static_cast<const uint16_t*>(v_new), static_cast<uint16_t*>(k_cache),
                           static_cast<uint16_t*>(v_cache), sh.hq, sh.hkv, sh.d, p.page_size, q_row,
                           kv_row, p.num_tokens, msrc, mdst, meta_n16);
    }
    return hipGetLastError();
}

}  // namespace ca

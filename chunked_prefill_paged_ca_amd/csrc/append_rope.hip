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
//   * the workgroup is sized to the token (one q/k rotation unit of N pairs per thread, 64 to
//     1024 threads), so every load is needed and all of them -- q/k as 16-byte vectors, V one
//     element per thread -- are issued before the first store (a thread writes back exactly
//     the elements it read, so q_out may alias q_in); q, k and v rows are read with their own
//     row strides, so they may be the column ranges of one packed projection output;
//   * V is stored as soon as it and the page id are in, before the angles are formed: one
//     element per thread, adjacent threads on adjacent dimensions, so that the 16 dimensions of
//     a V run (stride 4 in the 4-slot layout) go out as one partial write of one cache line,
//     not as 16 writes from 2 threads;
//   * the d/2 pair angles are formed in fp64 once per token, shared through LDS, and each
//     rotated element is computed in fp64 and rounded once to the storage type.

#include <hip/hip_runtime.h>

#include <type_traits>

#include "dtype.h"
#include "internal.h"

namespace ca {
namespace {


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

// NT: every store of the launch carries the non-temporal hint (nothing here reads what it
// wrote; the attention launch that follows reads it once).  That pays off for small appends and
// costs for large ones (launch_append_rope chooses; measured there).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <bool NT, typename T>
__device__ __forceinline__ void store16(T* p, const Vec<T>& v) {
    u32x4 raw;
    __builtin_memcpy(&raw, &v, sizeof(raw));
    if constexpr (NT) __builtin_nontemporal_store(raw, reinterpret_cast<u32x4*>(p));
    else *reinterpret_cast<u32x4*>(p) = raw;
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
// blockDim.x: a multiple of 64 in [64, 1024], at least D / 2 (the threads that form the angles).
// U: rotation units per thread in the first pass; each thread also loads U * 4 V elements
// before its first store.
template <typename T, int D, int U, bool NT>
__global__ void __launch_bounds__(1024) append_rope_kernel(
    const int32_t* __restrict__ row_pos, const int32_t* __restrict__ row_page,
    const double* __restrict__ inv_freq, const T* q_in, T* q_out, const T* __restrict__ k_new,
    const T* __restrict__ v_new, T* __restrict__ k_cache, T* __restrict__ v_cache, int hq,
    int hkv, int P, int64_t q_row, int64_t kv_row, int num_tokens,
    const uint4* __restrict__ meta_src, uint4* __restrict__ meta_dst, int64_t meta_n16) {
#pragma clang fp contract(off)
    constexpr int N = Vec<T>::N;
    constexpr int half = D / 2;
    constexpr int per_head = half / N;  // rotation units per head (each covers N pairs)
    constexpr int kV = 4 * U;           // V elements per thread in the first pass
    __shared__ double s_cos[half];
    __shared__ double s_sin[half];
    const int t = blockIdx.x;
    const int tid = threadIdx.x;
    const int nt = blockDim.x;
    // The position and page are read first, before anything else is set up: they come over PCIe
    // when the same launch copies the metadata, and every later step waits for them.  (A copy
    // workgroup reads row 0's, which exists: the launch has at least one token.)
    const int row = t < num_tokens ? t : 0;
    const int pos = row_pos[row];
    const int page = row_page[row];
    if (t >= num_tokens) {  // metadata copy workgroup (uniform branch)
        const int64_t stride = static_cast<int64_t>(gridDim.x - num_tokens) * nt;
        for (int64_t i = static_cast<int64_t>(t - num_tokens) * nt + tid; i < meta_n16; i += stride)
            meta_dst[i] = meta_src[i];
        return;
    }
    const int units = (hq + hkv) * per_head;
    const int vdims = hkv * D;

    // Every load of the first pass is issued before any value is used; indices past the end are
    // clamped into range (the loads stay unconditional, so they are in flight together) and only
    // the stores are predicated.  The frequency load goes first: waiting for it does not wait
    // for the q/k/v loads.
    const double freq = inv_freq[tid < half ? tid : half - 1];
    const T* vrow = v_new + t * kv_row;
    T vv[kV];
#pragma unroll
    for (int j = 0; j < kV; ++j) {
        const int e = tid + j * nt;
        vv[j] = vrow[e < vdims ? e : vdims - 1];
    }
    auto unit_src = [&](int u, int& h, int& i0) {
        h = u / per_head;
        i0 = (u - h * per_head) * N;
        return h < hq ? q_in + t * q_row + static_cast<int64_t>(h) * D
                      : k_new + t * kv_row + static_cast<int64_t>(h - hq) * D;
    };
    int hh[U], ii[U];
    Vec<T> a[U], b[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
        const int u = tid + j * nt;
        const T* src = unit_src(u < units ? u : units - 1, hh[j], ii[j]);
        a[j] = load16(src + ii[j]);
        b[j] = load16(src + ii[j] + half);
    }
    const int slot = pos % P;

    // V goes unrotated into its page: dim c of the slot lands in the run of 16-dim block c / 16
    // and 4-slot group slot / 4, at (c % 16) * 4 + slot % 4
    T* vpage = v_cache + static_cast<int64_t>(page) * hkv * P * D;
    auto v_store = [&](int e, T val) {
        const int g = e / D, c = e - g * D;
        T* dst = &vpage[static_cast<int64_t>(g) * P * D + (((c >> 4) * (P >> 2) + (slot >> 2)) * 16 + (c & 15)) * 4 +
                        (slot & 3)];
        if constexpr (NT) __builtin_nontemporal_store(val, dst);
        else *dst = val;
    };
#pragma unroll
    for (int j = 0; j < kV; ++j) {
        const int e = tid + j * nt;
        if (e < vdims) v_store(e, vv[j]);
    }
    for (int e = tid + kV * nt; e < vdims; e += nt) v_store(e, vrow[e]);

    if (tid < half) {
        double sn, cs;
        sincos(static_cast<double>(pos) * freq, &sn, &cs);
        s_cos[tid] = cs;
        s_sin[tid] = sn;
    }
    __syncthreads();

    auto rotate_store = [&](int u, int h, int i0, const Vec<T>& x, const Vec<T>& y) {
        Vec<T> rx, ry;
#pragma unroll
        for (int e = 0; e < N; ++e) {
            const double xe = widen<T>(x.e[e]), ye = widen<T>(y.e[e]);
            const double c = s_cos[i0 + e], s = s_sin[i0 + e];
            rx.e[e] = narrow<T>(xe * c - ye * s);
            ry.e[e] = narrow<T>(ye * c + xe * s);
        }
        if (u >= units) return;
        if (h < hq) {
            T* dst = q_out + (static_cast<int64_t>(t) * hq + h) * D;
            store16<NT>(dst + i0, rx);
            store16<NT>(dst + i0 + half, ry);
        } else {
            // K page: the slot's 8-dim runs, one per 8-dim block (a vector unit never straddles
            // two blocks: it starts at a multiple of its length, which divides 8)
            T* dst = k_cache + (static_cast<int64_t>(page) * hkv + (h - hq)) * P * D;
            const int e0 = i0, e1 = i0 + half;
            store16<NT>(dst + ((e0 >> 3) * P + slot) * 8 + (e0 & 7), rx);
            store16<NT>(dst + ((e1 >> 3) * P + slot) * 8 + (e1 & 7), ry);
        }
    };
    // a wave whose lanes all lie past the last unit skips the math (wave-uniform test)
    const int wave0 = __builtin_amdgcn_readfirstlane(tid & ~63);
#pragma unroll
    for (int j = 0; j < U; ++j)
        if (wave0 + j * nt < units) rotate_store(tid + j * nt, hh[j], ii[j], a[j], b[j]);
    for (int u0 = U * nt; u0 + wave0 < units; u0 += nt) {
        const int u = u0 + tid;
        int h, i0;
        const T* src = unit_src(u < units ? u : units - 1, h, i0);
        const Vec<T> x = load16(src + i0), y = load16(src + i0 + half);
        rotate_store(u, h, i0, x, y);
    }
}

// Threads per token workgroup for U rotation units per thread: enough that the first pass
// holds every rotation unit and (4 U per thread) every V element, and at least the D / 2 angle
// threads.
int append_threads(const Shape& sh, int U) {
    const int n = 16 / (sh.dtype == CA_FP32 ? 4 : 2);
    const int units = (sh.hq + sh.hkv) * (sh.d / 2 / n);
    const int vdims = sh.hkv * sh.d;
    int want = (units + U - 1) / U;
    const int vthreads = (vdims + 4 * U - 1) / (4 * U);
    want = want > vthreads ? want : vthreads;
    want = want > sh.d / 2 ? want : sh.d / 2;
    want = (want + 63) / 64 * 64;
    return want < 1024 ? want : 1024;
}

// Rotation units per thread: the smallest U in {1, 2} whose workgroups all fit on the CUs at once
// (32 resident waves per CU: 4 SIMDs x 8 waves, the kernel staying within 64 VGPRs for these),
// else 4.  One unit per thread keeps each thread's chain (loads -> angles -> rotation -> stores)
// shortest; when the token workgroups would not all be resident, fewer, longer-lived waves per
// token beat a second round of workgroups.
int append_units_per_thread(const Shape& sh, int64_t num_tokens, int num_cus) {
    for (int U = 1; U <= 2; U *= 2) {
        const int waves = append_threads(sh, U) / 64;
        if (num_tokens <= static_cast<int64_t>(num_cus) * (32 / waves)) return U;
    }
    return 4;
}

}  // namespace

hipError_t launch_append_rope(const DevPlan& p, const Shape& sh, const int32_t* row_pos,
                              const int32_t* row_page, const double* inv_freq, const void* q_in,
                              void* q_out, const void* k_new, const void* v_new, void* k_cache,
                              void* v_cache, int64_t q_row, int64_t kv_row, const void* meta_src,
                              void* meta_dst, int64_t meta_n16, int num_cus, hipStream_t stream,
                              const LaunchEvents& ev) {
    if (p.num_tokens <= 0) return hipSuccess;
    const int U = append_units_per_thread(sh, p.num_tokens, num_cus > 0 ? num_cus : 256);
    // Non-temporal stores while the step appends at most 16384 (token, kv head) pairs.  Measured
    // (same box, plain -> non-temporal): Mistral-7B step (4096 pairs) append 9.3 -> 9.2 us and
    // the attention launch after it 139.4 -> 136.0 us; LLaMA2-70B share (12288) append 23.8 ->
    // 27.2 us, attention 1024 -> 997 us; but a Llama-13B prompt (MHA, 40 kv heads) appended in
    // steps of 512 / 2048 / 8192 tokens (20480+ pairs) 15.6 -> 25 / 52 -> 105 / 191 -> 418 us per
    // step: the K and V slots of a token are 16-byte and 2-byte pieces of many cache lines, and
    // streamed past L2 such partial lines cost far more than merged ones.
    const bool nt = static_cast<int64_t>(p.num_tokens) * sh.hkv <= 16384;
    const int threads = append_threads(sh, U);
    // one 16-byte unit per copy thread: the staging is read over PCIe, where many small reads in
    // flight at once are what keeps the copy short
    const int64_t copy_wgs64 = meta_n16 > 0 ? (meta_n16 + threads - 1) / threads : 0;
    const int copy_wgs = static_cast<int>(copy_wgs64 < 256 ? copy_wgs64 : 256);
    const dim3 grid(p.num_tokens + copy_wgs), block(threads);
    const uint4* msrc = static_cast<const uint4*>(meta_src);
    uint4* mdst = static_cast<uint4*>(meta_dst);
    auto go = [&](auto tag, auto d_tag, auto u_tag, auto nt_tag) {
        using T = decltype(tag);
        constexpr int D = decltype(d_tag)::value, Uc = decltype(u_tag)::value;
        constexpr bool NTc = decltype(nt_tag)::value;
        hipExtLaunchKernelGGL(append_rope_kernel<T, D, Uc, NTc>, grid, block, 0, stream, ev.start, ev.stop, 0, row_pos,
                              row_page, inv_freq, static_cast<const T*>(q_in), static_cast<T*>(q_out),
                              static_cast<const T*>(k_new), static_cast<const T*>(v_new), static_cast<T*>(k_cache),
                              static_cast<T*>(v_cache), sh.hq, sh.hkv, p.page_size, q_row, kv_row, p.num_tokens,
                              msrc, mdst, meta_n16);
    };
    auto by_nt = [&](auto tag, auto d_tag, auto u_tag) {
        if (nt) go(tag, d_tag, u_tag, std::true_type{});
        else go(tag, d_tag, u_tag, std::false_type{});
    };
    auto by_u = [&](auto tag, auto d_tag) {
        if (U == 1) by_nt(tag, d_tag, std::integral_constant<int, 1>{});
        else if (U == 2) by_nt(tag, d_tag, std::integral_constant<int, 2>{});
        else by_nt(tag, d_tag, std::integral_constant<int, 4>{});
    };
    auto by_d = [&](auto tag) {
        if (sh.d == 128) by_u(tag, std::integral_constant<int, 128>{});
        else by_u(tag, std::integral_constant<int, 64>{});
    };
    if (sh.dtype == CA_FP32) by_d(0.0f);
    else by_d(uint16_t(0));
    return hipGetLastError();
}

}  // namespace ca

// mfma.h -- gfx950 bf16 MFMA fragments and wave helpers shared by the attention kernels.
//
// v_mfma_f32_16x16x32_bf16 (checked on the device): for lane l, with c = l % 16, q = l / 16,
//   A (16 x 32): row c, k = 8q .. 8q+7      B (32 x 16): column c, k = 8q .. 8q+7
//   C (16 x 16): column c, rows 4q .. 4q+3
// The kernels compute S^T = K Q^T (A = 16 keys x 32 dims, B = Q^T) and O^T = V^T P^T
// (A = 16 dims x 32 keys, B = P^T).  In both products the lane's C column is one query column,
// so the running max / sum of a query column never leaves its lane group.
//
// Key order inside a 32-key block (two pages a, b): S^T tile t is page t, its row r is slot r.
// Lane group q then holds the scores of slots 4q .. 4q+3 of page a (tile 0) and of page b
// (tile 1), and those eight keys, in that order, are the k range 8q .. 8q+7 of its P^T fragment
// in O^T = V^T P^T; the V^T fragment takes the same keys.  With the page layouts of the caches
// (8-dim blocks of 16 slots for K, 4-slot groups of 16 dims for V) every fragment a wavefront
// loads from a page is one contiguous run: lane l reads 16 bytes at 16 l for K, and 8 bytes at
// 8 l from each of the two pages for V.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace ca {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ floatx4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const floatx4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 16-byte global load of 8 bf16 as an MFMA fragment.
__device__ __forceinline__ bf16x8 load_frag(const uint16_t* p) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    bf16x8 r;
    __builtin_memcpy(&r, &v, sizeof(r));
    return r;
}

__device__ __forceinline__ bf16x8 zero_frag() {
    const uint4 v = make_uint4(0, 0, 0, 0);
    bf16x8 r;
    __builtin_memcpy(&r, &v, sizeof(r));
    return r;
}

// Two 8-byte loads (4 bf16 each: the lane's keys of page a, then of page b) as one fragment.
__device__ __forceinline__ bf16x8 load_frag_pair(const uint16_t* a, const uint16_t* b) {
    const uint2 x = *reinterpret_cast<const uint2*>(a);
    const uint2 y = *reinterpret_cast<const uint2*>(b);
    const uint4 v = make_uint4(x.x, x.y, y.x, y.y);
    bf16x8 r;
    __builtin_memcpy(&r, &v, sizeof(r));
    return r;
}

// The same loads with the non-temporal hint, for data read exactly once (the decode rows' K/V
// stream): measured on the part, a plain read stream runs ~10 % faster with it (6.1 -> 6.7 TB/s
// over 800 MiB), since the lines it brings in are not kept in the caches.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x8 load_frag_nt(const uint16_t* p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    bf16x8 r;
    __builtin_memcpy(&r, &v, sizeof(r));
    return r;
}

__device__ __forceinline__ bf16x8 load_frag_pair_nt(const uint16_t* a, const uint16_t* b) {
    const u32x2 x = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(a));
    const u32x2 y = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(b));
    const u32x4 v = {x.x, x.y, y.x, y.y};
    bf16x8 r;
    __builtin_memcpy(&r, &v, sizeof(r));
    return r;
}

// Zero fragment elements by key: element j < 4 is kept when j < va, element 4 + j when j < vb
// (va, vb: keys of the lane's page-a and page-b runs that are inside the range).
__device__ __forceinline__ bf16x8 mask_frag(bf16x8 f, int va, int vb) {
    uint4 v;
    __builtin_memcpy(&v, &f, sizeof(v));
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int n = i < 2 ? va : vb;
        const int j = 2 * (i & 1);
        const uint32_t keep = (j < n ? 0x0000ffffu : 0u) | (j + 1 < n ? 0xffff0000u : 0u);
        w[i] &= keep;
    }
    v = make_uint4(w[0], w[1], w[2], w[3]);
    __builtin_memcpy(&f, &v, sizeof(f));
    return f;
}

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f2bf(float f) {
    const __bf16 b = static_cast<__bf16>(f);
    uint16_t u;
    __builtin_memcpy(&u, &b, sizeof(u));
    return u;
}

__device__ __forceinline__ bf16x8 pack_frag(const float* x) {
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = static_cast<__bf16>(x[i]);
    return r;
}

// Lazy rescaling threshold of the online softmax, in log2 units: the running reference max of a
// query column only moves when a block's max exceeds it by more than this, so p = 2^(s - m)
// stays below 2^8 (exact enough in bf16, far from fp32 overflow) and the accumulator rescale
// is skipped for almost every block after the first.
constexpr float kRescaleSlack = 8.0f;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Max / sum over the four 16-lane rows of a wave for each column c = lane % 16; every lane gets
// the result of lanes c, c + 16, c + 32, c + 48.  v_permlane16_swap exchanges rows 1 <-> 0 and
// 3 <-> 2 of two copies, v_permlane32_swap rows {2, 3} <-> {0, 1} (checked on the device), so
// max/sum of the two swapped copies reduces over row pairs, then over halves.  They are VALU
// instructions: unlike ds_bpermute they leave the LDS/scalar-load counter alone, so a reduction
// does not wait for page-id scalar loads still in flight.
__device__ __forceinline__ float rows_max(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float rows_sum(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

}  // namespace ca

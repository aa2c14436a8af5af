// dtype.h -- storage-type conversions used by the kernels (device side).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace ca {

// bf16 is kept as its raw 16-bit pattern; widening to fp32 is exact (append 16 zero bits).
__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest, ties to even (NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// fp64 -> bf16 in one rounding (nearest, ties to even).  x is first rounded to fp32 with
// round-to-odd (truncate, then set the last bit if anything was cut off), then the hardware
// fp32 -> bf16 conversion rounds to nearest even.  Because fp32 keeps more than two extra bits
// beyond bf16's 8, the second rounding gives exactly the nearest-even bf16 of x (the
// round-to-odd double-rounding property: Boldo and Melquiond, "Emulation of FMA and correctly
// rounded sums: proved algorithms using rounding to odd", IEEE Trans. Computers 2008).
// Truncation is derived from the nearest-even conversion: if it moved away from zero, step one
// fp32 ulp back toward zero.  NaN stays NaN, overflow goes to infinity.
__device__ __forceinline__ uint16_t double_to_bf16_bits(double x) {
    const float f = static_cast<float>(x);
    const double back = static_cast<double>(f);
    uint32_t u = __float_as_uint(f);
    u -= __builtin_fabs(back) > __builtin_fabs(x) ? 1u : 0u;  // toward zero: truncation
    u |= back != x ? 1u : 0u;                                 // sticky bit: round to odd
    const __bf16 b = static_cast<__bf16>(__uint_as_float(u));
    uint16_t r;
    __builtin_memcpy(&r, &b, sizeof(r));
    return r;
}

template <typename T> struct Storage;

template <> struct Storage<float> {
    __device__ __forceinline__ static float load(const float* p) { return *p; }
    __device__ __forceinline__ static void store(float* p, float v) { *p = v; }
    __device__ __forceinline__ static void store_from_double(float* p, double v) { *p = static_cast<float>(v); }
};

template <> struct Storage<uint16_t> {
    __device__ __forceinline__ static float load(const uint16_t* p) { return bf16_bits_to_float(*p); }
    __device__ __forceinline__ static void store(uint16_t* p, float v) { *p = float_to_bf16_bits(v); }
    __device__ __forceinline__ static void store_from_double(uint16_t* p, double v) { *p = double_to_bf16_bits(v); }
};

}  // namespace ca

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

// fp64 -> bf16 in one rounding (nearest, ties to even), without passing through fp32.
// The top 18 bits of the fp64 magnitude (11 exponent + 7 fraction) are kept and the remaining
// 45 fraction bits decide the rounding; a carry into the exponent is handled by the integer add.
// Results below the bf16 normal range take the subnormal spacing 2^-133.
__device__ __forceinline__ uint16_t double_to_bf16_bits(double x) {
    const uint64_t u = static_cast<uint64_t>(__double_as_longlong(x));
    const uint32_t sign = static_cast<uint32_t>(u >> 63) << 15;
    const uint64_t mag = u & 0x7fffffffffffffffull;
    if (mag >= 0x7ff0000000000000ull) {  // inf or nan
        if (mag > 0x7ff0000000000000ull) return static_cast<uint16_t>(sign | 0x7fc0u);
        return static_cast<uint16_t>(sign | 0x7f80u);
    }
    const int exp_d = static_cast<int>(mag >> 52);  // biased fp64 exponent
    if (exp_d - 1023 < -126) {
        // subnormal (or zero) in bf16: multiples of 2^-133, rounded half to even
        const double scaled = __builtin_fabs(x) * 0x1p133;
        const double r = __builtin_rint(scaled);  // exact integer <= 2^7
        const uint32_t m = static_cast<uint32_t>(r);
        return static_cast<uint16_t>(sign | m);  // m == 128 lands on the smallest normal
    }
    uint64_t keep = mag >> 45;
    const uint64_t rem = mag & ((1ull << 45) - 1);
    const uint64_t half = 1ull << 44;
    if (rem > half || (rem == half && (keep & 1ull))) ++keep;
    const int exp_f = static_cast<int>(keep >> 7) - 1023 + 127;
    if (exp_f >= 255) return static_cast<uint16_t>(sign | 0x7f80u);
    return static_cast<uint16_t>(sign | (static_cast<uint32_t>(exp_f) << 7) | static_cast<uint32_t>(keep & 0x7f));
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

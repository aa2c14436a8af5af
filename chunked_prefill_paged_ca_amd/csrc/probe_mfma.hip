// probe_mfma.hip -- measure what this part sustains: the bf16 matrix pipe by operand data, and a
// plain HBM read stream.
//
// Not part of the attention path: a measurement aid for placing the kernels against ceilings
// they can actually reach.  Each workgroup (8 wavefronts, one per CU) keeps 16 A and 2 B
// fragments in registers, loaded once from a buffer the host fills, and issues 32
// v_mfma_f32_16x16x32_bf16 per iteration into 16 independent accumulators -- no memory traffic,
// no dependency stalls.  The rate still depends on the operand values: toggling data (random
// bf16) draws more power than constant data and the clock drops, so the same instruction stream
// runs slower.  Built into its own small library (libca_probe.so), exported with C linkage.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <random>
#include <vector>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 512;
constexpr int kFrags = 18;  // 16 A + 2 B fragments per lane

__global__ void __launch_bounds__(kThreads, 1) mfma_rate_kernel(const uint4* __restrict__ buf,
                                                                 float* __restrict__ out, int iters) {
    const int tid = threadIdx.x;
    const size_t base = (static_cast<size_t>(blockIdx.x) * kThreads + tid) * kFrags;
    bf16x8 a[16], b[2];
    for (int j = 0; j < 16; ++j) {
        const uint4 t = buf[base + j];
        __builtin_memcpy(&a[j], &t, 16);
    }
    for (int j = 0; j < 2; ++j) {
        const uint4 t = buf[base + 16 + j];
        __builtin_memcpy(&b[j], &t, 16);
    }
    floatx4 acc[16];
    for (int j = 0; j < 16; ++j) acc[j] = floatx4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j], b[0], acc[j], 0, 0, 0);
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[15 - j], b[1], acc[j], 0, 0, 0);
    }
    float r = 0.f;
    for (int j = 0; j < 16; ++j) r += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    out[static_cast<size_t>(blockIdx.x) * kThreads + tid] = r;  // keeps the loop live
}

// Plain read stream: each wavefront reads whole 16 KB chunks (16 loads of 16 bytes per lane in
// flight, each load one contiguous 1 KB run), chunks dealt round-robin over the waves, and folds
// the data into one word so the loads stay live.  n is a multiple of 1024 (16-byte units).  NT:
// the loads carry the non-temporal hint (streamed data not kept in the caches).
typedef uint32_t probe_u32x4 __attribute__((ext_vector_type(4)));
template <bool NT>
__global__ void __launch_bounds__(256) read_stream_kernel(const uint4* __restrict__ src, size_t n,
                                                          uint32_t* __restrict__ out) {
    const size_t gid = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const size_t wave = gid >> 6;
    const size_t nwaves = (static_cast<size_t>(gridDim.x) * blockDim.x) >> 6;
    const int lane = threadIdx.x & 63;
    uint32_t acc = 0;
    for (size_t c = wave; (c + 1) * 1024 <= n; c += nwaves) {
        const uint4* b = src + c * 1024;
        uint4 v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if constexpr (NT) {
                const probe_u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const probe_u32x4*>(b + i * 64 + lane));
                v[i] = make_uint4(t.x, t.y, t.z, t.w);
            } else {
                v[i] = b[i * 64 + lane];
            }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
    }
    out[gid] = acc;
}

// L2-resident read rate into a CU, by how the data lands: mode 0 / 2 load 16 bytes per lane into
// registers, mode 1 / 3 copy them straight into LDS (global->LDS DMA).  Modes 0 / 1 read 1 KB
// contiguous runs; modes 2 / 3 read 8 rows x 128 bytes per instruction with rows 8 KB apart (the
// tile rows of a GEMM over K = 4096 bf16); mode 4 loads 8 bytes per lane into registers (512-byte
// runs, two instructions per KB).  Every wave moves 16 KB per round (16 or 32 instructions), then
// waits for them, `iters` times; all addresses lie in the `window`-byte buffer (a multiple of
// 64 KB).
__global__ void __launch_bounds__(256) l2_rate_kernel(const uint4* __restrict__ src, size_t window,
                                                      int iters, int mode, uint32_t* __restrict__ out) {
    __shared__ __attribute__((aligned(16))) uint4 lds[4 * 16 * 64];  // 16 KB per wave
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const size_t gw = static_cast<size_t>(blockIdx.x) * 4 + w;
    const size_t nchunks = window / 1024;
    const size_t nrows = window / 8192;  // 8 KB rows, a multiple of 8
    uint32_t acc = 0;
    for (int it = 0; it < iters; ++it) {
        uint4 v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const size_t c = (gw * 16 + u + static_cast<size_t>(it) * 7) % nchunks;
            size_t off;  // in 16-byte units
            if (mode < 2) {
                off = c * 64 + lane;
            } else {
                const size_t row = (c * 8) % nrows + (lane >> 3);
                const size_t col = ((c * 8) / nrows) % 64;  // 128-byte column of the row
                off = row * 512 + col * 8 + (lane & 7);
            }
            if (mode == 1 || mode == 3) {
                __builtin_amdgcn_global_load_lds(src + off, lds + (w * 16 + u) * 64, 16, 0, 0);
            } else if (mode == 4) {
                const uint2* s2 = reinterpret_cast<const uint2*>(src + c * 64);
                const uint2 a = s2[lane], b = s2[64 + lane];
                v[u] = make_uint4(a.x, a.y, b.x, b.y);
            } else {
                v[u] = src[off];
            }
        }
        if (mode == 1 || mode == 3) {
            __builtin_amdgcn_s_waitcnt(0);
        } else {
#pragma unroll
            for (int u = 0; u < 16; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
        }
    }
    __syncthreads();
    out[blockIdx.x * 256 + threadIdx.x] = acc ^ lds[threadIdx.x].x;
}

uint16_t to_bf16(float x) {
    uint32_t u;
    std::memcpy(&u, &x, 4);
    return static_cast<uint16_t>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

}  // namespace

// Rate of back-to-back bf16 MFMAs on the current device for one operand distribution:
// mode 0 = all ones, 1 = all zeros, 2 = N(0, 1), 3 = exp(-|3 z|) with z ~ N(0, 1) (the range of
// softmax weights).  One workgroup per CU, `iters` iterations of 32 MFMAs per wave; best of 3
// timed launches after one warm-up.  Writes the rate in TFLOP/s and the time in ms; returns 0, or
// the HIP error code (nothing is left allocated either way).
extern "C" int ca_probe_mfma_rate(int mode, int iters, double* tflops, float* ms_out) {
    if (mode < 0 || mode > 3 || iters <= 0 || !tflops || !ms_out) return static_cast<int>(hipErrorInvalidValue);
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return static_cast<int>(e);
    const size_t nfrag = static_cast<size_t>(cus) * kThreads * kFrags;
    std::vector<uint16_t> host(nfrag * 8);
    std::mt19937 rng(12345u + static_cast<unsigned>(mode));
    std::normal_distribution<float> nd(0.f, 1.f);
    for (auto& h : host) {
        float x = mode == 0 ? 1.f : mode == 1 ? 0.f : nd(rng);
        if (mode == 3) x = std::exp(-std::fabs(3.f * x));
        h = to_bf16(x);
    }
    uint4* buf = nullptr;
    float* out = nullptr;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    float best = 1e30f;
    e = hipMalloc(&buf, nfrag * 16);
    if (e == hipSuccess) e = hipMalloc(&out, static_cast<size_t>(cus) * kThreads * sizeof(float));
    if (e == hipSuccess) e = hipMemcpy(buf, host.data(), nfrag * 16, hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipEventCreate(&e0);
    if (e == hipSuccess) e = hipEventCreate(&e1);
    for (int r = 0; r < 4 && e == hipSuccess; ++r) {
        e = hipEventRecord(e0, nullptr);
        if (e == hipSuccess) {
            hipLaunchKernelGGL(mfma_rate_kernel, dim3(cus), dim3(kThreads), 0, nullptr, buf, out, iters);
            e = hipGetLastError();
        }
        if (e == hipSuccess) e = hipEventRecord(e1, nullptr);
        if (e == hipSuccess) e = hipEventSynchronize(e1);
        float ms = 0.f;
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
        if (e == hipSuccess && r > 0 && ms < best) best = ms;
    }
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    if (buf) (void)hipFree(buf);
    if (out) (void)hipFree(out);
    if (e != hipSuccess) return static_cast<int>(e);
    const double flops = static_cast<double>(cus) * (kThreads / 64) * iters * 32 * 16384.0;
    *ms_out = best;
    *tflops = flops / (best * 1e-3) / 1e12;
    return 0;
}

// HBM read rate of the current device: a `bytes`-long buffer (rounded down to 16 KB, at least
// 1 MiB) read once per launch by 16 workgroups of 256 threads per CU, with plain or (nontemporal
// != 0) non-temporal loads; best of 5 timed launches after one warm-up.  Writes GB/s; returns 0
// or the HIP error code (nothing is left allocated either way).
extern "C" int ca_probe_read_rate(size_t bytes, int nontemporal, double* gbs) {
    if (bytes < (size_t(1) << 20) || !gbs) return static_cast<int>(hipErrorInvalidValue);
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return static_cast<int>(e);
    const size_t n = bytes / 16384 * 1024;
    const int grid = cus * 16, block = 256;
    uint4* src = nullptr;
    uint32_t* out = nullptr;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    float best = 1e30f;
    e = hipMalloc(&src, n * 16);
    if (e == hipSuccess) e = hipMalloc(&out, static_cast<size_t>(grid) * block * sizeof(uint32_t));
    if (e == hipSuccess) e = hipMemset(src, 0x5a, n * 16);
    if (e == hipSuccess) e = hipEventCreate(&e0);
    if (e == hipSuccess) e = hipEventCreate(&e1);
    for (int r = 0; r < 6 && e == hipSuccess; ++r) {
        e = hipEventRecord(e0, nullptr);
        if (e == hipSuccess) {
            if (nontemporal)
                hipLaunchKernelGGL(read_stream_kernel<true>, dim3(grid), dim3(block), 0, nullptr, src, n, out);
            else
                hipLaunchKernelGGL(read_stream_kernel<false>, dim3(grid), dim3(block), 0, nullptr, src, n, out);
            e = hipGetLastError();
        }
        if (e == hipSuccess) e = hipEventRecord(e1, nullptr);
        if (e == hipSuccess) e = hipEventSynchronize(e1);
        float ms = 0.f;
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
        if (e == hipSuccess && r > 0 && ms < best) best = ms;
    }
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    if (src) (void)hipFree(src);
    if (out) (void)hipFree(out);
    if (e != hipSuccess) return static_cast<int>(e);
    *gbs = static_cast<double>(n) * 16 / (best * 1e-3) / 1e9;
    return 0;
}

// Aggregate read rate (GB/s) of l2_rate_kernel for `mode` over a `window`-byte buffer (>= 64 KB, a
// multiple of 64 KB; small enough to stay in L2 it measures L2 -> CU delivery), `wgs_per_cu`
// workgroups of 4 waves per CU; best of 5 timed launches after one warm-up.  Returns 0 or the HIP
// error code (nothing left allocated).
extern "C" int ca_probe_l2_rate(int mode, size_t window, int iters, int wgs_per_cu, double* gbs) {
    if (mode < 0 || mode > 4 || window < 65536 || window % 65536 || iters <= 0 || wgs_per_cu < 1 ||
        wgs_per_cu > 4 || !gbs)
        return static_cast<int>(hipErrorInvalidValue);
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return static_cast<int>(e);
    const int grid = cus * wgs_per_cu;
    uint4* src = nullptr;
    uint32_t* out = nullptr;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    float best = 1e30f;
    e = hipMalloc(&src, window);
    if (e == hipSuccess) e = hipMalloc(&out, static_cast<size_t>(grid) * 256 * sizeof(uint32_t));
    if (e == hipSuccess) e = hipMemset(src, 0x5a, window);
    if (e == hipSuccess) e = hipEventCreate(&e0);
    if (e == hipSuccess) e = hipEventCreate(&e1);
    for (int r = 0; r < 6 && e == hipSuccess; ++r) {
        e = hipEventRecord(e0, nullptr);
        if (e == hipSuccess) {
            hipLaunchKernelGGL(l2_rate_kernel, dim3(grid), dim3(256), 0, nullptr, src, window, iters, mode, out);
            e = hipGetLastError();
        }
        if (e == hipSuccess) e = hipEventRecord(e1, nullptr);
        if (e == hipSuccess) e = hipEventSynchronize(e1);
        float ms = 0.f;
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
        if (e == hipSuccess && r > 0 && ms < best) best = ms;
    }
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    if (src) (void)hipFree(src);
    if (out) (void)hipFree(out);
    if (e != hipSuccess) return static_cast<int>(e);
    *gbs = static_cast<double>(grid) * 4 * iters * 16 * 1024 / (best * 1e-3) / 1e9;
    return 0;
}

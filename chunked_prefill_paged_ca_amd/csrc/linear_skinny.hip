// linear_skinny.hip -- the step's QKV projection for small token counts: every weight read once
// from HBM, straight into the matrix cores.
//
// bowenzhou.top "Sarathi：让解码搭上 prefill 的顺风车", section "Decode-maximal batching：顺车的账本":
// the linear layers of all tokens of a mixed step run as one product, so each weight is read once
// for all of them.  With few tokens (a decode-heavy step) that product is bound by reading the
// weights, (Hq + 2 Hkv) d x hidden bf16 values, and nothing else: the kernel below streams them
// at the HBM rate instead of tiling the product for arithmetic throughput.
//
//   out[T][N] = x[T][K] . w[N][K]^T  (bf16 operands, fp32 accumulation, bf16 result), T <= 16
//
// is computed as out^T = w x^T on v_mfma_f32_16x16x32_bf16: A = 16 weight rows x 32 of K (lane
// (c, q) holds 16 contiguous bytes of row c at k = 8q), B = x^T, 32 of K x 16 tokens (16 bytes of
// token row c; zero past T), C = 16 features x 16 tokens (lane (c, q) holds features 4q .. 4q+3
// of token c).  Workgroup = 32 weight rows (two A tiles) x all tokens; its 8 wavefronts take one
// eighth of K each and keep two batches of four 32-wide K steps of loads in flight (16 KB of
// weights per wave); the eight fp32 partial tiles are summed through LDS.
// Measured for the Mistral-7B projection (4096 -> 6144): 14.1 us at T = 1 (3.6 TB/s of weights)
// against 17.0 us for the library GEMM, level with it at T = 16.  Past 16 tokens the token rows,
// which every workgroup reads for its own weight rows, outgrow the weights in L2 traffic (at 80
// tokens ~4x), so a larger T is left to the library GEMM.

#include <hip/hip_runtime.h>

#include "internal.h"
#include "mfma.h"

namespace ca {
namespace {

constexpr int kWaves = 8;
constexpr int kRows = 32;   // weight rows per workgroup (two 16-row A tiles)
constexpr int kSteps = 4;   // 32-wide K steps per load batch (two batches in flight)

template <int TT>
__global__ void __launch_bounds__(64 * kWaves) skinny_kernel(const uint16_t* __restrict__ x,
                                                             const uint16_t* __restrict__ w,
                                                             uint16_t* __restrict__ out, int T,
                                                             int K, int N) {
    __shared__ floatx4 red[kWaves][2][TT][64];
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int c = lane & 15, q = lane >> 4;
    const int n0 = blockIdx.x * kRows;
    const int t0 = blockIdx.y * 16 * TT;
    const int kw = K / kWaves;  // this wave's K range: [wv kw, (wv + 1) kw)
    const int kb = wv * kw;

    const uint16_t* wa = w + static_cast<int64_t>(n0 + c) * K + kb + 8 * q;  // A tile 0, row c
    const uint16_t* wb = wa + static_cast<int64_t>(16) * K;                   // A tile 1, row c
    const uint16_t* xr[TT];
    bool ok[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        const int t = t0 + 16 * tt + c;
        ok[tt] = t < T;
        xr[tt] = x + static_cast<int64_t>(ok[tt] ? t : 0) * K + kb + 8 * q;
    }

    floatx4 acc[2][TT];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) acc[nt][tt] = floatx4{0.f, 0.f, 0.f, 0.f};

    // Register double buffer: the weight and token loads of the next kSteps K steps are issued
    // before the current ones are multiplied, so each wave keeps two batches (16 KB of weights)
    // in flight.
    struct Batch {
        bf16x8 a0[kSteps], a1[kSteps], b[kSteps][TT];
    };
    auto load = [&](Batch& bt, int k) {
#pragma unroll
        for (int u = 0; u < kSteps; ++u) {
            bt.a0[u] = load_frag(wa + k + 32 * u);
            bt.a1[u] = load_frag(wb + k + 32 * u);
        }
#pragma unroll
        for (int u = 0; u < kSteps; ++u)
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) bt.b[u][tt] = ok[tt] ? load_frag(xr[tt] + k + 32 * u) : zero_frag();
    };
    auto mul = [&](const Batch& bt) {
#pragma unroll
        for (int u = 0; u < kSteps; ++u)
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) {
                acc[0][tt] = mfma16x16x32(bt.a0[u], bt.b[u][tt], acc[0][tt]);
                acc[1][tt] = mfma16x16x32(bt.a1[u], bt.b[u][tt], acc[1][tt]);
            }
    };
    constexpr int KB = 32 * kSteps;  // K per batch; kw is a multiple of 2 KB
    Batch p0, p1;
    load(p0, 0);
    for (int k = 0; k < kw; k += 2 * KB) {
        load(p1, k + KB);
        mul(p0);
        if (k + 2 * KB < kw) load(p0, k + 2 * KB);
        mul(p1);
    }

#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) red[wv][nt][tt][lane] = acc[nt][tt];
    __syncthreads();
    // sum the eight K ranges of each (A tile, token tile, lane) and store 4 features of a token
    for (int i = threadIdx.x; i < 2 * TT * 64; i += 64 * kWaves) {
        const int ln = i & 63, tt = (i >> 6) % TT, nt = (i >> 6) / TT;
        floatx4 s = red[0][nt][tt][ln];
#pragma unroll
        for (int v = 1; v < kWaves; ++v) s += red[v][nt][tt][ln];
        const int t = t0 + 16 * tt + (ln & 15);
        if (t < T) {
            const int n = n0 + 16 * nt + 4 * (ln >> 4);
            const uint32_t lo = f2bf(s[0]) | (static_cast<uint32_t>(f2bf(s[1])) << 16);
            const uint32_t hi = f2bf(s[2]) | (static_cast<uint32_t>(f2bf(s[3])) << 16);
            *reinterpret_cast<uint2*>(out + static_cast<int64_t>(t) * N + n) = make_uint2(lo, hi);
        }
    }
}

}  // namespace

bool skinny_projection_fits(int64_t T, int64_t K, int64_t N) {
    return T >= 1 && T <= kSkinnyMaxTokens && K % (kWaves * 2 * 32 * kSteps) == 0 && N % kRows == 0 &&
           K <= INT32_MAX && N <= INT32_MAX;
}

hipError_t launch_skinny_projection(int64_t T, int64_t K, int64_t N, const void* x, const void* w,
                                    void* out, hipStream_t stream, const LaunchEvents& ev) {
    if (!skinny_projection_fits(T, K, N)) return hipErrorInvalidValue;
    const auto xx = static_cast<const uint16_t*>(x);
    const auto ww = static_cast<const uint16_t*>(w);
    auto oo = static_cast<uint16_t*>(out);
    const int t = static_cast<int>(T), k = static_cast<int>(K), n = static_cast<int>(N);
    const dim3 block(64 * kWaves);
    hipExtLaunchKernelGGL(skinny_kernel<1>, dim3(n / kRows, 1), block, 0, stream, ev.start, ev.stop, 0, xx,
                          ww, oo, t, k, n);
    return hipGetLastError();
}

}  // namespace ca

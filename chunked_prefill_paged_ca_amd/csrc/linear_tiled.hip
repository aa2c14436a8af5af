// linear_tiled.hip -- the step's QKV projection beyond 16 tokens: an LDS-tiled bf16 MFMA GEMM.
//
// bowenzhou.top "Sarathi：让解码搭上 prefill 的顺风车", section "Decode-maximal batching：顺车的账本":
// the linear layers of every token of a mixed step -- decode tokens and prefill-chunk tokens
// alike -- are one matrix product, so each weight is read once for all of them.  With a few
// hundred tokens that product is bound by arithmetic, not by the weight read:
//
//   out[T][N] = x[T][K] . w[N][K]^T  (bf16 operands, fp32 accumulation, bf16 result)
//
// Workgroup = one output tile of BM tokens x BN features over a range of K, 8 wavefronts: waves
// 0-3 (one per SIMD) split the tile 2 x 2, each BM/2 tokens x BN/2 features, and only compute;
// waves 4-7 only issue the stage copies.  A SIMD's vector-memory path takes ~15 bytes per
// clock, so issuing a stage's copies holds the issuing wave for hundreds of cycles; on a wave of
// its own that time runs beside the matrix work instead of before it (measured on the
// Mistral-7B projection: T = 512 51.4 -> 38.3-39.8 us, T = 256 40.7 -> 31.5 us, T = 128
// 27.6 -> 23.7 us, T = 100 26.6 -> 22.4 us; T <= 80 unchanged within the box's spread).  The product runs as
// out^T = w x^T on v_mfma_f32_16x16x32_bf16 (A = 16 weight rows x 32 of K, B = x^T: 32 of K x
// 16 tokens, C = 16 features x 16 tokens; lane (c, q) holds features 4q .. 4q+3 of token c).
//   * Operands reach LDS by 16-byte global->LDS DMA, no registers: a stage holds BK = 64 of K of
//     both tiles, and NST stages rotate (one barrier per stage, the next stages in flight).
//   * Each DMA instruction moves 8 whole 128-byte lines (8 rows x 64 of K); LDS holds the rows
//     as 128-byte rows whose 16-byte chunks are XOR-swizzled by row, so a fragment read (16 rows
//     x 16 bytes) touches 16 distinct bank groups.  (Fragment-major order -- 16 rows x 64 bytes
//     per instruction, half lines -- measured 30 % slower.)
//   * Blocks are dispatched round robin over the 8 XCDs; the block -> tile map puts the token
//     blocks that share a weight tile on the same XCD, so each weight byte is fetched from HBM
//     into one L2 and reused there.
//   * When the output tiles alone would leave most CUs idle (few tokens), K is split over
//     `nsplit` workgroups that write fp32 partials, summed in a fixed order by reduce_kernel
//     (deterministic; no atomics).
// Rows past T are loaded from row T - 1 (in bounds) and never stored.

#include <hip/hip_runtime.h>

#include <type_traits>

#include "internal.h"
#include "mfma.h"

namespace ca {
namespace {

// Tuning knobs fixed at build time (the defaults are the measured choice): K per LDS stage and
// the number of stages in the ring (0: the deepest ring that fits, see ring_stages).
#ifndef CA_TILED_BK
#define CA_TILED_BK 64
#endif
#ifndef CA_TILED_RING
#define CA_TILED_RING 0
#endif
// 1: operands go HBM/L2 -> VGPR -> LDS (two stages of loads in registers, two LDS slots) instead
// of global->LDS DMA
#ifndef CA_TILED_VGPR
#define CA_TILED_VGPR 0
#endif
static_assert(CA_TILED_VGPR == 0, "register staging is not built with copying waves");

constexpr int kThreads = 512;       // 4 computing wavefronts (2 x 2 over the tile) + 4 copying
constexpr int kBK = CA_TILED_BK;    // K per LDS stage
constexpr int kKS = kBK / 32;       // 32-wide MFMA steps per stage
static_assert(kBK % 32 == 0 && kKS >= 1 && kKS <= 8, "stage depth");

template <int BM, int BN>
struct TileShape {
    static constexpr int XF = BM / 16;             // token fragments per 32-wide K step
    static constexpr int WF = BN / 16;             // feature fragments per K step
    static constexpr int F = kKS * (XF + WF);      // 1 KB DMA instructions per stage
    static constexpr int HALVES = F * 512;         // bf16 elements per stage
    static constexpr int D = F / 4;                // DMA instructions per wave per stage
    static_assert(F % 4 == 0, "stage instructions must split evenly over the 4 waves");
};

// XOR swizzle of the 16-byte chunks of a 128-byte LDS row: the 16 rows of a fragment (row % 16)
// get distinct (row parity, chunk) pairs, i.e. distinct LDS bank groups.
__device__ __forceinline__ int swz(int row) {
    const int r = row & 15;
    return (r ^ (r >> 3)) & 7;
}

// s_waitcnt immediate: at most n vector-memory operations outstanding and every LDS read
// returned (expcnt not waited for)
constexpr int wait_vm_lgkm0(int n) { return (n & 0xf) | (0x7 << 4) | ((n >> 4) << 14); }

// The kernel body (a device function: the host compilation pass never instantiates it).
template <int BM, int BN, int NST>
__device__ __forceinline__ void tiled_body(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, uint16_t* __restrict__ out,
    float* __restrict__ part, int T, int K, int N, int ntb, int nfb, int nsplit) {
    using S = TileShape<BM, BN>;
    __shared__ __attribute__((aligned(16))) uint16_t st0[S::HALVES];
    __shared__ __attribute__((aligned(16))) uint16_t st1[S::HALVES];
    __shared__ __attribute__((aligned(16))) uint16_t st2[NST > 2 ? S::HALVES : 8];
    __shared__ __attribute__((aligned(16))) uint16_t st3[NST > 3 ? S::HALVES : 8];
    __shared__ __attribute__((aligned(16))) uint16_t st4[NST > 4 ? S::HALVES : 8];
    __shared__ __attribute__((aligned(16))) uint16_t st5[NST > 5 ? S::HALVES : 8];
    static_assert(NST >= 2 && NST <= 6, "2 to 6 stages");
    static_assert((NST - 2) * S::D <= 63, "vmcnt range");

    // block -> tile: the 8 XCDs take blocks b, b + 8, ...; logical tile ids run contiguously
    // inside one XCD's share, token block fastest
    const int per = static_cast<int>(gridDim.x) / 8;  // the grid is a multiple of 8
    const int logical = (blockIdx.x % 8) * per + blockIdx.x / 8;
    const int tb = logical % ntb;
    const int fb = (logical / ntb) % nfb;
    const int sp = logical / (ntb * nfb);
    if (sp >= nsplit) return;  // grid padding (uniform over the block)

    const int lane = threadIdx.x & 63;
    const int wv0 = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const bool copier = wv0 >= 4;  // waves 4-7 copy the stages, waves 0-3 compute
    const int wv = wv0 & 3;
    const int wr = wv >> 1, wc = wv & 1;
    const int c = lane & 15, q = lane >> 4;
    const int t0 = tb * BM, f0 = fb * BN;
    // split sp covers the K stages [sp KS / nsplit, (sp + 1) KS / nsplit) of the KS = K / kBK
    const int KS = K / kBK;
    const int s0 = static_cast<int>(static_cast<int64_t>(sp) * KS / nsplit);
    const int kbeg = s0 * kBK;
    const int nst = static_cast<int>(static_cast<int64_t>(sp + 1) * KS / nsplit) - s0;

    // This wave's DMA sources.  A stage holds the BM x rows, then the BN w rows, each row's kBK
    // values as one 2 kBK-byte LDS row.  DMA instruction u of the wave (stage instruction
    // g = wv D + u) fills rows 8 g .. 8 g + 7 (kBK = 64: one 128-byte line of each): lane l writes
    // LDS chunk p = l % 8 of row 8 g + l / 8 and reads global chunk p ^ swz(row) of that row, so
    // LDS chunk p of row r holds K offset 8 (p ^ swz(r)).  The XOR spreads the 16 rows of a
    // fragment over distinct bank groups.
    static_assert(kBK == 64, "8 rows of 128 bytes per DMA instruction");
    const uint16_t* src[S::D];
#pragma unroll
    for (int u = 0; u < S::D; ++u) {
        const int row = 8 * (wv * S::D + u) + (lane >> 3);  // stage row
        const int chunk = (lane & 7) ^ swz(row);
        if (row < BM) {
            int t = t0 + row;
            t = t < T ? t : T - 1;
            src[u] = x + static_cast<int64_t>(t) * K + kbeg + 8 * chunk;
        } else {
            src[u] = w + static_cast<int64_t>(f0 + row - BM) * K + kbeg + 8 * chunk;
        }
    }
    auto dma = [&](uint16_t* stage, int si) {
        if (!copier) return;
#pragma unroll
        for (int u = 0; u < S::D; ++u)
            __builtin_amdgcn_global_load_lds(src[u] + si * kBK, stage + 512 * (wv * S::D + u), 16, 0, 0);
    };

    constexpr int MI = BM / 32;  // token fragments of this wave
    constexpr int NJ = BN / 32;  // feature fragments of this wave
    floatx4 acc[NJ][MI];
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int i = 0; i < MI; ++i) acc[j][i] = floatx4{0.f, 0.f, 0.f, 0.f};

    // A fragment (16 rows from `r0`, 32-wide K step h): lane (c, q) reads row r0 + c, K offset
    // 32 h + 8 q, i.e. LDS chunk (4 h + q) ^ swz(r0 + c) of that row.
    const int fr_off = 64 * c + 8 * ((0 + q) ^ swz(c));  // h = 0 (r0 a multiple of 16)
    const int fr_off1 = 64 * c + 8 * ((4 + q) ^ swz(c));  // h = 1
    auto compute = [&](const uint16_t* stage) {
#pragma unroll
        for (int h = 0; h < kKS; ++h) {
            const int off = h == 0 ? fr_off : fr_off1;
            bf16x8 xf[MI], wf[NJ];
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                const uint4 v = *reinterpret_cast<const uint4*>(stage + 64 * 16 * (wr * MI + i) + off);
                __builtin_memcpy(&xf[i], &v, sizeof(v));
            }
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const uint4 v = *reinterpret_cast<const uint4*>(stage + 64 * (BM + 16 * (wc * NJ + j)) + off);
                __builtin_memcpy(&wf[j], &v, sizeof(v));
            }
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int i = 0; i < MI; ++i) acc[j][i] = mfma16x16x32(wf[j], xf[i], acc[j][i]);
        }
    };

    // Wait until at most `later` stages' DMAs of this wave are outstanding and this wave's LDS
    // reads have returned, then an execution barrier: the waited-for stage is complete in every
    // wave, and no wave still reads the slot about to be refilled.  (A __syncthreads() would be a
    // release fence that drains every DMA in flight.)
    auto wait_stage = [&](int later) {
        switch (later) {
            case 0: __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0)); break;
            case 1: __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(NST > 2 ? 1 * S::D : 0)); break;
            case 2: __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(NST > 3 ? 2 * S::D : 0)); break;
            case 3: __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(NST > 4 ? 3 * S::D : 0)); break;
            default: __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(NST > 5 ? 4 * S::D : 0)); break;
        }
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
    };
    auto slot = [&](auto I) -> uint16_t* {
        constexpr int i = decltype(I)::value % NST;
        if constexpr (i == 0) return st0;
        else if constexpr (i == 1) return st1;
        else if constexpr (i == 2) return st2;
        else if constexpr (i == 3) return st3;
        else if constexpr (i == 4) return st4;
        else return st5;
    };
    if constexpr (CA_TILED_VGPR != 0) {
        // Register staging: stage k's loads sit in reg[k % 2]; at step si the loads of stage
        // si + 1 (issued two steps earlier) are written to the LDS slot (si + 1) % 2 and that
        // register set is refilled with stage si + 3.  One barrier per stage: it publishes
        // stage si + 1 and frees slot si % 2 for stage si + 2.
        uint4 reg[2][S::D];
        auto load = [&](uint4 (&r)[S::D], int si) {
#pragma unroll
            for (int u = 0; u < S::D; ++u) r[u] = *reinterpret_cast<const uint4*>(src[u] + si * kBK);
        };
        auto store = [&](uint16_t* stage, const uint4 (&r)[S::D]) {
#pragma unroll
            for (int u = 0; u < S::D; ++u) *reinterpret_cast<uint4*>(stage + 512 * (wv * S::D + u) + 8 * lane) = r[u];
        };
        auto sync = [&]() {
            __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(63));  // LDS writes and reads done
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            __builtin_amdgcn_s_barrier();
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
        };
        load(reg[0], 0);
        if (1 < nst) load(reg[1], 1);
        store(st0, reg[0]);
        if (2 < nst) load(reg[0], 2);
        sync();
        auto vstep = [&](auto P, int si) {
            constexpr int p = decltype(P)::value;
            compute(p == 0 ? st0 : st1);
            if (si + 1 < nst) store(p == 0 ? st1 : st0, reg[1 - p]);
            if (si + 3 < nst) load(reg[1 - p], si + 3);
            sync();
        };
        for (int si = 0; si < nst; si += 2) {
            vstep(std::integral_constant<int, 0>{}, si);
            if (si + 1 >= nst) break;
            vstep(std::integral_constant<int, 1>{}, si + 1);
        }
    } else {
    // prologue: stages 0 .. NST-2 requested
    if (0 < nst) dma(st0, 0);
    if (NST > 2 && 1 < nst) dma(st1, 1);
    if (NST > 3 && 2 < nst) dma(st2, 2);
    if (NST > 4 && 3 < nst) dma(st3, 3);
    if (NST > 5 && 4 < nst) dma(st4, 4);
    // stage si sits in slot si % NST; at its wait, stages up to min(nst, si + NST - 1) - 1 were
    // requested, so min(nst - 1, si + NST - 2) - si of them may stay in flight; after the
    // barrier the slot of stage si - 1 is refilled with stage si + NST - 1
    auto step = [&](auto I, int si) {
        constexpr int i = decltype(I)::value;
        const int later = (nst - 1 < si + NST - 2 ? nst - 1 : si + NST - 2) - si;
        wait_stage(later);
        if (si + NST - 1 < nst) dma(slot(std::integral_constant<int, i + NST - 1>{}), si + NST - 1);
        if (!copier) compute(slot(std::integral_constant<int, i>{}));
    };
    for (int si = 0; si < nst; si += NST) {
        step(std::integral_constant<int, 0>{}, si);
        if (si + 1 >= nst) break;
        step(std::integral_constant<int, 1>{}, si + 1);
        if constexpr (NST > 2) {
            if (si + 2 >= nst) break;
            step(std::integral_constant<int, 2>{}, si + 2);
        }
        if constexpr (NST > 3) {
            if (si + 3 >= nst) break;
            step(std::integral_constant<int, 3>{}, si + 3);
        }
        if constexpr (NST > 4) {
            if (si + 4 >= nst) break;
            step(std::integral_constant<int, 4>{}, si + 4);
        }
        if constexpr (NST > 5) {
            if (si + 5 >= nst) break;
            step(std::integral_constant<int, 5>{}, si + 5);
        }
    }
    }

    if (copier) return;
    // C tile (j, i): features f0 + 16 (wc NJ + j) + 4 q .. + 3 of token t0 + 16 (wr MI + i) + c
#pragma unroll
    for (int i = 0; i < MI; ++i) {
        const int t = t0 + 16 * (wr * MI + i) + c;
        if (t >= T) continue;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int f = f0 + 16 * (wc * NJ + j) + 4 * q;
            if (nsplit == 1) {
                const uint32_t lo = f2bf(acc[j][i][0]) | (static_cast<uint32_t>(f2bf(acc[j][i][1])) << 16);
                const uint32_t hi = f2bf(acc[j][i][2]) | (static_cast<uint32_t>(f2bf(acc[j][i][3])) << 16);
                *reinterpret_cast<uint2*>(out + static_cast<int64_t>(t) * N + f) = make_uint2(lo, hi);
            } else {
                *reinterpret_cast<float4*>(part + (static_cast<int64_t>(sp) * T + t) * N + f) =
                    make_float4(acc[j][i][0], acc[j][i][1], acc[j][i][2], acc[j][i][3]);
            }
        }
    }
}

template <int BM, int BN, int NST>
__global__ void __launch_bounds__(kThreads) tiled_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, uint16_t* __restrict__ out,
    float* __restrict__ part, int T, int K, int N, int ntb, int nfb, int nsplit) {
    tiled_body<BM, BN, NST>(x, w, out, part, T, K, N, ntb, nfb, nsplit);
}

// out = sum over the nsplit partials, in split order, rounded once to bf16 (4 outputs per thread)
__global__ void __launch_bounds__(256) reduce_kernel(const float* __restrict__ part,
                                                     uint16_t* __restrict__ out, int64_t n4,
                                                     int64_t stride, int nsplit) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= n4) return;
    float4 s = reinterpret_cast<const float4*>(part)[i];
    for (int k = 1; k < nsplit; ++k) {
        const float4 v = reinterpret_cast<const float4*>(part + k * stride)[i];
        s.x += v.x;
        s.y += v.y;
        s.z += v.z;
        s.w += v.w;
    }
    const uint32_t lo = f2bf(s.x) | (static_cast<uint32_t>(f2bf(s.y)) << 16);
    const uint32_t hi = f2bf(s.z) | (static_cast<uint32_t>(f2bf(s.w)) << 16);
    reinterpret_cast<uint2*>(out)[i] = make_uint2(lo, hi);
}

// Stages of the ring (LDS per stage: kKS (bm + bn) / 16 KB): four when two workgroups then fit
// on a CU (160 KB of LDS), otherwise as many as one workgroup can hold, at most six.
constexpr int ring_stages(int bm, int bn) {
    const int kb = kKS * (bm / 16 + bn / 16);
    if (CA_TILED_VGPR != 0) return 2;
    if (CA_TILED_RING > 0) return CA_TILED_RING;
    if (4 * kb <= 80) return 4;
    int n = 2;
    while (n < 6 && (n + 1) * kb <= 160) ++n;
    return n;
}

using TiledFn = void (*)(const uint16_t*, const uint16_t*, uint16_t*, float*, int, int, int, int, int,
                         int);

// The kernel instance of a tile shape (nullptr for a shape not built).  Each instance is named
// here, in a plain host function, so both compilation passes instantiate it.
TiledFn tiled_fn(int bm, int bn) {
    switch (bm * 1000 + bn) {
        case 32064: return &tiled_kernel<32, 64, ring_stages(32, 64)>;
        case 32096: return &tiled_kernel<32, 96, ring_stages(32, 96)>;
        case 32128: return &tiled_kernel<32, 128, ring_stages(32, 128)>;
        case 64064: return &tiled_kernel<64, 64, ring_stages(64, 64)>;
        case 64096: return &tiled_kernel<64, 96, ring_stages(64, 96)>;
        case 64128: return &tiled_kernel<64, 128, ring_stages(64, 128)>;
        case 96064: return &tiled_kernel<96, 64, ring_stages(96, 64)>;
        case 96096: return &tiled_kernel<96, 96, ring_stages(96, 96)>;
        case 96128: return &tiled_kernel<96, 128, ring_stages(96, 128)>;
        case 128064: return &tiled_kernel<128, 64, ring_stages(128, 64)>;
        case 128096: return &tiled_kernel<128, 96, ring_stages(128, 96)>;
        case 128128: return &tiled_kernel<128, 128, ring_stages(128, 128)>;
        case 128192: return &tiled_kernel<128, 192, ring_stages(128, 192)>;
        case 128256: return &tiled_kernel<128, 256, ring_stages(128, 256)>;
        case 256096: return &tiled_kernel<256, 96, ring_stages(256, 96)>;
        case 256128: return &tiled_kernel<256, 128, ring_stages(256, 128)>;
        default: return nullptr;
    }
}

// Workgroups of a tile shape one CU holds at once (LDS- and register-limited), asked of the
// runtime once per shape.
int tiled_wgs_per_cu(int bm, int bn) {
    static int cache[9][7] = {};
    const int i = bm / 32, j = bn / 32 - 2;
    if (i < 1 || i > 8 || j < 0 || j > 6) return 1;
    int& c = cache[i][j];
    if (c == 0) {
        int blocks = 0;
        const TiledFn fn = tiled_fn(bm, bn);
        if (fn && hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, reinterpret_cast<const void*>(fn),
                                                               kThreads, 0) == hipSuccess && blocks > 0)
            c = blocks;
        else
            c = 1;
    }
    return c;
}

}  // namespace

// Tile shape and K split for T tokens: BM = T rounded up to 32 (at most 128); then, among the
// feature tiles (192, 128, 96, 64) that divide N, the one whose tile count fills the 256 CUs
// best (ties: the wider tile, fewer bytes moved per flop); K split as below.  Measured on the
// Mistral-7B projection: 1024 tokens 90.9 -> 65.5 us and 2048 tokens 141 -> 121 us with the
// 192-wide tile (one and two full rounds) against 128 (a round and a half, three rounds).  The
// 256-token tiles (256 x 96, 256 x 128, forced with CA_PROJECTION_TILE) were slower at every T.
TiledPlan plan_tiled_projection(int64_t T, int64_t K, int64_t N, int num_cus) {
    TiledPlan pl{};
    if (T < 1 || K % kBK != 0 || N % 64 != 0 || K > INT32_MAX || N > INT32_MAX || T > INT32_MAX) return pl;
    const int cus = num_cus > 0 ? num_cus : 256;
    pl.bm = T <= 32 ? 32 : (T <= 64 ? 64 : (T <= 96 ? 96 : 128));
    const int64_t ntb = (T + pl.bm - 1) / pl.bm;
    double best = -1.0;
    for (int bn : {192, 128, 96, 64}) {
        if (N % bn) continue;
        const int64_t tiles = ntb * (N / bn);
        const int64_t rounds = (tiles + cus - 1) / cus;
        const double util = static_cast<double>(tiles) / static_cast<double>(rounds * cus);
        if (util > best + 1e-9) {
            best = util;
            pl.bn = bn;
        }
    }
    // Fewer tiles than CUs (a few dozen tokens: the product is bound by reading the weights):
    // split K so that the workgroups fill every workgroup slot of the device once -- as many
    // splits as one round holds, not a count that leaves a partial second round (the splits need
    // not divide K evenly: split i takes K stages [i S / n, (i + 1) S / n)); at most 64, each at
    // least 256 of K.  Measured on the Mistral-7B projection at T = 80 (two workgroups per CU):
    // 8 even splits (768 workgroups, a round and a half) took 22.0 us, 5 uneven ones (480
    // workgroups, one round) 19.6 us.
    const int64_t tiles = ntb * (N / pl.bn);
    pl.nsplit = 1;
    if (tiles < cus) {
        const int64_t slots = static_cast<int64_t>(cus) * tiled_wgs_per_cu(pl.bm, pl.bn);
        int64_t n = slots / tiles;
        const int64_t by_k = K / 256;
        n = n < by_k ? n : by_k;
        n = n < 64 ? n : 64;
        pl.nsplit = static_cast<int>(n > 1 ? n : 1);
    }
    pl.ok = true;
    return pl;
}

bool tiled_shape_fits(const TiledPlan& pl, int64_t T, int64_t K, int64_t N) {
    return tiled_fn(pl.bm, pl.bn) != nullptr && T >= 1 && N % pl.bn == 0 && pl.nsplit >= 1 &&
           pl.nsplit <= 64 && K % kBK == 0 && K / kBK >= pl.nsplit;
}

size_t tiled_partial_bytes(const TiledPlan& pl, int64_t T, int64_t N) {
    return pl.nsplit > 1 ? static_cast<size_t>(pl.nsplit) * T * N * sizeof(float) : 0;
}

hipError_t launch_tiled_projection(const TiledPlan& pl, int64_t T, int64_t K, int64_t N, const void* x,
                                   const void* w, void* out, float* part, hipStream_t stream,
                                   const LaunchEvents& ev) {
    if (!pl.ok || (pl.nsplit > 1 && !part)) return hipErrorInvalidValue;
    const auto xx = static_cast<const uint16_t*>(x);
    const auto ww = static_cast<const uint16_t*>(w);
    auto oo = static_cast<uint16_t*>(out);
    const int t = static_cast<int>(T), k = static_cast<int>(K), n = static_cast<int>(N);
    // with a split, the start event goes on the GEMM and the stop event on the reduction
    hipEvent_t stop = pl.nsplit > 1 ? nullptr : ev.stop;
    const TiledFn fn = tiled_fn(pl.bm, pl.bn);
    if (!fn) return hipErrorInvalidValue;
    const int ntb = (t + pl.bm - 1) / pl.bm, nfb = n / pl.bn;
    const int blocks = ntb * nfb * pl.nsplit;
    const int grid = (blocks + 7) / 8 * 8;
    hipExtLaunchKernelGGL(fn, dim3(grid), dim3(kThreads), 0, stream, ev.start, stop, 0, xx, ww, oo, part, t, k,
                          n, ntb, nfb, pl.nsplit);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || pl.nsplit == 1) return e;
    const int64_t n4 = T * N / 4;
    hipExtLaunchKernelGGL(reduce_kernel, dim3(static_cast<unsigned>((n4 + 255) / 256)), dim3(256), 0, stream,
                          nullptr, ev.stop, 0, part, oo, n4, T * N, pl.nsplit);
    return hipGetLastError();
}

}  // namespace ca

// attn_chunk.hip -- causal paged attention for the prefill-chunk rows of a mixed step (bf16,
// MFMA, K/V pages staged in LDS), plus the merge of key splits.
//
// What it computes: pinghaoyang.com.cn "Sarathi-Serve 完全拆解", section "分块不等于截断上下文" --
// the chunk's query at absolute position p attends to keys 0..p of its request: the history pages
// written by earlier chunks and the pages the current chunk was just appended to, with the causal
// mask inside the chunk.  bowenzhou.top "Sarathi：让解码搭上 prefill 的顺风车", section
// "Chunked-prefills" notes that every later chunk re-reads the earlier chunks' K/V; here those
// reads are whole 4 KB (page, kv head) runs, coalesced, and shared by every query column of the
// workgroup through LDS.
//
// Work item = (sequence, kv head, block of rows, key range).  A workgroup is 4 wavefronts; each
// owns 64 query columns, a column being one (row, q head) pair of the kv head's group, so one K/V
// tile in LDS serves 4 x 64 columns.  Per 32-key block (two pages): the workgroup copies the two
// K pages and two V pages (16 KB) from HBM into LDS with 16-byte global->LDS DMA loads (no
// registers), issued for the next block before the current one is consumed; each wave then runs
// S^T = K Q^T and O^T = V^T P^T on
// v_mfma_f32_16x16x32_bf16 with an online softmax per column.  K rows in LDS are XOR-swizzled
// in 16-byte units so that the 16 keys an MFMA fragment reads fall on distinct banks.
// Only blocks that cross a row's diagonal need the mask; keys past a column's position get
// weight 0 and slots past the sequence end are zeroed before they reach the MFMA.

#include <hip/hip_runtime.h>

#include <cmath>

#include "internal.h"
#include "mfma.h"

namespace ca {
namespace {

constexpr int kWaves = 4;
constexpr int kTiles = 4;  // 16-column MFMA tiles per wave -> 64 columns
constexpr int kMaxItemPages = 2048;  // page ids of one workgroup's key range kept in LDS

// 16-byte unit swizzle of K row `key` (block key 0..31): spreads the 16 rows an S^T fragment
// reads (keys 8a + 4t + b, a, b in 0..3) over 16 distinct units.
__device__ __forceinline__ int kswz(int key) { return (key & 3) | (((key >> 3) & 3) << 2); }

// One stage = K block (32 keys x D, 16-byte units swizzled per key) then V block
// (2 pages x [d][16 slots]) = 64 D halves.  The two stages are separate __shared__ objects so
// the compiler can tell that the DMA filling one never aliases reads of the other (with one
// array indexed at run time it waits for every DMA before any LDS read).
__device__ __forceinline__ bf16x8 lds_frag(const uint16_t* p) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    bf16x8 r;
    __builtin_memcpy(&r, &v, sizeof(r));
    return r;
}


// Copy one 32-key block straight from HBM into LDS stage `stage` (16-byte DMA per lane, no
// registers).  The stage holds 8D 16-byte units: K units first (key-major, D/8 per key), then
// the two V pages.  Wave w, instruction u fills the contiguous units (w*U + u)*64 + lane; the
// lane picks the global unit that belongs there, which applies the K swizzle on the load side.
template <int D>
__device__ __forceinline__ void dma_block(uint16_t* stage, const uint16_t* __restrict__ k_cache,
                                          const uint16_t* __restrict__ v_cache, int pa, int pb,
                                          int g, int hkv, int w, int lane) {
    constexpr int U = 8 * D / 256;  // instructions per wave
    constexpr int KUNITS = 32 * D / 8;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int first = (w * U + u) * 64;
        const int x = first + lane;
        const uint16_t* src;
        if (x < KUNITS) {
            const int key = x / (D / 8);
            const int phys = x - key * (D / 8);
            const int unit = phys ^ (kswz(key) & (D / 8 - 1));
            const int page = (key >> 4) ? pb : pa;
            src = k_cache + ((static_cast<int64_t>(page) * hkv + g) * 16 + (key & 15)) * D + 8 * unit;
        } else {
            const int y = x - KUNITS;
            const int page = (y >= 2 * D) ? pb : pa;
            const int off = (y >= 2 * D) ? y - 2 * D : y;
            src = v_cache + (static_cast<int64_t>(page) * hkv + g) * 16 * D + 8 * off;
        }
        __builtin_amdgcn_global_load_lds(src, stage + 8 * first, 16, 0, 0);
    }
}

// items: two int4 per item: {seq, kv head, first row of the block, partial slot or -1},
//                           {key begin, key end, 0, 0}
template <int D>
__global__ void __launch_bounds__(64 * kWaves) chunk_kernel(
    DevPlan p, const int4* __restrict__ items, int rows_per_wave,
    const uint16_t* __restrict__ qg, const uint16_t* __restrict__ k_cache,
    const uint16_t* __restrict__ v_cache, int hq, int hkv, float scale_log2,
    float* __restrict__ part_acc, float2* __restrict__ part_ml, uint16_t* __restrict__ o,
    float* __restrict__ lse) {
    __shared__ __attribute__((aligned(16))) uint16_t stage0[64 * D];
    __shared__ __attribute__((aligned(16))) uint16_t stage1[64 * D];
    __shared__ int s_pages[kMaxItemPages];  // the item's page ids, so a block's ids are an LDS read
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int c = lane & 15, q = lane >> 4;
    const int4 it0 = items[2 * blockIdx.x];
    const int4 it1 = items[2 * blockIdx.x + 1];
    const int s = it0.x, g = it0.y, rb = it0.z, slot = it0.w;
    const int kb = it1.x, ke = it1.y;
    if (s < 0) return;  // grid padding (uniform across the workgroup)
    const int G = hq / hkv;
    const int P = 16;
    const int32_t* pages = p.kv_page_indices + p.kv_page_indptr[s];
    const int np = p.kv_page_indptr[s + 1] - p.kv_page_indptr[s];
    const int kv_len = (np - 1) * P + p.kv_last_page_len[s];
    const int q0 = p.qo_indptr[s];
    const int q_len = p.qo_indptr[s + 1] - q0;
    const int pos0 = kv_len - q_len;  // position of the chunk's first row
    // page ids of the item's key range [kb, ke) plus the page after it (clamped to the sequence)
    const int lp0 = kb >> 4;
    const int nlp = min(((ke + 31) >> 4) - lp0, np - lp0);  // <= kMaxItemPages (host-checked)
    for (int i = tid; i < nlp; i += 64 * kWaves) s_pages[i] = pages[lp0 + i];
    auto page_pair = [&](int key0, int* pa, int* pb) {
        const int lp = (key0 >> 4) - lp0;
        *pa = s_pages[lp];
        *pb = (lp0 + lp + 1 < np) ? s_pages[lp + 1] : *pa;  // a missing page is masked, never used
    };

    // columns of this wave: tile nt, column c -> (row, head) = (cw / G, cw % G), cw = 16 nt + c
    bf16x8 qf[kTiles][D / 32];
    int lim[kTiles];     // last key this column may see inside the item (-1: padding column)
    int wmin = 0x7fffffff;  // smallest lim over the wave's real columns
#pragma unroll
    for (int nt = 0; nt < kTiles; ++nt) {
        const int cw = 16 * nt + c;
        const int r = cw / G, j = cw - (cw / G) * G;
        const int row = rb + w * rows_per_wave + r;
        const bool ok = r < rows_per_wave && row < q_len;
        lim[nt] = ok ? min(pos0 + row, ke - 1) : -1;
        if (ok) wmin = min(wmin, lim[nt]);
        const uint16_t* qp = qg + (static_cast<int64_t>(q0 + (ok ? row : 0)) * hq + g * G + (ok ? j : 0)) * D + 8 * q;
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) qf[nt][kk] = ok ? load_frag(qp + 32 * kk) : zero_frag();
    }
#pragma unroll
    for (int o_ = 32; o_ >= 1; o_ >>= 1) wmin = min(wmin, __shfl_xor(wmin, o_, 64));

    floatx4 acc[kTiles][D / 16];
    float m[kTiles], l[kTiles];
#pragma unroll
    for (int nt = 0; nt < kTiles; ++nt) {
        m[nt] = -INFINITY;
        l[nt] = 0.0f;
#pragma unroll
        for (int mt = 0; mt < D / 16; ++mt) acc[nt][mt] = floatx4{0.f, 0.f, 0.f, 0.f};
    }

    // One 32-key block held in LDS stage `stg`.  Blocks wholly inside every column's visible
    // range (the common case) skip the causal mask; the mask test is wave-uniform.
    auto consume = [&](const uint16_t* stg, int key0) {
        floatx4 st[kTiles][2];
#pragma unroll
        for (int nt = 0; nt < kTiles; ++nt) st[nt][0] = st[nt][1] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int key = ((c >> 2) << 3) + 4 * t + (c & 3);
#pragma unroll
            for (int kk = 0; kk < D / 32; ++kk) {
                const int phys = (4 * kk + q) ^ (kswz(key) & (D / 8 - 1));
                const bf16x8 kf = lds_frag(stg + key * D + 8 * phys);
#pragma unroll
                for (int nt = 0; nt < kTiles; ++nt) st[nt][t] = mfma16x16x32(kf, qf[nt][kk], st[nt][t]);
            }
        }
        const bool full = key0 + 31 <= wmin;
        bf16x8 pf[kTiles];
#pragma unroll
        for (int nt = 0; nt < kTiles; ++nt) {
            float sc[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sc[i] = st[nt][0][i];
                sc[4 + i] = st[nt][1][i];
            }
            if (!full) {
                const int valid = lim[nt] - (key0 + 8 * q) + 1;
#pragma unroll
                for (int j = 0; j < 8; ++j) sc[j] = (j < valid) ? sc[j] : -INFINITY;
            }
            float bm = sc[0];
#pragma unroll
            for (int j = 1; j < 8; ++j) bm = fmaxf(bm, sc[j]);
            bm = fmaxf(bm, __shfl_xor(bm, 16, 64));
            bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
            bm *= scale_log2;
            const bool grow = bm > m[nt] + kRescaleSlack;
            if (__any(grow)) {
                const float alpha = grow ? exp2_fast(m[nt] - bm) : 1.0f;
                l[nt] *= alpha;
#pragma unroll
                for (int mt = 0; mt < D / 16; ++mt) acc[nt][mt] *= alpha;
                m[nt] = grow ? bm : m[nt];
            }
            const float m_use = (m[nt] == -INFINITY) ? 0.0f : m[nt];  // column with no key yet
            float pr[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                pr[j] = exp2_fast(__builtin_fmaf(sc[j], scale_log2, -m_use));
                l[nt] += pr[j];
            }
            pf[nt] = pack_frag(pr);
        }
        // O^T += V^T P^T; V fragments are read once and reused by all 4 tiles.  Slots past the
        // sequence end are zeroed (a stale or NaN slot must not meet p = 0).
        const bool vtail = key0 + 32 > kv_len;
        const int vvalid = kv_len - (key0 + 8 * q);
#pragma unroll
        for (int mt = 0; mt < D / 16; ++mt) {
            bf16x8 vf = lds_frag(stg + 32 * D + (q >> 1) * 16 * D + (16 * mt + c) * 16 + 8 * (q & 1));
            if (vtail) vf = mask_frag(vf, vvalid);
#pragma unroll
            for (int nt = 0; nt < kTiles; ++nt) acc[nt][mt] = mfma16x16x32(vf, pf[nt], acc[nt][mt]);
        }
    };

    // Two LDS stages, loop unrolled by two so each half names its stage at compile time: the
    // DMA for block i+1 (into one stage) runs while block i is consumed from the other; one
    // wait + barrier per block makes the DMA visible and frees the consumed stage.
    const int nblk = (ke - kb + 31) >> 5;
    __syncthreads();  // page ids in LDS
    int pa, pb;
    page_pair(kb, &pa, &pb);
    dma_block<D>(stage0, k_cache, v_cache, pa, pb, g, hkv, w, lane);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int bi = 0; bi < nblk; bi += 2) {
        const int key0 = kb + 32 * bi;
        if (bi + 1 < nblk) {
            page_pair(key0 + 32, &pa, &pb);
            dma_block<D>(stage1, k_cache, v_cache, pa, pb, g, hkv, w, lane);
        }
        consume(stage0, key0);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (bi + 1 >= nblk) break;
        if (bi + 2 < nblk) {
            page_pair(key0 + 64, &pa, &pb);
            dma_block<D>(stage0, k_cache, v_cache, pa, pb, g, hkv, w, lane);
        }
        consume(stage1, key0 + 32);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }

#pragma unroll
    for (int nt = 0; nt < kTiles; ++nt) {
        float lt = l[nt];
        lt += __shfl_xor(lt, 16, 64);
        lt += __shfl_xor(lt, 32, 64);
        const int cw = 16 * nt + c;
        const int r = cw / G, j = cw - (cw / G) * G;
        const int row = rb + w * rows_per_wave + r;
        if (!(r < rows_per_wave && row < q_len)) continue;
        const int h = g * G + j;
        const int64_t orow = static_cast<int64_t>(q0 + row) * hq + h;
        if (slot < 0) {
            const float inv = 1.0f / lt;
            uint16_t* op = o + orow * D + 4 * q;
#pragma unroll
            for (int mt = 0; mt < D / 16; ++mt) {
                const uint32_t lo = f2bf(acc[nt][mt][0] * inv) | (static_cast<uint32_t>(f2bf(acc[nt][mt][1] * inv)) << 16);
                const uint32_t hi = f2bf(acc[nt][mt][2] * inv) | (static_cast<uint32_t>(f2bf(acc[nt][mt][3] * inv)) << 16);
                *reinterpret_cast<uint2*>(op + 16 * mt) = make_uint2(lo, hi);
            }
            if (lse && q == 0) lse[orow] = (m[nt] + __log2f(lt)) * 0.69314718055994531f;
        } else {
            const int64_t col = static_cast<int64_t>(slot) * (64 * kWaves) + 64 * w + cw;
            float* ap = part_acc + col * D + 4 * q;
#pragma unroll
            for (int mt = 0; mt < D / 16; ++mt)
                *reinterpret_cast<float4*>(ap + 16 * mt) = make_float4(acc[nt][mt][0], acc[nt][mt][1], acc[nt][mt][2], acc[nt][mt][3]);
            if (q == 0) part_ml[col] = make_float2(m[nt], lt);
        }
    }
}

// One wavefront per (row block, column): combine the column's key splits.  A split that saw
// no key of the column has l = 0 and is skipped.  groups: two int4 per row block,
// {seq, kv head, first row of the block, first slot}, {number of splits, 0, 0, 0}.
template <int D>
__global__ void __launch_bounds__(256) chunk_merge_kernel(
    DevPlan p, const int4* __restrict__ groups, int num_groups, int rows_per_wave,
    const float* __restrict__ part_acc, const float2* __restrict__ part_ml, int hq, int hkv,
    uint16_t* __restrict__ o, float* __restrict__ lse) {
    constexpr int COLS = 64 * kWaves;
    const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (wid >= num_groups * COLS) return;
    const int grp = wid / COLS, col = wid - grp * COLS;
    const int4 g0 = groups[2 * grp];
    const int nsplit = groups[2 * grp + 1].x;
    const int s = g0.x, g = g0.y, rb = g0.z, first = g0.w;
    const int G = hq / hkv;
    const int q0 = p.qo_indptr[s];
    const int q_len = p.qo_indptr[s + 1] - q0;
    const int lane = threadIdx.x & 63;
    const int w = col >> 6, cw = col & 63;
    const int r = cw / G, j = cw - (cw / G) * G;
    const int row = rb + w * rows_per_wave + r;
    if (!(r < rows_per_wave && row < q_len)) return;
    // lane k holds split k's (max, sum); splits never exceed 64 here (checked on the host)
    float2 ml = make_float2(-INFINITY, 0.0f);
    if (lane < nsplit) ml = part_ml[static_cast<int64_t>(first + lane) * COLS + col];
    float mx = ml.y > 0.0f ? ml.x : -INFINITY;
#pragma unroll
    for (int o_ = 32; o_ >= 1; o_ >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o_, 64));
    const float wk = ml.y > 0.0f ? exp2_fast(ml.x - mx) : 0.0f;
    float L = wk * ml.y;
#pragma unroll
    for (int o_ = 32; o_ >= 1; o_ >>= 1) L += __shfl_xor(L, o_, 64);
    float a[D / 64] = {};
    const float* base = part_acc + (static_cast<int64_t>(first) * COLS + col) * D + lane;
#pragma unroll 4
    for (int k = 0; k < nsplit; ++k) {
        const float wgt = __shfl(wk, k, 64);
#pragma unroll
        for (int e = 0; e < D / 64; ++e) a[e] += wgt * base[static_cast<int64_t>(k) * COLS * D + 64 * e];
    }
    const int64_t orow = static_cast<int64_t>(q0 + row) * hq + g * G + j;
    const float inv = 1.0f / L;
#pragma unroll
    for (int e = 0; e < D / 64; ++e) o[orow * D + lane + 64 * e] = f2bf(a[e] * inv);
    if (lse && lane == 0) lse[orow] = (mx + __log2f(L)) * 0.69314718055994531f;
}

}  // namespace

int chunk_cols_per_block() { return 64 * kWaves; }
int chunk_max_split_keys() { return 16 * (kMaxItemPages - 2); }

hipError_t launch_chunk(const DevPlan& p, const Shape& sh, const int4* items, int num_items,
                        int rows_per_wave, const void* q, const void* k_cache, const void* v_cache,
                        float* part_acc, float2* part_ml, void* o, float* lse, hipStream_t stream) {
    if (num_items <= 0) return hipSuccess;
    const float scale_log2 = sh.scale * 1.4426950408889634f;
    auto qq = static_cast<const uint16_t*>(q);
    auto kc = static_cast<const uint16_t*>(k_cache);
    auto vc = static_cast<const uint16_t*>(v_cache);
    auto oo = static_cast<uint16_t*>(o);
    if (sh.d == 128)
        hipLaunchKernelGGL(chunk_kernel<128>, dim3(num_items), dim3(64 * kWaves), 0, stream, p, items,
                           rows_per_wave, qq, kc, vc, sh.hq, sh.hkv, scale_log2, part_acc, part_ml, oo, lse);
    else
        hipLaunchKernelGGL(chunk_kernel<64>, dim3(num_items), dim3(64 * kWaves), 0, stream, p, items,
                           rows_per_wave, qq, kc, vc, sh.hq, sh.hkv, scale_log2, part_acc, part_ml, oo, lse);
    return hipGetLastError();
}

hipError_t launch_chunk_merge(const DevPlan& p, const Shape& sh, const int4* groups, int num_groups,
                              int rows_per_wave, const float* part_acc, const float2* part_ml,
                              void* o, float* lse, hipStream_t stream) {
    if (num_groups <= 0) return hipSuccess;
    auto oo = static_cast<uint16_t*>(o);
    const dim3 grid((num_groups * 64 * kWaves + 3) / 4);
    if (sh.d == 128)
        hipLaunchKernelGGL(chunk_merge_kernel<128>, grid, dim3(256), 0, stream, p, groups, num_groups,
                           rows_per_wave, part_acc, part_ml, sh.hq, sh.hkv, oo, lse);
    else
        hipLaunchKernelGGL(chunk_merge_kernel<64>, grid, dim3(256), 0, stream, p, groups, num_groups,
                           rows_per_wave, part_acc, part_ml, sh.hq, sh.hkv, oo, lse);
    return hipGetLastError();
}

}  // namespace ca

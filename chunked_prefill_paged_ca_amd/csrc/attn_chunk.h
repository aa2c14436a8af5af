// attn_chunk.h -- causal paged attention for the prefill-chunk rows of a mixed step (bf16,
// MFMA, K/V pages staged in LDS): the per-workgroup work item, run by the attention kernel in
// attn_mixed.hip.  The merge of key splits is in merge.hip.
//
// What it computes: pinghaoyang.com.cn "Sarathi-Serve 完全拆解", section "分块不等于截断上下文" --
// the chunk's query at absolute position p attends to keys 0..p of its request: the history pages
// written by earlier chunks and the pages the current chunk was just appended to, with the causal
// mask inside the chunk.  bowenzhou.top "Sarathi：让解码搭上 prefill 的顺风车", section
// "Chunked-prefills" notes that every later chunk re-reads the earlier chunks' K/V; here those
// reads are whole 4 KB (page, kv head) runs, coalesced, and shared by every query column of the
// workgroup through LDS.
//
// Work item = (sequence, kv head, block of 256 query columns, key range).  A query column is one
// (row, q head) pair of the kv head's group, numbered row * G + head, so any group size packs the
// MFMA tiles without padding.  A workgroup is 8 wavefronts of 32 columns (two waves per SIMD:
// one wave's softmax overlaps the other's MFMAs), and one K/V tile in LDS serves all 256
// columns.  Per 32-key block (two pages) the workgroup copies the two K pages and two V pages
// (16 KB) from HBM into LDS with 16-byte global->LDS DMA loads (no registers), issued by one
// wave per SIMD while the SIMD's other wave computes; the blocks are
// copied and published four at a time (a 128-key LDS stage, one barrier each), the next stage
// in flight while one is consumed.  Each wave runs S^T = K Q^T and O^T = V^T P^T on
// v_mfma_f32_16x16x32_bf16 with an online softmax per column.  The pages keep
// their cache layout in LDS, where every fragment read is a bank-conflict-free contiguous run.
// Only blocks that cross a row's diagonal need the mask; keys past a column's position get
// weight 0, and V slots past the sequence end are zeroed in LDS before they reach the MFMA.

#pragma once

#include <hip/hip_runtime.h>

#include <cmath>

#include "internal.h"
#include "mfma.h"

namespace ca {
namespace chunk {

constexpr int kWaves = 8;
constexpr int kTiles = 2;  // 16-column MFMA tiles per wave -> 32 columns
constexpr int kCols = 16 * kTiles * kWaves;  // 256 columns per workgroup
constexpr int kMaxItemPages = 2048;  // page ids of one workgroup's key range kept in LDS

// One stage = the block's four page runs as they lie in the caches: K page a, K page b, V page
// a, V page b (16 D halves each, 64 D in all).  With the cache layouts every MFMA fragment read
// from a stage is then a contiguous run across the wave (16 bytes per lane for K, 8 bytes per
// lane and page for V), which is free of LDS bank conflicts without any swizzle.  The stages are
// separate __shared__ objects so the compiler can tell that the DMA filling one never aliases
// reads of another (with one array indexed at run time it waits for every DMA before any LDS
// read).

__device__ __forceinline__ bf16x8 lds_frag(const uint16_t* p) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    bf16x8 r;
    __builtin_memcpy(&r, &v, sizeof(r));
    return r;
}

__device__ __forceinline__ bf16x8 lds_frag_pair(const uint16_t* a, const uint16_t* b) {
    const uint2 x = *reinterpret_cast<const uint2*>(a);
    const uint2 y = *reinterpret_cast<const uint2*>(b);
    const uint4 v = make_uint4(x.x, x.y, y.x, y.y);
    bf16x8 r;
    __builtin_memcpy(&r, &v, sizeof(r));
    return r;
}

// Copy one 32-key block straight from HBM into LDS stage `stage` (16-byte DMA per lane, no
// registers).  The stage holds 8D 16-byte units, 2D per page run; copying wave w's instruction
// u fills the contiguous units (w*U + u)*64 + lane, all inside one run (2D is a multiple of 64),
// so every instruction copies 1 KB of one page run.  Only waves 0-3 copy, one per SIMD: a SIMD's
// vector-memory path takes ~15 bytes per clock, so issuing a stage's copies holds the issuing
// wave for ~1,000 cycles, and with one copying wave per SIMD the SIMD's other wave keeps the
// matrix core busy meanwhile (measured: Yi-34B chunk 459-466 -> 453-459 us, LLaMA2-70B chunk
// 285-287 -> 271-274 us, Llama-13B one-shot 757-791 -> 742-754 us; copies by two waves only
// took twice as long, by all eight or by halves alternating per stage no better).
constexpr int kCopyWaves = 4;
template <int D>
__device__ __forceinline__ void dma_block(uint16_t* stage, const uint16_t* __restrict__ k_cache,
                                          const uint16_t* __restrict__ v_cache, int pa, int pb,
                                          int g, int hkv, int w, int lane) {
    constexpr int U = 8 * D / (64 * kCopyWaves);  // instructions per copying wave
    static_assert(kCopyWaves <= kWaves && U >= 1, "copy split");
    if (w >= kCopyWaves) return;  // wave-uniform
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int first = (w * U + u) * 64;
        const int run = first / (2 * D);  // 0, 1: K of pages a, b; 2, 3: V of pages a, b
        const int page = (run & 1) ? pb : pa;
        const uint16_t* src = (run < 2 ? k_cache : v_cache) + (static_cast<int64_t>(page) * hkv + g) * 16 * D +
                              8 * (first - run * 2 * D + lane);
        __builtin_amdgcn_global_load_lds(src, stage + 8 * first, 16, 0, 0);
    }
}

// One LDS stage holds kSub 32-key blocks; each block keeps the four-run layout above.  kStages
// stages rotate: one is consumed while the others are in flight.  Measured on the part: the
// workgroup barrier, not the copy, is what the stage size trades against -- with one barrier
// per 32, 64, 96 and 128 keys the Yi-34B chunk took 588, 551, 523 and 502 us (192, 192, 96 and
// 64 KB in flight) -- so the stages are as large as LDS allows two of (2 x 64 KB at d = 128).
constexpr int kSub = 4;
constexpr int kStages = 2;
template <int D>
constexpr int kStageHalves = kSub * 64 * D;

// s_waitcnt immediate: wait until at most n vector memory operations are outstanding and
// every LDS read has returned (expcnt not waited for)
constexpr int waitcnt_vm_lgkm0(int n) { return (n & 0xf) | (0x7 << 4) | ((n >> 4) << 14); }

// items: two int4 per item: {seq, kv head, first column (row * G + head), partial slot or -1},
//                           {key begin, key end, 0, 0}   (seq -1: grid padding)
template <int D>
__device__ __forceinline__ void chunk_item(
    int item, DevPlan p, const int4* __restrict__ items,
    const uint16_t* __restrict__ qg, const uint16_t* __restrict__ k_cache,
    const uint16_t* __restrict__ v_cache, int hq, int hkv, float scale_log2,
    float* __restrict__ part_acc, float2* __restrict__ part_ml, uint16_t* __restrict__ o,
    float* __restrict__ lse) {
    __shared__ __attribute__((aligned(16))) uint16_t stage0[kStageHalves<D>];
    __shared__ __attribute__((aligned(16))) uint16_t stage1[kStageHalves<D>];
    __shared__ __attribute__((aligned(16))) uint16_t stage2[kStageHalves<D>];
    __shared__ __attribute__((aligned(16))) uint16_t stage3[kStageHalves<D>];
    // the item's page ids, so a stage's ids are one LDS read (at most 2048 pages: an item has at
    // most 1024 blocks, so the last stage's eight ids end at entry 2048; two spare entries)
    __shared__ __attribute__((aligned(16))) int s_pages[kMaxItemPages + 2];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 15, q = lane >> 4;
    const int4 it0 = items[2 * item];
    const int4 it1 = items[2 * item + 1];
    const int s = it0.x, g = it0.y, cb = it0.z, slot = it0.w;
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
    const int ncols = q_len * G;
    // page ids of the item's key range [kb, ke) plus the page after it (clamped to the sequence)
    const int lp0 = kb >> 4;
    const int nlp = min(((ke + 31) >> 4) - lp0, np - lp0);  // <= kMaxItemPages (host-checked)
    for (int i = tid; i < nlp; i += 64 * kWaves) s_pages[i] = pages[lp0 + i];

    // this wave's columns: tile nt, lane column c -> column cb + 32 w + 16 nt + c
    bf16x8 qf[kTiles][D / 32];
    int lim[kTiles];        // last key this column may see inside the item (-1: past the chunk)
    int wmin = 0x7fffffff;  // smallest lim over the wave's real columns
#pragma unroll
    for (int nt = 0; nt < kTiles; ++nt) {
        const int col = cb + 32 * w + 16 * nt + c;
        const bool ok = col < ncols;
        const int row = ok ? col / G : 0;
        const int j = ok ? col - row * G : 0;
        lim[nt] = ok ? min(pos0 + row, ke - 1) : -1;
        if (ok) wmin = min(wmin, lim[nt]);
        const uint16_t* qp = qg + (static_cast<int64_t>(q0 + row) * hq + g * G + j) * D + 8 * q;
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) qf[nt][kk] = ok ? load_frag(qp + 32 * kk) : zero_frag();
    }
#pragma unroll
    for (int o_ = 32; o_ >= 1; o_ >>= 1) wmin = min(wmin, __shfl_xor(wmin, o_, 64));
    // A wave whose 32 columns all lie past the chunk (the last column block of a chunk) only
    // helps with the copies and barriers; it skips the LDS reads, MFMAs and softmax.
    const bool active = wmin != 0x7fffffff;

    // Per column: running max m (log2 units), weight sum l (this lane's keys; summed over the
    // lane groups at the end) and the O^T accumulator.  m starts at a finite floor far below any
    // score, so a column that has seen no key yet needs no special case: its masked scores (-inf)
    // give weight 0, and the first real score always raises m.
    constexpr float kNoKey = -1.0e30f;
    floatx4 acc[kTiles][D / 16];
    float m[kTiles], l[kTiles];
#pragma unroll
    for (int nt = 0; nt < kTiles; ++nt) {
        m[nt] = kNoKey;
        l[nt] = 0.0f;
#pragma unroll
        for (int mt = 0; mt < D / 16; ++mt) acc[nt][mt] = floatx4{0.f, 0.f, 0.f, 0.f};
    }

    // The block loop is software-pipelined by one operand: block i's K fragments are read from
    // LDS while block i-1's PV MFMAs run, so the QK MFMAs of block i start as soon as the block
    // begins.  Per block: QK (K fragments already in registers) -> V fragment reads -> softmax
    // -> barrier (publishes block i+1, frees block i's stage) -> refill DMA -> block i+1's K
    // reads -> PV of block i.
    auto read_k = [&](bf16x8 (&kf)[2][D / 32], const uint16_t* stg) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int kk = 0; kk < D / 32; ++kk)
                // tile t = page t: row c = slot c, dims 32 kk + 8 q .. = 8-dim block 4 kk + q
                kf[t][kk] = lds_frag(stg + 16 * D * t + 512 * kk + 8 * lane);
    };
    auto qk = [&](const bf16x8 (&kf)[2][D / 32], floatx4 (&st)[kTiles][2]) {
#pragma unroll
        for (int nt = 0; nt < kTiles; ++nt) st[nt][0] = st[nt][1] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int kk = 0; kk < D / 32; ++kk)
#pragma unroll
                for (int nt = 0; nt < kTiles; ++nt) st[nt][t] = mfma16x16x32(kf[t][kk], qf[nt][kk], st[nt][t]);
    };
    // a V fragment's two halves (pages a and b) sit 16 D halves apart: read as one pair, kept
    // apart from the other fragments' reads so the pair is what gets merged into one
    // two-address LDS read, straight into the fragment's registers
    auto read_v = [&](bf16x8 (&vf)[D / 16], const uint16_t* stg) {
#pragma unroll
        for (int mt = 0; mt < D / 16; ++mt) {
            vf[mt] = lds_frag_pair(stg + 32 * D + 256 * mt + 4 * lane, stg + 48 * D + 256 * mt + 4 * lane);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // Online softmax of one block's scores into P^T fragments.  Blocks wholly inside every
    // column's visible range (the common case) skip the causal mask; the test is wave-uniform.
    auto softmax = [&](floatx4 (&st)[kTiles][2], int key0, bf16x8 (&pf)[kTiles]) {
        const bool full = key0 + 31 <= wmin;
#pragma unroll
        for (int nt = 0; nt < kTiles; ++nt) {
            float sc[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sc[i] = st[nt][0][i];
                sc[4 + i] = st[nt][1][i];
            }
            if (!full) {
                // keys key0 + 4q + j (page a) and key0 + 16 + 4q + j (page b) up to lim
                const int va = lim[nt] - (key0 + 4 * q) + 1;
                const int vb = va - 16;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    sc[jj] = (jj < va) ? sc[jj] : -INFINITY;
                    sc[4 + jj] = (jj < vb) ? sc[4 + jj] : -INFINITY;
                }
            }
            // Each lane checks its own 8 scores against the column's reference max; only when
            // some score of the wave exceeds it by more than the slack (the first block, and
            // rarely after) is the column max formed across the 4 lane groups and the
            // accumulator rescaled.  The common path needs no cross-lane traffic.
            float lmax = sc[0];
#pragma unroll
            for (int jj = 1; jj < 8; ++jj) lmax = fmaxf(lmax, sc[jj]);
            lmax *= scale_log2;
            if (__any(lmax > m[nt] + kRescaleSlack)) {
                float bm = rows_max(lmax);
                const bool grow = bm > m[nt] + kRescaleSlack;
                const float alpha = grow ? exp2_fast(m[nt] - bm) : 1.0f;
                l[nt] *= alpha;
#pragma unroll
                for (int mt = 0; mt < D / 16; ++mt) acc[nt][mt] *= alpha;
                m[nt] = grow ? bm : m[nt];
            }
            float pr[8];
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                pr[jj] = exp2_fast(__builtin_fmaf(sc[jj], scale_log2, -m[nt]));
                l[nt] += pr[jj];
            }
            pf[nt] = pack_frag(pr);
        }
    };
    // O^T += V^T P^T; each V fragment serves both tiles
    auto pv = [&](const bf16x8 (&vf)[D / 16], const bf16x8 (&pf)[kTiles]) {
#pragma unroll
        for (int mt = 0; mt < D / 16; ++mt)
#pragma unroll
            for (int nt = 0; nt < kTiles; ++nt) acc[nt][mt] = mfma16x16x32(vf[mt], pf[nt], acc[nt][mt]);
    };
    // The block holding the sequence's last key may carry stale (even non-finite) bytes in the
    // slots after it; they get p = 0, and 0 * NaN must not reach the accumulator, so those V
    // slots are zeroed in LDS once the block has landed (a wave-uniform, once-per-item branch).
    auto zero_v_tail = [&](uint16_t* stg, int key0) {
        if (key0 + 32 <= kv_len) return;
        const int first_bad = kv_len - key0;  // block slots [first_bad, 32) are past the end
        for (int i = tid; i < 2 * D * 16; i += 64 * kWaves) {
            // V page run element i: slot 4 ((i / 64) % 4) + i % 4 of page i / (16 D)
            const int slot = 16 * (i / (D * 16)) + 4 * ((i >> 6) & 3) + (i & 3);
            if (slot >= first_bad) stg[32 * D + i] = 0;
        }
        __syncthreads();
    };

    // kStages LDS stages of kSub 32-key blocks each, loop unrolled by kStages so each step
    // names its stages at compile time: while one stage is consumed the others are in flight
    // (DMA), which covers an L2/MALL or HBM round trip with several blocks of MFMA work.  One
    // wait and one barrier per stage (not per block): the wait covers only the stage about to be
    // read (the DMA count of the stages issued after it may stay outstanding), and the barrier
    // both publishes that stage and frees the one about to be refilled.
    static_assert(kStages >= 2 && kStages <= 4 && kSub >= 1 && kSub * (kStages - 2) <= 8, "stage shape");
    constexpr int U = 8 * D / (64 * kCopyWaves);  // DMA instructions per copying wave per 32-key block
    constexpr int SK = 32 * kSub;             // keys per stage
    const int nblk = (ke - kb + 31) >> 5;
    const int nst = (nblk + kSub - 1) / kSub;
    __syncthreads();  // page ids in LDS
    auto slot_of = [&](auto I) -> uint16_t* {
        constexpr int i = decltype(I)::value % kStages;
        if constexpr (i == 0) return stage0;
        else if constexpr (i == 1) return stage1;
        else if constexpr (i == 2) return stage2;
        else return stage3;
    };
    // copy stage si (its first min(kSub, blocks left) blocks) into `slot`.  The stage's 2 kSub
    // page ids are read from LDS at once (item ranges start on 32-key blocks, so the stage's
    // first page sits at lp = 2 kSub si past lp0, 16-byte aligned): one LDS round trip per stage
    // before its copies can be issued, not one per block.  Ids past the item's last page are
    // stale and never used (its blocks stop at nblk; a block's second page past the sequence is
    // replaced by its first and masked).
    auto dma_stage = [&](uint16_t* slot, int si) {
        static_assert(kSub == 4, "a stage's page ids are two int4");
        const int lp = 2 * kSub * si;
        const int4 ia = *reinterpret_cast<const int4*>(s_pages + lp);
        const int4 ib = *reinterpret_cast<const int4*>(s_pages + lp + 4);
        const int ids[2 * kSub] = {ia.x, ia.y, ia.z, ia.w, ib.x, ib.y, ib.z, ib.w};
#pragma unroll
        for (int j = 0; j < kSub; ++j) {
            if (kSub * si + j < nblk) {
                const int pa = ids[2 * j];
                const int pb = (lp0 + lp + 2 * j + 1 < np) ? ids[2 * j + 1] : pa;
                dma_block<D>(slot + 64 * D * j, k_cache, v_cache, pa, pb, g, hkv, w, lane);
            }
        }
    };
    // Wait until at most `later` blocks' DMAs of this wave are still outstanding and every LDS
    // read of this wave has returned, then an execution barrier.  __syncthreads() would also be
    // a release fence, which makes the compiler drain every outstanding DMA first; here
    // visibility is explicit: the waited-for stage's DMA is complete in every wave, and every
    // wave's reads of the stage about to be refilled have returned, when the barrier opens.  The
    // signal fence keeps the compiler from moving LDS accesses across it.
    auto wait_stage = [&](int later) {
        switch (later) {
            case 0: __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0)); break;
            case 1: __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(1 * U)); break;
            case 2: __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(2 * U)); break;
            case 3: __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(3 * U)); break;
            case 4: __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(4 * U)); break;
            case 5: __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(5 * U)); break;
            case 6: __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(6 * U)); break;
            case 7: __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(7 * U)); break;
            default: __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(8 * U)); break;
        }
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
    };
    // At step si's wait, stages 0 .. si+kStages-1 have been requested (blocks below
    // min(nblk, kSub (si + kStages))) and stage si+1 (blocks below kSub (si + 2)) must be
    // complete: the blocks requested after it may stay outstanding.
    auto later_blocks = [&](int si) { return max(0, min(nblk, kSub * (si + kStages)) - kSub * (si + 2)); };
    auto zero_stage_tail = [&](uint16_t* slot, int si) {
#pragma unroll
        for (int j = 0; j < kSub; ++j) zero_v_tail(slot + 64 * D * j, kb + SK * si + 32 * j);
    };
    // prologue: stages 0 .. kStages-2 requested, stage 0 waited for, then the last slot filled
#pragma unroll
    for (int i = 0; i + 1 < kStages; ++i)
        if (i < nst) dma_stage(i == 0 ? stage0 : i == 1 ? stage1 : stage2, i);
    wait_stage(max(0, min(nblk, kSub * (kStages - 1)) - kSub));  // stage 0 landed
    zero_stage_tail(stage0, 0);
    if (kStages - 1 < nst) dma_stage(slot_of(std::integral_constant<int, kStages - 1>{}), kStages - 1);

    // Stage si sits in `cur`, with its first block's K fragments already in kf; `nxt` holds
    // stage si+1; `cur` is refilled with stage si+kStages once every wave is past its reads.
    // Per block: QK -> V reads -> softmax -> (the next block's K reads) -> PV, so each block's K
    // reads go out under the previous block's PV MFMAs.  A wave whose columns all lie past the
    // chunk (ACT false: the last column block of a chunk) only helps with the copies and
    // barriers.
    bf16x8 kf[2][D / 32];
    auto step = [&](uint16_t* cur, uint16_t* nxt, int si, auto act) {
        constexpr bool ACT = decltype(act)::value;
        const int key0 = kb + SK * si;
        const int nb = min(kSub, nblk - kSub * si);  // blocks in this stage
        floatx4 st[kTiles][2];
        bf16x8 vf[D / 16];
        bf16x8 pf[kTiles];
        if constexpr (ACT) {
#pragma unroll
            for (int j = 0; j + 1 < kSub; ++j) {
                if (j < nb) {
                    qk(kf, st);
                    read_v(vf, cur + 64 * D * j);
                    softmax(st, key0 + 32 * j, pf);
                    if (j + 1 < nb) {
                        read_k(kf, cur + 64 * D * (j + 1));
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    pv(vf, pf);
                }
            }
            if (kSub - 1 < nb) {
                qk(kf, st);
                read_v(vf, cur + 64 * D * (kSub - 1));
                softmax(st, key0 + 32 * (kSub - 1), pf);
            }
        }
        __builtin_amdgcn_sched_barrier(0);  // the softmax completes before the barrier
        if (si + 1 < nst) {
            wait_stage(later_blocks(si));  // stage si+1 landed; later stages may still fly
            zero_stage_tail(nxt, si + 1);
            if (si + kStages < nst) dma_stage(cur, si + kStages);
            if constexpr (ACT) read_k(kf, nxt);
            __builtin_amdgcn_sched_barrier(0);  // the next block's K reads go out ahead of PV
        }
        if constexpr (ACT) {
            if (kSub - 1 < nb) pv(vf, pf);
        }
    };
    auto run = [&](auto act) {
        if constexpr (decltype(act)::value) read_k(kf, stage0);
        __builtin_amdgcn_sched_barrier(0);
        for (int si = 0; si < nst; si += kStages) {
            step(slot_of(std::integral_constant<int, 0>{}), slot_of(std::integral_constant<int, 1>{}), si, act);
            if (si + 1 >= nst) break;
            step(slot_of(std::integral_constant<int, 1>{}), slot_of(std::integral_constant<int, 2>{}), si + 1, act);
            if constexpr (kStages > 2) {
                if (si + 2 >= nst) break;
                step(slot_of(std::integral_constant<int, 2>{}), slot_of(std::integral_constant<int, 3>{}), si + 2, act);
            }
            if constexpr (kStages > 3) {
                if (si + 3 >= nst) break;
                step(slot_of(std::integral_constant<int, 3>{}), slot_of(std::integral_constant<int, 4>{}), si + 3, act);
            }
        }
    };
    if (active) run(std::true_type{});
    else run(std::false_type{});

#pragma unroll
    for (int nt = 0; nt < kTiles; ++nt) {
        const float lt = rows_sum(l[nt]);
        const int wc = 32 * w + 16 * nt + c;  // column within the workgroup
        const int col = cb + wc;
        if (col >= ncols) continue;
        const int row = col / G, j = col - (col / G) * G;
        const int64_t orow = static_cast<int64_t>(q0 + row) * hq + g * G + j;
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
            const int64_t pc = static_cast<int64_t>(slot) * kCols + wc;
            float* ap = part_acc + pc * D + 4 * q;
#pragma unroll
            for (int mt = 0; mt < D / 16; ++mt)
                *reinterpret_cast<float4*>(ap + 16 * mt) = make_float4(acc[nt][mt][0], acc[nt][mt][1], acc[nt][mt][2], acc[nt][mt][3]);
            if (q == 0) part_ml[pc] = make_float2(m[nt], lt);
        }
    }
}

}  // namespace chunk
}  // namespace ca

// attn_decode.h -- split-KV paged attention for the decode rows of a mixed step (bf16, MFMA):
// the per-wavefront work item, run by the attention kernel in attn_mixed.hip.
// The log-sum-exp merge of the splits is in merge.hip.
//
// What it computes: pinghaoyang.com.cn "Sarathi-Serve 完全拆解", section "分块不等于截断上下文" --
// a decode row is the query at position kv_len - 1; it attends to every key 0..kv_len-1 of its
// request.  Decode is bound by reading the whole history K/V once (magicnetworld.com
// "分块预填充与 Stall-free 调度", section 三: its arithmetic intensity is capped by the context
// length), so the kernel is organised around HBM traffic:
//   * the 32-key blocks of every (decode row, kv head), laid end to end, are cut into equal
//     shares, one per wavefront the chip holds at once, so every wave streams the same number of
//     bytes and there is no tail of short items; a share is a run of work items (decode row,
//     kv head, key range) processed back to back;
//   * the G query heads sharing a kv head are the columns of one MFMA tile, so each K/V byte is
//     read once for all of them;
//   * K and V fragments are loaded straight from HBM into registers, each load instruction one
//     contiguous run of a page (16 bytes per lane for K, 8 for V; the page layouts are chosen
//     for it), and the next 32-key block is requested before the current one is consumed
//     (register double buffer), so each wave keeps two blocks (16 KB) in flight; the loads
//     carry the non-temporal hint (each byte is read once per step), which keeps the stream
//     from displacing cached lines and measured ~10 % more read bandwidth on the part;
//   * QK^T and PV run on MFMA only so that the vector ALUs stay free: at G = 8 the fp32 vector
//     work of a VALU dot product would need most of the chip's non-packed vector rate just to keep
//     up with 8 TB/s of bf16 K/V.
// An item shorter than the whole context writes fp32 partials (unnormalised o, running max, sum);
// an item covering a whole (row, kv head) writes its normalised output directly.

#pragma once

#include <hip/hip_runtime.h>

#include <cmath>

#include "internal.h"
#include "mfma.h"

namespace ca {
namespace decode {

template <int D>
struct Block {
    bf16x8 k0[D / 32];  // S^T tile 0 (page a) A fragments, one per 32-dim k step
    bf16x8 k1[D / 32];  // S^T tile 1 (page b)
    bf16x8 v[D / 16];   // O^T A fragments, one per 16-dim output tile
};

// One 32-key block = pages pa, pb of kv head g.  Every load instruction of the wave reads one
// contiguous run: 1 KB (16 bytes per lane) of an 8-dim block of K, or 512 bytes (8 per lane) of
// a 16-dim block of V, the pair from pages a and b making one fragment.
template <int D>
__device__ __forceinline__ void load_block(Block<D>& b, const uint16_t* __restrict__ k_cache,
                                           const uint16_t* __restrict__ v_cache, int pa, int pb,
                                           int g, int hkv, int lane) {
    const int64_t ra = (static_cast<int64_t>(pa) * hkv + g) * 16 * D;
    const int64_t rb = (static_cast<int64_t>(pb) * hkv + g) * 16 * D;
    // tile row c = slot c, k = 8q + j = dim 32 kk + 8 q + j: 8-dim block 4 kk + q, slot c
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
        b.k0[kk] = load_frag_nt(k_cache + ra + 512 * kk + 8 * lane);
        b.k1[kk] = load_frag_nt(k_cache + rb + 512 * kk + 8 * lane);
    }
    // O^T row c = dim 16 mt + c, keys: slots 4q .. 4q+3 of page a, then of page b
#pragma unroll
    for (int mt = 0; mt < D / 16; ++mt)
        b.v[mt] = load_frag_pair_nt(v_cache + ra + 256 * mt + 4 * lane, v_cache + rb + 256 * mt + 4 * lane);
}

// One work item: the keys [kb, ke) of one (decode row, kv head).  rec0 = {kv head, kb, ke,
// partial slot or -1 for direct output}, rec1 = {row, offset of the row's page ids, page count, 0}.
template <int D>
__device__ __forceinline__ void decode_item(
    const int4 rec0, const int4 rec1, ConstPtr<int32_t> page_indices,
    const uint16_t* __restrict__ qg, const uint16_t* __restrict__ k_cache,
    const uint16_t* __restrict__ v_cache, int hq, int hkv, float scale_log2,
    float* __restrict__ part_acc, float2* __restrict__ part_ml, uint16_t* __restrict__ o,
    float* __restrict__ lse, int lane) {
    const int g = rec0.x, kb = rec0.y, ke = rec0.z, out = rec0.w;
    const int row = rec1.x;
    const ConstPtr<int32_t> pages = page_indices + rec1.y;
    const int np = rec1.z;
    const int G = hq / hkv;
    const int c = lane & 15, q = lane >> 4;

    // Q^T fragments: column c is q head g*G + c (zero beyond the group)
    bf16x8 qf[D / 32];
    {
        const uint16_t* qp = qg + (static_cast<int64_t>(row) * hq + g * G + (c < G ? c : 0)) * D + 8 * q;
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) qf[kk] = (c < G) ? load_frag(qp + 32 * kk) : zero_frag();
    }

    floatx4 acc[D / 16];
#pragma unroll
    for (int mt = 0; mt < D / 16; ++mt) acc[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, l = 0.0f;

    // One 32-key block: scores, online-softmax update, PV.  Lane group q holds the scores of
    // keys key0 + 4q .. key0 + 4q + 3 (page a) and key0 + 16 + 4q .. (page b) of query column c.
    // Only an item's last block can run past its end, so the masks are taken on that block alone
    // (the test is wave-uniform).
    auto consume = [&](const Block<D>& b, int key0) {
        floatx4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) {
            s0 = mfma16x16x32(b.k0[kk], qf[kk], s0);
            s1 = mfma16x16x32(b.k1[kk], qf[kk], s1);
        }
        const bool full = key0 + 32 <= ke;
        const int va = ke - (key0 + 4 * q);  // keys of this lane's page-a run inside the item
        const int vb = va - 16;               // and of its page-b run
        float sc[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sc[i] = s0[i];
            sc[4 + i] = s1[i];
        }
        if (!full) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                sc[j] = (j < va) ? sc[j] : -INFINITY;
                sc[4 + j] = (j < vb) ? sc[4 + j] : -INFINITY;
            }
        }
        float bm = sc[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) bm = fmaxf(bm, sc[j]);
        bm = rows_max(bm);
        bm *= scale_log2;  // finite: key0 < ke
        const bool grow = bm > m + kRescaleSlack;
        if (__any(grow)) {
            const float m_new = grow ? bm : m;
            const float alpha = exp2_fast(m - m_new);
            l *= alpha;
#pragma unroll
            for (int mt = 0; mt < D / 16; ++mt) acc[mt] *= alpha;
            m = m_new;
        }
        float pr[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            pr[j] = exp2_fast(__builtin_fmaf(sc[j], scale_log2, -m));
            l += pr[j];
        }
        const bf16x8 pf = pack_frag(pr);
        // slots past the item's end may hold stale or non-finite bytes: zero them so that
        // p = 0 cannot turn into 0 * NaN inside the MFMA
        if (full) {
#pragma unroll
            for (int mt = 0; mt < D / 16; ++mt) acc[mt] = mfma16x16x32(b.v[mt], pf, acc[mt]);
        } else {
#pragma unroll
            for (int mt = 0; mt < D / 16; ++mt) acc[mt] = mfma16x16x32(mask_frag(b.v[mt], va, vb), pf, acc[mt]);
        }
    };

    // Page ids of a 32-key block (two pages; past the sequence end the last page is read again
    // and never used).  They are scalar loads, fetched one block ahead of the K/V loads that
    // need them; the two loads are independent so that nothing waits for them before then.
    auto pages_of = [&](int key0, int& pa, int& pb) {
        const int lp = key0 >> 4 < np ? key0 >> 4 : np - 1;
        pa = pages[lp];
        pb = pages[lp + 1 < np ? lp + 1 : lp];
        // keep the scalar loads here, a block ahead: left alone, the scheduler sinks them to
        // just before their use and the wave then stalls on them with no K/V load issued
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
    };

    // Register double buffer: the next block's loads are in flight while a block is consumed.
    // Inside the loop every prefetch is unconditional (the last block or two are peeled off
    // below), so the compiler's load counter waits only for the block being consumed.
    const int nblk = (ke - kb + 31) >> 5;
    Block<D> ba, bb;
    int pa, pb;
    pages_of(kb, pa, pb);
    load_block<D>(ba, k_cache, v_cache, pa, pb, g, hkv, lane);
    if (nblk > 1) pages_of(kb + 32, pa, pb);
    int bi = 0;
    for (; bi + 2 < nblk; bi += 2) {
        load_block<D>(bb, k_cache, v_cache, pa, pb, g, hkv, lane);  // block bi + 1
        pages_of(kb + 32 * (bi + 2), pa, pb);
        consume(ba, kb + 32 * bi);
        load_block<D>(ba, k_cache, v_cache, pa, pb, g, hkv, lane);  // block bi + 2
        pages_of(kb + 32 * (bi + 3), pa, pb);  // clamped past the end, never used there
        consume(bb, kb + 32 * (bi + 1));
    }
    if (bi + 1 < nblk) {
        load_block<D>(bb, k_cache, v_cache, pa, pb, g, hkv, lane);
        consume(ba, kb + 32 * bi);
        consume(bb, kb + 32 * (bi + 1));
    } else {
        consume(ba, kb + 32 * bi);
    }
    l = rows_sum(l);

    if (c >= G) return;
    const int h = g * G + c;
    if (out < 0) {
        const float inv = 1.0f / l;
        uint16_t* op = o + (static_cast<int64_t>(row) * hq + h) * D + 4 * q;
#pragma unroll
        for (int mt = 0; mt < D / 16; ++mt) {
            const uint32_t lo = f2bf(acc[mt][0] * inv) | (static_cast<uint32_t>(f2bf(acc[mt][1] * inv)) << 16);
            const uint32_t hi = f2bf(acc[mt][2] * inv) | (static_cast<uint32_t>(f2bf(acc[mt][3] * inv)) << 16);
            *reinterpret_cast<uint2*>(op + 16 * mt) = make_uint2(lo, hi);
        }
        if (lse && q == 0) lse[static_cast<int64_t>(row) * hq + h] = (m + __log2f(l)) * 0.69314718055994531f;
    } else {
        float* ap = part_acc + (static_cast<int64_t>(out) * G + c) * D + 4 * q;
#pragma unroll
        for (int mt = 0; mt < D / 16; ++mt)
            *reinterpret_cast<float4*>(ap + 16 * mt) = make_float4(acc[mt][0], acc[mt][1], acc[mt][2], acc[mt][3]);
        if (q == 0) part_ml[static_cast<int64_t>(out) * G + c] = make_float2(m, l);
    }
}

}  // namespace decode
}  // namespace ca

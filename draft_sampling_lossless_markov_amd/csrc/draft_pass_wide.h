// draft_pass_wide.h -- the streaming draft pass (gfx950): per (request,
// 256-wide vocabulary tile) the partial of logit = base + E[prev] . W2^T for
// bf16 rows of 16-byte words -- what bias_pass_kernel<kSample | kGreedy>
// computes -- with two workgroups per CU.
//
// Four waves per workgroup, wave w owning 64 columns (two 32 x 32 MFMA tiles,
// its 128 W2 fragment registers held for the whole pass), within 256 registers
// a wave, so that two workgroups share a CU and each SIMD runs two waves.  A
// wave runs one block of 32 requests at a time -- its MFMA chain, then the
// block's logits and weights in place on the accumulators -- and the other
// workgroup's wave on the same SIMD fills what a single wave leaves idle (its
// MFMA chain while this one forms weights, its loads, LDS round trips and
// barrier waits).  Each embedding fragment read from LDS feeds two MFMAs.  A
// block's base logits and embedding rows are read a whole row segment per
// half-wave and reach the MFMA layout through LDS.
//
// Lane l holds request l % 32 of a block and, in tile t, the 16 contiguous
// columns [64 w + 32 t + 16 (l / 32), +16) (dp_arow maps MFMA rows to columns
// as for one 32-column tile).  Iteration i, one barrier: block i + 1's staged
// rows to LDS, block i + 2's logit words requested, block i's MFMA chain
// (sampling: block i - 1's last 16 weights among it, then its partial),
// logits, lane and wave maxima; barrier; block i + 2's embedding rows and block
// i + 3's tokens requested, block i - 1's partials merged and stored, block i's
// tile maximum taken and its first 16 weights summed.  All global traffic uses raw
// buffer instructions (draft_pass.h): rows past the end, bias rows that select
// none and idle lanes take out-of-range offsets, and a block's logit-word
// addresses are scalar.  Every logit is the same MFMA sequence (k-steps 0..15
// from zero) plus the base logit, as in the pick's tile rebuild; the weights
// take the tile maximum as their one reference.
#pragma once

#include "draft_pass.h"

namespace dsp {

constexpr int kDwWaves = 4;                  // waves per workgroup (two workgroups per CU)
constexpr int kDwThreads = 64 * kDwWaves;
constexpr int kDwRows = kPassBlock / (2 * kDwWaves);   // block rows a thread stages (E and logits)

union DraftWideLds {
    uint4 w2[2][64][kRankMax / 8];
    struct {
        uint16_t e[2][kPassBlock][kRankMax + kERowPad];
        uint16_t lg[2][kPassBlock][kVocabTile + kERowPad];
        Part red[2][kDwWaves][kPassBlock];
        float mx[2][kDwWaves][kPassBlock];
    } s;
};
static_assert(2 * sizeof(DraftWideLds) <= 160 * 1024, "two workgroups per CU share its 160 KB of LDS");

// The A fragments of wave w: tile t's W2 rows v0 + 64 w + 32 t + dp_arow(i),
// k-steps 0..15.  Quarter q (64 rows) of the tile is read contiguously into LDS
// and wave q takes both its tiles from it.
__device__ __forceinline__ void dw_stage_w2(const uint16_t* __restrict__ W2, int V, int r, int v0,
                                            DraftWideLds& L, bf16x8 (&a)[2][kKSteps])
{
    constexpr int kWordsRow = kRankMax / 8;                  // 32 words of 16 bytes
    constexpr int kPer = 64 * kWordsRow / kDwThreads;        // 8 words per quarter
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    uint4 cur[kPer], nxt[kPer];
    auto fetch = [&](int q, uint4* u) {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int f = i * kDwThreads + tid, rho = f / kWordsRow, c = f % kWordsRow;
            const int v = v0 + 64 * q + rho;
            u[i] = (v < V && 8 * c < r)
                       ? *reinterpret_cast<const uint4*>(W2 + (int64_t)v * r + 8 * c)
                       : make_uint4(0, 0, 0, 0);
        }
    };
    fetch(0, cur);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        if (q + 1 < 4) fetch(q + 1, nxt);
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int f = i * kDwThreads + tid, rho = f / kWordsRow, c = f % kWordsRow;
            L.w2[q & 1][rho][dp_slot(rho, c)] = cur[i];
        }
        lds_barrier();
        if (wave == q) {
            const int h = lane >> 5;
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int rho = 32 * t + dp_arow(lane & 31);
#pragma unroll
                for (int ks = 0; ks < kKSteps; ++ks)
                    a[t][ks] = as_bf16x8(L.w2[q & 1][rho][dp_slot(rho, 2 * ks + h)]);
            }
        }
#pragma unroll
        for (int i = 0; i < kPer; ++i) cur[i] = nxt[i];
    }
    lds_barrier();   // the buffers are reused for the embedding tiles
}

template <bool GREEDY, bool RNN>
__global__ __launch_bounds__(kDwThreads, 2) void draft_pass_wide_kernel(PassArgs a)
{
    __shared__ DraftWideLds L;
    auto& e_tile = L.s.e;
    auto& red = L.s.red;
    auto& mx = L.s.mx;
    if (a.ctl && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) a.ctl[0] = 0u;

    const int n_begin = blockIdx.y * a.req_per_wg;
    if (n_begin >= a.R) return;   // workgroup-uniform
    const int n_end = min(a.R, n_begin + a.req_per_wg);
    const int n_blk = (n_end - n_begin + kPassBlock - 1) / kPassBlock;

    const int vt = blockIdx.x;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int h = lane >> 5, c32 = lane & 31;
    const int V = a.V, r = a.r, gamma = a.gamma;
    // first of this lane's 16 columns in tile 0 (tile 1: 32 further)
    const int v_lane = vt * kVocabTile + 64 * wave + 16 * h;
    const Itl itL = fold_itl(a.inv_temp);

    bf16x8 afrag[2][kKSteps];
    dw_stage_w2(a.W2, V, r, vt * kVocabTile, L, afrag);

    // --- staging: thread t stages rows 8 w + 2 c + (l / 32), c < 4, word l % 32
    // of a block's embedding rows and of its logit rows (a half-wave reads one
    // whole row segment).  Rows past the end read zeros or row 0; their results
    // are never stored.
    const int sword = lane & 31;
    auto srow_of = [&](int c) { return 8 * wave + 2 * c + h; };
    const int kk = 8 * sword;
    const int cols = min(kVocabTile, V - vt * kVocabTile);

    const int32_t* tsrc = (a.k == 0) ? a.anchor : a.tok;
    const BufRsrc tok_rs = buf_rsrc(tsrc, (uint32_t)(a.R * ((a.k == 0) ? 1 : gamma)) * 4u);
    const uint32_t tstep = (uint32_t)(kPassBlock * ((a.k == 0) ? 1 : gamma)) * 4u;
    uint32_t toff = (uint32_t)((a.k == 0) ? n_begin + srow_of(0) : (n_begin + srow_of(0)) * gamma + (a.k - 1)) * 4u;
    const uint32_t tdc = (uint32_t)(2 * ((a.k == 0) ? 1 : gamma)) * 4u;   // rows 2 apart
    auto prev_raw = [&](int (&p)[kDwRows]) {
        if constexpr (!RNN) {
#pragma unroll
            for (int c = 0; c < kDwRows; ++c)
                p[c] = (int)__builtin_amdgcn_raw_buffer_load_b32(tok_rs, toff + c * tdc, 0, 0);
            toff += tstep;
        }
    };

    // embedding rows: a row outside [0, e_rows) -- a previous token outside the
    // vocabulary -- takes row e_rows, whose offset lies past the range (zeros);
    // columns past r take kBufOut
    const BufRsrc e_rsc = buf_rsrc(a.E, (uint32_t)((((int64_t)a.e_rows - 1) * a.e_rs + r) * 2));
    const uint32_t e_rs2 = (uint32_t)a.e_rs * 2u;
    const uint32_t kk2x = (kk < r) ? 2u * (uint32_t)kk : kBufOut;
    uint4 eu[kDwRows];
    auto load_e = [&](int blk, const int (&p)[kDwRows]) {
#pragma unroll
        for (int c = 0; c < kDwRows; ++c) {
            const int row = RNN ? n_begin + blk * kPassBlock + srow_of(c) : p[c];
            const uint32_t off = __umul24(min((uint32_t)row, (uint32_t)a.e_rows), e_rs2) + kk2x;
            eu[c] = buf_load16<0>(e_rsc, off);
        }
    };
    auto store_e = [&](auto Bc) {
        constexpr int b = decltype(Bc)::value;
#pragma unroll
        for (int c = 0; c < kDwRows; ++c) *reinterpret_cast<uint4*>(&e_tile[b][srow_of(c)][kk]) = eu[c];
    };

    const uint16_t* __restrict__ base = static_cast<const uint16_t*>(a.base);
    const uint32_t loff0 = (uint32_t)(srow_of(0) * a.bs.rs + kk) * 2u;
    const uint32_t ldc = (uint32_t)(2 * a.bs.rs) * 2u;   // rows 2 apart
    const uint16_t* lblk = base + (int64_t)n_begin * a.bs.rs + (int64_t)a.k * a.bs.ps + vt * kVocabTile;
    const int64_t lstep = (int64_t)kPassBlock * a.bs.rs;
    int lfirst = n_begin;
    uint4 rs[kDwRows];
    auto load_raw = [&]() {
        const int live = min(kPassBlock, n_end - lfirst);
        const uint32_t bytes = (live > 0) ? (uint32_t)(((int64_t)(live - 1) * a.bs.rs + cols) * 2) : 0u;
        const BufRsrc rb = buf_rsrc(lblk, bytes);
#pragma unroll
        for (int c = 0; c < kDwRows; ++c) rs[c] = buf_load16<kBufNt>(rb, loff0 + c * ldc);
        lblk += lstep;
        lfirst += kPassBlock;
    };
    const bool col_in = kk < cols;
    auto store_lg = [&](auto Bc) {
        constexpr int b = decltype(Bc)::value;
        if (cols < kVocabTile) {   // a partial tile (workgroup-uniform)
            constexpr uint32_t kNinf2 = 0xFF80FF80u;
            const uint32_t keep = col_in ? 0xFFFFFFFFu : 0u, put = kNinf2 & ~keep;
#pragma unroll
            for (int c = 0; c < kDwRows; ++c) {
                uint4& v = rs[c];
                v = make_uint4((v.x & keep) | put, (v.y & keep) | put, (v.z & keep) | put, (v.w & keep) | put);
            }
        }
#pragma unroll
        for (int c = 0; c < kDwRows; ++c) *reinterpret_cast<uint4*>(&L.s.lg[b][srow_of(c)][kk]) = rs[c];
    };

    // partials: lanes 0..7 of wave w store requests 8 w .. 8 w + 7 of a block.
    // A wave with no live row among them skips its stores: a store instruction
    // all of whose lanes fall out of range can retire ahead of older loads and
    // upset the waits on the in-order load counter.
    const uint32_t poff = (lane < 8) ? (uint32_t)((8 * wave + lane) * a.n_vt) * 16u : kBufOut;
    const uint32_t qoff = (lane < 8) ? (uint32_t)(8 * wave + lane) * 16u : kBufOut;
    // block j's partials (red[j % 2], written after the barrier of iteration j)
    // merged over the four waves and stored; j = -1 stores nothing
    const int jr = 8 * wave + (lane & 7);   // the request a lane merges
    auto merge = [&](int j, const Part (&pr)[kDwWaves]) {
        Part p = pr[0];
        float sq[kDwWaves];
        sq[0] = (float)p.s;
#pragma unroll
        for (int w = 1; w < kDwWaves; ++w) {
            const Part q = pr[w];
            if constexpr (GREEDY) {
                const ArgMax am = argmax_merge(ArgMax{p.m, p.idx}, ArgMax{q.m, q.idx});
                p.m = am.v;
                p.idx = am.i;
            } else {
                p.s += q.s;   // one reference (the tile maximum) throughout
                sq[w] = (float)q.s;
            }
        }
        const int n0 = n_begin + j * kPassBlock;
        const int live = (j >= 0) ? min(kPassBlock, n_end - n0) : 0;
        if (8 * wave < live) {
            Part* pb = a.part + (int64_t)n0 * a.n_vt + vt;
            const uint32_t pbytes = (uint32_t)(((int64_t)(live - 1) * a.n_vt + 1) * sizeof(Part));
            const BufRsrc rp = buf_rsrc(pb, pbytes);
            const uint64_t sb = (uint64_t)__double_as_longlong(p.s);
            const u32x4 pw = {__float_as_uint(p.m), (uint32_t)p.idx, (uint32_t)sb, (uint32_t)(sb >> 32)};
            __builtin_amdgcn_raw_buffer_store_b128(pw, rp, poff, 0, 0);
            if (!GREEDY && a.sub) {
                // the 64-column sums tile-major (sub[vt R + n]): a block's 32
                // requests are one contiguous 512-byte run
                const BufRsrc rq = buf_rsrc(a.sub + (int64_t)vt * a.R + n0, (uint32_t)live * 16u);
                const u32x4 qw = {__float_as_uint(sq[0]), __float_as_uint(sq[1]), __float_as_uint(sq[2]),
                                  __float_as_uint(sq[3])};
                __builtin_amdgcn_raw_buffer_store_b128(qw, rq, qoff, 0, 0);
            }
        }
    };

    // Sampling: a block's weights are summed in two halves -- slots 0..15 after
    // the barrier that publishes its maxima, slots 16..31 among the next block's
    // MFMAs, whose chain otherwise leaves the wave's VALU idle -- in two fp64
    // chains (even and odd slots, each in slot order).  Carried from one block
    // to the next: the last 16 logits, the reference, the tile maximum and the
    // two chains' sums.
    float zh[16], mh = 0.0f, mth = -INFINITY;
    double hc0 = 0.0, hc1 = 0.0;
#pragma unroll
    for (int s = 0; s < 16; ++s) zh[s] = -INFINITY;
    // the previous block's partial, once its second half is summed
    auto put_part = [&](auto Pc) {
        if constexpr (!GREEDY) {
            const Part res{mth, 0, xsum<32>(hc0 + hc1)};
            if (h == 0) red[decltype(Pc)::value][wave][c32] = res;
        }
    };

    // one block: its MFMA chain over e_tile[b] (sampling: the previous block's
    // second half of weights among it, its partial to red[Pc]), its logits (slot
    // s: tile s / 16, column s % 16) and lane maximum, and (sampling) the wave
    // maximum to mx[b]
    float z[32], m = -INFINITY;
    auto block_logits = [&](auto Bc, auto Pc) {
        constexpr int b = decltype(Bc)::value;
        const uint16_t* eb = &e_tile[b][c32][8 * h];
        floatx16 acc0 = floatx16{}, acc1 = floatx16{};
        // from here to the merge after the barrier the wave runs at raised issue
        // priority (the weights drop it): the other workgroup's wave on the SIMD
        // then fills its own weights into this wave's gaps rather than holding
        // back the chain, logits and maxima that all four waves of this
        // workgroup wait for at the barrier
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int ks = 0; ks < kKSteps; ++ks) {
            const bf16x8 bf = as_bf16x8(*reinterpret_cast<const uint4*>(eb + ks * kKStep));
            acc0 = mfma32_bf16(afrag[0][ks], bf, acc0);
            if constexpr (!GREEDY) {
                const double w = (double)wexp(zh[ks] - mh, itL);   // slot 16 + ks
                if (ks & 1) hc1 += w; else hc0 += w;
            }
            acc1 = mfma32_bf16(afrag[1][ks], bf, acc1);
        }
        if constexpr (!GREEDY) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
            for (int ks = 0; ks < kKSteps; ++ks) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (ks + 1 < kKSteps) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
            }
        }
        put_part(Pc);
        uint4 lw[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
            lw[q] = *reinterpret_cast<const uint4*>(&L.s.lg[b][c32][64 * wave + 32 * (q >> 1) + 16 * h + 8 * (q & 1)]);
#pragma unroll
        for (int s = 0; s < 16; ++s) {
            z[s] = Logit<uint16_t>::raw_at(lw + (s >> 3), s & 7) + acc0[s];
            z[16 + s] = Logit<uint16_t>::raw_at(lw + 2 + (s >> 3), s & 7) + acc1[s];
        }
        // lane maximum by a tree (five levels, not a chain of 31 dependent steps)
        float y[16];
#pragma unroll
        for (int s = 0; s < 16; ++s) y[s] = fmaxf(z[s], z[16 + s]);
#pragma unroll
        for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
            for (int s = 0; s < w; ++s) y[s] = fmaxf(y[s], y[s + w]);
        m = y[0];
        if constexpr (!GREEDY) {
            m = xmax<32>(m);
            if (h == 0) mx[b][wave][c32] = m;
        }
    };

    // block i's partial from z and (sampling) the four wave maxima, read after
    // the barrier that publishes them
    auto block_part = [&](auto Bc, const float (&mw)[kDwWaves]) {
        constexpr int b = decltype(Bc)::value;
        Part res;
        if constexpr (GREEDY) {
            int si = 31;
#pragma unroll
            for (int u = 30; u >= 0; --u) si = (z[u] == m) ? u : si;
            const int v = v_lane + ((si < 16) ? si : 16 + si);   // tile 1 starts 32 columns on
            ArgMax am{m, v < V ? v : 0x7fffffff};
            am = xargmax<32>(am);
            res = Part{am.v, am.i, 0.0};
            if (h == 0) red[b][wave][c32] = res;
        } else {
            // the first half of the weights (the second is summed among the next
            // block's MFMAs), in groups of eight kept apart for the scheduler
            const float mt = fmaxf(max3_lds(mw[0], mw[1], mw[2]), mw[3]);
            const float mref = (mt == -INFINITY) ? 0.0f : mt;
            hc0 = 0.0;
            hc1 = 0.0;
#pragma unroll
            for (int g = 0; g < 16; g += 8) {
#pragma unroll
                for (int s = g; s < g + 8; s += 2) {
                    hc0 += (double)wexp(z[s] - mref, itL);
                    hc1 += (double)wexp(z[s + 1] - mref, itL);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int s = 0; s < 16; ++s) zh[s] = z[16 + s];
            mh = mref;
            mth = mt;
        }
    };

    constexpr std::integral_constant<int, 0> kB0{};
    constexpr std::integral_constant<int, 1> kB1{};
    // prologue: block 0 staged; block 1's rows and block 2's tokens requested in
    // the order an iteration requests them (logit words, embedding rows,
    // tokens), so that the loop is entered with the loads in flight that it
    // carries round
    int p[kDwRows] = {};   // tokens of block i + 2 (the Markov head)
    {
        int p0[kDwRows] = {}, p1[kDwRows] = {};
        prev_raw(p0);
        prev_raw(p1);
        load_e(0, p0);
        load_raw();
        store_e(kB0);
        store_lg(kB0);
        load_raw();
        __builtin_amdgcn_sched_barrier(0);
        load_e(1, p1);
        prev_raw(p);
        __builtin_amdgcn_sched_barrier(0);
        lds_barrier();
    }

    // iteration i (buffers b = i % 2 hold block i, b ^ 1 receive block i + 1)
    auto iter = [&](int i, auto Bc, auto Nc) {
        store_e(Nc);             // block i + 1's rows: the buffers held block i - 1,
        store_lg(Nc);            // last read before the previous barrier
        load_raw();              // block i + 2's logit words
        __builtin_amdgcn_sched_barrier(0);
        block_logits(Bc, Nc);
        lds_barrier();
        // this block's wave maxima and the last block's partials, read together
        float mw[kDwWaves] = {};
        Part pr[kDwWaves];
#pragma unroll
        for (int w = 0; w < kDwWaves; ++w) {
            if constexpr (!GREEDY) mw[w] = mx[decltype(Bc)::value][w][c32];
            pr[w] = red[decltype(Nc)::value][w][jr];
        }
        load_e(i + 2, p);        // block i + 2's embedding rows
        prev_raw(p);             // block i + 3's tokens
        merge(i - 1, pr);
        __builtin_amdgcn_s_setprio(0);
        block_part(Bc, mw);
    };
    // whole pairs in the loop and an odd last block after it
    int i = 0;
    for (; i + 1 < n_blk; i += 2) {
        iter(i, kB0, kB1);
        iter(i + 1, kB1, kB0);
    }
    auto last_merge = [&](int j, auto Bc) {
        if constexpr (!GREEDY) {   // the last block's second half of weights
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                const double w = (double)wexp(zh[s] - mh, itL);
                if (s & 1) hc1 += w; else hc0 += w;
            }
            put_part(Bc);
        }
        lds_barrier();
        Part pr[kDwWaves];
#pragma unroll
        for (int w = 0; w < kDwWaves; ++w) pr[w] = red[decltype(Bc)::value][w][jr];
        merge(j, pr);
    };
    if (i < n_blk) {
        iter(i, kB0, kB1);
        last_merge(i, kB0);
    } else {
        last_merge(i - 1, kB1);
    }
}

}  // namespace dsp

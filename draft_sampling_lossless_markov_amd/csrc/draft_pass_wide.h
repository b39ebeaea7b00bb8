// draft_pass_wide.h -- the streaming draft pass at one wave per SIMD (gfx950).
//
// What bias_pass_kernel<kSample | kGreedy> computes for bf16 rows of 16-byte
// words -- per (request, 256-wide vocabulary tile) the partial of
// logit = base + E[prev] . W2^T -- software-pipelined for one wave per SIMD:
// four waves per workgroup, wave w owning 64 columns (two 32 x 32 MFMA tiles,
// 128 fragment registers in AGPRs, which only a single wave per SIMD can hold).
// Each embedding fragment read from LDS feeds two MFMAs, and four waves, not
// eight, meet at each block's barrier: with eight waves of 32 columns every
// wave reads the block's whole 16 KB embedding tile, and in a pass without its
// arithmetic those reads and the barrier took close to half of the time.
// bias_pass_kernel runs a block's MFMA chain and then its epilogue in each wave;
// here the next block's MFMAs are issued among the current block's weights.
//
// Lane l holds request l % 32 of a block and, in tile t, the 16 contiguous
// columns [64 w + 32 t + 16 (l / 32), +16) (dp_arow maps MFMA rows to columns
// as for one 32-column tile).  One barrier per block: in iteration i a wave
// runs block i + 1's 32 MFMAs with block i's 32 weights interleaved, stages
// block i + 2, publishes block i's partials and block i + 1's maxima; after the
// barrier it requests the blocks ahead, merges block i's partials and takes
// block i + 1's tile maximum.  All global traffic uses raw buffer instructions
// (draft_pass.h): rows past the end, bias rows that select none and idle lanes
// take out-of-range offsets, and a block's logit-word addresses are scalar.  Every logit is the same
// MFMA sequence (k-steps 0..15 from zero) plus the base logit, as in the pick's
// tile rebuild; the weights take the tile maximum as their one reference.
#pragma once

#include "draft_pass.h"

namespace dsp {

constexpr int kDwWaves = 4;                  // waves per workgroup (one per SIMD)
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
__global__ __launch_bounds__(kDwThreads, 1) void draft_pass_wide_kernel(PassArgs a)
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
    // whole row segment).  Rows past the end read zeros; their results are
    // never stored.
    const int sword = lane & 31;
    auto srow_of = [&](int c) { return 8 * wave + 2 * c + h; };
    const int kk = 8 * sword;
    const int cols = min(kVocabTile, V - vt * kVocabTile);

    const int32_t* tsrc = (a.k == 0) ? a.anchor : a.tok;
    const BufRsrc tok_rs = buf_rsrc(tsrc, (uint32_t)(a.R * ((a.k == 0) ? 1 : gamma)) * 4u);
    const uint32_t tstep = (uint32_t)(kPassBlock * ((a.k == 0) ? 1 : gamma)) * 4u;
    uint32_t toff[kDwRows];
#pragma unroll
    for (int c = 0; c < kDwRows; ++c) {
        const int row = n_begin + srow_of(c);
        toff[c] = (uint32_t)((a.k == 0) ? row : row * gamma + (a.k - 1)) * 4u;
    }
    auto prev_raw = [&](int (&p)[kDwRows]) {
        if constexpr (!RNN) {
#pragma unroll
            for (int c = 0; c < kDwRows; ++c) {
                p[c] = (int)__builtin_amdgcn_raw_buffer_load_b32(tok_rs, toff[c], 0, 0);
                toff[c] += tstep;
            }
        }
    };

    const BufRsrc e_rsc = buf_rsrc(a.E, (uint32_t)((((int64_t)a.e_rows - 1) * a.e_rs + r) * 2));
    const uint32_t e_rs2 = (uint32_t)a.e_rs * 2u, kk2 = 2u * (uint32_t)kk;
    const bool kk_ok = kk < r;
    uint4 eu[kDwRows];
    auto load_e = [&](int blk, const int (&p)[kDwRows]) {
#pragma unroll
        for (int c = 0; c < kDwRows; ++c) {
            const int row = RNN ? n_begin + blk * kPassBlock + srow_of(c) : p[c];
            const uint32_t off = ((unsigned)row < (unsigned)a.e_rows && kk_ok)
                                     ? __umul24((uint32_t)row, e_rs2) + kk2 : kBufOut;
            eu[c] = buf_load16<0>(e_rsc, off);
        }
    };
    auto store_e = [&](int b) {
#pragma unroll
        for (int c = 0; c < kDwRows; ++c) *reinterpret_cast<uint4*>(&e_tile[b][srow_of(c)][kk]) = eu[c];
    };

    const uint16_t* __restrict__ base = static_cast<const uint16_t*>(a.base);
    uint32_t loff[kDwRows];
#pragma unroll
    for (int c = 0; c < kDwRows; ++c) loff[c] = (uint32_t)(srow_of(c) * a.bs.rs + kk) * 2u;
    const uint16_t* lblk = base + (int64_t)n_begin * a.bs.rs + (int64_t)a.k * a.bs.ps + vt * kVocabTile;
    const int64_t lstep = (int64_t)kPassBlock * a.bs.rs;
    int lfirst = n_begin;
    uint4 rs[kDpRing][kDwRows];
    auto load_raw = [&](auto SLc) {
        constexpr int sl = decltype(SLc)::value;
        const int live = min(kPassBlock, n_end - lfirst);
        const uint32_t bytes = (live > 0) ? (uint32_t)(((int64_t)(live - 1) * a.bs.rs + cols) * 2) : 0u;
        const BufRsrc rb = buf_rsrc(lblk, bytes);
#pragma unroll
        for (int c = 0; c < kDwRows; ++c) rs[sl][c] = buf_load16<kBufNt>(rb, loff[c]);
        lblk += lstep;
        lfirst += kPassBlock;
    };
    const bool col_in = kk < cols;
    auto store_lg = [&](auto SLc) {
        constexpr int sl = decltype(SLc)::value, b = sl;
        if (cols < kVocabTile) {   // a partial tile (workgroup-uniform)
            constexpr uint32_t kNinf2 = 0xFF80FF80u;
            const uint32_t keep = col_in ? 0xFFFFFFFFu : 0u, put = kNinf2 & ~keep;
#pragma unroll
            for (int c = 0; c < kDwRows; ++c) {
                uint4& v = rs[sl][c];
                v = make_uint4((v.x & keep) | put, (v.y & keep) | put, (v.z & keep) | put, (v.w & keep) | put);
            }
        }
#pragma unroll
        for (int c = 0; c < kDwRows; ++c) *reinterpret_cast<uint4*>(&L.s.lg[b][srow_of(c)][kk]) = rs[sl][c];
    };

    // partials: lanes 0..7 of wave w store requests 8 w .. 8 w + 7 of a block.
    // A wave with no live row among them skips its stores: a store instruction
    // all of whose lanes fall out of range can retire ahead of older loads and
    // upset the waits on the in-order load counter.
    const uint32_t poff = (lane < 8) ? (uint32_t)((8 * wave + lane) * a.n_vt) * 16u : kBufOut;
    const uint32_t qoff = (lane < 8) ? (uint32_t)(8 * wave + lane) * 16u : kBufOut;
    Part* pblk = a.part + (int64_t)n_begin * a.n_vt + vt;
    const int64_t pstep = (int64_t)kPassBlock * a.n_vt;

    // logits of a block (slot s: tile s / 16, column s % 16) and their lane maximum
    float z[32], m = -INFINITY;
    auto logits = [&](int b, const floatx16& acc0, const floatx16& acc1) {
        uint4 lw[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
            lw[q] = *reinterpret_cast<const uint4*>(
                &L.s.lg[b][c32][64 * wave + 32 * (q >> 1) + 16 * h + 8 * (q & 1)]);
#pragma unroll
        for (int s = 0; s < 16; ++s) {
            z[s] = Logit<uint16_t>::raw_at(lw + (s >> 3), s & 7) + acc0[s];
            z[16 + s] = Logit<uint16_t>::raw_at(lw + 2 + (s >> 3), s & 7) + acc1[s];
        }
        m = z[0];
#pragma unroll
        for (int s = 1; s < 32; ++s) m = fmaxf(m, z[s]);
        if constexpr (!GREEDY) {
            m = xmax<32>(m);
            if (h == 0) mx[b][wave][c32] = m;
        }
    };
    float mt = 0.0f, mref = 0.0f;
    auto tile_max = [&](int b) {
        if constexpr (!GREEDY) {
            float mw[kDwWaves];
#pragma unroll
            for (int w = 0; w < kDwWaves; ++w) mw[w] = mx[b][w][c32];
            mt = fmaxf(max3_lds(mw[0], mw[1], mw[2]), mw[3]);
            mref = (mt == -INFINITY) ? 0.0f : mt;
        }
    };

    // prologue: blocks 0 and 1 staged (embedding rows and logits), block 0's
    // logits formed and its tile maximum taken; block 2's embedding rows,
    // block 3's tokens and the logit words of blocks 2 and 3 in flight
    constexpr std::integral_constant<int, 0> kSl0{};
    constexpr std::integral_constant<int, 1> kSl1{};
    floatx16 acc0, acc1;
    int p3[kDwRows] = {};   // raw tokens of block i + 3 (the Markov head)
    {
        int p0[kDwRows] = {}, p1[kDwRows] = {}, p2[kDwRows] = {};
        prev_raw(p0);
        prev_raw(p1);
        prev_raw(p2);
        load_e(0, p0);
        load_raw(kSl0);
        load_raw(kSl1);
        store_e(0);
        load_e(1, p1);
        store_lg(kSl0);
        store_lg(kSl1);
        store_e(1);
        // the last requests in the order an iteration makes them (words, then
        // embedding rows, tokens, words of the next block), so that the loop is
        // entered with the same loads in flight as it carries round
        load_raw(kSl0);   // block 2
        __builtin_amdgcn_sched_barrier(0);
        load_e(2, p2);
        prev_raw(p3);
        __builtin_amdgcn_sched_barrier(0);
        load_raw(kSl1);   // block 3
        __builtin_amdgcn_sched_barrier(0);
        lds_barrier();
        const uint16_t* eb = &e_tile[0][c32][8 * h];
        acc0 = floatx16{};
        acc1 = floatx16{};
#pragma unroll
        for (int ks = 0; ks < kKSteps; ++ks) {
            const bf16x8 bf = as_bf16x8(*reinterpret_cast<const uint4*>(eb + ks * kKStep));
            acc0 = mfma32_bf16(afrag[0][ks], bf, acc0);
            acc1 = mfma32_bf16(afrag[1][ks], bf, acc1);
        }
        logits(0, acc0, acc1);
        lds_barrier();
        tile_max(0);
    }

    // iteration i (SL = i % 2: ring slot and LDS buffers), entered with block
    // i's logits z, lane maximum m and (sampling) tile maximum mt:
    //   [B] block i + 1's 32 MFMAs with block i's 32 weights among them; block
    //       i + 2's embedding rows and logits to LDS; block i's partials to LDS;
    //       block i + 1's logits and maxima
    //   barrier
    //   [C] the requests of the blocks ahead; block i's partials merged and
    //       stored; block i + 1's tile maximum
    auto iter = [&](int i, auto SL) {
        constexpr int sl = decltype(SL)::value, b = sl;
        const int n0 = n_begin + i * kPassBlock;
        const bool more = i + 1 < n_blk;   // workgroup-uniform

        // sampling: a weight is wexp's exponential of its argument, in steps
        // staggered over the slots (slot s forms the argument of weight s + 2,
        // the exponential of weight s + 1 and adds weight s, into one of two fp64
        // chains), so that one wave's instructions between two MFMAs do not all
        // wait on each other; greedy: the lowest-index slot holding the lane
        // maximum, scanned from the top slot down
        double c2[2] = {0.0, 0.0};
        int si = 31;
        float ea[32], ew[32];
        auto arg_of = [&](int s) {
            const float d = z[s] - mref;
            ea[s] = fmaf(d, itL.hi, d * itL.lo);
        };
        auto exp_of = [&](int s) { ew[s] = __builtin_amdgcn_exp2f(ea[s]); };
        auto slot = [&](int s) {
            if constexpr (GREEDY) {
                const int u = 30 - s;   // 30 .. 0 over s = 0 .. 30
                if (u >= 0) si = (z[u] == m) ? u : si;
            } else {
                if (s + 2 < 32) arg_of(s + 2);
                if (s + 1 < 32) exp_of(s + 1);
                c2[s & 1] = (s < 2) ? (double)ew[s] : c2[s & 1] + (double)ew[s];   // (never -0)
            }
        };
        if constexpr (!GREEDY) {
            arg_of(0);
            arg_of(1);
            exp_of(0);
        }
        if (more) {
            // each embedding fragment (read two k-steps ahead) feeds both tiles'
            // MFMAs; one weight after each MFMA, in the order the scheduler is
            // asked to keep
            const uint16_t* eb = &e_tile[b ^ 1][c32][8 * h];
            uint4 bq[kKSteps];
            bq[0] = *reinterpret_cast<const uint4*>(eb);
            bq[1] = *reinterpret_cast<const uint4*>(eb + kKStep);
#pragma unroll
            for (int ks = 0; ks < kKSteps; ++ks) {
                if (ks + 2 < kKSteps) bq[ks + 2] = *reinterpret_cast<const uint4*>(eb + (ks + 2) * kKStep);
                acc0 = mfma32_bf16(afrag[0][ks], as_bf16x8(bq[ks]), ks == 0 ? floatx16{} : acc0);
                slot(2 * ks);
                acc1 = mfma32_bf16(afrag[1][ks], as_bf16x8(bq[ks]), ks == 0 ? floatx16{} : acc1);
                slot(2 * ks + 1);
            }
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
            for (int ks = 0; ks < kKSteps; ++ks) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (ks + 2 < kKSteps) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x402, GREEDY ? 2 : 6, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x402, GREEDY ? 2 : 6, 0);
            }
        } else {
#pragma unroll
            for (int s = 0; s < 32; ++s) slot(s);
        }
        Part res;
        if constexpr (GREEDY) {
            const int v = v_lane + ((si < 16) ? si : 16 + si);   // tile 1 starts 32 columns on
            ArgMax am{m, v < V ? v : 0x7fffffff};
            am = xargmax<32>(am);
            res = Part{am.v, am.i, 0.0};
        } else {
            res = Part{mt, 0, xsum<32>(c2[0] + c2[1])};
        }
        store_e(b);              // block i + 2's embedding rows
        store_lg(SL);            // block i + 2's logit words
        if (h == 0) red[b][wave][c32] = res;
        if (more) logits(b ^ 1, acc0, acc1);
        lds_barrier();

        // [C]
        load_e(i + 3, p3);       // block i + 3's embedding rows
        prev_raw(p3);            // block i + 4's tokens
        // the loads above are due before the logit words below: keep them ahead
        // in issue order (the load counter is in-order)
        __builtin_amdgcn_sched_barrier(0);
        load_raw(SL);            // block i + 4's logit words
        // every lane merges request 8 w + l % 8 of the block; lanes 0..7 store it
        // and (sampling) the four waves' 64-column sums, which let the pick
        // rebuild one 64-column quarter of the chosen tile instead of all of it
        {
            const int j = 8 * wave + (lane & 7);
            Part p = red[b][0][j];
            float sq[kDwWaves];
            sq[0] = (float)p.s;
#pragma unroll
            for (int w = 1; w < kDwWaves; ++w) {
                const Part q = red[b][w][j];
                if constexpr (GREEDY) {
                    const ArgMax am = argmax_merge(ArgMax{p.m, p.idx}, ArgMax{q.m, q.idx});
                    p.m = am.v;
                    p.idx = am.i;
                } else {
                    p.s += q.s;   // one reference (the tile maximum) throughout
                    sq[w] = (float)q.s;
                }
            }
            const int live = min(kPassBlock, n_end - n0);
            const uint32_t pbytes = (uint32_t)(((int64_t)(live - 1) * a.n_vt + 1) * sizeof(Part));
            const BufRsrc rp = buf_rsrc(pblk, pbytes);
            const uint64_t sb = (uint64_t)__double_as_longlong(p.s);
            const u32x4 pw = {__float_as_uint(p.m), (uint32_t)p.idx, (uint32_t)sb, (uint32_t)(sb >> 32)};
            if (8 * wave < live) __builtin_amdgcn_raw_buffer_store_b128(pw, rp, poff, 0, 0);
            if (!GREEDY && a.sub && 8 * wave < live) {
                // the sums tile-major (sub[vt R + n]): a block's 32 requests are
                // one contiguous 512-byte run
                const BufRsrc rq = buf_rsrc(a.sub + (int64_t)vt * a.R + n0, (uint32_t)live * 16u);
                const u32x4 qw = {__float_as_uint(sq[0]), __float_as_uint(sq[1]), __float_as_uint(sq[2]),
                                  __float_as_uint(sq[3])};
                __builtin_amdgcn_raw_buffer_store_b128(qw, rq, qoff, 0, 0);
            }
        }
        pblk += pstep;
        if (more) tile_max(b ^ 1);
    };
    // whole pairs in the loop and an odd last block after it (a conditional
    // second half would give the compiler a path back to the loop head on which
    // it waits for every load in flight)
    int i = 0;
    for (; i + 1 < n_blk; i += 2) {
        iter(i, kSl0);
        iter(i + 1, kSl1);
    }
    if (i < n_blk) iter(i, kSl0);
}

}  // namespace dsp

// draft_pass.h -- the streaming draft step's bias pass, software-pipelined (gfx950).
//
// What bias_pass_kernel<kSample | kGreedy> computes for bf16 rows of 16-byte
// words -- per (request, 256-wide vocabulary tile) the partial of
// logit = base + E[prev] . W2^T -- with every MFMA of the next request block
// issued among the VALU work of the current block's reduction.  bias_pass_kernel
// runs a block's MFMA chain and then its epilogue in each wave, so the matrix
// pipe and the vector ALUs of a SIMD are busy together only when its other wave
// happens to be in the other phase (measured at R 2048, V 262144: MFMA busy 22%
// of the cycles, VALU 46%, both at once 4%).
//
// Layout: 512 threads, eight waves; wave w owns vocabulary [256 vt + 32 w, +32)
// of the tile (one 32 x 32 MFMA tile per k-step, so that two accumulator sets
// fit two waves per SIMD); lane l holds request l % 32 of a block and the 16
// contiguous columns [16 (l / 32), +16) of the wave's 32 (see dp_arow); lanes l
// and l ^ 32 share a request.  A block's base logits and embedding rows reach
// that layout through LDS, read from memory a whole row segment per half-wave:
// per-lane reads of 16 bytes from 32 rows turn every lane into its own cache
// access and half-line request, and the pass then ran at the L1's limit of
// requests in flight.  One barrier per block: in iteration i a wave runs block
// i + 1's MFMA chain with block i's reduction interleaved, stages block i + 2,
// publishes block i's partials and block i + 1's maxima; after the barrier it
// requests the blocks ahead, merges block i's partials and takes block i + 1's
// tile maximum.
// Every logit is the sum of the same MFMA sequence (k-steps 0..15 from zero)
// and the base logit, as in bias_pass_kernel and the pick's tile rebuild; the
// tile's weights take the tile maximum as their one reference.  The sampling
// partial's fp64 sum adds the same weights in another order (a lane's 16 slots,
// its partner lane, then the waves).
#pragma once

#include "tile_pass.h"

namespace dsp {

constexpr int kDpWaves = 8;                 // waves per workgroup
constexpr int kDpThreads = 64 * kDpWaves;
constexpr int kDpRing = 2;                  // blocks of logit words held in registers

// LDS of a pipelined pass workgroup: the W2 tile in transit to the fragments,
// then the embedding and logit tiles, the cross-wave partials and block maxima.
union DraftPassLds {
    uint4 w2[2][64][kRankMax / 8];
    struct {
        uint16_t e[2][kPassBlock][kRankMax + kERowPad];
        uint16_t lg[2][kPassBlock][kVocabTile + kERowPad];   // base logits of a block
        Part red[2][kDpWaves][kPassBlock];
        float mx[2][kDpWaves][kPassBlock];
    } s;
};

// Vocabulary offset (within the wave's 32 columns) of MFMA row i: output
// register j of lane l is row 8 (j / 4) + 4 (l / 32) + j % 4, which this maps
// to column 16 (l / 32) + j.
__device__ __forceinline__ int dp_arow(int i) { return 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3); }

// slot of 16-byte word c of staged W2 row rho: each 16-lane phase of a fragment
// read (rows dp_arow(i) of one half) meets 16 distinct bank groups, and a row's
// words stay a permutation of its slots
__device__ __forceinline__ int dp_slot(int rho, int c) { return c ^ ((rho & 15) ^ (((rho >> 4) & 1) << 3)); }

// The A fragments of wave w: W2 rows v0 + 32 w + dp_arow(i), k-steps 0..15.  Each
// 64-row quarter of the 256-row tile is read contiguously into LDS; waves 2 q
// and 2 q + 1 then read their fragments from quarter q.
template <class Lds>   // an LDS union whose member w2 is [2][64][kRankMax / 8] words
__device__ __forceinline__ void dp_stage_w2(const uint16_t* __restrict__ W2, int V, int r, int v0,
                                            Lds& L, bf16x8 (&a)[kKSteps])
{
    constexpr int kWordsRow = kRankMax / 8;                  // 32 words of 16 bytes
    constexpr int kPer = 64 * kWordsRow / kDpThreads;        // 4 words per quarter
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    uint4 cur[kPer], nxt[kPer];
    auto fetch = [&](int q, uint4* u) {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int f = i * kDpThreads + tid, rho = f / kWordsRow, c = f % kWordsRow;
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
            const int f = i * kDpThreads + tid, rho = f / kWordsRow, c = f % kWordsRow;
            L.w2[q & 1][rho][dp_slot(rho, c)] = cur[i];
        }
        lds_barrier();
        if ((wave >> 1) == q) {
            const int rho = 32 * (wave & 1) + dp_arow(lane & 31), h = lane >> 5;
#pragma unroll
            for (int ks = 0; ks < kKSteps; ++ks) a[ks] = as_bf16x8(L.w2[q & 1][rho][dp_slot(rho, 2 * ks + h)]);
        }
#pragma unroll
        for (int i = 0; i < kPer; ++i) cur[i] = nxt[i];
    }
    lds_barrier();   // the buffers are reused for the embedding tiles
}

template <bool GREEDY>
__global__ __launch_bounds__(kDpThreads, 1) void draft_pass_kernel(PassArgs a)
{
    __shared__ DraftPassLds L;
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
    const int v_lane = vt * kVocabTile + 32 * wave + 16 * h;   // first of this lane's 16 columns
    // the partial of request n_begin + 4 w + l of block 0 (lanes l < 4 of wave w)
    Part* __restrict__ pnext = a.part + (int64_t)(n_begin + 4 * wave + (lane & 3)) * a.n_vt + vt;
    const int64_t pstep = (int64_t)kPassBlock * a.n_vt;
    const uint16_t* __restrict__ base = static_cast<const uint16_t*>(a.base);
    const Itl itL = fold_itl(a.inv_temp);

    bf16x8 afrag[kKSteps];
    dp_stage_w2(a.W2, V, r, vt * kVocabTile, L, afrag);

    // --- staging of a block's embedding rows and base logits: every load is a
    // whole row segment per half-wave (lanes 32 g .. 32 g + 31 read the 32
    // consecutive 16-byte words of one row), so that an instruction reads two
    // rows' full cache lines.  Thread t handles rows 4 w + 2 c + (l / 32) of a
    // block, c = 0, 1, word l % 32.
    const int sword = lane & 31;
    auto srow_of = [&](int c) { return 4 * wave + 2 * c + h; };
    // Per staging row c of the thread, its request in block 0, the index of its
    // previous token and the offset of its logit word.  The token and logit
    // requests go out block by block in order, so each adds a workgroup-uniform
    // running offset (no per-lane multiply in the loop).  Rows past the end read
    // the last request's token and the -inf words.
    const int vcol = vt * kVocabTile + 8 * sword;   // first column of this thread's word
    const bool col_in = vcol + 8 <= V;
    const int32_t* __restrict__ tsrc = (a.k == 0) ? a.anchor : a.tok;
    const int tstep = kPassBlock * ((a.k == 0) ? 1 : gamma);            // R * gamma < 2^30
    const int tlast = (a.k == 0) ? n_end - 1 : (n_end - 1) * gamma + (a.k - 1);
    const int64_t lstep = (int64_t)kPassBlock * a.bs.rs;
    int row0[2], tix0[2];
    int64_t lof0[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        row0[c] = n_begin + srow_of(c);
        tix0[c] = (a.k == 0) ? row0[c] : row0[c] * gamma + (a.k - 1);
        lof0[c] = (int64_t)row0[c] * a.bs.rs + (int64_t)a.k * a.bs.ps + vcol;
    }
    auto row_live = [&](int blk, int c) { return row0[c] + blk * kPassBlock < n_end; };
    // the raw tokens of this thread's two staging rows in the next block in
    // order (blk), validated where they are used
    int tnext = 0;
    // (recurrent head: the row of the bias table is the request itself)
    auto prev_raw = [&](int blk, int (&p)[2]) {
#pragma unroll
        for (int c = 0; c < 2; ++c)
            p[c] = a.rnn ? row0[c] + blk * kPassBlock : tsrc[row_live(blk, c) ? tix0[c] + tnext : tlast];
        tnext += tstep;
    };
    auto prev_ok = [&](int blk, int c, int p) -> bool {
        return row_live(blk, c) && (unsigned)p < (unsigned)a.e_rows;
    };
    const int e_rs = (int)a.e_rs;             // bias-table row stride (<= 64 x 256)
    const int kk = 8 * sword;                 // this thread's k-slice of an embedding row
    const int kk_in = (kk < r) ? kk : 0;      // ... clamped into the row
    uint4 eu[2];
    auto load_e = [&](int blk, const int (&p)[2]) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            // a row index below 2^24 and a stride below 2^15 whose product stays
            // below 2^31 (the library bounds both tables): a 24-bit multiply
            const int prev = prev_ok(blk, c, p[c]) ? p[c] : 0;
            eu[c] = *reinterpret_cast<const uint4*>(a.E + (__umul24(prev, e_rs) + kk_in));
        }
    };
    auto store_e = [&](int b, int blk, const int (&p)[2]) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            // a dead row or a k-slice past r stores zeros (masked, branch-free)
            const uint32_t mk = (prev_ok(blk, c, p[c]) && kk < r) ? 0xFFFFFFFFu : 0u;
            const uint4 v = eu[c];
            *reinterpret_cast<uint4*>(&e_tile[b][srow_of(c)][kk]) =
                make_uint4(v.x & mk, v.y & mk, v.z & mk, v.w & mk);
        }
    };

    // base logit words of a block (its rows' 256 columns of the tile) into ring
    // slot sl; rows past the end and words past V read the -inf words
    uint4 rs[kDpRing][2];
    const uint16_t* neg = reinterpret_cast<const uint16_t*>(kNegInfWords);
    int64_t lnext = 0;   // offset of the next block in order (blk)
    auto load_raw = [&](int blk, int sl) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const uint16_t* p = (row_live(blk, c) && col_in) ? base + (lof0[c] + lnext) : neg;
            rs[sl][c] = load_nt16(p);
        }
        lnext += lstep;
    };
    auto store_lg = [&](int b, int sl) {
#pragma unroll
        for (int c = 0; c < 2; ++c) *reinterpret_cast<uint4*>(&L.s.lg[b][srow_of(c)][8 * sword]) = rs[sl][c];
    };

    // logits of a block from its staged base logits and bias, and their lane
    // maximum
    float z[16], m = -INFINITY;
    auto logits = [&](int b, const floatx16& acc) {
        uint4 lw[2];
#pragma unroll
        for (int c = 0; c < 2; ++c)
            lw[c] = *reinterpret_cast<const uint4*>(&L.s.lg[b][c32][32 * wave + 16 * h + 8 * c]);
#pragma unroll
        for (int s = 0; s < 16; ++s) z[s] = Logit<uint16_t>::raw_at(lw + (s >> 3), s & 7) + acc[s];
        m = z[0];
#pragma unroll
        for (int s = 1; s < 16; ++s) m = fmaxf(m, z[s]);
        if constexpr (!GREEDY) {
            m = xmax<32>(m);
            if (h == 0) mx[b][wave][c32] = m;
        }
    };
    // the tile maximum of a block over the eight waves (sampling)
    float mt = 0.0f, mref = 0.0f;
    auto tile_max = [&](int b) {
        if constexpr (!GREEDY) {
            float mw[kDpWaves];
#pragma unroll
            for (int w = 0; w < kDpWaves; ++w) mw[w] = mx[b][w][c32];
            mt = fmaxf(fmaxf(fmaxf(mw[0], mw[1]), fmaxf(mw[2], mw[3])),
                       fmaxf(fmaxf(mw[4], mw[5]), fmaxf(mw[6], mw[7])));
            mref = (mt == -INFINITY) ? 0.0f : mt;   // an all-masked tile
        }
    };

    // prologue: blocks 0 and 1 staged (embedding rows and logits), block 0's
    // logits formed and its tile maximum taken; block 2's embedding rows,
    // block 3's tokens and the logit words of blocks 2 and 3 in flight
    floatx16 acc;
    int p2[2], p3[2];   // raw tokens of blocks i + 2 and i + 3
    {
        int p0[2], p1[2];
        prev_raw(0, p0);
        prev_raw(1, p1);
        prev_raw(2, p2);
        load_e(0, p0);
        load_raw(0, 0);
        load_raw(1, 1);
        store_e(0, 0, p0);
        load_e(1, p1);
        store_lg(0, 0);
        store_lg(1, 1);
        load_raw(2, 0);
        load_raw(3, 1);
        store_e(1, 1, p1);
        load_e(2, p2);
        prev_raw(3, p3);
        lds_barrier();
        const uint16_t* eb = &e_tile[0][c32][8 * h];
        acc = floatx16{};
#pragma unroll
        for (int ks = 0; ks < kKSteps; ++ks)
            acc = mfma32_bf16(afrag[ks], as_bf16x8(*reinterpret_cast<const uint4*>(eb + ks * kKStep)), acc);
        logits(0, acc);
        lds_barrier();
        tile_max(0);
    }

    // iteration i (SL = i % 2: ring slot and LDS buffers), entered with block
    // i's logits z, lane maximum m and (sampling) tile maximum mt:
    //   [B] block i + 1's MFMA chain with block i's reduction among it; block
    //       i + 2's embedding rows and logits to LDS; block i's partials to LDS;
    //       block i + 1's logits and maxima
    //   barrier
    //   [C] the requests of the blocks ahead; block i's partials merged and
    //       stored; block i + 1's tile maximum
    auto iter = [&](int i, auto SL) {
        constexpr int sl = decltype(SL)::value, b = sl;
        const int n0 = n_begin + i * kPassBlock;
        const bool more = i + 1 < n_blk;   // workgroup-uniform

        // [B] sampling: the weights and one fp64 chain in slot order; greedy: the
        // lowest-index slot holding the lane maximum (masked slots come last and
        // hold -inf), scanned from the top slot down
        double c = 0.0;
        int si = 15;
        auto slot = [&](int s) {
            if constexpr (GREEDY) {
                const int u = 14 - s;   // 14 .. 0 over s = 0 .. 14
                if (u >= 0) si = (z[u] == m) ? u : si;
            } else {
                c += (double)wexp(z[s] - mref, itL);
            }
        };
        if (more) {
            // one slot after each MFMA, in the order the scheduler is asked to
            // keep; the embedding fragment of k-step ks + 2 is read while k-step
            // ks issues
            const uint16_t* eb = &e_tile[b ^ 1][c32][8 * h];
            uint4 bq[kKSteps];
            bq[0] = *reinterpret_cast<const uint4*>(eb);
            bq[1] = *reinterpret_cast<const uint4*>(eb + kKStep);
#pragma unroll
            for (int ks = 0; ks < kKSteps; ++ks) {
                if (ks + 2 < kKSteps) bq[ks + 2] = *reinterpret_cast<const uint4*>(eb + (ks + 2) * kKStep);
                acc = mfma32_bf16(afrag[ks], as_bf16x8(bq[ks]), ks == 0 ? floatx16{} : acc);
                slot(ks);
            }
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
            for (int ks = 0; ks < kKSteps; ++ks) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (ks + 2 < kKSteps) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x402, GREEDY ? 2 : 6, 0);
            }
        } else {
#pragma unroll
            for (int s = 0; s < 16; ++s) slot(s);
        }
        Part res;
        if constexpr (GREEDY) {
            const int v = v_lane + si;
            ArgMax am{m, v < V ? v : 0x7fffffff};
            am = xargmax<32>(am);
            res = Part{am.v, am.i, 0.0};
        } else {
            res = Part{mt, 0, xsum<32>(c)};
        }
        store_e(b, i + 2, p2);   // rows past the end store zeros
        store_lg(b, sl);         // block i + 2's logits
        if (h == 0) red[b][wave][c32] = res;
        if (more) logits(b ^ 1, acc);
        lds_barrier();

        // [C]
        load_e(i + 3, p3);       // block i + 3's embedding rows
        p2[0] = p3[0];
        p2[1] = p3[1];
        prev_raw(i + 4, p3);     // block i + 4's tokens
        // the loads above are due before the logit words below: keep them ahead
        // in issue order (the load counter is in-order)
        __builtin_amdgcn_sched_barrier(0);
        load_raw(i + 4, sl);     // block i + 4's logit words
        // lanes 0..3 of wave w merge requests 4 w .. 4 w + 3 of the block
        const int j = 4 * wave + lane;
        if (lane < 4 && n0 + j < n_end) {
            Part p = red[b][0][j];
#pragma unroll
            for (int w = 1; w < kDpWaves; ++w) {
                const Part q = red[b][w][j];
                if constexpr (GREEDY) {
                    const ArgMax am = argmax_merge(ArgMax{p.m, p.idx}, ArgMax{q.m, q.idx});
                    p.m = am.v;
                    p.idx = am.i;
                } else {
                    p.s += q.s;   // one reference (the tile maximum) throughout
                }
            }
            *pnext = p;
        }
        pnext += pstep;
        if (more) tile_max(b ^ 1);
    };
    for (int i = 0; i < n_blk; i += 2) {
        iter(i, std::integral_constant<int, 0>{});
        if (i + 1 < n_blk) iter(i + 1, std::integral_constant<int, 1>{});
    }
}

}  // namespace dsp

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

// Raw buffer resources: a base in scalar registers, a 32-bit byte offset per
// lane and a range the hardware checks -- a load at or past the range returns
// zeros, a store there is dropped.  Rows past the end, bias rows that select
// none and idle lanes thus take offsets out of range instead of address masks
// and branches, and the per-block address arithmetic of the logit words is
// scalar.  Every range here stays below 2^31 bytes (dp_offsets_fit), so
// kBufOut lies outside all of them.
typedef __amdgpu_buffer_rsrc_t BufRsrc;
constexpr int kBufWord3 = 0x00020000;       // raw access, 32-bit data format
constexpr uint32_t kBufOut = 0x80000000u;

__device__ __forceinline__ BufRsrc buf_rsrc(const void* p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, kBufWord3);
}

// 16-byte loads: kBufNt streams (the logit words, read once)
constexpr int kBufNt = 2;
template <int AUX>
__device__ __forceinline__ uint4 buf_load16(BufRsrc r, uint32_t off)
{
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// the maximum of three values without the quieting of signalling NaNs that
// fmaxf adds to operands it did not compute itself (values read back from LDS)
__device__ __forceinline__ float max3_lds(float a, float b, float c)
{
    float d;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
    return d;
}

// Whether a call's tensors fit the pass's 32-bit offsets: the 32 rows of a
// block of logit words, and the bias table (whose row index also has to fit
// the 24-bit multiply).
__host__ __device__ inline bool dp_offsets_fit(RowStrides bs, int64_t e_rows, int64_t e_rs, int r)
{
    const int64_t lim = (int64_t)1 << 31;
    return bs.rs >= 0 && bs.ps >= 0 && (kPassBlock * bs.rs + kVocabTile) * 2 < lim &&
           e_rows < ((int64_t)1 << 24) && ((e_rows - 1) * e_rs + r) * 2 < lim;
}

template <bool GREEDY, bool RNN>
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
    const Itl itL = fold_itl(a.inv_temp);

    bf16x8 afrag[kKSteps];
    dp_stage_w2(a.W2, V, r, vt * kVocabTile, L, afrag);

    // --- staging of a block's embedding rows and base logits: every load is a
    // whole row segment per half-wave (lanes 32 g .. 32 g + 31 read the 32
    // consecutive 16-byte words of one row), so that an instruction reads two
    // rows' full cache lines.  Thread t handles rows 4 w + 2 c + (l / 32) of a
    // block, c = 0, 1, word l % 32.  Rows past the end (the last block of the
    // last chunk, and the blocks requested ahead past it) read zeros and their
    // results are never stored: a request's partial depends on its own row only.
    const int sword = lane & 31;
    auto srow_of = [&](int c) { return 4 * wave + 2 * c + h; };
    const int kk = 8 * sword;                         // this thread's k-slice of a bias row
    const int cols = min(kVocabTile, V - vt * kVocabTile);   // columns of this tile

    // previous tokens: byte offsets of this thread's rows' tokens in block 0,
    // advanced a block at a time (rows past the end fall past the array)
    const int32_t* tsrc = (a.k == 0) ? a.anchor : a.tok;
    const BufRsrc tok_rs = buf_rsrc(tsrc, (uint32_t)(a.R * ((a.k == 0) ? 1 : gamma)) * 4u);
    const uint32_t tstep = (uint32_t)(kPassBlock * ((a.k == 0) ? 1 : gamma)) * 4u;   // R gamma < 2^30
    uint32_t toff[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int row = n_begin + srow_of(c);
        toff[c] = (uint32_t)((a.k == 0) ? row : row * gamma + (a.k - 1)) * 4u;
    }
    auto prev_raw = [&](int (&p)[2]) {
        if constexpr (!RNN) {
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                p[c] = (int)__builtin_amdgcn_raw_buffer_load_b32(tok_rs, toff[c], 0, 0);
                toff[c] += tstep;
            }
        }
    };

    // bias rows: row p of the table at p e_rs (the previous token; the request
    // itself for the recurrent head); a row outside the table, or a k-slice
    // past r, reads zeros
    const BufRsrc e_rsc = buf_rsrc(a.E, (uint32_t)((((int64_t)a.e_rows - 1) * a.e_rs + r) * 2));
    const uint32_t e_rs2 = (uint32_t)a.e_rs * 2u, kk2 = 2u * (uint32_t)kk;
    const bool kk_ok = kk < r;
    uint4 eu[2];
    auto load_e = [&](int blk, const int (&p)[2]) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int row = RNN ? n_begin + blk * kPassBlock + srow_of(c) : p[c];
            // row < 2^24 and e_rs2 < 2^16: a 24-bit multiply (product < 2^31)
            const uint32_t off = ((unsigned)row < (unsigned)a.e_rows && kk_ok)
                                     ? __umul24((uint32_t)row, e_rs2) + kk2 : kBufOut;
            eu[c] = buf_load16<0>(e_rsc, off);
        }
    };
    auto store_e = [&](int b) {
#pragma unroll
        for (int c = 0; c < 2; ++c) *reinterpret_cast<uint4*>(&e_tile[b][srow_of(c)][kk]) = eu[c];
    };

    // base logit words of a block (its rows' 256 columns of the tile) into ring
    // slot sl (a compile-time index: the ring stays in registers).  The block's rows are one buffer based at its first row: each
    // thread's offset is fixed and the range ends with the block's last live
    // row, so that rows past the end read zeros; words past V (a last, partial
    // tile) read whatever lies there and are replaced by -inf words when staged.
    const uint16_t* __restrict__ base = static_cast<const uint16_t*>(a.base);
    uint32_t loff[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) loff[c] = (uint32_t)(srow_of(c) * a.bs.rs + kk) * 2u;
    const uint16_t* lblk = base + (int64_t)n_begin * a.bs.rs + (int64_t)a.k * a.bs.ps + vt * kVocabTile;
    const int64_t lstep = (int64_t)kPassBlock * a.bs.rs;
    int lfirst = n_begin;   // first request of the next block in order
    uint4 rs[kDpRing][2];
    auto load_raw = [&](auto SLc) {
        constexpr int sl = decltype(SLc)::value;
        const int live = min(kPassBlock, n_end - lfirst);   // <= 0 past the end
        const uint32_t bytes = (live > 0) ? (uint32_t)(((int64_t)(live - 1) * a.bs.rs + cols) * 2) : 0u;
        const BufRsrc rb = buf_rsrc(lblk, bytes);
#pragma unroll
        for (int c = 0; c < 2; ++c) rs[sl][c] = buf_load16<kBufNt>(rb, loff[c]);
        lblk += lstep;
        lfirst += kPassBlock;
    };
    const bool col_in = kk < cols;
    auto store_lg = [&](auto SLc) {
        constexpr int sl = decltype(SLc)::value, b = sl;
        if (cols < kVocabTile) {   // a partial tile (workgroup-uniform)
            // a blend with a mask: a select of whole words would become a load
            // through a selected address and move the ring to scratch memory
            constexpr uint32_t kNinf2 = 0xFF80FF80u;   // two bf16 -inf
            const uint32_t keep = col_in ? 0xFFFFFFFFu : 0u, put = kNinf2 & ~keep;
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                uint4& v = rs[sl][c];
                v = make_uint4((v.x & keep) | put, (v.y & keep) | put, (v.z & keep) | put, (v.w & keep) | put);
            }
        }
#pragma unroll
        for (int c = 0; c < 2; ++c) *reinterpret_cast<uint4*>(&L.s.lg[b][srow_of(c)][kk]) = rs[sl][c];
    };

    // partials: lanes 0..3 of wave w store requests 4 w .. 4 w + 3 of a block
    // (every lane merges request 4 w + l % 4; the others store out of range, as
    // do rows past the end)
    const uint32_t poff = (lane < 4) ? (uint32_t)((4 * wave + lane) * a.n_vt) * 16u : kBufOut;
    Part* pblk = a.part + (int64_t)n_begin * a.n_vt + vt;
    const int64_t pstep = (int64_t)kPassBlock * a.n_vt;

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
            mt = max3_lds(max3_lds(mw[0], mw[1], mw[2]), max3_lds(mw[3], mw[4], mw[5]),
                          fmaxf(mw[6], mw[7]));
            mref = (mt == -INFINITY) ? 0.0f : mt;   // an all-masked tile
        }
    };

    // prologue: blocks 0 and 1 staged (embedding rows and logits), block 0's
    // logits formed and its tile maximum taken; block 2's embedding rows,
    // block 3's tokens and the logit words of blocks 2 and 3 in flight
    constexpr std::integral_constant<int, 0> kSl0{};
    constexpr std::integral_constant<int, 1> kSl1{};
    floatx16 acc;
    int p3[2] = {0, 0};   // raw tokens of block i + 3 (the Markov head)
    {
        int p0[2] = {0, 0}, p1[2] = {0, 0}, p2[2] = {0, 0};
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
        store_e(b);              // block i + 2's embedding rows
        store_lg(SL);            // block i + 2's logits
        if (h == 0) red[b][wave][c32] = res;
        if (more) logits(b ^ 1, acc);
        lds_barrier();

        // [C]
        load_e(i + 3, p3);       // block i + 3's embedding rows
        prev_raw(p3);            // block i + 4's tokens
        // the loads above are due before the logit words below: keep them ahead
        // in issue order (the load counter is in-order)
        __builtin_amdgcn_sched_barrier(0);
        load_raw(SL);            // block i + 4's logit words
        // every lane merges request 4 w + l % 4 of the block; lanes 0..3 store it
        {
            const int j = 4 * wave + (lane & 3);
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
            const int live = min(kPassBlock, n_end - n0);
            const BufRsrc rp = buf_rsrc(pblk, (uint32_t)(((int64_t)(live - 1) * a.n_vt + 1) * sizeof(Part)));
            const uint64_t sb = (uint64_t)__double_as_longlong(p.s);
            const u32x4 pw = {__float_as_uint(p.m), (uint32_t)p.idx, (uint32_t)sb, (uint32_t)(sb >> 32)};
            __builtin_amdgcn_raw_buffer_store_b128(pw, rp, poff, 0, 0);
        }
        pblk += pstep;
        if (more) tile_max(b ^ 1);
    };
    // Whole pairs in the loop and an odd last block after it: with the second
    // half conditional inside the loop, the compiler also sees a path from the
    // first half straight back to the loop head, where the words that half has
    // just requested would be consumed, and waits for every load in flight.
    int i = 0;
    for (; i + 1 < n_blk; i += 2) {
        iter(i, std::integral_constant<int, 0>{});
        iter(i + 1, std::integral_constant<int, 1>{});
    }
    if (i < n_blk) iter(i, std::integral_constant<int, 0>{});
}

}  // namespace dsp

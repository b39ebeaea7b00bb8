// resid_pass.h -- the residual pass over queued (request, position) entries,
// software-pipelined like the draft pass (gfx950).
//
// What bias_pass_kernel<kResidual> computes for bf16 rows of 16-byte words: per
// (entry, 256-wide vocabulary tile) the sum over the tile of max(0, p_v - q_v),
// p the target row and q the draft row of the entry (base + bias by the bf16
// MFMA), both from their rows' (max, normaliser) -- the draws of verification
// (the first rejections) and the exact acceptance probability (every drafted
// position).  Layout and schedule as draft_pass_kernel: eight waves of 32
// columns, one 32 x 32 MFMA tile per k-step, the next block's MFMA chain issued
// one MFMA per slot of the current block's reduction, one barrier per block;
// draft rows, target rows and bias rows read a whole row segment per half-wave
// and staged through LDS.  No maximum is exchanged: every row's reference is
// known beforehand, so each wave reduces on its own.
//
// An entry's rows and statistics come from a record written before the pass
// (resid_prep_kernel): the element offsets of its draft and target rows, its
// bias row, and (M_d, 1/Z_d, M_t, 1/Z_t) rounded as the pick's rescan rounds
// them, so that no load of the pass depends on another.
#pragma once

#include "draft_pass.h"

namespace dsp {

// the per-entry record of a residual pass (three arrays indexed by entry)
struct ResidRecs {
    const int64_t* roff;   // [N, 2] element offsets of the draft row and the target row
    const int* erow;       // [N] bias row (-1: none)
    const float4* rst;     // [N] (M_d, 1/Z_d, M_t, 1/Z_t)
};

// One thread per entry e < *count: its record.  M_d and Z_d are the draft row's
// statistics (stats[n, m]), M_t and Z_t the target row's (row_m/row_z indexed by
// entry or by request); 1/Z in fp64, then fp32 (as the pick's rescan).
__global__ void resid_prep_kernel(const int* __restrict__ list, const int* __restrict__ list_m,
                                  const int* __restrict__ list_prev, const int* __restrict__ count,
                                  const double* __restrict__ stats, const float* __restrict__ row_m,
                                  const double* __restrict__ row_z, int row_by_entry, RowStrides bs,
                                  RowStrides ts, int gamma, int64_t* __restrict__ roff,
                                  int* __restrict__ erow, float4* __restrict__ rst)
{
    const int e = blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= *count) return;
    const int n = list[e], m = list_m[e];
    const int rs = row_by_entry ? e : n;
    const double* st = stats + 2 * ((int64_t)n * gamma + m);
    roff[2 * (int64_t)e] = (int64_t)n * bs.rs + (int64_t)m * bs.ps;
    roff[2 * (int64_t)e + 1] = (int64_t)n * ts.rs + (int64_t)m * ts.ps;
    erow[e] = list_prev[e];
    rst[e] = make_float4((float)st[0], (float)(1.0 / st[1]), row_m[rs], (float)(1.0 / row_z[rs]));
}

union ResidPassLds {
    uint4 w2[2][64][kRankMax / 8];
    struct {
        uint16_t e[2][kPassBlock][kRankMax + kERowPad];
        uint16_t ld[2][kPassBlock][kVocabTile + kERowPad];   // draft base logits of a block
        uint16_t lt[2][kPassBlock][kVocabTile + kERowPad];   // target logits of a block
        Part red[2][kDpWaves][kPassBlock];
    } s;
};

__global__ __launch_bounds__(kDpThreads, 1) void resid_pass_kernel(PassArgs a, ResidRecs rec)
{
    __shared__ ResidPassLds L;
    auto& e_tile = L.s.e;
    auto& red = L.s.red;

    const int count = *a.count;
    const int n_begin = blockIdx.y * a.req_per_wg;
    if (n_begin >= count) return;   // workgroup-uniform
    const int n_end = min(count, n_begin + a.req_per_wg);
    const int n_blk = (n_end - n_begin + kPassBlock - 1) / kPassBlock;

    const int vt = blockIdx.x;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int h = lane >> 5, c32 = lane & 31;
    const int V = a.V, r = a.r;
    const uint16_t* __restrict__ base = static_cast<const uint16_t*>(a.base);
    const uint16_t* __restrict__ target = static_cast<const uint16_t*>(a.target);
    const Itl itL = fold_itl(a.inv_temp);

    bf16x8 afrag[kKSteps];
    dp_stage_w2(a.W2, V, r, vt * kVocabTile, L, afrag);

    // --- staging: thread t handles rows 4 w + 2 c + (l / 32) of a block, 16-byte
    // word l % 32 of each
    const int sword = lane & 31;
    auto srow_of = [&](int c) { return 4 * wave + 2 * c + h; };
    const int vcol = vt * kVocabTile + 8 * sword;
    const bool col_in = vcol + 8 <= V;
    const int kk = 8 * sword;
    const int kk_in = (kk < r) ? kk : 0;
    auto entry_of = [&](int blk, int c) { return min(n_begin + blk * kPassBlock + srow_of(c), n_end - 1); };
    auto row_live = [&](int blk, int c) { return n_begin + blk * kPassBlock + srow_of(c) < n_end; };

    // records of the staging rows of a block: the row offsets of the next block
    // whose words are to be requested, the bias rows of two blocks (slot blk % 2)
    int64_t ro[2][2];      // [c][draft, target]
    int er[2][2];          // [slot][c]
    auto load_meta = [&](int blk, int sl) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int e = entry_of(blk, c);
            const int4 w = *reinterpret_cast<const int4*>(rec.roff + 2 * (int64_t)e);
            ro[c][0] = ((int64_t)(uint32_t)w.x) | ((int64_t)w.y << 32);
            ro[c][1] = ((int64_t)(uint32_t)w.z) | ((int64_t)w.w << 32);
            er[sl][c] = rec.erow[e];
        }
    };
    uint4 eu[2];
    auto load_e = [&](int blk, int sl) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int p = er[sl][c];
            const int prev = (row_live(blk, c) && (unsigned)p < (unsigned)a.e_rows) ? p : 0;
            eu[c] = *reinterpret_cast<const uint4*>(a.E + (int64_t)prev * a.e_rs + kk_in);
        }
    };
    auto store_e = [&](int b, int blk, int sl) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int p = er[sl][c];
            const bool ok = row_live(blk, c) && (unsigned)p < (unsigned)a.e_rows;
            const uint32_t mk = (ok && kk < r) ? 0xFFFFFFFFu : 0u;
            const uint4 v = eu[c];
            *reinterpret_cast<uint4*>(&e_tile[b][srow_of(c)][kk]) = make_uint4(v.x & mk, v.y & mk, v.z & mk, v.w & mk);
        }
    };
    // draft and target words of a block's rows (one block in flight), from the
    // row offsets last loaded (rows past the end and words past V read -inf words)
    uint4 rd[2], rt[2];
    const uint16_t* neg = reinterpret_cast<const uint16_t*>(kNegInfWords);
    auto load_raw = [&](int blk) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const bool live = row_live(blk, c) && col_in;
            rd[c] = load_nt16(live ? base + (ro[c][0] + vcol) : neg);
            rt[c] = load_nt16(live ? target + (ro[c][1] + vcol) : neg);
        }
    };
    auto store_lg = [&](int b) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            *reinterpret_cast<uint4*>(&L.s.ld[b][srow_of(c)][8 * sword]) = rd[c];
            *reinterpret_cast<uint4*>(&L.s.lt[b][srow_of(c)][8 * sword]) = rt[c];
        }
    };
    // the statistics of this lane's entry (request c32 of the block), two-block ring
    float4 stq[2];
    auto load_st = [&](int blk, int sl) {
        stq[sl] = rec.rst[min(n_begin + blk * kPassBlock + c32, n_end - 1)];
    };

    // a block's draft logits (base + bias) and target words into registers
    float zd[16];
    uint4 wt[2];
    auto logits = [&](int b, const floatx16& acc) {
        uint4 wd[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            wd[c] = *reinterpret_cast<const uint4*>(&L.s.ld[b][c32][32 * wave + 16 * h + 8 * c]);
            wt[c] = *reinterpret_cast<const uint4*>(&L.s.lt[b][c32][32 * wave + 16 * h + 8 * c]);
        }
#pragma unroll
        for (int s = 0; s < 16; ++s) zd[s] = Logit<uint16_t>::raw_at(wd + (s >> 3), s & 7) + acc[s];
    };

    // prologue: blocks 0 and 1 staged, block 0's logits formed; the records of
    // blocks 2 and 3, block 2's bias rows and words, the statistics of blocks 0
    // and 1 requested
    floatx16 acc;
    {
        // (the row offsets hold one block: each block's records are loaded right
        // before its words are requested)
        load_meta(0, 0);
        load_e(0, 0);
        load_raw(0);
        load_meta(1, 1);
        store_e(0, 0, 0);
        store_lg(0);
        load_e(1, 1);
        load_raw(1);
        load_st(0, 0);
        load_meta(2, 0);
        store_e(1, 1, 1);
        store_lg(1);
        // the last requests in the order an iteration makes them, so that the
        // loop is entered with the same loads in flight as it carries round
        __builtin_amdgcn_sched_barrier(0);
        load_e(2, 0);
        load_raw(2);
        __builtin_amdgcn_sched_barrier(0);
        load_st(1, 1);
        load_meta(3, 1);
        __builtin_amdgcn_sched_barrier(0);
        lds_barrier();
        const uint16_t* eb = &e_tile[0][c32][8 * h];
        acc = floatx16{};
#pragma unroll
        for (int ks = 0; ks < kKSteps; ++ks)
            acc = mfma32_bf16(afrag[ks], as_bf16x8(*reinterpret_cast<const uint4*>(eb + ks * kKStep)), acc);
        logits(0, acc);
    }

    // iteration i (SL = i % 2), entered with block i's logits in registers, the
    // bias rows of blocks i + 2 (slot i % 2) and i + 3 (the other) and block
    // i + 3's row offsets, block i + 2's bias rows and words, the statistics of
    // blocks i and i + 1:
    //   [B] block i + 1's MFMA chain with block i's reduction among it; block
    //       i + 2's rows to LDS; block i's partials to LDS; block i + 1's logits
    //   barrier
    //   [C] block i + 3's bias rows and words, block i + 2's statistics and block
    //       i + 4's records requested (each from a record loaded an iteration
    //       earlier); block i's partials merged and stored
    auto iter = [&](int i, auto SL) {
        constexpr int sl = decltype(SL)::value, b = sl;
        const bool more = i + 1 < n_blk;   // workgroup-uniform
        const float Md = stq[sl].x, invZd = stq[sl].y, Mt = stq[sl].z, invZt = stq[sl].w;
        double d = 0.0;
        auto slot = [&](int s) {
            const float xt = Logit<uint16_t>::raw_at(wt + (s >> 3), s & 7);
            d += resid_w(wexp(xt - Mt, itL), invZt, wexp(zd[s] - Md, itL), invZd);
        };
        if (more) {
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
                __builtin_amdgcn_sched_group_barrier(0x402, 12, 0);
            }
        } else {
#pragma unroll
            for (int s = 0; s < 16; ++s) slot(s);
        }
        const Part res{0.0f, 0, xsum<32>(d)};
        store_e(b, i + 2, sl);   // block i + 2's bias rows (rows past the end: zeros)
        store_lg(b);             // block i + 2's draft and target words
        if (h == 0) red[b][wave][c32] = res;
        if (more) logits(b ^ 1, acc);
        lds_barrier();

        // [C]
        load_e(i + 3, sl ^ 1);
        load_raw(i + 3);
        __builtin_amdgcn_sched_barrier(0);
        load_st(i + 2, sl);
        load_meta(i + 4, sl);
        // lanes 0..3 of wave w merge entries 4 w .. 4 w + 3 of the block
        const int n0 = n_begin + i * kPassBlock;
        const int j = 4 * wave + lane;
        if (lane < 4 && n0 + j < n_end) {
            Part p = red[b][0][j];
#pragma unroll
            for (int w = 1; w < kDpWaves; ++w) p.s += red[b][w][j].s;
            a.part[(int64_t)(n0 + j) * a.n_vt + vt] = p;
        }
    };
    // whole pairs in the loop and an odd last block after it (a conditional
    // second half would give the compiler a path back to the loop head on which
    // it waits for every load in flight)
    int i = 0;
    for (; i + 1 < n_blk; i += 2) {
        iter(i, std::integral_constant<int, 0>{});
        iter(i + 1, std::integral_constant<int, 1>{});
    }
    if (i < n_blk) iter(i, std::integral_constant<int, 0>{});
}

}  // namespace dsp

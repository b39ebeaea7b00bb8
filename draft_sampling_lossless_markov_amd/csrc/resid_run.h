// resid_run.h -- the residual draws of lossless verification in one persistent
// launch (gfx950), where the draft's W2 slice fits on chip.
//
// After the first rejection at position m of request n, the correction token is
// drawn from max(0, p_m - q_m) normalised, q_m being the draft's biased row at m
// (page "DSpark.让每一轮计算，多走几步", lossless section; page "为什么DSpark
// 可以加速推理？", section on the mathematics of speculative decoding).  The
// requests without a rejection draw their bonus token from target row l (same
// sections).  This kernel replaces the streaming residual pass and the verify
// pick with one persistent launch laid out like draft_run_kernel:
//   W2 slice staged once per workgroup (one per CU);
//   phase 1: the queued requests (rejections found by verify_accept) in blocks
//     of 32: q_m rebuilt by MFMA from the resident slice plus the base logits,
//     the target row added, sum over each tile of max(0, p - q) written to the
//     request's slot (fp64 bits) -- verify_accept marked the slots empty;
//   phase 2: workgroup n mod G draws request n (the grid has one workgroup per
//     request where CUs are free beyond the tiles; those past the tiles run
//     phase 1 on empty tiles, writing nothing): waits for its slots, combines
//     them, locates the tile, rebuilds its residual with the same arithmetic
//     as verify_pick and scans it; without a rejection (or with no residual
//     mass) it draws from target row l (or m) through verify_rows' partials.
#pragma once

#include "draft_run.h"

namespace dsp {

struct ResidArgs {
    const uint16_t* base;    // bf16 draft base logits
    RowStrides bs;
    const uint16_t* target;  // bf16 target logits
    RowStrides ts;
    const uint16_t* E;
    const uint16_t* W2;
    const double* stats;     // [R, gamma, 2] draft (M, Z)
    const int32_t* len;      // [R]
    const int32_t* n_accept; // [R]
    int32_t* y;              // [R]
    int R, gamma, V, r;
    float inv_temp;
    uint64_t seed;
    uint32_t round;
    int n_t;                 // tiles of 32 TU columns
    int n_vt;                // verify_rows' 256-column tiles
    const int* count;        // queued rejections
    const int* list;         // [count] request of each queue slot
    const int* list_m;       // [count] its first rejection
    const int* list_prev;    // [count] the token before it (-1: no bias)
    const int* slot_of;      // [R] queue slot of each request (-1: none)
    const float* row_m;      // [R] target row max at the rejection
    const double* row_z;     // [R] target row normaliser at the rejection
    const Part* rowpart;     // [R, gamma+1, n_vt] verify_rows' tile partials
    uint64_t* slots;         // [count][n_t] residual mass per tile (fp64 bits)
    unsigned* ctl;           // [0] error word
};

template <int NL>
struct ResidLds {
    uint4 w2[4][NL > 0 ? NL : 1][32][kRankMax / 8];
    uint16_t e[kPassBlock][kRankMax + kERowPad];
    uint16_t e_row[kRankMax];
    PickScratch sh;
};

template <int TU>
__global__ __launch_bounds__(256, 1) void resid_run_kernel(ResidArgs a)
{
    constexpr int NR = TU < kRunRegUnits ? TU : kRunRegUnits;
    constexpr int NL = TU - NR;
    __shared__ ResidLds<NL> L;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int h = lane >> 5, c32 = lane & 31;
    const int V = a.V, r = a.r, R = a.R, gamma = a.gamma, n_t = a.n_t;
    const int G = gridDim.x;
    const int tw = 4 * (int)blockIdx.x + wave;
    const int v_tile = tw * 32 * TU;
    const Itl itL = fold_itl(a.inv_temp);
    const int prow = unit_row_col(c32);

    // ================= phase 1: residual mass of every (queued request, tile) ====
    // Loads run ahead so that no block waits on a chain of them: the queue entries
    // two blocks ahead, the rows and embedding rows (which need the entries) one
    // block ahead, under the MFMAs of the block before (two-slot register rings).
    const int count = *a.count;
    const int srow = tid & 31, sq = tid >> 5;
    // queue entries of a block: this lane's request and rejection (row c32) and
    // the token before the rejection of row srow
    int qn[2], qm[2], qp[2];
    auto load_entries = [&](int n0, auto SL) {
        constexpr int sl = decltype(SL)::value & 1;
        const int ee = n0 + c32, e = n0 + srow;
        qn[sl] = (ee < count) ? a.list[ee] : 0;
        qm[sl] = (ee < count) ? a.list_m[ee] : 0;
        qp[sl] = (e < count) ? a.list_prev[e] : -1;
    };
    // embedding rows of the tokens before the block's rejections
    uint4 eu[4];
    auto load_e = [&](int p) {
        const bool pok = p >= 0 && p < V;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int kk = (sq * 4 + c) * 8;
            eu[c] = (pok && kk < r) ? *reinterpret_cast<const uint4*>(a.E + (int64_t)p * r + kk)
                                    : make_uint4(0, 0, 0, 0);
        }
    };
    // this lane's target and draft words, its row statistics: two slots of each
    // up to four units per wave; at five the registers hold two slots of target
    // words but one of draft words, so the next block's draft words are requested
    // after this block's epilogue.  Ordinary cached loads: the two lanes of a
    // request read 32 bytes of a row per instruction and the next instruction the
    // rest of its 64-byte segment, which a streaming load would fetch again (the
    // words are whole 16-byte words of the row or read as -inf: V % 8 == 0 here)
    constexpr int RING = 2;                      // target words, statistics
    constexpr int RING_D = (TU >= 5) ? 1 : 2;    // draft words
    uint4 dw[RING_D][TU][2], xw[RING][TU][2];
    float Md[RING], invZd[RING], Mt[RING], invZt[RING];
    auto load_target = [&](int n0, int n, int m, auto SL) {
        constexpr int sl = decltype(SL)::value % RING;
        const bool ok = n0 + c32 < count;
        const uint16_t* trow = a.target + (int64_t)n * a.ts.rs + (int64_t)m * a.ts.ps;
#pragma unroll
        for (int u = 0; u < TU; ++u)
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const int v0 = v_tile + 32 * u + 16 * c + 8 * h;
                const bool in = ok && v0 + 8 <= V;
                xw[sl][u][c] = *reinterpret_cast<const uint4*>(in ? trow + v0 : reinterpret_cast<const uint16_t*>(kNegInfWords));
            }
        Md[sl] = ok ? (float)a.stats[2 * ((int64_t)n * gamma + m)] : 0.0f;
        invZd[sl] = ok ? (float)(1.0 / a.stats[2 * ((int64_t)n * gamma + m) + 1]) : 0.0f;
        Mt[sl] = ok ? a.row_m[n] : 0.0f;
        invZt[sl] = ok ? (float)(1.0 / a.row_z[n]) : 0.0f;
    };
    auto load_draft = [&](int n0, int n, int m, auto SL) {
        constexpr int sl = decltype(SL)::value % RING_D;
        const bool ok = n0 + c32 < count;
        const uint16_t* drow = a.base + (int64_t)n * a.bs.rs + (int64_t)m * a.bs.ps;
#pragma unroll
        for (int u = 0; u < TU; ++u)
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const int v0 = v_tile + 32 * u + 16 * c + 8 * h;
                const bool in = ok && v0 + 8 <= V;
                dw[sl][u][c] = *reinterpret_cast<const uint4*>(in ? drow + v0 : reinterpret_cast<const uint16_t*>(kNegInfWords));
            }
    };
    auto load_rows = [&](int n0, int n, int m, auto SL) {
        load_draft(n0, n, m, SL);
        load_target(n0, n, m, SL);
    };
    load_entries(0, std::integral_constant<int, 0>{});
    load_entries(kPassBlock, std::integral_constant<int, 1>{});

    bf16x8 afrag[NR][kKSteps];
    stage_w2_slice<TU, NR>(a.W2, V, r, v_tile, L.w2[wave], afrag);

    if (count > 0) {
        load_e(qp[0]);
        load_rows(0, qn[0], qm[0], std::integral_constant<int, 0>{});
    }

    auto block = [&](int n0, auto SL) {
        constexpr int sl = decltype(SL)::value % RING;
        const int ee = n0 + c32;
        const bool ok = ee < count;
        lds_barrier();   // the previous block's embedding tile is read
#pragma unroll
        for (int c = 0; c < 4; ++c) *reinterpret_cast<uint4*>(&L.e[srow][(sq * 4 + c) * 8]) = eu[c];
        lds_barrier();
        constexpr int qs = decltype(SL)::value & 1;   // entry slot of this block
        if (n0 + kPassBlock < count) {
            // block b + 1 from the entries in slot qs ^ 1; then block b + 2's
            // entries into slot qs (this block's are used up)
            load_e(qp[qs ^ 1]);
            load_target(n0 + kPassBlock, qn[qs ^ 1], qm[qs ^ 1], std::integral_constant<int, sl ^ 1>{});
            if constexpr (RING_D == 2)
                load_draft(n0 + kPassBlock, qn[qs ^ 1], qm[qs ^ 1], std::integral_constant<int, sl ^ 1>{});
            if (n0 + 2 * kPassBlock < count) load_entries(n0 + 2 * kPassBlock, std::integral_constant<int, qs>{});
        }

        floatx16 acc[TU];
#pragma unroll
        for (int u = 0; u < TU; ++u)
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[u][j] = 0.0f;
        // LDS operands requested two k-steps ahead of their MFMAs and the order
        // pinned per k-step (one wave per SIMD: nothing else hides an LDS read);
        // the register units' fragments are read by the MFMAs from AGPRs
        {
            constexpr int NLU = TU - NR > 0 ? TU - NR : 1;
            constexpr int D = 2, S = D + 1;
            uint4 pb[S];
            uint4 pa[S][NLU];
            auto fetch = [&](int ks, int slot) {
                pb[slot] = *reinterpret_cast<const uint4*>(&L.e[c32][ks * kKStep + 8 * h]);
#pragma unroll
                for (int u = NR; u < TU; ++u)
                    pa[slot][u - NR < NLU ? u - NR : 0] = L.w2[wave][u >= NR ? u - NR : 0][prow][w2_slot(prow, 2 * ks + h)];
            };
#pragma unroll
            for (int ks = 0; ks < D; ++ks) fetch(ks, ks);
#pragma unroll
            for (int ks = 0; ks < kKSteps; ++ks) {
                if (ks + D < kKSteps) fetch(ks + D, (ks + D) % S);
                const bf16x8 bv = as_bf16x8(pb[ks % S]);
#pragma unroll
                for (int u = 0; u < TU; ++u) {
                    if (u < NR) asm volatile("" : "+a"(afrag[u < NR ? u : 0][ks]));
                    const bf16x8 av = (u < NR) ? afrag[u < NR ? u : 0][ks] : as_bf16x8(pa[ks % S][u >= NR ? u - NR : 0]);
                    acc[u] = mfma32_bf16(av, bv, acc[u]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // max(0, p - q) per column with the arithmetic of the streaming residual
        // pass (fp32 weights, fp64 products, difference and sums)
        double d2[2] = {0.0, 0.0};
#pragma unroll
        for (int u = 0; u < TU; ++u)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const float zd = Logit<uint16_t>::raw_at(&dw[sl % RING_D][u][j >> 3], j & 7) + acc[u][j];
                const float xt = Logit<uint16_t>::raw_at(&xw[sl][u][j >> 3], j & 7);
                d2[j & 1] += resid_w(wexp(xt - Mt[sl], itL), invZt[sl], wexp(zd - Md[sl], itL), invZd[sl]);
            }
        const double sum = xsum<32>(d2[0] + d2[1]);
        if (h == 0 && ok && tw < n_t)
            dev_store_u64(a.slots + (int64_t)ee * n_t + tw, (uint64_t)__double_as_longlong(sum));
        if constexpr (RING_D == 1) {
            if (n0 + kPassBlock < count)
                load_draft(n0 + kPassBlock, qn[qs ^ 1], qm[qs ^ 1], std::integral_constant<int, 0>{});
        }
    };
    for (int n0 = 0; n0 < count; n0 += 2 * kPassBlock) {
        block(n0, std::integral_constant<int, 0>{});
        if (n0 + kPassBlock < count) block(n0 + kPassBlock, std::integral_constant<int, 1>{});
    }

    // ================= phase 2: one workgroup per request ======================
    constexpr int PER = kRunTilesMax / 256;
    for (int n = blockIdx.x; n < R; n += G) {
        const int l = min(max(a.len[n], 0), gamma);
        const int m = min(max(a.n_accept[n], 0), l);
        const int slot = a.slot_of[n];
        const double u = uniform24(a.seed, a.round, (uint32_t)n, (uint32_t)m, 2u);
        bool done = false;
        if (slot >= 0) {   // workgroup-uniform
            const uint64_t* ps = a.slots + (int64_t)slot * n_t;
            uint64_t wv[PER];
            bool miss = false;
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                const int t = tid * PER + i;
                wv[i] = (t < n_t) ? dev_load_u64(ps + t) : 0ull;
                miss |= (wv[i] == kRunSlotEmpty);
            }
            for (unsigned spins = 1; miss; ++spins) {
                __builtin_amdgcn_s_sleep(2);
                if ((spins & 127u) == 0u && run_give_up(a.ctl, spins)) break;
                miss = false;
#pragma unroll
                for (int i = 0; i < PER; ++i) {
                    const int t = tid * PER + i;
                    if (wv[i] == kRunSlotEmpty) wv[i] = dev_load_u64(ps + t);
                    miss |= (wv[i] == kRunSlotEmpty);
                }
            }
            double w[PER];
            double ls = 0.0;
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                w[i] = (tid * PER + i < n_t && wv[i] != kRunSlotEmpty)
                           ? __longlong_as_double((long long)wv[i]) : 0.0;
                ls += w[i];
            }
            const double rsum = block_sum256(ls, L.sh);
            if (rsum > 0.0) {   // workgroup-uniform
                const double tgt = u * rsum;
                double before;
                const int tsel = block_locate<PER>(w, tgt, &before, L.sh, 0);
                // the tile's draft logits rebuilt as phase 1 computed them, and
                // the target row's; the residual per column as verify_pick has it
                const int vt0 = tsel * 32 * TU;
                const int pv = a.list_prev[slot];
                const bool pok = pv >= 0 && pv < V;
                uint4 ev = make_uint4(0, 0, 0, 0);
                if (tid < kRankMax / 8 && pok && 8 * tid < r)
                    ev = *reinterpret_cast<const uint4*>(a.E + (int64_t)pv * r + 8 * tid);
                const uint16_t* drow = a.base + (int64_t)n * a.bs.rs + (int64_t)m * a.bs.ps;
                const uint16_t* trow = a.target + (int64_t)n * a.ts.rs + (int64_t)m * a.ts.ps;
                const int v = vt0 + tid;
                const bool vin = tid < 32 * TU && v < V;
                const float xb = vin ? Logit<uint16_t>::at(drow, v) : -INFINITY;
                const float xt = vin ? Logit<uint16_t>::at(trow, v) : -INFINITY;
                // the rows' statistics, requested with the tile's words
                const double sd0 = a.stats[2 * ((int64_t)n * gamma + m)];
                const double sd1 = a.stats[2 * ((int64_t)n * gamma + m) + 1];
                const float Mt = a.row_m[n];
                const double zt = a.row_z[n];
                constexpr int NU = (TU + 3) / 4;
                uint4 af[NU][kKSteps];
#pragma unroll
                for (int j = 0; j < NU; ++j) {
                    const int vr = vt0 + 32 * (wave + 4 * j) + prow;
                    const bool uin = wave + 4 * j < TU && vr < V;
#pragma unroll
                    for (int ks = 0; ks < kKSteps; ++ks) {
                        const int kk = ks * kKStep + 8 * h;
                        af[j][ks] = (uin && kk < r)
                                        ? *reinterpret_cast<const uint4*>(a.W2 + (int64_t)vr * r + kk)
                                        : make_uint4(0, 0, 0, 0);
                    }
                }
                if (tid < kRankMax / 8) *reinterpret_cast<uint4*>(L.e_row + 8 * tid) = ev;
                lds_barrier();
                // the wave's units as independent MFMA chains issued side by side
                // (a wave without a second unit runs its chain on zero fragments)
                floatx16 acc[NU];
#pragma unroll
                for (int j = 0; j < NU; ++j)
#pragma unroll
                    for (int jj = 0; jj < 16; ++jj) acc[j][jj] = 0.0f;
#pragma unroll
                for (int ks = 0; ks < kKSteps; ++ks) {
                    const uint4 bu = (c32 == 0) ? *reinterpret_cast<const uint4*>(L.e_row + ks * kKStep + 8 * h)
                                                : make_uint4(0, 0, 0, 0);
#pragma unroll
                    for (int j = 0; j < NU; ++j) acc[j] = mfma32_bf16(as_bf16x8(af[j][ks]), as_bf16x8(bu), acc[j]);
                }
#pragma unroll
                for (int j = 0; j < NU; ++j) {
                    const int uu = wave + 4 * j;
                    if (uu < TU && c32 == 0) {
#pragma unroll
                        for (int jj = 0; jj < 16; ++jj) L.sh.lg[32 * uu + unit_acc_col(h, jj)] = acc[j][jj];
                    }
                }
                lds_barrier();
                // the rows' statistics exactly as phase 1 used them
                const float Md = (float)sd0;
                const float invZd = (float)(1.0 / sd1);
                const float invZt = (float)(1.0 / zt);
                double rho[1] = {0.0};
                if (vin) {
                    const float zd = xb + L.sh.lg[tid];
                    rho[0] = resid_w(wexp(xt - Mt, itL), invZt, wexp(zd - Md, itL), invZd);
                }
                double b2;
                const int loc = block_locate<1>(rho, tgt - before, &b2, L.sh, 1);
                if (tid == 0) a.y[n] = vt0 + loc;
                done = true;
            }
        }
        if (!done) {
            // bonus draw from target row l, or the zero-residual fallback from row m
            const int row_j = (slot >= 0) ? m : l;
            const Part* pp = a.rowpart + ((int64_t)n * (gamma + 1) + row_j) * a.n_vt;
            float mt[PER];
            double st[PER];
            float M = -INFINITY;
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                const int t = tid * PER + i;
                mt[i] = -INFINITY;
                st[i] = 0.0;
                if (t < a.n_vt) {
                    mt[i] = pp[t].m;
                    st[i] = pp[t].s;
                }
                M = fmaxf(M, mt[i]);
            }
            M = block_max256(M, L.sh);
            double w[PER];
            double ls = 0.0;
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                w[i] = st[i] * rescale64(mt[i], M, a.inv_temp);
                ls += w[i];
            }
            const double Z = block_sum256(ls, L.sh);
            const double tgt = u * Z;
            double before;
            const int tsel = block_locate<PER>(w, tgt, &before, L.sh, 0);
            const uint16_t* trow = a.target + (int64_t)n * a.ts.rs + (int64_t)row_j * a.ts.ps;
            const int v = tsel * kVocabTile + tid;
            // verify_rows' own weights: relative to the tile maximum, moved onto M
            const float m_t = pp[tsel].m;
            const float mref = (m_t == -INFINITY) ? 0.0f : m_t;
            double e1[1] = {(v < V) ? (double)wexp(Logit<uint16_t>::at(trow, v) - mref, itL) *
                                          rescale64(m_t, M, a.inv_temp)
                                    : 0.0};
            double b2;
            const int loc = block_locate<1>(e1, tgt - before, &b2, L.sh, 1);
            if (tid == 0) a.y[n] = tsel * kVocabTile + loc;
        }
        lds_barrier();   // the pick scratch is reused by the next request
    }
}

}  // namespace dsp

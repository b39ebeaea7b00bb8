// draft_run.h -- every draft position of a call in one persistent launch (gfx950).
//
// The Markov head makes draft position k depend on the token sampled at k - 1,
// so the positions of a round run in sequence, and each one needs the bias
// E[x_{k-1}] . W2^T over the whole vocabulary.  Re-reading W2 (V x r bf16) for
// every position dominates the traffic of a small batch, so this kernel reads it
// once per call: one workgroup per CU (all resident at once: the grid has at most
// one per CU and the kernel's registers and LDS admit exactly one), each
// holding its slice of W2 on chip -- three 32-column units per wave in registers as
// MFMA fragments and up to two in LDS.  Per position:
//   phase 1 (every workgroup): the previous tokens of all requests, then per
//     32-request block the bias by MFMA from the resident slice plus the base
//     logits, reduced to one partial per (request, tile) and published;
//   phase 2 (workgroup n mod G for request n): wait for the request's partials,
//     combine them, draw u, locate the tile, rebuild its logits with the same
//     MFMA sequence and scan them (the steps of draft_pick_kernel), publish the
//     token.
// There is no grid-wide barrier: the published values themselves are the
// signals.  Partial slots (double-buffered by position parity) and the tokens
// of the call's positions hold "empty" markers before they are written (a clear
// kernel sets them before the launch; a pick re-marks its request's slots for
// two positions later), and readers poll until the marker is gone.  A pick
// publishes its token only after its earlier stores -- those re-marks included
// -- are complete, and a writer reads the tokens before it writes the next
// partials, so a slot is never re-marked after its new value lands.
//
// DSpark pages: the sequential head adds a bias from the previous token before
// each sample (page "DSpark.让每一轮计算，多走几步", Markov-head paragraph); it is
// a low-rank matrix (page "DeepSeek联合北大最新文章DSpark", two-stage design).
//
// Values exchanged between workgroups are written and read with device-scope
// relaxed atomics, which gfx950 performs coherently across its XCDs (no L2
// writeback or invalidate is needed).  Every wait is bounded: one that exceeds
// the limit sets the error word, and every later wait then returns at once, so
// the grid always drains (a resident grid never gets there).
#pragma once

#include "tile_pass.h"

namespace dsp {

constexpr int kRunUnitsMax = 5;      // 32-column units per wave (one tile per wave)
constexpr int kRunRegUnits = 3;      // units held in registers (AGPRs); the rest in LDS
constexpr int kRunTilesMax = 1024;   // tiles of one launch (four per workgroup)
constexpr int kRunReqMax = 2048;     // requests of one launch (their tokens sit in LDS)
constexpr unsigned kRunSpinLimit = 1u << 22;
constexpr uint64_t kRunSlotEmpty = ~0ull;          // a partial slot not yet written
constexpr int32_t kRunTokEmpty = (int32_t)0x80000000u;   // a token not yet drawn

struct RunArgs {
    const uint16_t* base;    // bf16 base logits, rows 16-byte aligned
    RowStrides bs;
    const uint16_t* E;       // [V, r]
    const uint16_t* W2;      // [V, r]
    const int32_t* anchor;   // [R]
    int32_t* tok;            // [R, gamma]
    float* q;                // [R, gamma]
    double* stats;           // [R, gamma, 2]
    int R, gamma, V, r, k0, n_steps;
    float inv_temp;
    uint64_t seed;
    uint32_t round;
    int n_t;                 // tiles of 32 * TU columns
    uint64_t* slots;         // [2][R][n_t][2] partials: words (max, 0) and the fp64 sum
                             // of weights relative to the max, or (max, index) and 0
    unsigned* ctl;           // [0] error word
};

// MFMA row i of a 32-column unit -> column of the unit.  With this placement,
// lane half h holds columns [8 h, 8 h + 8) in accumulator registers 0..7 and
// [16 + 8 h, 16 + 8 h + 8) in registers 8..15, so the two 8-column words of a
// request that a lane pair loads are 32 contiguous bytes.
__host__ __device__ inline int unit_row_col(int i)
{
    const int h = (i >> 2) & 1, j = 4 * (i >> 3) + (i & 3);
    return 8 * h + (j & 7) + 16 * (j >> 3);
}

// column of accumulator register j of lane half h
__host__ __device__ inline int unit_acc_col(int h, int j) { return 8 * h + (j & 7) + 16 * (j >> 3); }

// ---------------------------------------------------------------------------
// coherent exchange between the workgroups of one launch
// ---------------------------------------------------------------------------
__device__ __forceinline__ void dev_store_i32(int32_t* p, int32_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ int32_t dev_load_i32(const int32_t* p)
{
    return __hip_atomic_load(const_cast<int32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void dev_store_u64(uint64_t* p, uint64_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t dev_load_u64(const uint64_t* p)
{
    return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// every store this wave issued has completed (is visible to coherent loads)
__device__ __forceinline__ void stores_done() { __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// a wait gave up (or another one did): record it; true when waiting should stop
__device__ __forceinline__ bool run_give_up(unsigned* ctl, unsigned spins)
{
    if (spins > kRunSpinLimit) {
        __hip_atomic_store(&ctl[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return true;
    }
    return __hip_atomic_load(&ctl[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u;
}

__device__ __forceinline__ int32_t poll_tok(const int32_t* p, unsigned* ctl)
{
    int32_t v = dev_load_i32(p);
    for (unsigned spins = 1; v == kRunTokEmpty; ++spins) {
        __builtin_amdgcn_s_sleep(2);
        if ((spins & 127u) == 0u && run_give_up(ctl, spins)) break;
        v = dev_load_i32(p);
    }
    return v;
}

// partial slot words
__device__ __forceinline__ uint64_t pack2(float m, uint32_t x) { return (uint64_t)__float_as_uint(m) | ((uint64_t)x << 32); }
__device__ __forceinline__ float slot_m(uint64_t w) { return __uint_as_float((uint32_t)w); }
__device__ __forceinline__ uint32_t slot_x(uint64_t w) { return (uint32_t)(w >> 32); }

template <int NL>
struct RunLds {
    uint4 w2[4][NL > 0 ? NL : 1][32][kRankMax / 8];   // LDS-resident units (first: staging)
    uint16_t e[kPassBlock][kRankMax + kERowPad];       // embedding rows of a request block
    uint16_t e_row[kRankMax];                          // the picked request's embedding row
    int32_t tokl[kRunReqMax];                          // previous tokens of every request
    PickScratch sh;
    uint64_t pw[2][kPassBlock][4][2];   // a block's words per (request, wave), stored by the workgroup
};

// The wave's W2 units (the 32 TU columns from v_tile): units 0 .. NR-1 into
// MFMA A fragments, the others into the wave's LDS slots (unit NR + i in slot
// i).  Each unit is read contiguously (an instruction covers two whole rows)
// into the wave's first LDS slot and the fragments are read from there; the
// LDS-resident units are written straight to their slots.  Called by every
// wave of the workgroup (it holds workgroup barriers).
template <int TU, int NR, int NLA>
__device__ __forceinline__ void stage_w2_slice(const uint16_t* __restrict__ W2, int V, int r, int v_tile,
                                               uint4 (&w2)[NLA][32][kRankMax / 8],
                                               bf16x8 (&afrag)[NR][kKSteps])
{
    constexpr int kWordsRow = kRankMax / 8;   // 16-byte words of a staged W2 row
    const int lane = threadIdx.x & 63, h = lane >> 5;
    const int prow = unit_row_col(lane & 31);
    uint4 cur[16], nxt[16];
    auto fetch = [&](int u, uint4* w) {
        const int v0 = v_tile + 32 * u;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int f = i * 64 + lane, rho = f / kWordsRow, c = f % kWordsRow;
            const int v = v0 + rho;
            w[i] = (v < V && 8 * c < r) ? *reinterpret_cast<const uint4*>(W2 + (int64_t)v * r + 8 * c)
                                        : make_uint4(0, 0, 0, 0);
        }
    };
    auto put = [&](int slot, const uint4* w) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int f = i * 64 + lane, rho = f / kWordsRow, c = f % kWordsRow;
            w2[slot][rho][w2_slot(rho, c)] = w[i];
        }
    };
    fetch(0, cur);
#pragma unroll
    for (int u = 0; u < TU; ++u) {
        if (u + 1 < TU) fetch(u + 1, nxt);
        if (u < NR) {
            put(0, cur);
            lds_barrier();
#pragma unroll
            for (int ks = 0; ks < kKSteps; ++ks)
                afrag[u < NR ? u : 0][ks] = as_bf16x8(w2[0][prow][w2_slot(prow, 2 * ks + h)]);
            lds_barrier();
        } else {
            put(u - NR, cur);
        }
        if (u + 1 < TU) {
#pragma unroll
            for (int i = 0; i < 16; ++i) cur[i] = nxt[i];
        }
    }
    lds_barrier();
}

// ---------------------------------------------------------------------------
// draft_run_kernel: grid max(ceil(n_t / 4), min(R, CUs)) (at most one workgroup
// per CU), 256 threads; wave w owns tile 4 blockIdx.x + w, i.e. the 32 TU columns
// from 32 TU (4 blockIdx.x + w).  Workgroups past the tiles (added so that no
// workgroup draws two requests of a position where CUs are free) run phase 1 on
// empty tiles -- guarded loads, no HBM traffic, no partials written -- and pick.
// Lane l holds request l % 32 of a 32-request block.
// ---------------------------------------------------------------------------
template <bool GREEDY, int TU>
__global__ __launch_bounds__(256, 1) void draft_run_kernel(RunArgs a)
{
    constexpr int NR = TU < kRunRegUnits ? TU : kRunRegUnits;
    constexpr int NL = TU - NR;
    __shared__ RunLds<NL> L;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int h = lane >> 5, c32 = lane & 31;
    const int V = a.V, r = a.r, R = a.R, gamma = a.gamma, n_t = a.n_t;
    const int G = gridDim.x;
    const int tw = 4 * (int)blockIdx.x + wave;
    const int v_tile = tw * 32 * TU;
    const Itl itL = fold_itl(a.inv_temp);
    const int prow = unit_row_col(c32);   // unit row of this lane's A fragments

    bf16x8 afrag[NR][kKSteps];
    stage_w2_slice<TU, NR>(a.W2, V, r, v_tile, L.w2[wave], afrag);

    const int srow = tid & 31, sq = tid >> 5;   // embedding staging: row, word group
    const int RB = (R + kPassBlock - 1) / kPassBlock;
    for (int s = 0; s < a.n_steps; ++s) {
        const int k = a.k0 + s;
        uint64_t* slots = a.slots + (int64_t)(k & 1) * R * n_t * 2;

        // base words of this lane's request: its two 8-column words of each unit.
        // Ordinary cached loads: the two lanes of a request read 32 bytes of a row
        // per instruction and the next instruction the rest of its 64-byte
        // segment, which a streaming (non-temporal) load would fetch again.  The
        // words do not depend on the tokens, so the first block's are requested
        // before the wait for them.  (V is a multiple of 8 here: a word lies
        // wholly inside the row or wholly past it and then reads as -inf.)
        constexpr int RING = (TU >= 5) ? 1 : 2;
        uint4 bw[RING][TU][2];
        auto load_base = [&](int n0, auto SL) {
            constexpr int sl = decltype(SL)::value % RING;
            const int n = n0 + c32;
            const bool nok = n < R;
            const uint16_t* row = a.base + (int64_t)(nok ? n : 0) * a.bs.rs + (int64_t)k * a.bs.ps;
#pragma unroll
            for (int u = 0; u < TU; ++u)
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    const int v0 = v_tile + 32 * u + 16 * c + 8 * h;
                    const bool in = nok && v0 + 8 <= V;
                    const uint16_t* p = in ? row + v0 : reinterpret_cast<const uint16_t*>(kNegInfWords);
                    bw[sl][u][c] = *reinterpret_cast<const uint4*>(p);
                }
        };
        load_base(0, std::integral_constant<int, 0>{});

        // ---- the previous token of every request (drawn in this launch: wait
        // for it; the anchor or an earlier call's token: read it)
        lds_barrier();   // the previous position's readers of tokl are done
        for (int n = tid; n < R; n += 256) {
            int t;
            if (k == 0) t = a.anchor[n];
            else if (s == 0) t = a.tok[(int64_t)n * gamma + k - 1];
            else t = poll_tok(a.tok + (int64_t)n * gamma + k - 1, a.ctl);
            L.tokl[n] = t;
        }
        lds_barrier();

        // ================= phase 1: partials of every (request, tile) =========
        uint4 eu[4];
        auto load_e = [&](int n0) {
            const int ne = n0 + srow;
            const int p = (ne < R) ? L.tokl[ne] : -1;
            const bool pok = p >= 0 && p < V;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int kk = (sq * 4 + c) * 8;
                eu[c] = (pok && kk < r) ? *reinterpret_cast<const uint4*>(a.E + (int64_t)p * r + kk)
                                        : make_uint4(0, 0, 0, 0);
            }
        };
        load_e(0);

        // A block's words are staged in LDS by each wave and stored by the
        // workgroup after the next barrier: thread t writes request n0 + t / 4's
        // pair of tile 4 blockIdx.x + t % 4, so that a request's four tiles (64
        // contiguous bytes) leave together instead of as four scattered 16-byte
        // stores (each written through at a whole segment's cost)
        auto store_words = [&](int n0, int par) {
            if (tid < 4 * kPassBlock) {
                const int nl = tid >> 2, j = tid & 3;
                const int n = n0 + nl, t = 4 * (int)blockIdx.x + j;
                if (n < R && t < n_t) {
                    uint64_t* sp = slots + 2 * ((int64_t)n * n_t + t);
                    dev_store_u64(sp, L.pw[par][nl][j][0]);
                    dev_store_u64(sp + 1, L.pw[par][nl][j][1]);
                }
            }
        };
        // one request block; SL (block parity) is the base-word ring slot
        auto block = [&](int b, auto SL) {
            constexpr int sl = decltype(SL)::value % RING;
            const int n0 = b * kPassBlock;
            lds_barrier();   // the previous block's embedding tile is read
            if (b > 0) store_words(n0 - kPassBlock, (b - 1) & 1);
#pragma unroll
            for (int c = 0; c < 4; ++c)
                *reinterpret_cast<uint4*>(&L.e[srow][(sq * 4 + c) * 8]) = eu[c];
            lds_barrier();
            if (b + 1 < RB) {   // the next block's rows, under this block's MFMAs
                load_e(n0 + kPassBlock);
                if constexpr (RING == 2) load_base(n0 + kPassBlock, std::integral_constant<int, sl ^ 1>{});
            }

            // units in two groups (registers, then LDS), each reduced on its own
            // and the two partials merged: fewer accumulators live at once
            float gm[2] = {-INFINITY, -INFINITY};
            double gs[2] = {0.0, 0.0};
            int gi[2] = {0x7fffffff, 0x7fffffff};
            auto group = [&](auto U0, auto U1) {
                constexpr int u0 = decltype(U0)::value, u1 = decltype(U1)::value, nu = u1 - u0;
                constexpr int gidx = u0 == 0 ? 0 : 1;
                floatx16 acc[nu];
#pragma unroll
                for (int u = 0; u < nu; ++u)
#pragma unroll
                    for (int j = 0; j < 16; ++j) acc[u][j] = 0.0f;
                // LDS operands (the embedding fragment; the W2 fragments of LDS
                // units) requested D k-steps ahead of their MFMAs and the order
                // pinned per k-step: at one wave per SIMD nothing else hides an LDS
                // read, and left to itself the compiler issues each one right before
                // its MFMA.  The register units' fragments stay in AGPRs, read there
                // by the MFMAs (no copies into VGPRs), which leaves the VGPRs for the
                // prefetch (D = 2 would spill at five units).
                constexpr bool kLds = u0 >= NR;
                constexpr int D = (kLds && TU < 5) ? 2 : 1, S = D + 1;
                uint4 pb[S];
                uint4 pa[S][kLds ? nu : 1];
                auto fetch = [&](int ks, int slot) {
                    pb[slot] = *reinterpret_cast<const uint4*>(&L.e[c32][ks * kKStep + 8 * h]);
                    if constexpr (kLds) {
#pragma unroll
                        for (int u = 0; u < nu; ++u)
                            pa[slot][u] = L.w2[wave][u0 + u >= NR ? u0 + u - NR : 0][prow][w2_slot(prow, 2 * ks + h)];
                    }
                };
#pragma unroll
                for (int ks = 0; ks < D; ++ks) fetch(ks, ks);
#pragma unroll
                for (int ks = 0; ks < kKSteps; ++ks) {
                    if (ks + D < kKSteps) fetch(ks + D, (ks + D) % S);
                    const bf16x8 bv = as_bf16x8(pb[ks % S]);
#pragma unroll
                    for (int u = 0; u < nu; ++u) {
                        const int uu = u0 + u;
                        if constexpr (!kLds) asm volatile("" : "+a"(afrag[uu < NR ? uu : 0][ks]));
                        const bf16x8 av = kLds ? as_bf16x8(pa[ks % S][kLds ? u : 0]) : afrag[uu < NR ? uu : 0][ks];
                        acc[u] = mfma32_bf16(av, bv, acc[u]);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
                // logits of the group's columns for this lane's request
#pragma unroll
                for (int u = 0; u < nu; ++u)
#pragma unroll
                    for (int j = 0; j < 16; ++j)
                        acc[u][j] = Logit<uint16_t>::raw_at(&bw[sl][u0 + u][j >> 3], j & 7) + acc[u][j];
                // with one ring slot, the next block's words as soon as the last
                // group has read this block's
                if constexpr (RING == 1 && u1 == TU) {
                    if (b + 1 < RB) load_base(n0 + kPassBlock, std::integral_constant<int, 0>{});
                }
                float m = -INFINITY;
#pragma unroll
                for (int u = 0; u < nu; ++u)
#pragma unroll
                    for (int j = 0; j < 16; ++j) m = fmaxf(m, acc[u][j]);
                if constexpr (GREEDY) {
                    // the lowest column holding the lane maximum (columns grow
                    // with u, then j); masked columns hold -inf and come last
                    int best = 0x7fffffff;
#pragma unroll
                    for (int u = nu - 1; u >= 0; --u)
#pragma unroll
                        for (int j = 15; j >= 0; --j)
                            best = (acc[u][j] == m) ? 32 * u + unit_acc_col(h, j) : best;
                    best = (best == 0x7fffffff) ? best : v_tile + 32 * u0 + best;
                    gm[gidx] = m;
                    gi[gidx] = best < V ? best : 0x7fffffff;
                } else {
                    m = xmax<32>(m);
                    // fp32 weights relative to the group maximum (a pick's rescan forms
                    // the same ones), summed in fp64 element by element.  A reference
                    // at the group's maximum keeps the dominant weights' exponents near
                    // 0, where the argument's rounding (relative to its size) costs least
                    const float mref = (m == -INFINITY) ? 0.0f : m;   // an all-masked group
                    double sd = 0.0;
#pragma unroll
                    for (int u = 0; u < nu; ++u) {
                        float zu[16];
#pragma unroll
                        for (int j = 0; j < 16; ++j) zu[j] = acc[u][j];
                        sd += sum_w64(zu, mref, itL);
                    }
                    gm[gidx] = m;
                    gs[gidx] = xsum<32>(sd);
                }
            };
            group(std::integral_constant<int, 0>{}, std::integral_constant<int, NR>{});
            if constexpr (NL > 0) group(std::integral_constant<int, NR>{}, std::integral_constant<int, TU>{});

            uint64_t word, word2;
            if constexpr (GREEDY) {
                ArgMax am{gm[0], gi[0]};
                if constexpr (NL > 0) am = argmax_merge(am, ArgMax{gm[1], gi[1]});
                am = xargmax<32>(am);
                word = pack2(am.v, (uint32_t)am.i);
                word2 = 0ull;
            } else {
                float m = gm[0];
                double sum = gs[0];
                if constexpr (NL > 0) {
                    // the group holding the maximum keeps its sum, the other is moved
                    // onto that reference (one fp64 exponential)
                    const bool first = gm[0] >= gm[1];
                    const float mm = first ? gm[0] : gm[1];
                    const double f = rescale64(first ? gm[1] : gm[0], mm, a.inv_temp);
                    if (mm != -INFINITY) sum = first ? gs[0] + gs[1] * f : gs[0] * f + gs[1];
                    m = mm;
                }
                word = pack2(m, 0u);
                word2 = (uint64_t)__double_as_longlong(sum);
            }
            if (h == 0) {
                L.pw[b & 1][c32][wave][0] = word;
                L.pw[b & 1][c32][wave][1] = word2;
            }
        };
        for (int b = 0; b < RB; b += 2) {
            block(b, std::integral_constant<int, 0>{});
            if (b + 1 < RB) block(b + 1, std::integral_constant<int, 1>{});
        }
        lds_barrier();
        store_words((RB - 1) * kPassBlock, (RB - 1) & 1);

        // ================= phase 2: one workgroup per request ==================
        for (int n = blockIdx.x; n < R; n += G) {
            const int64_t out = (int64_t)n * gamma + k;
            uint64_t* ps = slots + 2 * (int64_t)n * n_t;
            constexpr int PER = kRunTilesMax / 256;
            // the request's partials: wait until both words of every tile's have
            // landed (word 2 i + 1 of thread t belongs to tile t PER + i)
            uint64_t wv[PER], ws2[PER];
            {
                bool miss = false;
#pragma unroll
                for (int i = 0; i < PER; ++i) {
                    const int t = tid * PER + i;
                    wv[i] = (t < n_t) ? dev_load_u64(ps + 2 * t) : 0ull;
                    ws2[i] = (t < n_t) ? dev_load_u64(ps + 2 * t + 1) : 0ull;
                    miss |= (wv[i] == kRunSlotEmpty) || (ws2[i] == kRunSlotEmpty);
                }
                for (unsigned spins = 1; miss; ++spins) {
                    __builtin_amdgcn_s_sleep(2);
                    if ((spins & 127u) == 0u && run_give_up(a.ctl, spins)) break;
                    miss = false;
#pragma unroll
                    for (int i = 0; i < PER; ++i) {
                        const int t = tid * PER + i;
                        if (wv[i] == kRunSlotEmpty) wv[i] = dev_load_u64(ps + 2 * t);
                        if (ws2[i] == kRunSlotEmpty) ws2[i] = dev_load_u64(ps + 2 * t + 1);
                        miss |= (wv[i] == kRunSlotEmpty) || (ws2[i] == kRunSlotEmpty);
                    }
                }
            }
            int tok_out = 0, tok_thread = 0;
            float q_out = 1.0f;
            double st0 = 0.0, st1 = 0.0;
            if constexpr (GREEDY) {
                ArgMax am{-INFINITY, 0x7fffffff};
#pragma unroll
                for (int i = 0; i < PER; ++i)
                    if (tid * PER + i < n_t) am = argmax_merge(am, ArgMax{slot_m(wv[i]), (int)slot_x(wv[i])});
                am = wave_argmax(am);
                if (lane == 0) {
                    L.sh.wmax[wave] = am.v;
                    L.sh.hit[0][wave] = am.i;
                }
                lds_barrier();
                ArgMax b{L.sh.wmax[0], L.sh.hit[0][0]};
#pragma unroll
                for (int w = 1; w < 4; ++w) b = argmax_merge(b, ArgMax{L.sh.wmax[w], L.sh.hit[0][w]});
                tok_out = b.i;
                st0 = b.v;
            } else {
                float mt[PER];
                double sw[PER];
                float M = -INFINITY;
#pragma unroll
                for (int i = 0; i < PER; ++i) {
                    // (a word left empty by a wait that gave up reads as an empty tile)
                    const bool in = tid * PER + i < n_t && wv[i] != kRunSlotEmpty && ws2[i] != kRunSlotEmpty;
                    mt[i] = in ? slot_m(wv[i]) : -INFINITY;
                    sw[i] = in ? __longlong_as_double((long long)ws2[i]) : 0.0;
                    M = fmaxf(M, mt[i]);
                }
                M = block_max256(M, L.sh);
#pragma unroll
                for (int i = 0; i < PER; ++i) sw[i] = sw[i] * rescale64(mt[i], M, a.inv_temp);
                // the row total from the locating scan itself (target = u Z)
                const double u = uniform24(a.seed, a.round, (uint32_t)n, (uint32_t)k, 0u);
                double before, Z;
                const int tsel = block_locate_u<PER>(sw, u, &Z, &before, L.sh, 0);
                const double target = u * Z;

                // rebuild the tile's 32 TU logits (thread t: column vt0 + t); the
                // embedding row, the base logit and this wave's W2 fragments
                // (units w and w + 4) are requested together
                const int vt0 = tsel * 32 * TU;
                const int pv = L.tokl[n];
                const bool pok = pv >= 0 && pv < V;
                uint4 ev = make_uint4(0, 0, 0, 0);
                if (tid < kRankMax / 8 && pok && 8 * tid < r)
                    ev = *reinterpret_cast<const uint4*>(a.E + (int64_t)pv * r + 8 * tid);
                // (the base logit's address clamped into the row and its value
                // masked where used, so that no wait follows its load; the W2
                // addresses clamped the same way: a clamped row only feeds masked
                // columns, a clamped k-step meets zeros of the embedding row)
                const uint16_t* row = a.base + (int64_t)n * a.bs.rs + (int64_t)k * a.bs.ps;
                const int v = vt0 + tid;
                const bool vin = tid < 32 * TU && v < V;
                const float xb = Logit<uint16_t>::at(row, min(v, V - 1));
                constexpr int NU = (TU + 3) / 4;   // units per wave in a rebuild
                uint4 af[NU][kKSteps];
#pragma unroll
                for (int j = 0; j < NU; ++j) {
                    const uint16_t* wrow = a.W2 + (int64_t)min(vt0 + 32 * (wave + 4 * j) + prow, V - 1) * r;
#pragma unroll
                    for (int ks = 0; ks < kKSteps; ++ks)
                        af[j][ks] = (wave + 4 * j < TU)   // wave-uniform: the wave has unit j
                                        ? *reinterpret_cast<const uint4*>(wrow + min(ks * kKStep + 8 * h, r - 8))
                                        : make_uint4(0, 0, 0, 0);
                }
                if (tid < kRankMax / 8) *reinterpret_cast<uint4*>(L.e_row + 8 * tid) = ev;
                lds_barrier();
                // the embedding row as B fragments (column 0 of the N-tile), read
                // once for the wave's units
                // once for the wave's unit (with two units per wave there is no room
                // for them: then each k-step reads its own)
                constexpr bool kBfHeld = (NU == 1);
                uint4 bf[kBfHeld ? kKSteps : 1];
                auto b_frag = [&](int ks) -> uint4 {
                    return (c32 == 0) ? *reinterpret_cast<const uint4*>(L.e_row + ks * kKStep + 8 * h)
                                      : make_uint4(0, 0, 0, 0);
                };
                if constexpr (kBfHeld) {
#pragma unroll
                    for (int ks = 0; ks < kKSteps; ++ks) bf[ks] = b_frag(ks);
                }
                // the wave's units as independent MFMA chains issued side by side
                // (a wave without a second unit runs its chain on zero fragments)
                floatx16 acc[NU];
#pragma unroll
                for (int j = 0; j < NU; ++j)
#pragma unroll
                    for (int jj = 0; jj < 16; ++jj) acc[j][jj] = 0.0f;
#pragma unroll
                for (int ks = 0; ks < kKSteps; ++ks) {
                    const uint4 bu = kBfHeld ? bf[kBfHeld ? ks : 0] : b_frag(ks);
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
                const float z = vin ? xb + L.sh.lg[tid] : -INFINITY;
                // the pass's own weights: relative to the maximum of the column's
                // unit group (units 0 .. NR-1 in registers, NR .. TU-1 in LDS), moved
                // onto the tile's reference by the same factor as the pass (1 for the
                // group holding the maximum), then onto the row's
                const int g1 = (tid >= 32 * NR) ? 1 : 0;
                float gmx[2];
                block_max2(g1 == 0 ? z : -INFINITY, g1 == 1 ? z : -INFINITY, gmx, L.sh);
                const float mg = gmx[g1];
                const bool first = gmx[0] >= gmx[1];
                const float m_t = first ? gmx[0] : gmx[1];
                const double fg = ((g1 == 0) == first) ? 1.0 : rescale64(mg, m_t, a.inv_temp);
                const float mref = (mg == -INFINITY) ? 0.0f : mg;
                double e1[1] = {vin ? (double)wexp(z - mref, itL) * fg * rescale64(m_t, M, a.inv_temp)
                                    : 0.0};
                double b2;
                const int loc = block_locate<1>(e1, target - before, &b2, L.sh, 1);
                tok_out = vt0 + loc;
                tok_thread = loc;
                q_out = (float)(e1[0] / Z);
                st0 = M;
                st1 = Z;
            }
            // publish: this workgroup's earlier stores (the slot re-marks of the
            // previous position among them) complete first
            stores_done();
            lds_barrier();
            if (tid == tok_thread) {
                dev_store_i32(a.tok + out, tok_out);
                a.q[out] = q_out;
                a.stats[2 * out] = st0;
                a.stats[2 * out + 1] = st1;
            }
            // re-mark the request's slots of this parity for position k + 2
            if (s + 2 < a.n_steps) {
#pragma unroll
                for (int i = 0; i < PER; ++i) {
                    const int t = tid * PER + i;
                    if (t < n_t) {
                        dev_store_u64(ps + 2 * t, kRunSlotEmpty);
                        dev_store_u64(ps + 2 * t + 1, kRunSlotEmpty);
                    }
                }
            }
        }
    }
}

}  // namespace dsp

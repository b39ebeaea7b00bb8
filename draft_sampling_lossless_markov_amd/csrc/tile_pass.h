// tile_pass.h -- the two building blocks every sampling step of the path uses:
//
//   bias_pass_kernel  one streaming pass over [requests x vocabulary] that
//     computes the Markov bias E[prev] . W2^T with bf16 MFMA (W2 rows in
//     registers, embedding rows in LDS), adds the logit row(s) loaded before the
//     MFMA chain, and reduces each 256-wide vocabulary tile to a partial:
//       kSample   (max logit, sum exp((logit - max) / T))
//       kGreedy   (max logit, lowest index of the max)
//       kResidual sum over the tile of max(0, p_v - q_v) with p the target row,
//                 q the biased draft row (lossless-verification residual)
//   pick_kernel  one workgroup per request: combine the tile partials in fp64,
//     locate the tile where the cumulative mass crosses u * Z, rebuild that
//     tile's 256 weights (recomputing the bias with the identical MFMA sequence)
//     and scan them in vocabulary order.
//
// Tile partials are 256 columns wide everywhere, so a pick rescans 256 values.
#pragma once

#include <type_traits>

#include "bias_tile.h"
#include "dsp_device.h"
#include "dsp_launch.h"

namespace dsp {

enum PassKind : int { kSample = 0, kGreedy = 1, kResidual = 2 };

// ---------------------------------------------------------------------------
// Softmax weights exp((z - ref) / T) = 2^((z - ref) log2(e) / T), z <= ref (z =
// -inf gives 0), by the hardware exp2 (on gfx950 correctly rounded for ~95% of
// arguments, within 0.8 ulp for all, measured).  log2(e) / T is carried as an
// fp32 pair hi + lo folded once per kernel, and the argument formed with one
// rounding: fl32(log2 e / T) alone is off by up to 6e-8 relative, a systematic
// change of temperature that shifts a whole row's CDF.  Every pass, combine and
// rescan of a row forms its weights this same way, so partials and rescans agree.
// ---------------------------------------------------------------------------
struct Itl {
    float hi, lo;
};

// hi is taken strictly below log2(e) / T, so lo > 0: a masked logit (d = -inf)
// then forms -inf * lo = -inf and the weight 0 (a negative lo would give
// -inf * hi + inf = NaN)
__host__ __device__ inline Itl fold_itl(float inv_temp)
{
    const double t = (double)inv_temp * 1.4426950408889634074;   // log2(e) / T
    float hi = (float)t;
    if ((double)hi >= t) hi = nextafterf(hi, 0.0f);
    return Itl{hi, (float)(t - (double)hi)};
}

__device__ __forceinline__ float wexp(float d, Itl itL)
{
    return __builtin_amdgcn_exp2f(fmaf(d, itL.hi, d * itL.lo));
}

// exp((m0 - m1) / T) in fp64: the factor that moves a sum of weights taken
// relative to m0 onto the reference m1 (0 for an empty sum, m0 = -inf).  Every
// merge of partials, every combine and every rescan of a row uses it, so a
// rescan reproduces the pass's sums up to fp64 rounding.
__device__ __forceinline__ double rescale64(float m0, float m1, float inv_temp)
{
    return (m0 == -INFINITY) ? 0.0 : exp(((double)m0 - (double)m1) * (double)inv_temp);
}

// Sum of a lane's fp32 softmax weights exp((z_s - ref) / T), accumulated in fp64
// element by element as they are produced (one chain: no weight array and no
// second accumulator is kept live).  An fp32 tree over a tile's weights rounds at the magnitude of its
// dominant weights, and that rounding alone moves the inverse-CDF boundaries of
// a 1.5e5-word row by ~1.5e-9 on average -- enough to flip ~2e-4 of the draws
// against an fp64 reference; the weights' own rounding moves them ~5x less.
template <int N>
__device__ __forceinline__ double sum_w64(const float (&z)[N], float ref, Itl itL)
{
    // in groups of eight kept apart for the scheduler, so that it does not hoist
    // every exponential ahead of the chain and hold all their results live
    static_assert(N % 8 == 0, "groups of eight");
    double c = 0.0;
#pragma unroll
    for (int g = 0; g < N; g += 8) {
#pragma unroll
        for (int s = g; s < g + 8; ++s) c += (double)wexp(z[s] - ref, itL);
        __builtin_amdgcn_sched_barrier(0);
    }
    return c;
}

// One column's residual max(0, p - q) from its fp32 target and draft weights
// (relative to the rows' maxima) and the rows' fp32 inverse normalisers: the
// products and the difference in fp64, so that cancellation between p and q
// costs no precision beyond the weights' own.
__device__ __forceinline__ double resid_w(float wt, float invZt, float wd, float invZd)
{
    return fmax((double)wt * (double)invZt - (double)wd * (double)invZd, 0.0);
}

// Partial of one 256-wide vocabulary tile of one row.
//   softmax pass: m = max logit, s = sum exp((logit - m) / T) (fp64)
//   greedy pass:  m = max logit, idx = lowest index of the max
//   residual:     s = sum max(0, p - q)
struct __attribute__((aligned(16))) Part {
    float m;
    int idx;
    double s;
};

struct PassArgs {
    const void* base;        // [R, gamma, V] draft base logits
    const void* target;      // [R, gamma+1, V] target logits (kResidual)
    RowStrides bs, ts;       // element strides of base and target rows
    // The table of bias rows (r bf16 values each): row p at E + p * e_rs, valid
    // for 0 <= p < e_rows.  Markov head: the embedding E, e_rs = r, e_rows = V,
    // row = the previous token.  Recurrent head: its states S [R, gamma, r];
    // a draft pass at position k takes E = S + k r, e_rs = gamma r, e_rows = R and
    // row = the request (rnn = 1); a residual pass takes E = S, e_rs = r,
    // e_rows = R gamma and the queue's list_prev = n gamma + m.
    const uint16_t* E;
    int64_t e_rs;
    int e_rows;
    int rnn;
    const uint16_t* W2;
    const int32_t* anchor;
    const int32_t* tok;
    // kResidual: queued requests, their first-rejection position and the token
    // before it (prev), all indexed by queue slot
    const int* list;         // [count] request ids
    const int* list_m;       // [count] first-rejection position
    const int* list_prev;    // [count] token before it (-1: no bias)
    const int* count;        // device scalar
    const int32_t* n_accept; // [R]
    const double* stats;     // [R, gamma, 2] draft (M, Z)
    const float* row_m;      // [R] target row max at the rejection
    const double* row_z;     // [R] target row normaliser at the rejection
    int R, gamma, V, r, k;
    float inv_temp;
    int n_vt, req_per_wg;
    Part* part;              // [R, n_vt] (kResidual: [queue slot, n_vt])
    float4* sub;             // [n_vt, R] or null: a sampling tile's four 64-column sums
                             // (fp32, relative to the tile maximum), for the pick
    unsigned* ctl;           // error word of the call's workspace, set to 0 by the
                             // first pass of a call (nullptr: left alone)
    int row_by_entry;        // kResidual: row_m / row_z indexed by queue slot (else by request)
};

// ---------------------------------------------------------------------------
// bias_pass_kernel: grid (n_vt, request chunks), 256 threads; wave w owns
// vocabulary [256 vt + 64 w, +64) and walks the workgroup's requests in blocks of
// 32 (one N-tile).  Lane l holds request l % 32 of the block and the 32
// contiguous vocabulary columns [32 (l / 32), +32) of the wave's 64 (see
// a_row_voff); lanes l and l ^ 32 share a request.
//
// Per block i, per wave: MFMA (bias of 64 columns x 32 requests, embedding rows
// from LDS), then the epilogue, which in this order
//   consumes block i's logit words (loaded two blocks earlier),
//   stores block i+1's embedding rows (loaded one block earlier) to LDS,
//   requests block i+2's embedding rows, block i+3's previous tokens and
//   block i+2's logit words,
//   reduces the block to partials;
// then an LDS barrier and the merge of the four waves' partials.  Global loads
// are thus issued in the order they are consumed: every wait on the in-order
// load counter covers only data that is due, the barrier orders LDS only, and
// the logit stream stays two blocks ahead.  Every load is unconditional
// (clamped addresses, masked afterwards), so the load count is the same on
// every path and the waits stay exact across the loop.
// ---------------------------------------------------------------------------
constexpr int kPassBlock = 32;   // requests per block (one 32-wide N-tile)

// Two workgroups per CU for the bf16 passes on 16-byte-aligned rows (their
// registers fit 256 per lane); fp32 rows and the element-wise loads of other
// vocabulary sizes need more and run one.
template <typename LT, int KIND, bool VEC>
constexpr int pass_min_blocks() { return (sizeof(LT) == 2 && VEC) ? 2 : 1; }

// 32 bytes of -inf in either logit type: the source of every logit word that
// falls outside the row (or belongs to a request past the end of the list).
// Never written; declared without const so that it lives in the global address
// space like the rows: a select between a row and a constant-space array would
// turn the loads into flat loads, which the LDS wait counter also tracks.
__device__ __attribute__((aligned(16))) uint32_t kNegInfWords[8] = {
    0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u,
    0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u};
__device__ __attribute__((aligned(16))) uint32_t kNegInfF32[8] = {
    0xFF800000u, 0xFF800000u, 0xFF800000u, 0xFF800000u,
    0xFF800000u, 0xFF800000u, 0xFF800000u, 0xFF800000u};

// Raw words of 8 consecutive logits from v0 of a row (ok: the row belongs to a
// live request; in: the chunk lies inside the row).  VEC (V % 8 == 0): a chunk
// lies wholly inside or wholly outside the row, and an outside chunk or a dead
// row reads the -inf words instead, without a branch.  Otherwise element by
// element, each bounded by V.
template <typename LT, bool VEC>
__device__ __forceinline__ void load8_any(const LT* row, int v0, int V, bool ok, bool in, uint4* r)
{
    if constexpr (VEC) {
        in = in && ok;
        const LT* neg = (sizeof(LT) == 2) ? reinterpret_cast<const LT*>(kNegInfWords)
                                          : reinterpret_cast<const LT*>(kNegInfF32);
        const LT* p = in ? row + v0 : neg;
        r[0] = load_nt16(p);
        if constexpr (Logit<LT>::kRaw == 2) r[1] = load_nt16(p + 4);
    } else {
        Logit<LT>::load8_raw(row, ok ? v0 : V, V, false, r);   // bounds per element
    }
}

// LDS of a bias-pass workgroup: first the W2 tile in transit to the MFMA
// fragments (two 64-row quarter buffers, 16-byte slots XOR-swizzled per row),
// then the embedding tiles and the cross-wave partials.
union PassLds {
    uint4 w2[2][64][kRankMax / 8];
    struct {
        uint16_t e[2][kPassBlock][kRankMax + kERowPad];
        Part red[2][4][kPassBlock];
        float mx[2][4][kPassBlock];   // softmax: each wave's block maxima
    } s;
};

// slot of 16-byte word c of staged W2 row rho: the swizzle spreads the 32 rows an
// A-fragment read touches (a_row_voff) over distinct banks, and keeps a row's
// words a permutation of its slots
__device__ __forceinline__ int w2_slot(int rho, int c) { return c ^ ((rho & 31) ^ (((rho >> 5) & 1) << 3)); }

// The A fragments of the workgroup's 256-row W2 tile (rows v0 .. v0 + 255; wave w
// takes rows 64 w .. 64 w + 63): each 64-row quarter is read contiguously (a
// wave instruction covers two whole rows) into LDS, then the owning wave reads
// its fragments.  Same values as the direct loads of tile_logit, at the
// streaming rate of W2.
__device__ __forceinline__ void stage_w2_frags(const uint16_t* __restrict__ W2, int V, int r,
                                               int v0, PassLds& L, bf16x8 a[2][kKSteps])
{
    constexpr int kWordsRow = kRankMax / 8;                    // 32 words of 16 bytes
    constexpr int kPerThread = 64 * kWordsRow / 256;           // 8 words per quarter
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    uint4 cur[kPerThread], nxt[kPerThread];
    auto fetch = [&](int q, uint4* u) {
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) {
            const int f = i * 256 + tid, rho = f / kWordsRow, c = f % kWordsRow;
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
        for (int i = 0; i < kPerThread; ++i) {
            const int f = i * 256 + tid, rho = f / kWordsRow, c = f % kWordsRow;
            L.w2[q & 1][rho][w2_slot(rho, c)] = cur[i];
        }
        lds_barrier();
        if (wave == q) {
            const int i32 = lane & 31, h = lane >> 5;
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int rho = a_row_voff(t, i32);
#pragma unroll
                for (int ks = 0; ks < kKSteps; ++ks)
                    a[t][ks] = as_bf16x8(L.w2[q & 1][rho][w2_slot(rho, 2 * ks + h)]);
            }
        }
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) cur[i] = nxt[i];
    }
    lds_barrier();   // the buffers are reused for the embedding tiles
}

template <typename LT, int KIND, bool VEC>
__global__ __launch_bounds__(256, (pass_min_blocks<LT, KIND, VEC>())) void bias_pass_kernel(PassArgs a)
{
    __shared__ PassLds L;
    auto& e_tile = L.s.e;
    auto& red = L.s.red;
    auto& mx = L.s.mx;
    constexpr int RW = Logit<LT>::kRaw;
    constexpr bool RES = (KIND == kResidual);

    if (a.ctl && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) a.ctl[0] = 0u;
    const int count = RES ? *a.count : a.R;
    const int n_begin = blockIdx.y * a.req_per_wg;
    if (n_begin >= count) return;   // workgroup-uniform
    const int n_end = min(count, n_begin + a.req_per_wg);
    const int n_blk = (n_end - n_begin + kPassBlock - 1) / kPassBlock;

    const int vt = blockIdx.x;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int h = lane >> 5, c32 = lane & 31;
    const int V = a.V, r = a.r, gamma = a.gamma;
    const int v_blk = vt * kVocabTile + wave * 64;
    const int v_lane = v_blk + 32 * h;   // first of this lane's 32 columns
    const LT* __restrict__ base = static_cast<const LT*>(a.base);
    const LT* __restrict__ target = static_cast<const LT*>(a.target);
    const Itl itL = fold_itl(a.inv_temp);

    bf16x8 afrag[2][kKSteps];
    stage_w2_frags(a.W2, V, r, vt * kVocabTile, L, afrag);

    // --- embedding rows: thread t stages row t % 32 of a block, 16-byte words
    // [4 q, 4 q + 4) of it, q = t / 32, so a wave's stores hit 32 rows at two
    // columns (no bank conflicts with the 264-element row pitch)
    const int srow = threadIdx.x & 31, sq = threadIdx.x >> 5;
    // the raw token of this thread's staging row in block blk (unconditional
    // load, clamped index); it is validated only where it is used, a block
    // later, so that nothing waits for it early
    auto prev_raw = [&](int blk) -> int {
        const int ec = min(n_begin + blk * kPassBlock + srow, n_end - 1);
        if constexpr (RES) return a.list_prev[ec];
        else if (a.rnn) return ec;
        else return (a.k == 0) ? a.anchor[ec] : a.tok[(int64_t)ec * gamma + (a.k - 1)];
    };
    // the row index selects a bias row: a live request and a row of the table
    auto prev_ok = [&](int blk, int p) -> bool {
        return n_begin + blk * kPassBlock + srow < n_end && (unsigned)p < (unsigned)a.e_rows;
    };
    constexpr int kWords = kRankMax / 8 / 8;   // 16-byte words per thread (4)
    uint4 eu[kWords];
    auto load_e = [&](int blk, int praw) {
        const int prev = prev_ok(blk, praw) ? praw : 0;
        const uint16_t* rowp = a.E + (int64_t)prev * a.e_rs;
#pragma unroll
        for (int c = 0; c < kWords; ++c) {
            const int kk = (sq * kWords + c) * 8;
            eu[c] = *reinterpret_cast<const uint4*>(rowp + (kk < r ? kk : 0));
        }
    };
    auto store_e = [&](int b, int blk, int praw) {
        const bool ok = prev_ok(blk, praw);
#pragma unroll
        for (int c = 0; c < kWords; ++c) {
            const int kk = (sq * kWords + c) * 8;
            // a dead row or a k-step past r stores zeros (masked, branch-free)
            const uint32_t mk = (ok && kk < r) ? 0xFFFFFFFFu : 0u;
            const uint4 v = eu[c];
            *reinterpret_cast<uint4*>(&e_tile[b][srow][kk]) = make_uint4(v.x & mk, v.y & mk, v.z & mk, v.w & mk);
        }
    };

    // --- logit words of block blk for this lane (its request, its 32 columns
    // as four 8-element chunks) into ring slot sl
    // The softmax and greedy passes keep a two-block ring of logit words.  The
    // residual pass (a few blocks of rejected rows) fetches a block's draft and
    // target words at the block's start, under its MFMA chain, which keeps its
    // registers within two workgroups per CU.
    constexpr int kRing = RES ? 1 : 2;
    uint4 rs[kRing][4 * RW];
    const LT* trow = nullptr;
    uint4 rt[RES ? 4 * RW : 1];
    auto load_raw = [&](int blk, int sl) {
        const int e = n_begin + blk * kPassBlock + c32;
        const bool ok = e < n_end;
        int n = min(e, n_end - 1), m = a.k;
        if constexpr (RES) {
            m = a.list_m[n];
            n = a.list[n];
        }
        const LT* row = base + (int64_t)n * a.bs.rs + (int64_t)m * a.bs.ps;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int v0 = v_lane + 8 * c;
            load8_any<LT, VEC>(row, v0, V, ok, v0 + 8 <= V, rs[sl] + c * RW);
        }
        if constexpr (RES) {
            trow = target + (int64_t)n * a.ts.rs + (int64_t)m * a.ts.ps;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int v0 = v_lane + 8 * c;
                load8_any<LT, VEC>(trow, v0, V, ok, v0 + 8 <= V, rt + c * RW);
            }
        }
    };

    // prologue: block 0's rows staged, then the loads in flight in the same
    // order as at the end of every later block (logit words of the block after
    // next ... embedding rows, tokens, logit words of the last one), so that the
    // loop is entered with the load queue it leaves with
    int prev1, prev2;   // raw tokens of blocks i + 1 and i + 2
    {
        const int prev0 = prev_raw(0);
        prev1 = prev_raw(1);
        load_e(0, prev0);
        store_e(0, 0, prev0);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (!RES) load_raw(0, 0);
        __builtin_amdgcn_sched_barrier(0);
        load_e(1, prev1);
        prev2 = prev_raw(2);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (!RES) load_raw(1, 1);
    }
    lds_barrier();

    // one block; SL = i % 2 is both the ring slot and the LDS buffer, a
    // compile-time constant so the ring stays in registers
    auto step = [&](int i, auto SL) {
        constexpr int sl = decltype(SL)::value, b = sl;
        const int n0 = n_begin + i * kPassBlock;

        // bias of the block: all sixteen k-steps (fragments past r are zero on
        // both sides, so they add exact zeros)
        if constexpr (RES) load_raw(i, 0);
        floatx16 acc[2];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[t][j] = 0.0f;
#pragma unroll
        for (int ks = 0; ks < kKSteps; ++ks) {
            const bf16x8 bv = as_bf16x8(*reinterpret_cast<const uint4*>(
                &e_tile[b][c32][ks * kKStep + 8 * h]));
#pragma unroll
            for (int t = 0; t < 2; ++t) acc[t] = mfma32_bf16(afrag[t][ks], bv, acc[t]);
        }
        // keep the embedding-fragment reads four k-steps ahead of their MFMAs
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int ks = 0; ks < kKSteps - 4; ++ks) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);

        // epilogue: consume, stage, request, reduce
        float z[32];
#pragma unroll
        for (int s = 0; s < 32; ++s)
            z[s] = Logit<LT>::raw_at(rs[RES ? 0 : sl] + (s >> 3) * RW, s & 7) + acc[s >> 4][s & 15];
        if (i + 1 < n_blk) store_e(b ^ 1, i + 1, prev1);
        load_e(i + 2, prev2);         // block i + 2's embedding rows
        prev1 = prev2;
        prev2 = prev_raw(i + 3);      // block i + 3's tokens
        // the loads above are due one block earlier than the logit words below:
        // keep them ahead in issue order (the load counter is in-order)
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (!RES) load_raw(i + 2, sl);   // block i + 2's logit words

        Part res;
        if constexpr (KIND == kGreedy) {
            // slots map to increasing vocabulary ids: the first slot holding the
            // lane maximum is the lane's lowest-index argmax (masked slots come
            // last and hold -inf)
            float m = z[0];
#pragma unroll
            for (int s = 1; s < 32; ++s) m = fmaxf(m, z[s]);
            int si = 31;
#pragma unroll
            for (int s = 30; s >= 0; --s) si = (z[s] == m) ? s : si;
            const int v = v_lane + si;
            ArgMax am{m, v < V ? v : 0x7fffffff};
            am = xargmax<32>(am);
            res = Part{am.v, am.i, 0.0};
        } else if constexpr (KIND == kSample) {
            float m = z[0];
#pragma unroll
            for (int s = 1; s < 32; ++s) m = fmaxf(m, z[s]);
            m = xmax<32>(m);
            // the tile maximum over the four waves' blocks: every weight of the
            // tile then has one reference, the tile's, which the partial records
            // and a pick's rescan uses as it is
            if (h == 0) mx[b][wave][c32] = m;
            lds_barrier();
            m = fmaxf(fmaxf(mx[b][0][c32], mx[b][1][c32]), fmaxf(mx[b][2][c32], mx[b][3][c32]));
            const float mref = (m == -INFINITY) ? 0.0f : m;   // an all-masked tile
            res = Part{m, 0, xsum<32>(sum_w64(z, mref, itL))};
        } else {   // kResidual
            const int e = min(n0 + c32, n_end - 1);
            const int n = a.list[e];
            const int m = a.list_m[e];
            const int rs = a.row_by_entry ? e : n;
            const float Md = (float)a.stats[2 * ((int64_t)n * gamma + m)];
            const float invZd = (float)(1.0 / a.stats[2 * ((int64_t)n * gamma + m) + 1]);
            const float Mt = a.row_m[rs];
            const float invZt = (float)(1.0 / a.row_z[rs]);
            // max(0, p - q) per column: fp32 weights, then the products, the
            // difference and the sums in fp64 (the rescan of a pick repeats it)
            double d2[2] = {0.0, 0.0};
#pragma unroll
            for (int s = 0; s < 32; ++s) {
                const float xt = Logit<LT>::raw_at(rt + (s >> 3) * RW, s & 7);
                d2[s & 1] += resid_w(wexp(xt - Mt, itL), invZt, wexp(z[s] - Md, itL), invZd);
            }
            res = Part{0.f, 0, xsum<32>(d2[0] + d2[1])};
        }
        if (h == 0) red[b][wave][c32] = res;
        lds_barrier();

        // merge the four waves' partials: lanes 0..7 of wave w take requests
        // 8 w .. 8 w + 7 of the block
        const int j = 8 * wave + lane;
        if (lane < 8 && n0 + j < n_end) {
            Part p = red[b][0][j];
#pragma unroll
            for (int w = 1; w < 4; ++w) {
                const Part q = red[b][w][j];
                if constexpr (KIND == kGreedy) {
                    const ArgMax mm = argmax_merge(ArgMax{p.m, p.idx}, ArgMax{q.m, q.idx});
                    p.m = mm.v;
                    p.idx = mm.i;
                } else if constexpr (KIND == kSample) {
                    p.s += q.s;   // one reference (the tile maximum) throughout
                } else {
                    p.s += q.s;
                }
            }
            a.part[(int64_t)(n0 + j) * a.n_vt + vt] = p;
        }
    };
    for (int i = 0; i < n_blk; i += 2) {
        step(i, std::integral_constant<int, 0>{});
        if (i + 1 < n_blk) step(i + 1, std::integral_constant<int, 1>{});
    }
}

// ---------------------------------------------------------------------------
// block-wide helpers for 256-thread pick workgroups.  Wave-level work runs on
// DPP and row swaps; each helper call owns its LDS slots, so a call needs one
// LDS barrier (two for a locate) and none to release its slots.
// ---------------------------------------------------------------------------
struct PickScratch {
    float wmax[4];
    float wmax2[2][4];
    double wsum[4];
    double scan[2][4];
    int hit[2][4];
    double hb[2][4];
    int last[2][4];
    double fb[2];
    float lg[kVocabTile];
};

__device__ __forceinline__ float block_max256(float v, PickScratch& sh)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    v = wave_max_f(v);
    if (lane == 0) sh.wmax[wave] = v;
    lds_barrier();
    return fmaxf(fmaxf(sh.wmax[0], sh.wmax[1]), fmaxf(sh.wmax[2], sh.wmax[3]));
}

// two block maxima at once (one LDS barrier): out[i] = max over the block of v_i
__device__ __forceinline__ void block_max2(float v0, float v1, float (&out)[2], PickScratch& sh)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    v0 = wave_max_f(v0);
    v1 = wave_max_f(v1);
    if (lane == 0) {
        sh.wmax2[0][wave] = v0;
        sh.wmax2[1][wave] = v1;
    }
    lds_barrier();
#pragma unroll
    for (int i = 0; i < 2; ++i)
        out[i] = fmaxf(fmaxf(sh.wmax2[i][0], sh.wmax2[i][1]), fmaxf(sh.wmax2[i][2], sh.wmax2[i][3]));
}

__device__ __forceinline__ double block_sum256(double v, PickScratch& sh)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    v = wave_sum_d(v);
    if (lane == 0) sh.wsum[wave] = v;
    lds_barrier();
    return (sh.wsum[0] + sh.wsum[1]) + (sh.wsum[2] + sh.wsum[3]);
}

// Locate the first of the block's consecutive weights (thread t owns items
// [t * PER, t * PER + PER)) whose inclusive cumulative sum exceeds target.
// w[] holds the thread's weights (zeros past the end).  Returns the item and
// the cumulative mass before it; falls back to the last positive item when
// rounding leaves the target beyond the total.  slot: 0 or 1, one per call.
// FROM_U: the target is u times the total, the total taken from the scan's own
// wave sums (one block reduction fewer than summing first) and returned in *total.
template <int PER, bool FROM_U>
__device__ __forceinline__ int block_locate_impl(const double (&w)[PER], double target, double* before,
                                                 PickScratch& sh, int slot, double* total)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    double ls = 0.0;
#pragma unroll
    for (int i = 0; i < PER; ++i) ls += w[i];
    const double incl = wave_scan_d(ls);
    if (lane == kWave - 1) sh.scan[slot][wave] = incl;
    lds_barrier();
    if constexpr (FROM_U) {
        const double z = (sh.scan[slot][0] + sh.scan[slot][1]) + (sh.scan[slot][2] + sh.scan[slot][3]);
        *total = z;
        target *= z;
    }
    double off = 0.0;
    for (int w2 = 0; w2 < wave; ++w2) off += sh.scan[slot][w2];
    const double c0 = off + incl - ls;
    double c = c0;
    int hit = 0x7fffffff, last = -1;
    double hit_before = 0.0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const double nc = c + w[i];
        // a hit needs positive weight: a zero-weight item (a masked column, a tile
        // past the end) is never chosen even where scan rounding puts the crossing
        if (hit == 0x7fffffff && w[i] > 0.0 && nc > target) {
            hit = (int)threadIdx.x * PER + i;
            hit_before = c;
        }
        if (w[i] > 0.0) last = (int)threadIdx.x * PER + i;
        c = nc;
    }
    const int hmin = wave_minmax_i<false>(hit);
    const int lmax = wave_minmax_i<true>(last);
    if (lane == 0) {
        sh.hit[slot][wave] = hmin;
        sh.last[slot][wave] = lmax;
    }
    if (hmin != 0x7fffffff && hit == hmin) sh.hb[slot][wave] = hit_before;
    lds_barrier();
#pragma unroll
    for (int w2 = 0; w2 < 4; ++w2) {
        const int h = sh.hit[slot][w2];
        if (h != 0x7fffffff) {
            *before = sh.hb[slot][w2];
            return h;
        }
    }
    // no crossing (block-uniform): the last positive item and the mass before it
    const int l = max(max(sh.last[slot][0], sh.last[slot][1]), max(sh.last[slot][2], sh.last[slot][3]));
    if (l >= 0 && (int)threadIdx.x == l / PER) {
        double cc = c0;
        for (int i = 0; i < PER; ++i) {
            if ((int)threadIdx.x * PER + i == l) break;
            cc += w[i];
        }
        sh.fb[slot] = cc;
    }
    lds_barrier();
    *before = (l >= 0) ? sh.fb[slot] : 0.0;
    return l < 0 ? 0 : l;
}

template <int PER>
__device__ __forceinline__ int block_locate(const double (&w)[PER], double target, double* before,
                                            PickScratch& sh, int slot)
{
    return block_locate_impl<PER, false>(w, target, before, sh, slot, nullptr);
}

// The same with the target u * Z, Z the weights' total (returned in *Z).
template <int PER>
__device__ __forceinline__ int block_locate_u(const double (&w)[PER], double u, double* Z, double* before,
                                              PickScratch& sh, int slot)
{
    return block_locate_impl<PER, true>(w, u, before, sh, slot, Z);
}


// One request's logits over the 256-wide tile at v0 (thread t: column v0 + t),
// bit-identical to the bias pass (same W2 fragments, same MFMA sequence, the
// request in column 0 of the N-tile), then the base logit added.  xb: the
// thread's base logit (-inf past V); e_row: the embedding row in LDS (zeros
// when the previous token selects none), written before the call.  The A
// fragments are loaded straight from W2 into registers:
// wave w's rows v0 + 64 w + a_row_voff(t, i), k-steps 16 ks + 8 h.  Addresses
// are clamped into the rows and the loads issued unconditionally: a clamped
// row (past V) only feeds columns whose base logit is -inf, and a clamped
// k-step (past r) meets zeros of the embedding row, so the products are those
// of the staged fragments.
__device__ __forceinline__ float tile_logit(const uint16_t* __restrict__ W2, int V, int r, int v0,
                                            const uint16_t* e_row, float xb, PickScratch& sh)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int h = lane >> 5, c32 = lane & 31;
    // the fragments in two halves of the k-steps (64 registers each, not 128):
    // the pick kernels then fit four waves per SIMD instead of two
    constexpr int kHalf = kKSteps / 2;
    const uint16_t* wrow[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
        wrow[t] = W2 + (int64_t)min(v0 + 64 * wave + a_row_voff(t, c32), V - 1) * r;
    uint4 af[2][kHalf];
    auto fetch = [&](int half) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < kHalf; ++i)
                af[t][i] = *reinterpret_cast<const uint4*>(
                    wrow[t] + min((half * kHalf + i) * kKStep + 8 * h, r - 8));
    };
    fetch(0);
    lds_barrier();   // e_row is written
    floatx16 acc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[t][j] = 0.0f;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        if (half == 1) {
            __builtin_amdgcn_sched_barrier(0);
            fetch(1);
        }
#pragma unroll
        for (int i = 0; i < kHalf; ++i) {
            const int ks = half * kHalf + i;
            uint4 u = make_uint4(0, 0, 0, 0);
            if (c32 == 0) u = *reinterpret_cast<const uint4*>(e_row + ks * kKStep + 8 * h);
            const bf16x8 bv = as_bf16x8(u);
#pragma unroll
            for (int t = 0; t < 2; ++t) acc[t] = mfma32_bf16(as_bf16x8(af[t][i]), bv, acc[t]);
        }
    }
    if (c32 == 0) {
#pragma unroll
        for (int s = 0; s < 32; ++s) sh.lg[wave * 64 + 32 * h + s] = acc[s >> 4][s & 15];
    }
    lds_barrier();
    return xb + sh.lg[threadIdx.x];
}

// One request's logits over the 64 columns at v0 (thread t < 64: column v0 + t),
// bit-identical to tile_logit and the passes (each column the same MFMA sequence):
// waves 0 and 1 run M-tiles 0 and 1 of the 64-block (the rows a_row_voff
// places), waves 2 and 3 only meet the barriers.  Same conventions as
// tile_logit; threads 64.. get the logit of column v0 + t % 64.
__device__ __forceinline__ float sub_logit(const uint16_t* __restrict__ W2, int V, int r, int v0,
                                           const uint16_t* e_row, float xb, PickScratch& sh)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int h = lane >> 5, c32 = lane & 31;
    constexpr int kHalf = kKSteps / 2;
    const bool live = wave < 2;   // wave-uniform
    const uint16_t* wrow = W2 + (int64_t)min(v0 + a_row_voff(wave & 1, c32), V - 1) * r;
    uint4 af[kHalf];
    auto fetch = [&](int half) {
#pragma unroll
        for (int i = 0; i < kHalf; ++i)
            af[i] = *reinterpret_cast<const uint4*>(wrow + min((half * kHalf + i) * kKStep + 8 * h, r - 8));
    };
    if (live) fetch(0);
    lds_barrier();   // e_row is written
    if (live) {
        floatx16 acc;
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[j] = 0.0f;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            if (half == 1) {
                __builtin_amdgcn_sched_barrier(0);
                fetch(1);
            }
#pragma unroll
            for (int i = 0; i < kHalf; ++i) {
                const int ks = half * kHalf + i;
                uint4 u = make_uint4(0, 0, 0, 0);
                if (c32 == 0) u = *reinterpret_cast<const uint4*>(e_row + ks * kKStep + 8 * h);
                acc = mfma32_bf16(as_bf16x8(af[i]), as_bf16x8(u), acc);
            }
        }
        if (c32 == 0) {
#pragma unroll
            for (int j = 0; j < 16; ++j) sh.lg[32 * h + 16 * wave + j] = acc[j];
        }
    }
    lds_barrier();
    return xb + sh.lg[threadIdx.x & 63];
}

}  // namespace dsp

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

#include "bias_tile.h"
#include "dsp_device.h"

namespace dsp {

enum PassKind : int { kSample = 0, kGreedy = 1, kResidual = 2 };

// ---------------------------------------------------------------------------
// softmax weight exp(x), x <= 0 (x = -inf gives 0): the hardware exp2 of
// x log2 e.  Accuracy budget: the sums these weights enter are accumulated in
// fp64, which is what keeps the inverse-CDF decisions in step with an fp64
// reference at vocabularies of 10^5; a more careful argument reduction did not
// change a single decision in measurement and costs four times the ALU work.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float exp_w(float x)
{
    return __builtin_amdgcn_exp2f(x * 1.44269502162933349609375f);
}

// exp((z - ref) / T) with itL = log2(e) / T folded once per kernel; every pass,
// combine and rescan of a row uses this same form so partials and rescans agree.
__device__ __forceinline__ float wexp(float d, float itL) { return __builtin_amdgcn_exp2f(d * itL); }

__host__ __device__ inline float fold_itl(float inv_temp) { return inv_temp * 1.44269502162933349609375f; }

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
    const uint16_t* E;
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
};

// ---------------------------------------------------------------------------
// bias_pass_kernel: grid (n_vt, request chunks), 256 threads; wave w owns
// vocabulary [256 vt + 64 w, +64) of every 64-request sub-block.  Lane l holds
// request column l % 16 of each N-tile and the 16 vocabulary slots of lane group
// l / 16 (bias_voff / slot_voff); the logit rows for those slots are prefetched
// as raw 16-byte words before the MFMA chain.
// ---------------------------------------------------------------------------
// Two workgroups per CU for the bf16 softmax / greedy passes (their registers
// fit 256 per lane); the residual pass and fp32 rows need more and run one.
template <typename LT, int KIND>
constexpr int pass_min_blocks() { return (sizeof(LT) == 2 && KIND != kResidual) ? 2 : 1; }

template <typename LT, int KIND>
__global__ __launch_bounds__(256, (pass_min_blocks<LT, KIND>())) void bias_pass_kernel(PassArgs a)
{
    // double-buffered embedding tiles and cross-wave partials: sub-block i + 1 is
    // staged and its logit rows requested while sub-block i is computed
    __shared__ __attribute__((aligned(16))) uint16_t e_tile[2][kReqBlock][kRankMax + kERowPad];
    __shared__ Part red[2][4][kReqBlock];
    constexpr int RW = Logit<LT>::kRaw;

    const int count = (KIND == kResidual) ? *a.count : a.R;
    const int n_begin = blockIdx.y * a.req_per_wg;
    if (n_begin >= count) return;   // workgroup-uniform
    const int n_end = min(count, n_begin + a.req_per_wg);

    const int vt = blockIdx.x;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int g = lane >> 4, c16 = lane & 15;
    const int V = a.V, r = a.r, gamma = a.gamma;
    const int v_blk = vt * kVocabTile + wave * 64;
    const int ksteps = (r + kKStep - 1) / kKStep;
    const LT* __restrict__ base = static_cast<const LT*>(a.base);
    const LT* __restrict__ target = static_cast<const LT*>(a.target);
    const bool vec_ok = (V % Logit<LT>::kVecAlign) == 0;
    const int va = v_blk + 8 * g, vb = v_blk + 32 + 8 * g;
    const bool fa = vec_ok && va + 8 <= V, fb = vec_ok && vb + 8 <= V;
    const float it = a.inv_temp;
    const float itL = fold_itl(it);

    bf16x8 afrag[4][kKSteps];
    load_w2_frags(a.W2, V, r, v_blk, lane, afrag);

    // embedding rows of sub-block n0 into buffer b: thread t owns row t % 64 and
    // the quarter t / 64 of it, so a wave writes 64 different rows at one column
    // (conflict-free LDS stores); two halves keep the staging registers small
    auto stage_e = [&](int n0, int b) {
        const int row = threadIdx.x & 63, q4 = threadIdx.x >> 6;
        const int e = n0 + row;
        int prev = -1;
        if (e < n_end) {
            if constexpr (KIND == kResidual) prev = a.list_prev[e];
            else prev = prev_token(a.anchor, a.tok, e, gamma, a.k, V);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            uint4 u[kRankMax / 64];
#pragma unroll
            for (int c = 0; c < kRankMax / 64; ++c) {
                const int kk = (q4 * (kRankMax / 32) + h * (kRankMax / 64) + c) * 8;
                u[c] = make_uint4(0, 0, 0, 0);
                if (prev >= 0 && kk < r) u[c] = *reinterpret_cast<const uint4*>(a.E + (int64_t)prev * r + kk);
            }
#pragma unroll
            for (int c = 0; c < kRankMax / 64; ++c)
                *reinterpret_cast<uint4*>(
                    &e_tile[b][row][(q4 * (kRankMax / 32) + h * (kRankMax / 64) + c) * 8]) = u[c];
        }
    };
    // raw logit words of N-tile tn of sub-block n0 (request rows for this lane)
    auto load_raw = [&](int n0, int tn, uint4* rs_tn, uint4* rt_tn) {
        const int e = n0 + 16 * tn + c16;
        const bool ok = e < n_end;
        int n = e, m = a.k;
        if constexpr (KIND == kResidual) {
            n = ok ? a.list[e] : 0;
            m = ok ? a.list_m[e] : 0;
        }
        const LT* row = base + ((int64_t)(ok ? n : 0) * gamma + m) * V;
        Logit<LT>::load8_raw(row, ok ? va : V, V, ok && fa, rs_tn);
        Logit<LT>::load8_raw(row, ok ? vb : V, V, ok && fb, rs_tn + RW);
        if constexpr (KIND == kResidual) {
            const LT* trow = target + ((int64_t)(ok ? n : 0) * (gamma + 1) + m) * V;
            Logit<LT>::load8_raw(trow, ok ? va : V, V, ok && fa, rt_tn);
            Logit<LT>::load8_raw(trow, ok ? vb : V, V, ok && fb, rt_tn + RW);
        }
    };

    uint4 rs[4][2 * RW];
    uint4 rt[KIND == kResidual ? 4 : 1][2 * RW];
    stage_e(n_begin, 0);
#pragma unroll
    for (int tn = 0; tn < 4; ++tn) load_raw(n_begin, tn, rs[tn], rt[KIND == kResidual ? tn : 0]);
    lds_barrier();

    int buf = 0;
    for (int n0 = n_begin; n0 < n_end; n0 += kReqBlock, buf ^= 1) {
        const int n1 = n0 + kReqBlock;
        const bool more = n1 < n_end;

        // two halves of two N-tiles each: half the accumulators live at a time, and
        // the embedding rows of the next sub-block are staged between the halves
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
        floatx4 acc[2][4];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int t = 0; t < 4; ++t) acc[i][t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < kKSteps; ++ks) {
            if (ks < ksteps) {
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const bf16x8 b = as_bf16x8(*reinterpret_cast<const uint4*>(
                        &e_tile[buf][16 * (2 * hf + i) + c16][ks * kKStep + 8 * g]));
#pragma unroll
                    for (int t = 0; t < 4; ++t) acc[i][t] = mfma_bf16(afrag[t][ks], b, acc[i][t]);
                }
            }
        }
        if (hf == 0 && more) stage_e(n1, buf ^ 1);

#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int tn = 2 * hf + i;
            float z[16];
#pragma unroll
            for (int s = 0; s < 16; ++s)
                z[s] = Logit<LT>::raw_at(rs[tn] + (s >> 3) * RW, s & 7) + acc[i][s >> 2][s & 3];
            float xt[KIND == kResidual ? 16 : 1];
            if constexpr (KIND == kResidual) {
#pragma unroll
                for (int s = 0; s < 16; ++s) xt[s] = Logit<LT>::raw_at(rt[tn] + (s >> 3) * RW, s & 7);
            }
            // the next sub-block's rows reuse this N-tile's registers
            if (more) load_raw(n1, tn, rs[tn], rt[KIND == kResidual ? tn : 0]);
            Part res;
            if constexpr (KIND == kGreedy) {
                // slot s maps to increasing vocabulary ids, so the first slot holding
                // the lane maximum is the lane's lowest-index argmax; masked slots
                // (past V) come last and carry -inf
                float m = z[0];
#pragma unroll
                for (int s = 1; s < 16; ++s) m = fmaxf(m, z[s]);
                int si = 15;
#pragma unroll
                for (int s = 14; s >= 0; --s) si = (z[s] == m) ? s : si;
                const int v = v_blk + slot_voff(g, si);
                ArgMax am{m, v < V ? v : 0x7fffffff};
#pragma unroll
                for (int o = 16; o < 64; o <<= 1) {
                    ArgMax b;
                    b.v = __shfl_xor(am.v, o, kWave);
                    b.i = __shfl_xor(am.i, o, kWave);
                    am = argmax_merge(am, b);
                }
                res = Part{am.v, am.i, 0.0};
            } else if constexpr (KIND == kSample) {
                float m = z[0];
#pragma unroll
                for (int s = 1; s < 16; ++s) m = fmaxf(m, z[s]);
                m = fmaxf(m, __shfl_xor(m, 16, kWave));
                m = fmaxf(m, __shfl_xor(m, 32, kWave));
                const float mref = (m == -INFINITY) ? 0.0f : m;   // an all-masked block
                double sum = 0.0;
#pragma unroll
                for (int s = 0; s < 16; s += 2)
                    sum += (double)(wexp(z[s] - mref, itL) + wexp(z[s + 1] - mref, itL));
                sum += __shfl_xor(sum, 16, kWave);
                sum += __shfl_xor(sum, 32, kWave);
                res = Part{m, 0, sum};
            } else {   // kResidual
                const int e = n0 + 16 * tn + c16;
                double sum = 0.0;
                if (e < n_end) {
                    const int n = a.list[e];
                    const int m = a.list_m[e];
                    const float Md = (float)a.stats[2 * ((int64_t)n * gamma + m)];
                    const double invZd = 1.0 / a.stats[2 * ((int64_t)n * gamma + m) + 1];
                    const float Mt = a.row_m[n];
                    const double invZt = 1.0 / a.row_z[n];
#pragma unroll
                    for (int s = 0; s < 16; ++s) {
                        const double pv = (double)wexp(xt[s] - Mt, itL) * invZt;
                        const double qv = (double)wexp(z[s] - Md, itL) * invZd;
                        sum += fmax(pv - qv, 0.0);
                    }
                }
                sum += __shfl_xor(sum, 16, kWave);
                sum += __shfl_xor(sum, 32, kWave);
                res = Part{0.f, 0, sum};
            }
            if (g == 0) red[buf][wave][16 * tn + c16] = res;
        }
        }
        lds_barrier();
        if (threadIdx.x < kReqBlock) {
            const int e = n0 + threadIdx.x;
            if (e < n_end) {
                Part p = red[buf][0][threadIdx.x];
#pragma unroll
                for (int w = 1; w < 4; ++w) {
                    const Part b = red[buf][w][threadIdx.x];
                    if constexpr (KIND == kGreedy) {
                        const ArgMax m = argmax_merge(ArgMax{p.m, p.idx}, ArgMax{b.m, b.idx});
                        p.m = m.v;
                        p.idx = m.i;
                    } else if constexpr (KIND == kSample) {
                        const float mm = fmaxf(p.m, b.m);
                        if (mm != -INFINITY)
                            p.s = p.s * (double)wexp(p.m - mm, itL) + b.s * (double)wexp(b.m - mm, itL);
                        p.m = mm;
                    } else {
                        p.s += b.s;
                    }
                }
                a.part[(int64_t)e * a.n_vt + vt] = p;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// block-wide helpers for 256-thread pick workgroups
// ---------------------------------------------------------------------------
struct PickScratch {
    double wsum[4];
    float wmax[4];
    double scan[4];
    int hit[4];
    float lg[kVocabTile];
    float wt[kVocabTile];
};

__device__ __forceinline__ float block_max256(float v, PickScratch& sh)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    v = wave_max(v);
    if (lane == 0) sh.wmax[wave] = v;
    __syncthreads();
    const float r = fmaxf(fmaxf(sh.wmax[0], sh.wmax[1]), fmaxf(sh.wmax[2], sh.wmax[3]));
    __syncthreads();
    return r;
}

// Locate the first of n_items consecutive weights (thread t owns items
// [t * per, t * per + per)) whose inclusive cumulative sum exceeds target.
// w[] holds the thread's weights (zeros past the end).  Returns the item and
// the cumulative mass before it; falls back to the last positive item.
template <int PER>
__device__ __forceinline__ int block_locate(const double (&w)[PER], double target, double* before,
                                            PickScratch& sh)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    double ls = 0.0;
#pragma unroll
    for (int i = 0; i < PER; ++i) ls += w[i];
    const double incl = wave_incl_scan(ls, lane);
    if (lane == kWave - 1) sh.scan[wave] = incl;
    __syncthreads();
    double off = 0.0;
    for (int w2 = 0; w2 < wave; ++w2) off += sh.scan[w2];
    __syncthreads();
    double c = off + incl - ls;
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
    int h = wave_min_i(hit);
    if (lane == 0) sh.hit[wave] = h;
    __syncthreads();
    h = min(min(sh.hit[0], sh.hit[1]), min(sh.hit[2], sh.hit[3]));
    __syncthreads();
    if (h == 0x7fffffff) {
        // rounding left the target beyond the total: take the last positive item
        int l = wave_max_i(last);
        if (lane == 0) sh.hit[wave] = l;
        __syncthreads();
        h = max(max(sh.hit[0], sh.hit[1]), max(sh.hit[2], sh.hit[3]));
        __syncthreads();
        // cumulative mass before it
        double b = 0.0;
        if ((int)threadIdx.x == h / PER) {
            double cc = off + incl - ls;
            for (int i = 0; i < PER; ++i) { if ((int)threadIdx.x * PER + i == h) break; cc += w[i]; }
            sh.scan[0] = cc;
        }
        __syncthreads();
        b = sh.scan[0];
        __syncthreads();
        *before = b;
        return h < 0 ? 0 : h;
    }
    if ((int)threadIdx.x == h / PER) sh.scan[0] = hit_before;
    __syncthreads();
    *before = sh.scan[0];
    __syncthreads();
    return h;
}

}  // namespace dsp

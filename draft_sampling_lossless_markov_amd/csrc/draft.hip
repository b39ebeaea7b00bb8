// draft.hip -- semi-autoregressive draft step with the Markov head (gfx950).
//
// One draft position k for all R requests, in two launches:
//   draft_partials: per (request, 256-vocabulary tile) online-softmax partials
//     (max, sum exp) -- or (max, argmax) in greedy mode -- of
//     logit = base[n, k, :] + E[prev_n] . W2^T, the bias computed by bf16 MFMA
//     with W2 held in registers and embedding rows staged through LDS.  The bias
//     tile never leaves registers.
//   draft_pick: per request, combine the tile partials (fp64), draw u from
//     Philox, locate the tile whose cumulative mass crosses u * Z, recompute that
//     one tile's logits with the identical MFMA sequence and scan it in order.
//
// DSpark pages: the sequential head adds a bias from the previous token before
// each sample (page "DSpark.让每一轮计算，多走几步", Markov-head paragraph); it is
// a low-rank matrix (page "DeepSeek联合北大最新文章DSpark", two-stage design);
// only the token id is carried to the next position (page "DeepSeek DSpark 技术
// 解析", section 四).
#include "bias_tile.h"
#include "dsp_device.h"
#include "dsp_launch.h"

namespace dsp {

// ---------------------------------------------------------------------------
// draft_partials
// grid: (n_vt, n_req_chunks); block: 256 = 4 waves, wave w owns vocabulary
// [256 vt + 64 w, +64).  Each workgroup walks its request chunk in sub-blocks
// of 64 requests (4 N-tiles).
// part[n * n_vt + vt] = (m, s) or (max value, argmax index bits)
// ---------------------------------------------------------------------------
template <typename LT, bool GREEDY>
__global__ __launch_bounds__(256) void draft_partials_kernel(
    const LT* __restrict__ base, const uint16_t* __restrict__ E, const uint16_t* __restrict__ W2,
    const int32_t* __restrict__ anchor, const int32_t* __restrict__ tok, int R, int gamma, int V,
    int r, int k, float inv_temp, int n_vt, int req_per_wg, float2* __restrict__ part)
{
    __shared__ __attribute__((aligned(16))) uint16_t e_tile[kReqBlock][kRankMax + kERowPad];
    __shared__ float2 red[4][kReqBlock];

    const int vt = blockIdx.x;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int g = lane >> 4, c16 = lane & 15;
    const int v_blk = vt * kVocabTile + wave * 64;
    const int ksteps = (r + kKStep - 1) / kKStep;

    bf16x8 afrag[4][kKSteps];
    load_w2_frags(W2, V, r, v_blk, lane, afrag);

    const bool vec_ok = (V % Logit<LT>::kVecAlign) == 0;
    const int n_begin = blockIdx.y * req_per_wg;
    const int n_end = min(R, n_begin + req_per_wg);

    for (int n0 = n_begin; n0 < n_end; n0 += kReqBlock) {
        // stage the embedding rows E[prev] of 64 requests (zero rows past the end)
        const int chunks = kRankMax / 8;
        for (int idx = threadIdx.x; idx < kReqBlock * chunks; idx += blockDim.x) {
            const int row = idx / chunks, ch = idx % chunks;
            const int n = n0 + row;
            uint4 u = make_uint4(0, 0, 0, 0);
            if (n < n_end && ch * 8 < r) {
                const int prev = prev_token(anchor, tok, n, gamma, k, V);
                if (prev >= 0) u = *reinterpret_cast<const uint4*>(E + (int64_t)prev * r + ch * 8);
            }
            *reinterpret_cast<uint4*>(&e_tile[row][ch * 8]) = u;
        }
        __syncthreads();

        floatx4 acc[4][4];
#pragma unroll
        for (int tn = 0; tn < 4; ++tn)
#pragma unroll
            for (int t = 0; t < 4; ++t) acc[tn][t] = floatx4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
        for (int ks = 0; ks < kKSteps; ++ks) {
            if (ks < ksteps) {
#pragma unroll
                for (int tn = 0; tn < 4; ++tn) {
                    const uint4 bu =
                        *reinterpret_cast<const uint4*>(&e_tile[16 * tn + c16][ks * kKStep + 8 * g]);
                    const bf16x8 b = as_bf16x8(bu);
#pragma unroll
                    for (int t = 0; t < 4; ++t) acc[tn][t] = mfma_bf16(afrag[t][ks], b, acc[tn][t]);
                }
            }
        }

        // epilogue: biased logits -> per-request partial over this wave's 64 columns
#pragma unroll
        for (int tn = 0; tn < 4; ++tn) {
            const int n = n0 + 16 * tn + c16;
            float x[16];
            if (n < n_end) {
                const LT* row = base + ((int64_t)n * gamma + k) * V;
                const int va = v_blk + 8 * g, vb = v_blk + 32 + 8 * g;
                Logit<LT>::load8(row, va, V, vec_ok && va + 8 <= V, x);
                Logit<LT>::load8(row, vb, V, vec_ok && vb + 8 <= V, x + 8);
            } else {
#pragma unroll
                for (int s = 0; s < 16; ++s) x[s] = -INFINITY;
            }
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                const float b = acc[tn][s >> 2][s & 3];
                x[s] = (x[s] == -INFINITY) ? -INFINITY : x[s] + b;
            }
            float2 res;
            if constexpr (GREEDY) {
                ArgMax am{-INFINITY, 0x7fffffff};
#pragma unroll
                for (int s = 0; s < 16; ++s) {
                    const int v = v_blk + slot_voff(g, s);
                    if (v < V) am = argmax_merge(am, ArgMax{x[s], v});
                }
#pragma unroll
                for (int o = 16; o < 64; o <<= 1) {
                    ArgMax b;
                    b.v = __shfl_xor(am.v, o, kWave);
                    b.i = __shfl_xor(am.i, o, kWave);
                    am = argmax_merge(am, b);
                }
                res = make_float2(am.v, __int_as_float(am.i));
            } else {
                float m = -INFINITY;
#pragma unroll
                for (int s = 0; s < 16; ++s) m = fmaxf(m, x[s]);
                float sum = 0.f;
                if (m != -INFINITY) {
#pragma unroll
                    for (int s = 0; s < 16; ++s) sum += __expf((x[s] - m) * inv_temp);
                }
                res = make_float2(m, sum);
#pragma unroll
                for (int o = 16; o < 64; o <<= 1) {
                    float2 b;
                    b.x = __shfl_xor(res.x, o, kWave);
                    b.y = __shfl_xor(res.y, o, kWave);
                    res = lse_merge(res, b, inv_temp);
                }
            }
            if (g == 0) red[wave][16 * tn + c16] = res;
        }
        __syncthreads();
        if (threadIdx.x < kReqBlock) {
            const int n = n0 + threadIdx.x;
            if (n < n_end) {
                float2 a = red[0][threadIdx.x];
#pragma unroll
                for (int w = 1; w < 4; ++w) {
                    const float2 b = red[w][threadIdx.x];
                    if constexpr (GREEDY) {
                        const ArgMax m = argmax_merge(ArgMax{a.x, __float_as_int(a.y)},
                                                      ArgMax{b.x, __float_as_int(b.y)});
                        a = make_float2(m.v, __int_as_float(m.i));
                    } else {
                        a = lse_merge(a, b, inv_temp);
                    }
                }
                part[(int64_t)n * n_vt + vt] = a;
            }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// draft_pick: one wave per request.
// ---------------------------------------------------------------------------
template <typename LT, bool GREEDY>
__global__ __launch_bounds__(256) void draft_pick_kernel(
    const LT* __restrict__ base, const uint16_t* __restrict__ E, const uint16_t* __restrict__ W2,
    const int32_t* __restrict__ anchor, int32_t* __restrict__ tok, float* __restrict__ q,
    float* __restrict__ stats, int R, int gamma, int V, int r, int k, float inv_temp,
    uint64_t seed, uint32_t round, int n_vt, const float2* __restrict__ part)
{
    __shared__ float lg_s[4][kVocabTile];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n = blockIdx.x * 4 + wave;
    const bool active = n < R;   // wave-uniform
    const float2* pp = part + (int64_t)(active ? n : 0) * n_vt;
    const int64_t out = (int64_t)n * gamma + k;

    if constexpr (GREEDY) {
        if (!active) return;   // no barrier on this path
        ArgMax am{-INFINITY, 0x7fffffff};
        for (int t = lane; t < n_vt; t += kWave) {
            const float2 p = pp[t];
            am = argmax_merge(am, ArgMax{p.x, __float_as_int(p.y)});
        }
        am = wave_argmax(am);
        if (lane == 0) {
            tok[out] = am.i;
            q[out] = 1.0f;
            stats[2 * out] = am.v;
            stats[2 * out + 1] = 0.0f;
        }
    } else {
        float M = -INFINITY;
        double Z = 0.0, target = 0.0, before = 0.0;
        int tsel = 0;
        if (active) {
            for (int t = lane; t < n_vt; t += kWave) M = fmaxf(M, pp[t].x);
            M = wave_max(M);
            // tile masses s_t exp((m_t - M) / T) in fp64, summed in tile order
            for (int t0 = 0; t0 < n_vt; t0 += kWave) {
                const int t = t0 + lane;
                double w = 0.0;
                if (t < n_vt) {
                    const float2 p = pp[t];
                    if (p.x != -INFINITY) w = (double)p.y * exp(((double)p.x - (double)M) * (double)inv_temp);
                }
                Z += wave_sum(w);
            }
            const double u = uniform24(seed, round, (uint32_t)n, (uint32_t)k, 0u);
            target = u * Z;
            double run = 0.0, before_last = 0.0;
            int hit_t = -1, tlast = 0;
            for (int t0 = 0; t0 < n_vt && hit_t < 0; t0 += kWave) {
                const int t = t0 + lane;
                double w = 0.0;
                if (t < n_vt) {
                    const float2 p = pp[t];
                    if (p.x != -INFINITY) w = (double)p.y * exp(((double)p.x - (double)M) * (double)inv_temp);
                }
                const double incl = wave_incl_scan(w, lane) + run;
                const int hit = wave_min_i((incl > target) ? t : 0x7fffffff);
                const int lastpos = wave_max_i((w > 0.0) ? t : -1);
                if (lastpos >= 0) {
                    tlast = lastpos;
                    before_last = __shfl(incl - w, lastpos - t0, kWave);
                }
                if (hit != 0x7fffffff) {
                    hit_t = hit;
                    before = __shfl(incl - w, hit - t0, kWave);
                }
                run = __shfl(incl, kWave - 1, kWave);
            }
            if (hit_t < 0) { hit_t = tlast; before = before_last; }
            tsel = hit_t;
            const int prev = prev_token(anchor, tok, n, gamma, k, V);
            const LT* row = base + ((int64_t)n * gamma + k) * V;
            tile_logits<LT>(row, E, W2, V, r, prev, tsel, lane, lg_s[wave]);
        }
        __syncthreads();
        if (active) {
            float wsel;
            const int loc = tile_inverse_cdf(lg_s[wave], M, inv_temp, before, target, lane, &wsel);
            if (lane == 0) {
                tok[out] = tsel * kVocabTile + loc;
                q[out] = (float)((double)wsel / Z);
                stats[2 * out] = M;
                stats[2 * out + 1] = (float)Z;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
size_t draft_workspace_bytes(int R, int V)
{
    const size_t n_vt = (size_t)((V + kVocabTile - 1) / kVocabTile);
    return (size_t)R * n_vt * sizeof(float2);
}

template <typename LT>
static hipError_t launch_draft_t(const LT* base, const uint16_t* E, const uint16_t* W2,
                                 const int32_t* anchor, int32_t* tok, float* q, float* stats, int R,
                                 int gamma, int V, int r, int k, float temperature, uint64_t seed,
                                 uint32_t round, void* ws, hipStream_t s)
{
    const int n_vt = (V + kVocabTile - 1) / kVocabTile;
    float2* part = static_cast<float2*>(ws);
    const bool greedy = (temperature == 0.0f);
    const float inv_temp = greedy ? 1.0f : 1.0f / temperature;
    // requests per workgroup: whole 64-request blocks, split into enough balanced
    // chunks that the grid has about 2048 workgroups (8 per CU)
    const int blocks = (R + kReqBlock - 1) / kReqBlock;
    const int want = std::max(1, std::min(blocks, (2048 + n_vt - 1) / n_vt));
    const int req_per_wg = ((blocks + want - 1) / want) * kReqBlock;
    const dim3 g1(n_vt, (R + req_per_wg - 1) / req_per_wg);
    if (greedy)
        hipLaunchKernelGGL((draft_partials_kernel<LT, true>), g1, dim3(256), 0, s, base, E, W2,
                           anchor, tok, R, gamma, V, r, k, inv_temp, n_vt, req_per_wg, part);
    else
        hipLaunchKernelGGL((draft_partials_kernel<LT, false>), g1, dim3(256), 0, s, base, E, W2,
                           anchor, tok, R, gamma, V, r, k, inv_temp, n_vt, req_per_wg, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 g2((R + 3) / 4);
    if (greedy)
        hipLaunchKernelGGL((draft_pick_kernel<LT, true>), g2, dim3(256), 0, s, base, E, W2, anchor,
                           tok, q, stats, R, gamma, V, r, k, inv_temp, seed, round, n_vt, part);
    else
        hipLaunchKernelGGL((draft_pick_kernel<LT, false>), g2, dim3(256), 0, s, base, E, W2, anchor,
                           tok, q, stats, R, gamma, V, r, k, inv_temp, seed, round, n_vt, part);
    return hipGetLastError();
}

hipError_t launch_draft_step(const void* base, bool bf16, const uint16_t* E, const uint16_t* W2,
                             const int32_t* anchor, int32_t* tok, float* q, float* stats, int R,
                             int gamma, int V, int r, int k, float temperature, uint64_t seed,
                             uint32_t round, void* ws, hipStream_t s)
{
    if (bf16)
        return launch_draft_t(static_cast<const uint16_t*>(base), E, W2, anchor, tok, q, stats, R,
                              gamma, V, r, k, temperature, seed, round, ws, s);
    return launch_draft_t(static_cast<const float*>(base), E, W2, anchor, tok, q, stats, R, gamma,
                          V, r, k, temperature, seed, round, ws, s);
}

}  // namespace dsp

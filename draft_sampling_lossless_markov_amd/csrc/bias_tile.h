// bias_tile.h -- one request's Markov-biased draft logits for one
// 256-vocabulary tile, recomputed with exactly the MFMA sequence of the draft
// kernel, plus the in-order inverse-CDF scan of such a tile.
#pragma once

#include "dsp_device.h"

namespace dsp {

// x_{k-1} of request n: the anchor for k = 0.  A token outside [0, V) carries no
// Markov bias (-1).
__device__ __forceinline__ int prev_token(const int32_t* __restrict__ anchor,
                                          const int32_t* __restrict__ tok, int n, int gamma, int k,
                                          int V)
{
    const int p = (k == 0) ? anchor[n] : tok[(int64_t)n * gamma + (k - 1)];
    return (p >= 0 && p < V) ? p : -1;
}

// ---------------------------------------------------------------------------
// Biased logits of one 256-vocabulary tile for one request, computed by one wave
// with the same MFMA sequence as draft_partials (request in column 0 of the
// N-tile).  Writes lg[0..255] (vocabulary order, -inf past V) to LDS.
// ---------------------------------------------------------------------------
template <typename LT>
__device__ __forceinline__ void tile_logits(const LT* __restrict__ row, const uint16_t* __restrict__ E,
                            const uint16_t* __restrict__ W2, int V, int r, int prev, int tile,
                            int lane, float* __restrict__ lg)
{
    const int g = lane >> 4, c16 = lane & 15;
    const int ksteps = (r + kKStep - 1) / kKStep;
    for (int wb = 0; wb < 4; ++wb) {
        const int v_blk = tile * kVocabTile + wb * 64;
        bf16x8 afrag[4][kKSteps];
        load_w2_frags(W2, V, r, v_blk, lane, afrag);
        floatx4 acc[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < kKSteps; ++ks) {
            if (ks < ksteps) {
                const int kk = ks * kKStep + 8 * g;
                uint4 u = make_uint4(0, 0, 0, 0);
                if (c16 == 0 && prev >= 0 && kk < r)
                    u = *reinterpret_cast<const uint4*>(E + (int64_t)prev * r + kk);
                const bf16x8 b = as_bf16x8(u);
#pragma unroll
                for (int t = 0; t < 4; ++t) acc[t] = mfma_bf16(afrag[t][ks], b, acc[t]);
            }
        }
        if (c16 == 0) {
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                const int voff = slot_voff(g, s);
                const int v = v_blk + voff;
                lg[wb * 64 + voff] = (v < V) ? Logit<LT>::at(row, v) + acc[s >> 2][s & 3] : -INFINITY;
            }
        }
    }
}

// In-order inverse-CDF scan of a 256-wide tile whose weights w[4] are held by
// the lanes (lane l owns tile positions 4l .. 4l+3): the first v with
// cum_before + sum_{i<=v} w_i > target; falls back to the last positive weight of
// the tile.  Returns the tile-local index and its weight in *w_out.
__device__ __forceinline__ int tile_inverse_cdf_w(const float w[4], double cum_before,
                                                  double target, int lane, float* w_out)
{
    double ls = 0.0;
#pragma unroll
    for (int e = 0; e < 4; ++e) ls += (double)w[e];
    const double incl = wave_incl_scan(ls, lane);
    double c = cum_before + (incl - ls);
    int hit = 0x7fffffff, last = -1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        c += (double)w[e];
        if (hit == 0x7fffffff && c > target) hit = 4 * lane + e;
        if (w[e] > 0.f) last = 4 * lane + e;
    }
    hit = wave_min_i(hit);
    if (hit == 0x7fffffff) hit = wave_max_i(last);
    const int src = hit >> 2;
    float wsel = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float t = __shfl(w[e], src, kWave);
        if ((hit & 3) == e) wsel = t;
    }
    *w_out = wsel;
    return hit;
}

// Softmax weights exp((lg - M) / T) of the tile positions a lane owns.
__device__ __forceinline__ int tile_inverse_cdf(const float* __restrict__ lg, float M, float it,
                                                double cum_before, double target, int lane,
                                                float* w_out)
{
    float w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float z = lg[4 * lane + e];
        w[e] = (z == -INFINITY) ? 0.f : __expf((z - M) * it);
    }
    return tile_inverse_cdf_w(w, cum_before, target, lane, w_out);
}

}  // namespace dsp

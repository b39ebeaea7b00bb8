// bias_tile.h -- one request's Markov-biased draft logits for one 64-wide
// vocabulary block, recomputed with exactly the MFMA sequence of the bias pass
// (same fragments, same K order, accumulation from zero), so every element is
// bit-identical to the value the pass reduced.
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

// lg[0..63] = base row [v_blk, v_blk + 64) + bias (fp32); -inf past V.  Called by
// one whole wave; the request sits in column 0 of the N-tile.
template <typename LT>
__device__ __forceinline__ void block_logits64(const LT* __restrict__ row,
                                               const uint16_t* __restrict__ E,
                                               const uint16_t* __restrict__ W2, int V, int r,
                                               int prev, int v_blk, int lane, float* __restrict__ lg)
{
    const int g = lane >> 4, c16 = lane & 15;
    const int ksteps = (r + kKStep - 1) / kKStep;
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
            lg[voff] = (v < V) ? Logit<LT>::at(row, v) + acc[s >> 2][s & 3] : -INFINITY;
        }
    }
}

}  // namespace dsp

// bias_tile.h -- one request's Markov-biased draft logits for one 64-wide
// vocabulary block, recomputed with exactly the MFMA sequence of the bias pass
// (same fragments, same K order, accumulation from zero, then the base logit
// added), so every element is bit-identical to the value the pass reduced.
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
// one whole wave; the request sits in column 0 of the N-tile (lanes 0 and 32).
template <typename LT>
__device__ __forceinline__ void block_logits64(const LT* __restrict__ row,
                                               const uint16_t* __restrict__ E,
                                               const uint16_t* __restrict__ W2, int V, int r,
                                               int prev, int v_blk, int lane, float* __restrict__ lg)
{
    const int h = lane >> 5, c32 = lane & 31;
    bf16x8 afrag[2][kKSteps];
    load_w2_frags(W2, V, r, v_blk, lane, afrag);
    floatx16 acc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[t][j] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
        const int kk = ks * kKStep + 8 * h;
        uint4 u = make_uint4(0, 0, 0, 0);
        if (c32 == 0 && prev >= 0 && kk < r)
            u = *reinterpret_cast<const uint4*>(E + (int64_t)prev * r + kk);
        const bf16x8 b = as_bf16x8(u);
#pragma unroll
        for (int t = 0; t < 2; ++t) acc[t] = mfma32_bf16(afrag[t][ks], b, acc[t]);
    }
    if (c32 == 0) {
#pragma unroll
        for (int s = 0; s < 32; ++s) {
            const int voff = 32 * h + s;
            const int v = v_blk + voff;
            lg[voff] = (v < V) ? Logit<LT>::at(row, v) + acc[s >> 4][s & 15] : -INFINITY;
        }
    }
}

}  // namespace dsp

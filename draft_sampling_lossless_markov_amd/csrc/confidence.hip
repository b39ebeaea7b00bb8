// confidence.hip -- confidence head with sequential temperature scaling (gfx950).
//
// Page "DeepSeek联合北大最新文章DSpark", section 2.1: c_k estimates the chance that
// draft token k is accepted given that all earlier ones were, as a sigmoid of a
// linear map of the backbone state h_k concatenated with the Markov embedding of
// x_{k-1}; per-position temperatures fitted left to right calibrate it.
//
// One wave per (request, position) row: a d + r long dot product accumulated in
// fp64 (bf16 x fp32 products are exact in fp64), then the sigmoid in fp64 and one
// rounding to fp32.  Bound by streaming h once.  Without temperatures (T null)
// the kernel writes the sigmoid's argument instead: the raw logit that the
// temperatures are fitted on.
#include "dsp_device.h"
#include "dsp_launch.h"

namespace dsp {

__global__ __launch_bounds__(256) void confidence_kernel(
    const uint16_t* __restrict__ h, const uint16_t* __restrict__ E,
    const int32_t* __restrict__ anchor, const int32_t* __restrict__ tok,
    const float* __restrict__ w, const float* __restrict__ T, const float* __restrict__ offset,
    float* __restrict__ c, int R, int gamma, int d, int V, int r)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + wave;
    if (row >= (int64_t)R * gamma) return;
    const int n = (int)(row / gamma), k = (int)(row % gamma);
    const uint16_t* hr = h + row * d;
    double acc = 0.0;
    if ((d & 7) == 0) {
        // issue up to four 16-byte loads per lane before accumulating
        for (int i0 = lane * 8; i0 < d; i0 += 4 * kWave * 8) {
            uint4 u[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int i = i0 + t * kWave * 8;
                u[t] = (i < d) ? load_nt16(hr + i) : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int i = i0 + t * kWave * 8;
                if (i >= d) break;
                const float4 w0 = *reinterpret_cast<const float4*>(w + i);
                const float4 w1 = *reinterpret_cast<const float4*>(w + i + 4);
                acc += (double)w0.x * (double)__uint_as_float(u[t].x << 16);
                acc += (double)w0.y * (double)__uint_as_float(u[t].x & 0xFFFF0000u);
                acc += (double)w0.z * (double)__uint_as_float(u[t].y << 16);
                acc += (double)w0.w * (double)__uint_as_float(u[t].y & 0xFFFF0000u);
                acc += (double)w1.x * (double)__uint_as_float(u[t].z << 16);
                acc += (double)w1.y * (double)__uint_as_float(u[t].z & 0xFFFF0000u);
                acc += (double)w1.z * (double)__uint_as_float(u[t].w << 16);
                acc += (double)w1.w * (double)__uint_as_float(u[t].w & 0xFFFF0000u);
            }
        }
    } else {
        for (int i = lane; i < d; i += kWave) acc += (double)w[i] * (double)bf16_to_f32(hr[i]);
    }
    const int prev = (k == 0) ? anchor[n] : tok[row - 1];
    if (prev >= 0 && prev < V) {
        const uint16_t* er = E + (int64_t)prev * r;
        for (int i = lane; i < r; i += kWave) acc += (double)w[d + i] * (double)bf16_to_f32(er[i]);
    }
    acc = wave_sum(acc);
    if (lane == 0) {
        const double y = acc + (offset ? (double)offset[n] : 0.0);
        c[row] = T ? (float)(1.0 / (1.0 + exp(-y / (double)T[k]))) : (float)y;
    }
}

hipError_t launch_confidence(const uint16_t* h, const uint16_t* E, const int32_t* anchor,
                             const int32_t* tok, const float* w, const float* T,
                             const float* offset, float* c, int R, int gamma, int d, int V, int r,
                             hipStream_t s)
{
    const int64_t rows = (int64_t)R * gamma;
    const dim3 grid((unsigned)((rows + 3) / 4));
    hipLaunchKernelGGL(confidence_kernel, grid, dim3(256), 0, s, h, E, anchor, tok, w, T, offset,
                       c, R, gamma, d, V, r);
    return hipGetLastError();
}

}  // namespace dsp

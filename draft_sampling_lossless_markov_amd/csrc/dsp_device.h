// dsp_device.h -- device-side building blocks shared by the gfx950 kernels of
// libdsp: wave64 reductions, the Philox4x32-10 counter generator, bf16 loads
// and the bf16 MFMA fragment types.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsp {

constexpr int kWave = 64;
constexpr int kRankMax = 256;             // largest Markov rank r the bias kernels hold
constexpr int kKStep = 32;                // K of one v_mfma_f32_16x16x32_bf16
constexpr int kKSteps = kRankMax / kKStep;
constexpr int kVocabTile = 256;           // vocabulary columns per draft workgroup
constexpr int kReqBlock = 64;             // requests per MFMA sub-block (4 N-tiles of 16)
constexpr int kERowPad = 8;               // bf16 padding of an LDS embedding row
constexpr int kVerifyChunk = 8192;        // vocabulary per verify row work item

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming load that does not allocate in the caches (logit rows are
// read once; keeping them out of L2/MALL leaves room for E and W2).
__device__ __forceinline__ uint4 load_nt16(const void* p)
{
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Workgroup barrier that orders LDS only.  __syncthreads() also waits for every
// outstanding global load of the calling wave, which would drain the logit rows
// prefetched for the next sub-block at each barrier; kernels whose global loads
// land in registers (never read by another wave) use this one instead.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u)
{
    bf16x8 r;
    __builtin_memcpy(&r, &u, sizeof(r));
    return r;
}

__device__ __forceinline__ floatx4 mfma_bf16(bf16x8 a, bf16x8 b, floatx4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon et al., SC'11): 10 rounds of two 32x32 multiplies with
// a Weyl-sequence key schedule.  counter = (round, request, position, purpose),
// key = (seed low, seed high); u = (word0 >> 8) / 2^24.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t philox_word0(uint64_t seed, uint32_t c0, uint32_t c1,
                                                 uint32_t c2, uint32_t c3)
{
    uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
#pragma unroll
    for (int i = 0; i < 10; ++i) {
        const uint32_t a_hi = __umulhi(0xD2511F53u, c0), a_lo = 0xD2511F53u * c0;
        const uint32_t b_hi = __umulhi(0xCD9E8D57u, c2), b_lo = 0xCD9E8D57u * c2;
        const uint32_t n0 = b_hi ^ c1 ^ k0;
        const uint32_t n2 = a_hi ^ c3 ^ k1;
        c0 = n0; c1 = b_lo; c2 = n2; c3 = a_lo;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return c0;
}

__device__ __forceinline__ double uniform24(uint64_t seed, uint32_t round, uint32_t req,
                                            uint32_t pos, uint32_t purpose)
{
    return (double)(philox_word0(seed, round, req, pos, purpose) >> 8) * (1.0 / 16777216.0);
}

// ---------------------------------------------------------------------------
// wave64 reductions
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

__device__ __forceinline__ double wave_sum(double v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

__device__ __forceinline__ int wave_min_i(int v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, kWave));
    return v;
}

__device__ __forceinline__ int wave_max_i(int v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, kWave));
    return v;
}

// inclusive prefix sum over the 64 lanes, in lane order
__device__ __forceinline__ double wave_incl_scan(double v, int lane)
{
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const double t = __shfl_up(v, o, kWave);
        if (lane >= o) v += t;
    }
    return v;
}

// (value, index) argmax: larger value wins, the lower index on ties.
struct ArgMax {
    float v;
    int i;
};

__device__ __forceinline__ ArgMax argmax_merge(ArgMax a, ArgMax b)
{
    if (b.v > a.v || (b.v == a.v && b.i < a.i)) return b;
    return a;
}

__device__ __forceinline__ ArgMax wave_argmax(ArgMax a)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        ArgMax b;
        b.v = __shfl_xor(a.v, o, kWave);
        b.i = __shfl_xor(a.i, o, kWave);
        a = argmax_merge(a, b);
    }
    return a;
}

// Online-softmax partial (m, s): s = sum exp((x - m) * it) over a set of
// logits with maximum m (m = -inf, s = 0 for the empty set).
__device__ __forceinline__ float2 lse_merge(float2 a, float2 b, float it)
{
    const float m = fmaxf(a.x, b.x);
    if (m == -INFINITY) return make_float2(-INFINITY, 0.0f);
    const float s = a.y * __expf((a.x - m) * it) + b.y * __expf((b.x - m) * it);
    return make_float2(m, s);
}

// ---------------------------------------------------------------------------
// logit loads (fp32 or bf16 rows), 8 consecutive values.  `load8` unpacks to
// fp32; `load8_raw` keeps the loaded bits (one 16-byte word per 8 bf16 values,
// two per 8 fp32 values) and `raw_at` unpacks element e later, so prefetched
// rows occupy half the registers for bf16.  Columns past V read as -inf.
// ---------------------------------------------------------------------------
template <typename LT>
struct Logit;

template <>
struct Logit<float> {
    static constexpr int kVecAlign = 4;   // elements per 16 bytes
    static constexpr int kRaw = 2;        // 16-byte words per 8 elements
    __device__ static __forceinline__ float at(const float* p, int64_t i) { return p[i]; }
    __device__ static __forceinline__ void load8_raw(const float* row, int v0, int V, bool fast,
                                                     uint4 r[2])
    {
        if (fast) {
            r[0] = load_nt16(row + v0);
            r[1] = load_nt16(row + v0 + 4);
        } else {
            uint32_t w[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                w[e] = (v0 + e < V) ? __float_as_uint(row[v0 + e]) : 0xFF800000u;
            r[0] = make_uint4(w[0], w[1], w[2], w[3]);
            r[1] = make_uint4(w[4], w[5], w[6], w[7]);
        }
    }
    __device__ static __forceinline__ float raw_at(const uint4 r[2], int e)
    {
        const uint4 q = r[e >> 2];
        const uint32_t w = ((e & 3) == 0) ? q.x : ((e & 3) == 1) ? q.y : ((e & 3) == 2) ? q.z : q.w;
        return __uint_as_float(w);
    }
    __device__ static __forceinline__ void load8(const float* row, int v0, int V, bool fast,
                                                 float x[8])
    {
        uint4 r[2];
        load8_raw(row, v0, V, fast, r);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = raw_at(r, e);
    }
};

template <>
struct Logit<uint16_t> {
    static constexpr int kVecAlign = 8;
    static constexpr int kRaw = 1;
    __device__ static __forceinline__ float at(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
    __device__ static __forceinline__ void load8_raw(const uint16_t* row, int v0, int V, bool fast,
                                                     uint4 r[1])
    {
        if (fast) {
            r[0] = load_nt16(row + v0);
        } else {
            uint32_t w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t lo = (v0 + 2 * e < V) ? row[v0 + 2 * e] : 0xFF80u;
                const uint32_t hi = (v0 + 2 * e + 1 < V) ? row[v0 + 2 * e + 1] : 0xFF80u;
                w[e] = lo | (hi << 16);
            }
            r[0] = make_uint4(w[0], w[1], w[2], w[3]);
        }
    }
    __device__ static __forceinline__ float raw_at(const uint4 r[1], int e)
    {
        const uint4 q = r[0];
        const uint32_t w = ((e >> 1) == 0) ? q.x : ((e >> 1) == 1) ? q.y : ((e >> 1) == 2) ? q.z : q.w;
        return (e & 1) ? __uint_as_float(w & 0xFFFF0000u) : __uint_as_float(w << 16);
    }
    __device__ static __forceinline__ void load8(const uint16_t* row, int v0, int V, bool fast,
                                                 float x[8])
    {
        uint4 r[1];
        load8_raw(row, v0, V, fast, r);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = raw_at(r, e);
    }
};

// ---------------------------------------------------------------------------
// The Markov-bias MFMA tile shared by every kernel that needs biased draft
// logits.  A wave computes a 64-vocabulary x 16-request block per N-tile:
//   out[v, n] = sum_i W2[v, i] * E[prev_n, i]
// with W2 rows as the A operand (M = vocabulary) and embedding rows as the B
// operand (N = requests).  Lane l of the 16x16 output tile holds request column
// l % 16 and rows 4 (l / 16) + 0..3.  The vocabulary order inside the 64-block
// is permuted so that lane group g = l / 16 owns the 16 columns
// {8g .. 8g+7} and {32+8g .. 32+8g+7}: two 16-byte logit loads per request.
// Every caller issues the same K order (k-steps 0..ceil(r/32)-1 accumulated
// into a zero tile), so a vocabulary element's bias is bit-identical wherever
// it is recomputed.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int bias_voff(int t, int m)
{
    // output slot s of M-tile t, row m: lane group m / 4, position 4 t + m % 4
    const int s = 4 * t + (m & 3);
    const int g = m >> 2;
    return (s < 8) ? (8 * g + s) : (32 + 8 * g + (s - 8));
}

// value slot s (0..15) of lane group g -> vocabulary offset inside the 64-block
__device__ __forceinline__ int slot_voff(int g, int s) { return (s < 8) ? (8 * g + s) : (24 + 8 * g + s); }

// Load the A fragments (W2 rows) of a 64-vocabulary block starting at v_blk.
__device__ __forceinline__ void load_w2_frags(const uint16_t* __restrict__ W2, int V, int r,
                                              int v_blk, int lane, bf16x8 a[4][kKSteps])
{
    const int m = lane & 15, g = lane >> 4;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int v = v_blk + bias_voff(t, m);
#pragma unroll
        for (int ks = 0; ks < kKSteps; ++ks) {
            const int kk = ks * kKStep + 8 * g;
            uint4 u = make_uint4(0, 0, 0, 0);
            if (v < V && kk < r) u = *reinterpret_cast<const uint4*>(W2 + (int64_t)v * r + kk);
            a[t][ks] = as_bf16x8(u);
        }
    }
}

}  // namespace dsp

// dsp_device.h -- device-side building blocks shared by the gfx950 kernels of
// libdsp: wave64 reductions, the Philox4x32-10 counter generator, bf16 loads
// and the bf16 MFMA fragment types.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsp {

constexpr int kWave = 64;
constexpr int kRankMax = 256;             // largest Markov rank r the bias kernels hold
constexpr int kKStep = 16;                // K of one v_mfma_f32_32x32x16_bf16
constexpr int kKSteps = kRankMax / kKStep;
constexpr int kVocabTile = 256;           // vocabulary columns per draft workgroup
constexpr int kReqBlock = 64;             // requests per MFMA sub-block (4 N-tiles of 16)
constexpr int kERowPad = 8;               // bf16 padding of an LDS embedding row
constexpr int kVerifyChunk = 8192;        // vocabulary per verify row work item

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
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

// D = A B + C with A 32x16 (W2 rows), B 16x32 (embedding rows), fp32 C.  On
// gfx950 this form issues at twice the rate of the 16x16x32 one.  Lane l holds
// A row l % 32 and B column l % 32 at k = 8 (l / 32) .. +7, and D column l % 32
// at rows 8 (j / 4) + 4 (l / 32) + j % 4, j = 0..15.
__device__ __forceinline__ floatx16 mfma32_bf16(bf16x8 a, bf16x8 b, floatx16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
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

// ---------------------------------------------------------------------------
// Combines across lanes l ^ 16 and l ^ 32 with the gfx950 row-swap instructions
// (v_permlane16_swap / v_permlane32_swap): a register-to-register exchange, no
// LDS round trip.  permlane16_swap(x, x) returns, in every lane, the values of
// lanes l and l ^ 16 (in row order), permlane32_swap(x, x) those of l and l ^ 32.
// Every combine below is commutative, so all lanes of a pair get identical bits.
// ---------------------------------------------------------------------------
template <int O>
__device__ __forceinline__ void xswap(uint32_t x, uint32_t& p, uint32_t& q)
{
    static_assert(O == 16 || O == 32, "row swaps exist for 16 and 32 only");
    if constexpr (O == 16) {
        const auto v = __builtin_amdgcn_permlane16_swap(x, x, false, false);
        p = v[0];
        q = v[1];
    } else {
        const auto v = __builtin_amdgcn_permlane32_swap(x, x, false, false);
        p = v[0];
        q = v[1];
    }
}

template <int O>
__device__ __forceinline__ float xmax(float x)
{
    uint32_t p, q;
    xswap<O>(__float_as_uint(x), p, q);
    return fmaxf(__uint_as_float(p), __uint_as_float(q));
}

template <int O>
__device__ __forceinline__ double xsum(double x)
{
    const uint64_t b = (uint64_t)__double_as_longlong(x);
    uint32_t p0, q0, p1, q1;
    xswap<O>((uint32_t)b, p0, q0);
    xswap<O>((uint32_t)(b >> 32), p1, q1);
    const double a = __longlong_as_double((long long)(((uint64_t)p1 << 32) | p0));
    const double c = __longlong_as_double((long long)(((uint64_t)q1 << 32) | q0));
    return a + c;
}

template <int O>
__device__ __forceinline__ ArgMax xargmax(ArgMax x)
{
    uint32_t pv, qv, pi, qi;
    xswap<O>(__float_as_uint(x.v), pv, qv);
    xswap<O>((uint32_t)x.i, pi, qi);
    return argmax_merge(ArgMax{__uint_as_float(pv), (int)pi}, ArgMax{__uint_as_float(qv), (int)qi});
}

// ---------------------------------------------------------------------------
// Whole-wave reductions and scans on DPP row operations (quad permutes, row
// mirrors, row shifts and row broadcasts) plus the row swaps above: VALU work,
// no LDS round trips.  Every lane gets the result.
// ---------------------------------------------------------------------------
template <int CTRL, int ROW_MASK = 0xF, bool ZERO_FILL = false>
__device__ __forceinline__ uint32_t dpp32(uint32_t x)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROW_MASK, 0xF, ZERO_FILL);
}

template <int CTRL, int ROW_MASK = 0xF, bool ZERO_FILL = false>
__device__ __forceinline__ double dpp64(double x)
{
    const uint64_t b = (uint64_t)__double_as_longlong(x);
    const uint32_t lo = dpp32<CTRL, ROW_MASK, ZERO_FILL>((uint32_t)b);
    const uint32_t hi = dpp32<CTRL, ROW_MASK, ZERO_FILL>((uint32_t)(b >> 32));
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

constexpr int kDppXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7 - i within 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15 - i within 16

__device__ __forceinline__ float wave_max_f(float x)
{
    x = fmaxf(x, __uint_as_float(dpp32<kDppXor1>(__float_as_uint(x))));
    x = fmaxf(x, __uint_as_float(dpp32<kDppXor2>(__float_as_uint(x))));
    x = fmaxf(x, __uint_as_float(dpp32<kDppHalfMirror>(__float_as_uint(x))));
    x = fmaxf(x, __uint_as_float(dpp32<kDppMirror>(__float_as_uint(x))));
    return xmax<32>(xmax<16>(x));
}

__device__ __forceinline__ double wave_sum_d(double x)
{
    x += dpp64<kDppXor1>(x);
    x += dpp64<kDppXor2>(x);
    x += dpp64<kDppHalfMirror>(x);
    x += dpp64<kDppMirror>(x);
    return xsum<32>(xsum<16>(x));
}

template <bool MAX>
__device__ __forceinline__ int wave_minmax_i(int x)
{
    auto op = [](int a, int b) { return MAX ? max(a, b) : min(a, b); };
    x = op(x, (int)dpp32<kDppXor1>((uint32_t)x));
    x = op(x, (int)dpp32<kDppXor2>((uint32_t)x));
    x = op(x, (int)dpp32<kDppHalfMirror>((uint32_t)x));
    x = op(x, (int)dpp32<kDppMirror>((uint32_t)x));
    uint32_t p, q;
    xswap<16>((uint32_t)x, p, q);
    x = op((int)p, (int)q);
    xswap<32>((uint32_t)x, p, q);
    return op((int)p, (int)q);
}

// inclusive prefix sum over the 64 lanes: Hillis-Steele within each 16-lane row
// (row shifts by 1, 2, 4, 8 with zero fill), then the row totals carried by the
// row broadcasts of lane 15 (to rows 1 and 3) and lane 31 (to rows 2 and 3)
__device__ __forceinline__ double wave_scan_d(double x)
{
    x += dpp64<0x111, 0xF, true>(x);
    x += dpp64<0x112, 0xF, true>(x);
    x += dpp64<0x114, 0xF, true>(x);
    x += dpp64<0x118, 0xF, true>(x);
    x += dpp64<0x142, 0xA>(x);
    x += dpp64<0x143, 0xC>(x);
    return x;
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
// logits.  A wave computes a 64-vocabulary x 32-request block per N-tile:
//   out[v, n] = sum_i W2[v, i] * E[prev_n, i]
// with W2 rows as the A operand (two 32-row M-tiles) and embedding rows as the
// B operand (N = requests).  The W2 rows are placed in the M-tiles in an order
// that gives lane l (half h = l / 32) the 32 contiguous vocabulary columns
// [32 h, 32 h + 32) of the 64-block in its accumulators: slot s = 16 t + j of
// M-tile t, register j, is column 32 h + s.  Lanes l and l ^ 32 hold the two
// halves of one request's 64 columns.  Every caller issues the same K order
// (k-steps 0..15 accumulated into a zero tile; fragments past r are zero), so
// a vocabulary element's bias is bit-identical wherever it is recomputed.
// ---------------------------------------------------------------------------
// A row i of M-tile t -> vocabulary offset in the 64-block (inverse of the
// accumulator placement above: row 8 q + 4 h + e holds column 32 h + 16 t + 4 q + e)
__device__ __forceinline__ int a_row_voff(int t, int i)
{
    const int q = i >> 3, h = (i >> 2) & 1, e = i & 3;
    return 32 * h + 16 * t + 4 * q + e;
}

// Load the A fragments (W2 rows) of a 64-vocabulary block starting at v_blk.
__device__ __forceinline__ void load_w2_frags(const uint16_t* __restrict__ W2, int V, int r,
                                              int v_blk, int lane, bf16x8 a[2][kKSteps])
{
    const int i = lane & 31, h = lane >> 5;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int v = v_blk + a_row_voff(t, i);
#pragma unroll
        for (int ks = 0; ks < kKSteps; ++ks) {
            const int kk = ks * kKStep + 8 * h;
            uint4 u = make_uint4(0, 0, 0, 0);
            if (v < V && kk < r) u = *reinterpret_cast<const uint4*>(W2 + (int64_t)v * r + kk);
            a[t][ks] = as_bf16x8(u);
        }
    }
}

}  // namespace dsp

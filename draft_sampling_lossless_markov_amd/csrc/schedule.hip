// schedule.hip -- hardware-aware prefix scheduler (gfx950), one workgroup.
//
// Page "DeepSeek联合北大最新文章DSpark", section 2.2: pick the verify lengths that
// maximise Theta = tau * SPS(B), B = sum (1 + l_r), tau = sum of admitted survival
// probabilities, by sorting every candidate by survival probability, admitting
// them in that order and stopping when throughput stops rising.  Page "DSpark.让
// 每一轮计算，多走几步", section 写得长，不如验得值: a_j = c_1 x ... x c_j, so a
// request's candidates never overtake their own prefix in the sort.
//
// Steps, all in LDS of one 1024-thread workgroup:
//   1. a = running fp32 product of c along each request (also written out)
//   2. stable LSD radix sort (4 passes of 8 bits) of the candidate indices by the
//      key ~bits(a): a descending, then index (r, j) ascending; ranks inside a
//      wave come from ballots, so the sort is deterministic and stable
//   3. Q48 fixed-point prefix sums of a in sorted order (exact, so the order of
//      the parallel scan cannot change them), Theta_n = double(S_n 2^-48) SPS(R+n)
//   4. first n whose Theta does not rise (or R + n > B_max) -> admitted count
//   5. per-request counts of the admitted prefix -> l_r, B
#include "dsp_device.h"
#include "dsp_launch.h"

namespace dsp {

namespace {
constexpr int kSchedThreads = 1024;
constexpr int kSchedWaves = kSchedThreads / kWave;
constexpr int kRadixBits = 8;
constexpr int kBuckets = 1 << kRadixBits;

__device__ __forceinline__ uint32_t sort_key(float a) { return ~__float_as_uint(a); }

__device__ __forceinline__ uint64_t q48(float a)
{
    return (uint64_t)((double)a * 281474976710656.0);   // a >= 0: truncation = floor
}

struct SortLds {
    uint32_t hist[kSchedWaves][kBuckets];   // per-wave digit counts, then offsets
    uint32_t digit_tot[kBuckets];
};

// Stable LSD radix sort (4 passes of 8 bits) of candidate indices idx[cur][0..N)
// by the key ~bits(a[idx]): a descending, then index ascending.  Wave w owns a
// contiguous segment of the current order; offsets are laid out (digit, wave) so
// segment order is kept; ranks inside a wave come from ballots (deterministic).
// Returns the buffer holding the sorted order.  Called by the whole workgroup.
__device__ int sort_desc(const float* a_s, uint16_t (&idx_s)[2][kSchedMaxCand], int N, SortLds& L)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int seg = ((N + kSchedWaves - 1) / kSchedWaves + kWave - 1) / kWave * kWave;
    const int seg_begin = min(N, wave * seg);
    const int seg_end = min(N, seg_begin + seg);
    const uint64_t lanes_below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int cur = 0;
    for (int shift = 0; shift < 32; shift += kRadixBits) {
        for (int b = lane; b < kBuckets; b += kWave) L.hist[wave][b] = 0;
        __syncthreads();
        for (int e = seg_begin + lane; e < seg_end; e += kWave) {
            const uint32_t dgt = (sort_key(a_s[idx_s[cur][e]]) >> shift) & (kBuckets - 1);
            atomicAdd(&L.hist[wave][dgt], 1u);
        }
        __syncthreads();
        if (tid < kBuckets) {
            uint32_t run = 0;
            for (int w = 0; w < kSchedWaves; ++w) {
                const uint32_t t = L.hist[w][tid];
                L.hist[w][tid] = run;
                run += t;
            }
            L.digit_tot[tid] = run;
        }
        __syncthreads();
        if (wave == 0) {
            // exclusive scan of the 256 digit totals, 4 consecutive digits per lane
            uint32_t v[4], sm = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) { v[e] = L.digit_tot[4 * lane + e]; sm += v[e]; }
            uint32_t incl = sm;
#pragma unroll
            for (int o = 1; o < kWave; o <<= 1) {
                const uint32_t t = __shfl_up(incl, o, kWave);
                if (lane >= o) incl += t;
            }
            uint32_t run = incl - sm;
#pragma unroll
            for (int e = 0; e < 4; ++e) { L.digit_tot[4 * lane + e] = run; run += v[e]; }
        }
        __syncthreads();
        if (tid < kBuckets) {
            const uint32_t b = L.digit_tot[tid];
            for (int w = 0; w < kSchedWaves; ++w) L.hist[w][tid] += b;
        }
        __syncthreads();
        // scatter, one 64-element round at a time in segment order
        for (int e0 = seg_begin; e0 < seg_end; e0 += kWave) {
            const int e = e0 + lane;
            const bool valid = e < seg_end;
            const uint16_t id = valid ? idx_s[cur][e] : 0;
            const uint32_t dgt = valid ? (sort_key(a_s[id]) >> shift) & (kBuckets - 1) : 0;
            uint64_t same = __ballot(valid);
#pragma unroll
            for (int bit = 0; bit < kRadixBits; ++bit) {
                const uint64_t bb = __ballot((dgt >> bit) & 1u);
                same &= ((dgt >> bit) & 1u) ? bb : ~bb;
            }
            const uint32_t rank = (uint32_t)__popcll(same & lanes_below);
            const uint32_t cnt = (uint32_t)__popcll(same);
            uint32_t base = 0;
            if (valid) base = L.hist[wave][dgt];
            if (valid) idx_s[cur ^ 1][base + rank] = id;
            if (valid && rank + 1 == cnt) L.hist[wave][dgt] = base + cnt;
        }
        __syncthreads();
        cur ^= 1;
    }
    return cur;
}

// The Q48 prefix sums of the sorted survival values, as each thread's exclusive
// start over its contiguous chunk [p0, p0 + items): S0 + sum of the q48 values
// before p0.  Called by the whole workgroup.
__device__ uint64_t chunk_prefix(const float* a_s, const uint16_t* order, int N, uint64_t S0, int p0,
                                 int items, uint64_t* wave_tot)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint64_t local = 0;
    for (int p = p0; p < min(N, p0 + items); ++p) local += q48(a_s[order[p]]);
    uint64_t incl = local;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const uint64_t t = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += t;
    }
    if (lane == kWave - 1) wave_tot[wave] = incl;
    __syncthreads();
    if (tid == 0) {
        uint64_t run = 0;
        for (int w = 0; w < kSchedWaves; ++w) {
            const uint64_t t = wave_tot[w];
            wave_tot[w] = run;
            run += t;
        }
    }
    __syncthreads();
    return S0 + wave_tot[wave] + (incl - local);
}
}  // namespace

__global__ __launch_bounds__(kSchedThreads) void schedule_kernel(
    const float* __restrict__ c, const float* __restrict__ sps, int B_max, uint64_t S0, int mode,
    int32_t* __restrict__ len, float* __restrict__ a_out, int32_t* __restrict__ B_out, int R,
    int gamma)
{
    __shared__ float a_s[kSchedMaxCand];                 // survival; later per-request counts
    __shared__ uint16_t idx_s[2][kSchedMaxCand];         // candidate index ping-pong
    __shared__ SortLds sl;
    __shared__ uint64_t wave_tot[kSchedWaves];
    __shared__ int stop_at;

    const int tid = threadIdx.x;
    const int N = R * gamma;

    // 1. survival products, left to right
    for (int rr = tid; rr < R; rr += kSchedThreads) {
        float prod = 1.0f;
        for (int j = 0; j < gamma; ++j) {
            prod = __fmul_rn(prod, c[(int64_t)rr * gamma + j]);
            a_out[(int64_t)rr * gamma + j] = prod;
            if (mode != 0) a_s[rr * gamma + j] = prod;
        }
    }
    if (mode == 0) {
        for (int rr = tid; rr < R; rr += kSchedThreads) len[rr] = gamma;
        if (tid == 0) *B_out = R * (1 + gamma);
        return;
    }
    for (int i = tid; i < N; i += kSchedThreads) idx_s[0][i] = (uint16_t)i;
    if (tid == 0) stop_at = N;
    __syncthreads();

    // 2. stable radix sort: a descending, then (r, j) ascending
    const int cur = sort_desc(a_s, idx_s, N, sl);

    // 3-4. Q48 prefix sums in sorted order and the first non-rising Theta
    const int items = (N + kSchedThreads - 1) / kSchedThreads;
    const int p0 = tid * items;
    uint64_t S = chunk_prefix(a_s, idx_s[cur], N, S0, p0, items, wave_tot);
    const double inv_scale = 1.0 / 281474976710656.0;
    for (int p = p0; p < min(N, p0 + items); ++p) {
        if (R + p + 1 > B_max) { atomicMin(&stop_at, p); break; }
        const uint64_t S_next = S + q48(a_s[idx_s[cur][p]]);
        const double th_prev = ((double)S * inv_scale) * (double)sps[R + p - 1];
        const double th = ((double)S_next * inv_scale) * (double)sps[R + p];
        if (!(th > th_prev)) { atomicMin(&stop_at, p); break; }
        S = S_next;
    }
    __syncthreads();
    const int n_adm = stop_at;

    // 5. lengths = admitted candidates per request (a_s reused as counters)
    int* cnt = reinterpret_cast<int*>(a_s);
    for (int rr = tid; rr < R; rr += kSchedThreads) cnt[rr] = 0;
    __syncthreads();
    for (int p = tid; p < n_adm; p += kSchedThreads) atomicAdd(&cnt[idx_s[cur][p] / gamma], 1);
    __syncthreads();
    for (int rr = tid; rr < R; rr += kSchedThreads) len[rr] = cnt[rr];
    if (tid == 0) *B_out = R + n_adm;
}

// ---------------------------------------------------------------------------
// Asynchronous scheduler (page "DeepSeek联合北大最新文章DSpark", 挑战2: the capacity
// comes from the confidences of two steps back, the candidates are ranked by the
// newest ones, and the capacity barrier lets the search drop the early stop).
//   capacity: survival products of c_hist, sorted as above; Theta_n for every
//     n <= min(N, B_max - R), K = the smallest n with the maximum Theta
//   admission: survival products of c (written to a), sorted; the first K
//     candidates admitted; l_r, B = R + K, K
// ---------------------------------------------------------------------------
struct ThetaBest {
    double th;
    int n;
};

__device__ __forceinline__ ThetaBest theta_better(ThetaBest x, ThetaBest y)
{
    return (y.th > x.th || (y.th == x.th && y.n < x.n)) ? y : x;
}

__global__ __launch_bounds__(kSchedThreads) void schedule_async_kernel(
    const float* __restrict__ c, const float* __restrict__ c_hist, const float* __restrict__ sps,
    int B_max, uint64_t S0, int32_t* __restrict__ len, float* __restrict__ a_out,
    int32_t* __restrict__ B_out, int32_t* __restrict__ K_out, int R, int gamma)
{
    __shared__ float a_s[kSchedMaxCand];
    __shared__ uint16_t idx_s[2][kSchedMaxCand];
    __shared__ SortLds sl;
    __shared__ uint64_t wave_tot[kSchedWaves];
    __shared__ ThetaBest best_w[kSchedWaves];
    __shared__ int K_s;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int N = R * gamma;
    const int n_max = min(N, B_max - R);
    const double inv_scale = 1.0 / 281474976710656.0;

    // capacity from the earlier round's confidences
    for (int rr = tid; rr < R; rr += kSchedThreads) {
        float prod = 1.0f;
        for (int j = 0; j < gamma; ++j) {
            prod = __fmul_rn(prod, c_hist[(int64_t)rr * gamma + j]);
            a_s[rr * gamma + j] = prod;
        }
    }
    for (int i = tid; i < N; i += kSchedThreads) idx_s[0][i] = (uint16_t)i;
    __syncthreads();
    int cur = sort_desc(a_s, idx_s, N, sl);
    const int items = (N + kSchedThreads - 1) / kSchedThreads;
    const int p0 = tid * items;
    uint64_t S = chunk_prefix(a_s, idx_s[cur], N, S0, p0, items, wave_tot);
    // Theta_0 (nothing admitted) on thread 0, then Theta_n for n = p + 1 of the chunk
    ThetaBest b{-1.0, 0x7fffffff};
    if (tid == 0) b = ThetaBest{((double)S0 * inv_scale) * (double)sps[R - 1], 0};
    for (int p = p0; p < min(n_max, p0 + items); ++p) {
        S += q48(a_s[idx_s[cur][p]]);
        b = theta_better(b, ThetaBest{((double)S * inv_scale) * (double)sps[R + p], p + 1});
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        ThetaBest y;
        y.th = __shfl_xor(b.th, o, kWave);
        y.n = __shfl_xor(b.n, o, kWave);
        b = theta_better(b, y);
    }
    if (lane == 0) best_w[wave] = b;
    __syncthreads();
    if (tid == 0) {
        ThetaBest t = best_w[0];
        for (int w = 1; w < kSchedWaves; ++w) t = theta_better(t, best_w[w]);
        K_s = t.n;
    }

    // admission by the current confidences
    for (int rr = tid; rr < R; rr += kSchedThreads) {
        float prod = 1.0f;
        for (int j = 0; j < gamma; ++j) {
            prod = __fmul_rn(prod, c[(int64_t)rr * gamma + j]);
            a_out[(int64_t)rr * gamma + j] = prod;
            a_s[rr * gamma + j] = prod;
        }
    }
    for (int i = tid; i < N; i += kSchedThreads) idx_s[0][i] = (uint16_t)i;
    __syncthreads();
    cur = sort_desc(a_s, idx_s, N, sl);
    const int K = K_s;
    int* cnt = reinterpret_cast<int*>(a_s);
    for (int rr = tid; rr < R; rr += kSchedThreads) cnt[rr] = 0;
    __syncthreads();
    for (int p = tid; p < K; p += kSchedThreads) atomicAdd(&cnt[idx_s[cur][p] / gamma], 1);
    __syncthreads();
    for (int rr = tid; rr < R; rr += kSchedThreads) len[rr] = cnt[rr];
    if (tid == 0) {
        *B_out = R + K;
        *K_out = K;
    }
}

hipError_t launch_schedule(const float* c, const float* sps, int B_max, uint64_t S0, int mode,
                           int32_t* len, float* a, int32_t* B, int R, int gamma, hipStream_t s)
{
    hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(kSchedThreads), 0, s, c, sps, B_max, S0,
                       mode, len, a, B, R, gamma);
    return hipGetLastError();
}

hipError_t launch_schedule_async(const float* c, const float* c_hist, const float* sps, int B_max,
                                 uint64_t S0, int32_t* len, float* a, int32_t* B, int32_t* K, int R,
                                 int gamma, hipStream_t s)
{
    hipLaunchKernelGGL(schedule_async_kernel, dim3(1), dim3(kSchedThreads), 0, s, c, c_hist, sps,
                       B_max, S0, len, a, B, K, R, gamma);
    return hipGetLastError();
}

}  // namespace dsp

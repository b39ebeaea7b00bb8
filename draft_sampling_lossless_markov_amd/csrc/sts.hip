// sts.hip -- sequential temperature scaling fit and calibration error (gfx950).
//
// Page "DeepSeek联合北大最新文章DSpark", section 2.1: the raw confidences are
// overconfident, so that the cumulative prefix survival is overestimated; the
// temperatures are calibrated on held-out data position by position from left
// to right, and the calibration error (ECE) falls to about 1%.  The page names
// no objective; here T_k, with the earlier temperatures fixed, minimises the
// binary cross-entropy of the cumulative survival a_k = a_{k-1} sigma(z_k / T_k)
// against "prefix accepted through k", over two grids of beta = 1 / T.
//
// Per position k (five launches, stream-ordered, no host round trip):
//   sts_obj_kernel (stage 1)  grid of 256 candidates x sample chunks: thread g of
//                             a workgroup adds the loss of every sample of the
//                             chunk at candidate g (samples staged through LDS
//                             and read by all threads at once) -> partial[chunk][g]
//   sts_pick_kernel           sums the chunks in order, takes the lowest-index
//                             minimum, sets the second grid (the best point's
//                             neighbours)
//   sts_obj_kernel, sts_pick_kernel (stage 2) -> beta_k, T_k, the loss at beta_k
//   sts_update_kernel         carries ln a and b = 1 - a of every sample through k
// Everything in fp64: the loss of one (sample, candidate) takes two to four
// exp/log evaluations, so the fit is bound by the fp64 ALUs.
#include "dsp_device.h"
#include "dsp_launch.h"

namespace dsp {

// ln sigma(x), without overflow
__device__ __forceinline__ double log_sigmoid_d(double x)
{
    return -(fmax(-x, 0.0) + log1p(exp(-fabs(x))));
}

// Cross-entropy of one cumulative survival a sigma(x) against outcome s, from
// la = ln a and b = 1 - a:  s = 1: -(ln a + ln sigma(x));
// s = 0: -ln(1 - a sigma(x)) = -ln(b + a sigma(-x)).
__device__ __forceinline__ double survival_bce_d(double x, bool s, double la, double b)
{
    return s ? -(la + log_sigmoid_d(x)) : -log(b + exp(la + log_sigmoid_d(-x)));
}

struct StsCtl {
    double lo[2];     // first grid point of each stage
    double step[2];   // grid spacing of each stage
    double beta;      // fitted beta of the current position
};

struct StsWs {
    double* la;       // [N] ln a
    double* b;        // [N] 1 - a
    double* partial;  // [nb, kStsGrid]
    StsCtl* ctl;
    int nb, per;      // sample chunks and samples per chunk
};

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static void sts_chunks(int N, int& nb, int& per)
{
    nb = std::min((N + kStsGrid - 1) / kStsGrid, kStsMaxChunks);
    per = (N + nb - 1) / nb;
}

size_t sts_workspace_bytes(int N)
{
    int nb, per;
    sts_chunks(N, nb, per);
    return 2 * align256((size_t)N * sizeof(double)) + align256((size_t)nb * kStsGrid * sizeof(double)) +
           align256(sizeof(StsCtl));
}

static StsWs carve_sts(void* ws, int N)
{
    StsWs w;
    sts_chunks(N, w.nb, w.per);
    char* p = static_cast<char*>(ws);
    w.la = reinterpret_cast<double*>(p);
    p += align256((size_t)N * sizeof(double));
    w.b = reinterpret_cast<double*>(p);
    p += align256((size_t)N * sizeof(double));
    w.partial = reinterpret_cast<double*>(p);
    p += align256((size_t)w.nb * kStsGrid * sizeof(double));
    w.ctl = reinterpret_cast<StsCtl*>(p);
    return w;
}

__global__ __launch_bounds__(256) void sts_init_kernel(double* __restrict__ la, double* __restrict__ b,
                                                       int N, StsCtl* __restrict__ ctl, double lo, double step)
{
    const int n = blockIdx.x * 256 + threadIdx.x;
    if (n < N) {
        la[n] = 0.0;
        b[n] = 0.0;
    }
    if (n == 0) {
        ctl->lo[0] = lo;
        ctl->step[0] = step;
    }
}

// partial[chunk][g] = sum over the chunk's samples, in order, of the loss at
// beta_g = fma(g, step, lo) of the stage
__global__ __launch_bounds__(kStsGrid) void sts_obj_kernel(
    const float* __restrict__ z, const int32_t* __restrict__ acc, const double* __restrict__ la,
    const double* __restrict__ b, int N, int gamma, int k, int per, int stage,
    const StsCtl* __restrict__ ctl, double* __restrict__ partial)
{
    __shared__ double sz[kStsGrid], sla[kStsGrid], sb[kStsGrid];
    __shared__ int ss[kStsGrid];
    const int g = threadIdx.x;
    const double beta = fma((double)g, ctl->step[stage], ctl->lo[stage]);
    const int n0 = blockIdx.x * per, n1 = min(N, n0 + per);
    double f = 0.0;
    for (int base = n0; base < n1; base += kStsGrid) {
        const int n = base + g;
        if (n < n1) {
            sz[g] = (double)z[(int64_t)n * gamma + k];
            sla[g] = la[n];
            sb[g] = b[n];
            ss[g] = acc[n] > k;
        }
        __syncthreads();
        const int cnt = min(kStsGrid, n1 - base);
        for (int i = 0; i < cnt; ++i) f += survival_bce_d(beta * sz[i], ss[i] != 0, sla[i], sb[i]);
        __syncthreads();
    }
    partial[(int64_t)blockIdx.x * kStsGrid + g] = f;
}

// objective of candidate g = chunk partials added in chunk order; the lowest-
// index minimum (a NaN counts as +inf) picks the stage's point
__global__ __launch_bounds__(kStsGrid) void sts_pick_kernel(const double* __restrict__ partial, int nb,
                                                            int stage, int k, StsCtl* __restrict__ ctl,
                                                            float* __restrict__ T, double* __restrict__ nll)
{
    __shared__ double sf[kStsGrid];
    __shared__ int sg[kStsGrid];
    const int g = threadIdx.x;
    double f = 0.0;
    for (int c = 0; c < nb; ++c) f += partial[(int64_t)c * kStsGrid + g];
    if (isnan(f)) f = INFINITY;
    sf[g] = f;
    sg[g] = g;
    __syncthreads();
    for (int off = kStsGrid / 2; off > 0; off >>= 1) {
        if (g < off) {
            const double f2 = sf[g + off];
            const int g2 = sg[g + off];
            if (f2 < sf[g] || (f2 == sf[g] && g2 < sg[g])) {
                sf[g] = f2;
                sg[g] = g2;
            }
        }
        __syncthreads();
    }
    if (g == 0) {
        const int best = sg[0];
        const double lo = ctl->lo[stage], step = ctl->step[stage];
        if (stage == 0) {
            const double lo2 = fma((double)(best > 0 ? best - 1 : 0), step, lo);
            const double hi2 = fma((double)(best < kStsGrid - 1 ? best + 1 : kStsGrid - 1), step, lo);
            ctl->lo[1] = lo2;
            ctl->step[1] = (hi2 - lo2) / (double)(kStsGrid - 1);
        } else {
            const double beta = fma((double)best, step, lo);
            ctl->beta = beta;
            T[k] = (float)(1.0 / beta);
            if (nll) nll[k] = sf[0];
        }
    }
}

// the survival of every sample carried through position k at the fitted beta
__global__ __launch_bounds__(256) void sts_update_kernel(const float* __restrict__ z, double* __restrict__ la,
                                                         double* __restrict__ b, int N, int gamma, int k,
                                                         const StsCtl* __restrict__ ctl)
{
    const int n = blockIdx.x * 256 + threadIdx.x;
    if (n >= N) return;
    const double x = ctl->beta * (double)z[(int64_t)n * gamma + k];
    const double l = la[n];
    b[n] = b[n] + exp(l + log_sigmoid_d(-x));
    la[n] = l + log_sigmoid_d(x);
}

hipError_t launch_sts_fit(const float* z, const int32_t* acc, int N, int gamma, double t_lo,
                          double t_hi, float* T, double* nll, void* ws, hipStream_t s)
{
    const StsWs w = carve_sts(ws, N);
    const double lo = 1.0 / t_hi, hi = 1.0 / t_lo;
    const dim3 gN((unsigned)((N + 255) / 256));
    hipLaunchKernelGGL(sts_init_kernel, gN, dim3(256), 0, s, w.la, w.b, N, w.ctl, lo,
                       (hi - lo) / (double)(kStsGrid - 1));
    for (int k = 0; k < gamma; ++k) {
        for (int stage = 0; stage < 2; ++stage) {
            hipLaunchKernelGGL(sts_obj_kernel, dim3(w.nb), dim3(kStsGrid), 0, s, z, acc, w.la, w.b, N,
                               gamma, k, w.per, stage, w.ctl, w.partial);
            hipLaunchKernelGGL(sts_pick_kernel, dim3(1), dim3(kStsGrid), 0, s, w.partial, w.nb, stage, k,
                               w.ctl, T, nll);
        }
        if (k + 1 < gamma)
            hipLaunchKernelGGL(sts_update_kernel, gN, dim3(256), 0, s, z, w.la, w.b, N, gamma, k, w.ctl);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// ECE of the cumulative survival: every (sample, position) pair is a prediction
// a = prod_{j <= k} sigma(z_j / T_j) of "prefix accepted through k", binned by
// min(floor(a M), M - 1); ECE = sum_bins |sum (s - a)| / (N gamma).  Bin sums
// are exact integers (a in units of 2^-40, at most 2^23 predictions), so the
// result does not depend on the order of the atomic adds.
// ---------------------------------------------------------------------------
struct EceAcc {
    unsigned long long sa[kEceMaxBins];   // sum of a, units of 2^-40
    unsigned long long ss[kEceMaxBins];   // accepted predictions
};

size_t ece_workspace_bytes() { return align256(sizeof(EceAcc)); }

__global__ void ece_zero_kernel(EceAcc* __restrict__ acc)
{
    const int i = threadIdx.x;
    if (i < kEceMaxBins) {
        acc->sa[i] = 0ull;
        acc->ss[i] = 0ull;
    }
}

__global__ __launch_bounds__(256) void ece_kernel(const float* __restrict__ z, const int32_t* __restrict__ nacc,
                                                  const float* __restrict__ T, int N, int gamma, int M,
                                                  EceAcc* __restrict__ out)
{
    __shared__ unsigned long long lsa[kEceMaxBins], lss[kEceMaxBins];
    const int t = threadIdx.x;
    if (t < kEceMaxBins) {
        lsa[t] = 0ull;
        lss[t] = 0ull;
    }
    __syncthreads();
    const int n = blockIdx.x * 256 + t;
    if (n < N) {
        const int na = nacc[n];
        double a = 1.0;
        for (int k = 0; k < gamma; ++k) {
            double x = (double)z[(int64_t)n * gamma + k];
            if (T) x = x / (double)T[k];
            a = a * exp(log_sigmoid_d(x));
            int bin = (int)floor(a * (double)M);
            bin = min(max(bin, 0), M - 1);
            atomicAdd(&lsa[bin], (unsigned long long)(a * 0x1p40));
            if (na > k) atomicAdd(&lss[bin], 1ull);
        }
    }
    __syncthreads();
    if (t < M) {
        if (lsa[t]) atomicAdd(&out->sa[t], lsa[t]);
        if (lss[t]) atomicAdd(&out->ss[t], lss[t]);
    }
}

__global__ void ece_final_kernel(const EceAcc* __restrict__ acc, int M, double count, double* __restrict__ ece)
{
    if (threadIdx.x != 0) return;
    double e = 0.0;
    for (int m = 0; m < M; ++m)
        e += fabs((double)acc->ss[m] - (double)acc->sa[m] * 0x1p-40);
    *ece = e / count;
}

hipError_t launch_ece(const float* z, const int32_t* nacc, const float* T, int N, int gamma, int M,
                      double* ece, void* ws, hipStream_t s)
{
    EceAcc* acc = static_cast<EceAcc*>(ws);
    hipLaunchKernelGGL(ece_zero_kernel, dim3(1), dim3(kEceMaxBins), 0, s, acc);
    hipLaunchKernelGGL(ece_kernel, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, s, z, nacc, T, N,
                       gamma, M, acc);
    hipLaunchKernelGGL(ece_final_kernel, dim3(1), dim3(64), 0, s, acc, M, (double)N * (double)gamma, ece);
    return hipGetLastError();
}

}  // namespace dsp

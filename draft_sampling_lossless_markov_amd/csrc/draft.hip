// draft.hip -- semi-autoregressive draft step with the Markov head (gfx950).
//
// Draft positions k .. k + n_steps - 1 for all R requests.  Where the
// vocabulary slice of W2 fits on chip (bf16 rows), one persistent launch runs
// every position (draft_run.h); otherwise each position takes two launches:
//   bias_pass_kernel<kSample | kGreedy>: per (request, 256-wide vocabulary tile)
//     partials of logit = base[n, k, :] + E[prev_n] . W2^T (bias by bf16 MFMA,
//     never stored);
//   draft_pick_kernel: one workgroup per request combines the partials in fp64,
//     draws u from Philox, locates the tile whose cumulative mass crosses u * Z,
//     recomputes that tile's 256 logits and scans them in order.
//
// DSpark pages: the sequential head adds a bias from the previous token before
// each sample (page "DSpark.让每一轮计算，多走几步", Markov-head paragraph); it is
// a low-rank matrix (page "DeepSeek联合北大最新文章DSpark", two-stage design);
// only the token id is carried to the next position (page "DeepSeek DSpark 技术
// 解析", section 四).
#include <atomic>

#include "bias_tile.h"
#include "draft_pass.h"
#include "draft_pass_wide.h"
#include "draft_run.h"
#include "dsp_device.h"
#include "dsp_launch.h"
#include "tile_pass.h"

namespace dsp {

// ---------------------------------------------------------------------------
// draft_pick: grid R, 256 threads; thread t owns tiles [t * PER, t * PER + PER).
// Sampling: combine the tile partials in fp64 -> (M, Z); u from Philox; locate
// the tile whose cumulative mass crosses u Z; rebuild its 256 logits exactly as
// the pass computed them; locate the token inside it.  The tile's base logits
// and the embedding row are requested before the W2 fetch so their latencies
// overlap.
// ---------------------------------------------------------------------------
template <typename LT, bool GREEDY, int PER, bool SUB>
__global__ __launch_bounds__(256, 4) void draft_pick_kernel(
    const LT* __restrict__ base, RowStrides bs, const uint16_t* __restrict__ E,
    const uint16_t* __restrict__ W2,
    const int32_t* __restrict__ anchor, int32_t* __restrict__ tok, float* __restrict__ q,
    double* __restrict__ stats, int R, int gamma, int V, int r, int k, float inv_temp,
    uint64_t seed, uint32_t round, int n_vt, const Part* __restrict__ part,
    const float4* __restrict__ sub, const uint16_t* __restrict__ S)
{
    __shared__ PickScratch sh;
    const int n = blockIdx.x;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const Part* pp = part + (int64_t)n * n_vt;
    const int64_t out = (int64_t)n * gamma + k;

    if constexpr (GREEDY) {
        ArgMax am{-INFINITY, 0x7fffffff};
        for (int t = tid; t < n_vt; t += 256) am = argmax_merge(am, ArgMax{pp[t].m, pp[t].idx});
        am = wave_argmax(am);
        if (lane == 0) { sh.wmax[wave] = am.v; sh.hit[0][wave] = am.i; }
        lds_barrier();
        if (tid == 0) {
            ArgMax b{sh.wmax[0], sh.hit[0][0]};
            for (int w = 1; w < 4; ++w) b = argmax_merge(b, ArgMax{sh.wmax[w], sh.hit[0][w]});
            tok[out] = b.i;
            q[out] = 1.0f;
            stats[2 * out] = b.v;
            stats[2 * out + 1] = 0.0;
        }
        return;
    } else {
        __shared__ __attribute__((aligned(16))) uint16_t e_row[kRankMax];
        const int prev = prev_token(anchor, tok, n, gamma, k, V);   // issued early
        float mt[PER];
        double st[PER];
        float M = -INFINITY;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int t = tid * PER + i;
            mt[i] = -INFINITY;
            st[i] = 0.0;
            if (t < n_vt) { mt[i] = pp[t].m; st[i] = pp[t].s; }
            M = fmaxf(M, mt[i]);
        }
        M = block_max256(M, sh);
        double w[PER];
        double ls = 0.0;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            w[i] = st[i] * rescale64(mt[i], M, inv_temp);
            ls += w[i];
        }
        const double Z = block_sum256(ls, sh);
        const double u = uniform24(seed, round, (uint32_t)n, (uint32_t)k, 0u);
        const double target = u * Z;
        double before;
        const int tsel = block_locate<PER>(w, target, &before, sh, 0);

        const float m_t = pp[tsel].m;   // the tile's reference in the partial
        const double f = rescale64(m_t, M, inv_temp);
        // SUB: the quarter of the tile whose cumulative mass crosses the target,
        // from the pass's four 64-column sums (the first with positive mass that
        // crosses, else the last with positive mass); only it is rebuilt
        int v0 = tsel * kVocabTile, width = kVocabTile;
        double before_t = before;
        if constexpr (SUB) {
            const float4 sw = sub[(int64_t)tsel * R + n];   // tile-major
            const float sv[4] = {sw.x, sw.y, sw.z, sw.w};
            int js = -1, jl = 0;
            double cum = before, cj = before, cl = before;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const double wj = (double)sv[j] * f;
                if (js < 0 && wj > 0.0 && cum + wj > target) {
                    js = j;
                    cj = cum;
                }
                if (wj > 0.0) {
                    jl = j;
                    cl = cum;
                }
                cum += wj;
            }
            if (js < 0) {
                js = jl;
                cj = cl;
            }
            v0 += 64 * js;
            width = 64;
            before_t = cj;
        }
        // rebuild the chosen columns' logits (thread t: column v0 + t, t < width)
        const LT* row = base + (int64_t)n * bs.rs + (int64_t)k * bs.ps;
        const int v = v0 + tid;
        const bool in_tile = tid < width;
        const float xb = (v < V && in_tile) ? Logit<LT>::at(row, v) : -INFINITY;
        if (tid < kRankMax / 8) {
            // the bias row: E[x_{k-1}] (Markov head) or the state S[n, k]
            const uint16_t* er = S ? S + ((int64_t)n * gamma + k) * r
                                   : (prev >= 0 ? E + (int64_t)prev * r : nullptr);
            const int kk = 8 * tid;
            uint4 ev = make_uint4(0, 0, 0, 0);
            if (er && kk < r) ev = *reinterpret_cast<const uint4*>(er + kk);
            *reinterpret_cast<uint4*>(e_row + kk) = ev;
        }
        const float z = SUB ? sub_logit(W2, V, r, v0, e_row, xb, sh)
                            : tile_logit(W2, V, r, v0, e_row, xb, sh);
        // the pass's own weights: relative to the tile maximum, moved onto the
        // row's reference by the partials' fp64 factor
        const float mref = (m_t == -INFINITY) ? 0.0f : m_t;
        double e1[1] = {(v < V && in_tile) ? (double)wexp(z - mref, fold_itl(inv_temp)) * f : 0.0};
        double b2;
        const int loc = block_locate<1>(e1, target - before_t, &b2, sh, 1);
        if (tid == loc) {
            tok[out] = v0 + loc;
            q[out] = (float)(e1[0] / Z);
            stats[2 * out] = M;
            stats[2 * out + 1] = Z;
        }
    }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
constexpr size_t kRunCtlBytes = 256;

// partials of either path (the streaming path's 256-column tiles, 16 bytes each,
// then the pipelined pass's four 64-column sums per tile, 16 bytes each; or a
// persistent run's tiles: two positions' slots of two 8-byte words), then the
// error word
static size_t draft_part_bytes(int R, int V)
{
    const size_t n_vt = (size_t)((V + kVocabTile - 1) / kVocabTile);
    const size_t n_run = std::min<size_t>((size_t)((V + 31) / 32), (size_t)kRunTilesMax);
    const size_t b = (size_t)R * std::max(n_vt * (sizeof(Part) + sizeof(float4)),
                                          n_run * 4 * sizeof(uint64_t));
    return (b + 255) / 256 * 256;
}

size_t draft_workspace_bytes(int R, int V) { return draft_part_bytes(R, V) + kRunCtlBytes; }

const unsigned* draft_error_word(const void* ws, int R, int V)
{
    return reinterpret_cast<const unsigned*>(static_cast<const char*>(ws) + draft_part_bytes(R, V));
}

// requests per workgroup of a bias pass: whole 64-request blocks, split into
// balanced chunks so the grid has about 1024 workgroups (two rounds at two per
// CU; every chunk re-reads its W2 tile, so fewer chunks move fewer bytes)
int pass_req_per_wg(int count_max, int n_vt)
{
    const int blocks = (count_max + kReqBlock - 1) / kReqBlock;
    const int want = std::max(1, std::min(blocks, (1024 + n_vt - 1) / n_vt));
    return ((blocks + want - 1) / want) * kReqBlock;
}

template <typename LT, bool GREEDY, int PER>
static void launch_pick(const LT* base, RowStrides bs, const uint16_t* E, const uint16_t* W2,
                        const int32_t* anchor, int32_t* tok, float* q, double* stats, int R,
                        int gamma, int V, int r, int k, float it, uint64_t seed, uint32_t round,
                        int n_vt, const Part* part, const float4* sub, const uint16_t* S,
                        hipStream_t s)
{
    if (sub)
        hipLaunchKernelGGL((draft_pick_kernel<LT, GREEDY, PER, true>), dim3(R), dim3(256), 0, s, base, bs,
                           E, W2, anchor, tok, q, stats, R, gamma, V, r, k, it, seed, round, n_vt, part,
                           sub, S);
    else
        hipLaunchKernelGGL((draft_pick_kernel<LT, GREEDY, PER, false>), dim3(R), dim3(256), 0, s, base, bs,
                           E, W2, anchor, tok, q, stats, R, gamma, V, r, k, it, seed, round, n_vt, part,
                           sub, S);
}

template <typename LT>
static hipError_t launch_draft_t(const LT* base, RowStrides bs, const uint16_t* E, const uint16_t* W2,
                                 const int32_t* anchor, int32_t* tok, float* q, double* stats,
                                 int R, int gamma, int V, int r, int k, float temperature,
                                 uint64_t seed, uint32_t round, void* ws, unsigned* ctl,
                                 const uint16_t* S, hipStream_t s)
{
    const int n_vt = (V + kVocabTile - 1) / kVocabTile;
    Part* part = static_cast<Part*>(ws);
    const bool greedy = (temperature == 0.0f);
    const float it = greedy ? 1.0f : 1.0f / temperature;
    PassArgs a{};
    a.base = base; a.bs = bs; a.W2 = W2; a.anchor = anchor; a.tok = tok;
    if (S) {   // recurrent head: row n of position k's states
        a.E = S + (int64_t)k * r; a.e_rs = (int64_t)gamma * r; a.e_rows = R; a.rnn = 1;
    } else {   // Markov head: row x_{k-1} of the embedding
        a.E = E; a.e_rs = r; a.e_rows = V; a.rnn = 0;
    }
    a.R = R; a.gamma = gamma; a.V = V; a.r = r; a.k = k; a.inv_temp = it;
    a.n_vt = n_vt;
    a.req_per_wg = pass_req_per_wg(R, n_vt);
    a.part = part;
    a.ctl = ctl;
    const dim3 g1(n_vt, (R + a.req_per_wg - 1) / a.req_per_wg);
    const bool vec = rows_vec(bs, V, 8);
    const bool piped = sizeof(LT) == 2 && vec && dp_offsets_fit(bs, a.e_rows, a.e_rs, r);
    // the pipelined pass's 64-column sums (sampling, tile-major [n_vt, R]), after
    // the partials
    float4* sub = (piped && !greedy)
                      ? reinterpret_cast<float4*>(part + (size_t)R * n_vt) : nullptr;
    a.sub = sub;
    if (piped) {
        // bf16 rows of 16-byte words: the software-pipelined pass
#define DSP_DP(G, H) hipLaunchKernelGGL((draft_pass_wide_kernel<G, H>), g1, dim3(kDwThreads), 0, s, a)
        if (greedy) { if (S) DSP_DP(true, true); else DSP_DP(true, false); }
        else { if (S) DSP_DP(false, true); else DSP_DP(false, false); }
#undef DSP_DP
    } else if (greedy && vec)
        hipLaunchKernelGGL((bias_pass_kernel<LT, kGreedy, true>), g1, dim3(256), 0, s, a);
    else if (greedy)
        hipLaunchKernelGGL((bias_pass_kernel<LT, kGreedy, false>), g1, dim3(256), 0, s, a);
    else if (vec)
        hipLaunchKernelGGL((bias_pass_kernel<LT, kSample, true>), g1, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((bias_pass_kernel<LT, kSample, false>), g1, dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int per = (n_vt + 255) / 256;
#define DSP_PICK(P)                                                                              \
    (greedy ? launch_pick<LT, true, P>(base, bs, E, W2, anchor, tok, q, stats, R, gamma, V, r, k, \
                                       it, seed, round, n_vt, part, sub, S, s)                   \
            : launch_pick<LT, false, P>(base, bs, E, W2, anchor, tok, q, stats, R, gamma, V, r, k, \
                                        it, seed, round, n_vt, part, sub, S, s))
    if (per <= 1) DSP_PICK(1);
    else if (per <= 2) DSP_PICK(2);
    else if (per <= 4) DSP_PICK(4);
    else DSP_PICK(8);
#undef DSP_PICK
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// persistent path
// ---------------------------------------------------------------------------
// Marks every partial slot of a launch and the tokens of its positions empty,
// and sets the error word: 0, or 1 under the give-up test hook (every wait of
// the launch then returns at once).
__global__ void run_clear_kernel(uint64_t* slots, int64_t n_slots, int32_t* tok, int R, int gamma,
                                 int k0, int n_steps, unsigned* ctl, unsigned ctl0)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (int64_t i = i0; i < n_slots; i += stride) slots[i] = kRunSlotEmpty;
    const int64_t n_tok = (int64_t)R * n_steps;
    for (int64_t i = i0; i < n_tok; i += stride)
        tok[(i / n_steps) * gamma + k0 + (i % n_steps)] = kRunTokEmpty;
    if (i0 == 0) ctl[0] = ctl0;
}

namespace {

// compute units of the current device (cached per device)
int device_cus()
{
    constexpr int kDevs = 64;
    static std::atomic<int> ncu[kDevs];
    int d = 0;
    if (hipGetDevice(&d) != hipSuccess) return 0;
    if (d >= 0 && d < kDevs) {
        const int c = ncu[d].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, d) != hipSuccess) n = 0;
    if (d >= 0 && d < kDevs && n > 0) ncu[d].store(n, std::memory_order_relaxed);
    return n;
}

// the fewest 32-column units per wave for which the tiles (four per
// workgroup, one workgroup per CU) cover V; 0 when none does
int run_units(int V, int ncu, int* n_t)
{
    for (int tu = 1; tu <= kRunUnitsMax; ++tu) {
        const int nt = (V + 32 * tu - 1) / (32 * tu);
        if (nt <= kRunTilesMax && (nt + 3) / 4 <= ncu) {
            *n_t = nt;
            return tu;
        }
    }
    return 0;
}

template <bool GREEDY, int TU>
hipError_t launch_run_t(const RunArgs& ra, int G, int ncu, bool give_up, hipStream_t s,
                        bool* launched)
{
    *launched = false;
    static std::atomic<int> occ{-1};
    if (occ.load(std::memory_order_relaxed) < 0) {
        int o = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, draft_run_kernel<GREEDY, TU>, 256, 0) !=
            hipSuccess)
            o = 0;
        occ.store(o, std::memory_order_relaxed);
    }
    if (G > occ.load(std::memory_order_relaxed) * ncu) return hipSuccess;
    const int64_t n_slots = 4 * (int64_t)ra.R * ra.n_t;
    const int64_t n_clear = std::max<int64_t>(n_slots, (int64_t)ra.R * ra.n_steps);
    const int cg = (int)std::min<int64_t>(1024, (n_clear + 255) / 256);
    hipLaunchKernelGGL(run_clear_kernel, dim3(cg), dim3(256), 0, s, ra.slots, n_slots, ra.tok, ra.R,
                       ra.gamma, ra.k0, ra.n_steps, ra.ctl, give_up ? 1u : 0u);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // an ordinary launch: the grid has at most one workgroup per CU and the
    // kernel's registers and LDS admit exactly one, so every workgroup is
    // resident at once (a cooperative launch would guarantee the same at ~18 us
    // more per launch, measured on MI355X)
    hipLaunchKernelGGL((draft_run_kernel<GREEDY, TU>), dim3(G), dim3(256), 0, s, ra);
    e = hipGetLastError();
    if (e == hipSuccess) *launched = true;
    return e;
}

// one persistent launch for every position, when the shapes and the device allow
hipError_t try_launch_run(const uint16_t* base, RowStrides bs, const uint16_t* E, const uint16_t* W2,
                          const int32_t* anchor, int32_t* tok, float* q, double* stats, int R,
                          int gamma, int V, int r, int k0, int n_steps, float temperature,
                          uint64_t seed, uint32_t round, void* ws, bool give_up, hipStream_t s,
                          bool* launched)
{
    *launched = false;
    if (!rows_vec(bs, V, 8) || R > kRunReqMax) return hipSuccess;
    RunGeometry geo;
    if (!run_geometry(V, &geo)) return hipSuccess;
    const int tu = geo.tu, n_t = geo.n_t;
    const bool greedy = (temperature == 0.0f);
    RunArgs ra{};
    ra.base = base; ra.bs = bs; ra.E = E; ra.W2 = W2; ra.anchor = anchor; ra.tok = tok; ra.q = q;
    ra.stats = stats; ra.R = R; ra.gamma = gamma; ra.V = V; ra.r = r; ra.k0 = k0;
    ra.n_steps = n_steps; ra.inv_temp = greedy ? 1.0f : 1.0f / temperature; ra.seed = seed;
    ra.round = round; ra.n_t = n_t;
    ra.slots = static_cast<uint64_t*>(ws);
    ra.ctl = reinterpret_cast<unsigned*>(static_cast<char*>(ws) + draft_part_bytes(R, V));
    // one workgroup per request where CUs are free beyond the tile workgroups:
    // no workgroup then draws two requests of a position
    const int G = std::max((n_t + 3) / 4, std::min(R, geo.ncu));
#define DSP_RUN(TU)                                                                            \
    return greedy ? launch_run_t<true, TU>(ra, G, geo.ncu, give_up, s, launched)               \
                  : launch_run_t<false, TU>(ra, G, geo.ncu, give_up, s, launched)
    switch (tu) {
    case 1: DSP_RUN(1);
    case 2: DSP_RUN(2);
    case 3: DSP_RUN(3);
    case 4: DSP_RUN(4);
    default: DSP_RUN(5);
    }
#undef DSP_RUN
}

}  // namespace

// ---------------------------------------------------------------------------
// Static scratch of the allocation-free draft entry point: one array per device,
// holding what the workspace argument holds for dsp_draft_step.  In host code the
// array's name is not a device address: the address comes from
// hipGetSymbolAddress, looked up once per device with that device current.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

hipError_t static_scratch(void** ptr)
{
    constexpr int kDevs = 64;
    static std::atomic<void*> addr[kDevs];
    int d = 0;
    hipError_t e = hipGetDevice(&d);
    if (e != hipSuccess) return e;
    if (d < 0 || d >= kDevs) return hipErrorInvalidDevice;
    void* p = addr[d].load(std::memory_order_acquire);
    if (!p) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[d].store(p, std::memory_order_release);
    }
    *ptr = p;
    return hipSuccess;
}

bool run_geometry(int V, RunGeometry* g)
{
    const int ncu = device_cus();
    int n_t = 0;
    const int tu = run_units(V, ncu, &n_t);
    *g = RunGeometry{tu, n_t, ncu};
    return tu > 0;
}

// ---------------------------------------------------------------------------
// Recurrent head state of position k: S[n, k] = bf16(tanh(A S[n, k-1] +
// E[x_{k-1}])), S[n, -1] = 0, the E term dropped for x outside [0, V).  One
// workgroup per kRnnReq requests; thread i computes element i of each: its row
// of A in registers, the previous states in LDS, the dot product in fp64 in
// index order (bf16 x bf16 products are exact), tanh in fp64, then one rounding
// to the nearest bf16 (ties to even) directly from fp64.
// ---------------------------------------------------------------------------
constexpr int kRnnReq = 8;

__device__ __forceinline__ uint16_t bf16_rne_f64(double x)
{
    // the two bf16 values around x: the truncation of x's nearest float and the
    // next one up in magnitude (rounding to float never crosses a bf16 value)
    const uint32_t u = __float_as_uint((float)x);
    const uint32_t lo = u & 0xFFFF0000u, hi = lo + 0x10000u;
    const double dlo = fabs(x - (double)__uint_as_float(lo));
    const double dhi = fabs((double)__uint_as_float(hi) - x);
    const uint32_t pick = (dlo < dhi) ? lo : (dhi < dlo) ? hi : (((lo >> 16) & 1u) ? hi : lo);
    return (uint16_t)(pick >> 16);
}

__global__ __launch_bounds__(256) void rnn_state_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ E, const int32_t* __restrict__ anchor,
    const int32_t* __restrict__ tok, uint16_t* __restrict__ S, int R, int gamma, int V, int r, int k)
{
    __shared__ __attribute__((aligned(16))) uint16_t sp[kRnnReq][kRankMax];
    const int n0 = blockIdx.x * kRnnReq;
    const int t = threadIdx.x;
    // previous states of the workgroup's requests (zero for position 0)
    for (int w = t; w < kRnnReq * (kRankMax / 8); w += 256) {
        const int j = w / (kRankMax / 8), c = 8 * (w % (kRankMax / 8)), n = n0 + j;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (k > 0 && n < R && c < r)
            v = *reinterpret_cast<const uint4*>(S + ((int64_t)n * gamma + (k - 1)) * r + c);
        *reinterpret_cast<uint4*>(&sp[j][c]) = v;
    }
    __syncthreads();
    if (t >= r) return;
    uint4 arow[kRankMax / 8];
#pragma unroll
    for (int c = 0; c < kRankMax / 8; ++c)
        arow[c] = (8 * c < r) ? *reinterpret_cast<const uint4*>(A + (int64_t)t * r + 8 * c)
                              : make_uint4(0, 0, 0, 0);
    for (int j = 0; j < kRnnReq; ++j) {
        const int n = n0 + j;
        if (n >= R) break;
        const int x = (k == 0) ? anchor[n] : tok[(int64_t)n * gamma + (k - 1)];
        double u = 0.0;
#pragma unroll
        for (int c = 0; c < kRankMax / 8; ++c) {
            if (8 * c >= r) break;
            const uint4 sv = *reinterpret_cast<const uint4*>(&sp[j][8 * c]);
            const uint32_t aw[4] = {arow[c].x, arow[c].y, arow[c].z, arow[c].w};
            const uint32_t sw[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                u = fma((double)__uint_as_float(aw[e] << 16), (double)__uint_as_float(sw[e] << 16), u);
                u = fma((double)__uint_as_float(aw[e] & 0xFFFF0000u),
                        (double)__uint_as_float(sw[e] & 0xFFFF0000u), u);
            }
        }
        if (x >= 0 && x < V) u += (double)bf16_to_f32(E[(int64_t)x * r + t]);
        S[((int64_t)n * gamma + k) * r + t] = bf16_rne_f64(tanh(u));
    }
}

hipError_t launch_draft_step(const void* base, RowStrides bs, bool bf16, const uint16_t* E,
                             const uint16_t* W2,
                             const int32_t* anchor, int32_t* tok, float* q, double* stats, int R,
                             int gamma, int V, int r, int k, int n_steps, int path,
                             bool give_up, float temperature, uint64_t seed, uint32_t round,
                             void* ws, hipStream_t s, const uint16_t* A, uint16_t* S)
{
    if (S) {   // recurrent head: streaming launches only, each position after its state
        if (path == kPathPersistent) return hipErrorNotSupported;
        unsigned* ctl = const_cast<unsigned*>(draft_error_word(ws, R, V));
        for (int i = 0; i < n_steps; ++i) {
            hipLaunchKernelGGL(rnn_state_kernel, dim3((unsigned)((R + kRnnReq - 1) / kRnnReq)), dim3(256),
                               0, s, A, E, anchor, tok, S, R, gamma, V, r, k + i);
            unsigned* c = (i == 0) ? ctl : nullptr;
            const hipError_t e =
                bf16 ? launch_draft_t(static_cast<const uint16_t*>(base), bs, E, W2, anchor, tok, q, stats,
                                      R, gamma, V, r, k + i, temperature, seed, round, ws, c, S, s)
                     : launch_draft_t(static_cast<const float*>(base), bs, E, W2, anchor, tok, q, stats,
                                      R, gamma, V, r, k + i, temperature, seed, round, ws, c, S, s);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    if (path != kPathStream && bf16) {
        bool launched = false;
        const hipError_t e = try_launch_run(static_cast<const uint16_t*>(base), bs, E, W2, anchor, tok,
                                            q, stats, R, gamma, V, r, k, n_steps, temperature, seed,
                                            round, ws, give_up, s, &launched);
        if (launched || e != hipSuccess) return e;
    }
    if (path == kPathPersistent) return hipErrorNotSupported;
    // the streaming launches have no waits: the first pass clears the error word
    unsigned* ctl = const_cast<unsigned*>(draft_error_word(ws, R, V));
    for (int i = 0; i < n_steps; ++i) {
        unsigned* c = (i == 0) ? ctl : nullptr;
        const hipError_t e =
            bf16 ? launch_draft_t(static_cast<const uint16_t*>(base), bs, E, W2, anchor, tok, q, stats,
                                  R, gamma, V, r, k + i, temperature, seed, round, ws, c, nullptr, s)
                 : launch_draft_t(static_cast<const float*>(base), bs, E, W2, anchor, tok, q, stats,
                                  R, gamma, V, r, k + i, temperature, seed, round, ws, c, nullptr, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace dsp

// verify.hip -- lossless verification of the scheduled draft prefixes (gfx950).
//
// Acceptance min(1, p/q), the residual max(0, p - q) normalised after the first
// rejection, and the extra token from the next target row when the whole block
// passed: page "DSpark.让每一轮计算，多走几步", lossless section; page "为什么
// DSpark 可以加速推理？", section on the mathematics of speculative decoding.
// Greedy verification keeps a draft token only if it is the target's choice
// (same lossless section).
//
// Launches (sampling; greedy stops after the second):
//   verify_rows      stream every verified target row (r, j <= l_r) once:
//                    per 256-wide tile (max, sum exp) -- or argmax -- partials,
//                    and the target logit at the drafted token
//   verify_accept    one workgroup per request: row normalisers (fp64), p_j(x_j),
//                    the accept tests, the first rejection, greedy tokens; queue
//                    the requests that need a residual draw
//   bias_pass<kResidual>  residual mass per (queued request, tile), the draft row
//                    rebuilt with the draft step's MFMA bias
//   verify_pick      one workgroup per request: locate the tile of the residual
//                    (or of the bonus / zero-residual fallback row) and scan it
// Where the draft's W2 slice fits on chip (bf16 rows), resid_run_kernel
// (resid_run.h) replaces the last two launches with one persistent launch.
#include "bias_tile.h"
#include "dsp_device.h"
#include "dsp_launch.h"
#include "resid_pass.h"
#include "resid_run.h"
#include "tile_pass.h"

#include <atomic>
#include <type_traits>

namespace dsp {

namespace {

constexpr int kSpanTiles = 32;   // tiles per verify_rows work item (8192 columns)

struct VerifyWs {
    Part* rowpart;       // [R, gamma+1, n_vt]
    Part* spanpart;      // [R, gamma+1, 4 spans] the same rows, 8 tiles combined
    float* zx;           // [R, gamma] target logit at the drafted token
    int* resid_cnt;      // [1]
    int* resid_list;     // [R] request of each queue slot
    int* resid_m;        // [R] its first rejection position
    int* resid_prev;     // [R] the token before that position
    int* resid_slot;     // [R] queue slot of each request (-1: none)
    double* row_z;       // [R] normaliser of target row n_accept (rejecting requests)
    float* row_m;        // [R] max logit of that row
    Part* resid_part;    // [R, n_vt]
    uint64_t* run_slots; // [R, n_t] residual mass of the persistent residual launch
    unsigned* run_ctl;   // its error word
    int64_t* resid_roff; // [R, 2] records of the queued entries for resid_pass_kernel
    int* resid_erow;     // [R]
    float4* resid_rst;   // [R]
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

inline VerifyWs carve(void* ws, int R, int gamma, int V, size_t* total)
{
    const size_t n_vt = (size_t)((V + kVocabTile - 1) / kVocabTile);
    char* p = static_cast<char*>(ws);
    size_t off = 0;
    VerifyWs w;
    const size_t spans = (n_vt + kSpanTiles - 1) / kSpanTiles;
    w.rowpart = reinterpret_cast<Part*>(p + off);     off += align256((size_t)R * (gamma + 1) * n_vt * sizeof(Part));
    w.spanpart = reinterpret_cast<Part*>(p + off);    off += align256((size_t)R * (gamma + 1) * 4 * spans * sizeof(Part));
    w.zx = reinterpret_cast<float*>(p + off);         off += align256((size_t)R * gamma * sizeof(float));
    w.resid_cnt = reinterpret_cast<int*>(p + off);    off += align256(sizeof(int));
    w.resid_list = reinterpret_cast<int*>(p + off);   off += align256((size_t)R * sizeof(int));
    w.resid_m = reinterpret_cast<int*>(p + off);      off += align256((size_t)R * sizeof(int));
    w.resid_prev = reinterpret_cast<int*>(p + off);   off += align256((size_t)R * sizeof(int));
    w.resid_slot = reinterpret_cast<int*>(p + off);   off += align256((size_t)R * sizeof(int));
    w.row_z = reinterpret_cast<double*>(p + off);     off += align256((size_t)R * sizeof(double));
    w.row_m = reinterpret_cast<float*>(p + off);      off += align256((size_t)R * sizeof(float));
    w.resid_part = reinterpret_cast<Part*>(p + off);  off += align256((size_t)R * n_vt * sizeof(Part));
    const size_t n_run = std::min<size_t>((size_t)((V + 31) / 32), (size_t)kRunTilesMax);
    w.run_slots = reinterpret_cast<uint64_t*>(p + off); off += align256((size_t)R * n_run * sizeof(uint64_t));
    w.run_ctl = reinterpret_cast<unsigned*>(p + off); off += 256;
    w.resid_roff = reinterpret_cast<int64_t*>(p + off); off += align256((size_t)R * 2 * sizeof(int64_t));
    w.resid_erow = reinterpret_cast<int*>(p + off);   off += align256((size_t)R * sizeof(int));
    w.resid_rst = reinterpret_cast<float4*>(p + off); off += align256((size_t)R * sizeof(float4));
    if (total) *total = off;
    return w;
}

__device__ __forceinline__ int clamp_len(const int32_t* len, int n, int gamma)
{
    return min(max(len[n], 0), gamma);
}

}  // namespace

// ---------------------------------------------------------------------------
// verify_rows: one workgroup per (request, 32-tile span), looping over the
// request's verified rows j = 0 .. l_r (so no workgroup is launched for a row
// that is not verified); the next row's words are requested before the current
// row is reduced.  Wave w covers tiles [32 sp + 8 w, +8): lanes 8i .. 8i+7 own
// tile i of the wave, 32 values each (load k reads columns k*64 + 8*(l%8) .. +7
// of the tile, so each load instruction moves eight whole 128-byte runs).
// VEC (rows of whole 16-byte words): every load is one unconditional 16-byte
// load from the row or, past V, from the -inf words, so the compiler keeps the
// next row's loads in flight while the current row is reduced; a load behind a
// branch (the per-element path, or the drafted token's logit) made it wait for
// them before every reduction.
// ---------------------------------------------------------------------------
template <typename LT, bool GREEDY, bool VEC>
__global__ __launch_bounds__(256) void verify_rows_kernel(
    const LT* __restrict__ target, RowStrides ts, const int32_t* __restrict__ tok,
    const int32_t* __restrict__ len, int R, int gamma, int V, float inv_temp, int n_vt,
    VerifyWs ws, unsigned ctl0)
{
    constexpr int RW = Logit<LT>::kRaw;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const Itl itL = fold_itl(inv_temp);
    // the error word of the call: 0, or 1 under the give-up test hook (every wait
    // of the persistent residual launch then returns at once)
    if (blockIdx.x == 0 && tid == 0) {
        *ws.resid_cnt = 0;
        ws.run_ctl[0] = ctl0;
    }
    const int spans = (n_vt + kSpanTiles - 1) / kSpanTiles;
    const int n = blockIdx.x / spans;
    const int sp = blockIdx.x - n * spans;
    const int l = clamp_len(len, n, gamma);
    const int t = sp * kSpanTiles + wave * 8 + (lane >> 3);
    const int sub = lane & 7;

    // VEC: row j through a buffer resource of the whole row (a row past l has a
    // zero range: the loads are still issued, read nothing and return zeros),
    // each lane at fixed offsets; words past V read zeros and become -inf words
    // in the last span
    const bool tail_span = (sp + 1) * kSpanTiles * kVocabTile > V;   // workgroup-uniform
    auto load_row = [&](int j, uint4 (&raw)[4][RW]) {
        if constexpr (VEC) {
            const LT* row = target + (int64_t)n * ts.rs + (int64_t)min(j, l) * ts.ps;
            const BufRsrc rr = buf_rsrc(row, (j <= l) ? (uint32_t)V * (uint32_t)sizeof(LT) : 0u);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t off = (uint32_t)(t * kVocabTile + k * 64 + sub * 8) * (uint32_t)sizeof(LT);
#pragma unroll
                for (int w = 0; w < RW; ++w) raw[k][w] = buf_load16<kBufNt>(rr, off + 16u * w);
            }
        } else {
            const LT* row = target + (int64_t)n * ts.rs + (int64_t)j * ts.ps;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int v0 = t * kVocabTile + k * 64 + sub * 8;
                Logit<LT>::load8_raw(row, min(v0, V), V, false, raw[k]);
            }
        }
    };
    auto mask_tail = [&](uint4 (&raw)[4][RW]) {
        if (VEC && tail_span) {
            const uint32_t ninf = (sizeof(LT) == 2) ? 0xFF80FF80u : 0xFF800000u;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const bool in = t * kVocabTile + k * 64 + sub * 8 < V;   // whole words: in or past V
                const uint32_t keep = in ? 0xFFFFFFFFu : 0u, put = ninf & ~keep;
#pragma unroll
                for (int w = 0; w < RW; ++w) {
                    uint4& u = raw[k][w];
                    u = make_uint4((u.x & keep) | put, (u.y & keep) | put, (u.z & keep) | put, (u.w & keep) | put);
                }
            }
        }
    };
    auto reduce_row = [&](int j, const uint4 (&raw)[4][RW]) {
        Part* out = ws.rowpart + ((int64_t)n * (gamma + 1) + j) * n_vt;
        if constexpr (GREEDY) {
            ArgMax am{-INFINITY, 0x7fffffff};
#pragma unroll
            for (int k = 0; k < 4; ++k)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int v = t * kVocabTile + k * 64 + sub * 8 + e;
                    if (v < V) am = argmax_merge(am, ArgMax{Logit<LT>::raw_at(raw[k], e), v});
                }
#pragma unroll
            for (int o = 1; o < 8; o <<= 1) {
                ArgMax b;
                b.v = __shfl_xor(am.v, o, kWave);
                b.i = __shfl_xor(am.i, o, kWave);
                am = argmax_merge(am, b);
            }
            const Part pt{am.v, am.i, 0.0};
            // the wave's 8 tiles (lane groups) combined: one partial per wave
            ArgMax b8;
            b8.v = __shfl_xor(am.v, 8, kWave);
            b8.i = __shfl_xor(am.i, 8, kWave);
            am = xargmax<32>(xargmax<16>(argmax_merge(am, b8)));
            if (sub == 0 && t < n_vt) out[t] = pt;
            if (lane == 0)
                ws.spanpart[(((int64_t)n * (gamma + 1) + j) * spans + sp) * 4 + wave] = Part{am.v, am.i, 0.0};
        } else {
            float m = -INFINITY;
#pragma unroll
            for (int k = 0; k < 4; ++k)
#pragma unroll
                for (int e = 0; e < 8; ++e) m = fmaxf(m, Logit<LT>::raw_at(raw[k], e));
#pragma unroll
            for (int o = 1; o < 8; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
            const float mref = (m == -INFINITY) ? 0.0f : m;
            // fp32 weights relative to the tile maximum (the reference a pick's
            // rescan recomputes), summed in fp64 per lane and across the tile's lanes
            float x[32];
#pragma unroll
            for (int k = 0; k < 4; ++k)
#pragma unroll
                for (int e = 0; e < 8; ++e) x[8 * k + e] = Logit<LT>::raw_at(raw[k], e);
            double s = sum_w64(x, mref, itL);
#pragma unroll
            for (int o = 1; o < 8; o <<= 1) s += __shfl_xor(s, o, kWave);
            const Part pt{m, 0, s};
            // the wave's 8 tiles (lane groups) rescaled to their max and summed:
            // one partial per wave (an fp32 factor: these partials only give each
            // row's normaliser, to ~1e-7; the draws use the tile partials and rescans)
            float mw = fmaxf(m, __shfl_xor(m, 8, kWave));
            mw = xmax<32>(xmax<16>(mw));
            double sw = (m == -INFINITY) ? 0.0 : s * (double)wexp(m - mw, itL);
            sw += __shfl_xor(sw, 8, kWave);
            sw = xsum<32>(xsum<16>(sw));
            // (ordinary exec-masked stores: a buffer store whose every lane falls out
            // of range -- a wave of tiles past V -- upset the in-order load
            // counter the compiler's waits assume, measured as wrong row sums)
            if (sub == 0 && t < n_vt) out[t] = pt;
            if (lane == 0)
                ws.spanpart[(((int64_t)n * (gamma + 1) + j) * spans + sp) * 4 + wave] = Part{mw, 0, sw};
        }
    };
    uint4 ra[4][RW], rb[4][RW];
    load_row(0, ra);
    for (int j = 0; j <= l; j += 2) {
        // VEC: unconditional requests (a row past l reads nothing)
        if (VEC || j + 1 <= l) load_row(j + 1, rb);
        mask_tail(ra);
        reduce_row(j, ra);
        if (j + 1 > l) break;
        if (VEC || j + 2 <= l) load_row(j + 2, ra);
        mask_tail(rb);
        reduce_row(j + 1, rb);
    }
    // sampling: the target logit at each drafted token of this span (thread j,
    // row j), for the accept test
    if constexpr (!GREEDY) {
        const int j = tid;
        if (j < l) {
            const int xj = tok[(int64_t)n * gamma + j];
            const int lo = sp * kSpanTiles * kVocabTile;
            if (xj >= lo && xj < min(V, lo + kSpanTiles * kVocabTile))
                ws.zx[(int64_t)n * gamma + j] = Logit<LT>::at(target + (int64_t)n * ts.rs + (int64_t)j * ts.ps, xj);
        }
    }
}

// ---------------------------------------------------------------------------
// verify_accept: one workgroup per request; wave w combines rows j = w, w+4, ...
// from their 8-tile partials (lane l: partials [l * PER, l * PER + PER); at
// most 256 per row).
// ---------------------------------------------------------------------------
template <bool GREEDY, int PER>
__global__ __launch_bounds__(256) void verify_accept_kernel(
    const int32_t* __restrict__ anchor, int V,
    const int32_t* __restrict__ tok, const float* __restrict__ q, const int32_t* __restrict__ len,
    int8_t* __restrict__ accept, int32_t* __restrict__ n_accept, int32_t* __restrict__ y,
    float* __restrict__ p_out, int R, int gamma, float inv_temp, uint64_t seed, uint32_t round,
    int n_vt, VerifyWs ws, int run_n_t, int rnn)
{
    __shared__ int slot_s;
    __shared__ int acc_s[kGammaMax + 1];
    __shared__ float pj_s[kGammaMax + 1];
    __shared__ float m_s[kGammaMax + 1];
    __shared__ double z_s[kGammaMax + 1];
    __shared__ int am_s[kGammaMax + 1];
    __shared__ int tk_s[kGammaMax + 1];
    const int n = blockIdx.x;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int l = clamp_len(len, n, gamma);
    const int np = 4 * ((n_vt + kSpanTiles - 1) / kSpanTiles);
    const Part* rows = ws.spanpart + (int64_t)n * (gamma + 1) * np;
    const int last_row = GREEDY ? l : l - 1;
    const int anchor_n = (!GREEDY && tid == 0) ? anchor[n] : 0;   // x_{-1}, for the queue
    for (int j = wave; j <= last_row; j += 4) {
        const Part* pp = rows + (int64_t)j * np;
        // the accept test's inputs, requested with the row's partials (sampling:
        // j < l here, so (n, j) is a drafted position)
        const int64_t o = (int64_t)n * gamma + j;
        float zx_j = 0.0f, q_j = 0.0f;
        int tk_j = 0;
        if constexpr (!GREEDY) {
            zx_j = ws.zx[o];
            q_j = q[o];
            tk_j = tok[o];
        }
        Part pt[PER];
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int t = lane * PER + i;
            pt[i] = (t < np) ? pp[t] : Part{-INFINITY, 0x7fffffff, 0.0};
        }
        if constexpr (GREEDY) {
            ArgMax am{-INFINITY, 0x7fffffff};
#pragma unroll
            for (int i = 0; i < PER; ++i) am = argmax_merge(am, ArgMax{pt[i].m, pt[i].idx});
            am = wave_argmax(am);
            if (lane == 0) {
                am_s[j] = am.i;
                if (j < l) {
                    const int a = (tok[(int64_t)n * gamma + j] == am.i);
                    acc_s[j] = a;
                    pj_s[j] = a ? 1.0f : 0.0f;
                }
            }
        } else {
            float M = -INFINITY;
#pragma unroll
            for (int i = 0; i < PER; ++i) M = fmaxf(M, pt[i].m);
            M = wave_max_f(M);
            double Z = 0.0;
#pragma unroll
            for (int i = 0; i < PER; ++i)
                Z += pt[i].s * rescale64(pt[i].m, M, inv_temp);
            Z = wave_sum_d(Z);
            if (lane == 0) {
                const double p = exp(((double)zx_j - (double)M) * (double)inv_temp) / Z;
                const double u = uniform24(seed, round, (uint32_t)n, (uint32_t)j, 1u);
                acc_s[j] = (u * (double)q_j <= p);
                tk_s[j] = tk_j;
                pj_s[j] = (float)p;
                m_s[j] = M;
                z_s[j] = Z;
            }
        }
    }
    __syncthreads();
    int nacc = l;
    for (int j = 0; j < l; ++j)
        if (!acc_s[j]) { nacc = j; break; }
    for (int j = tid; j < gamma; j += 256) {
        const int64_t o = (int64_t)n * gamma + j;
        accept[o] = (j < l) ? (int8_t)acc_s[j] : (int8_t)-1;
        p_out[o] = (j < l) ? pj_s[j] : 0.0f;
    }
    if (tid == 0) {
        n_accept[n] = nacc;
        slot_s = -1;
        if constexpr (GREEDY) {
            y[n] = am_s[nacc];
        } else {
            if (nacc < l) {
                const int slot = atomicAdd(ws.resid_cnt, 1);
                slot_s = slot;
                ws.resid_list[slot] = n;
                ws.resid_m[slot] = nacc;
                // the bias row of the rejected position: the token before it
                // (drafted positions j < l are in tk_s), or for the recurrent
                // head the state row (n, nacc)
                const int pv = (nacc == 0) ? anchor_n : tk_s[nacc - 1];
                ws.resid_prev[slot] = rnn ? n * gamma + nacc : (pv >= 0 && pv < V) ? pv : -1;
                ws.resid_slot[n] = slot;
                ws.row_m[n] = m_s[nacc];
                ws.row_z[n] = z_s[nacc];
            } else {
                ws.resid_slot[n] = -1;
            }
        }
    }
    if constexpr (!GREEDY) {
        // a persistent residual launch follows: its slots of this request start empty
        if (run_n_t > 0) {
            __syncthreads();
            const int slot = slot_s;
            if (slot >= 0)
                for (int t = tid; t < run_n_t; t += 256) ws.run_slots[(int64_t)slot * run_n_t + t] = kRunSlotEmpty;
        }
    }
}

// ---------------------------------------------------------------------------
// verify_pick: one workgroup per request (sampling)
// ---------------------------------------------------------------------------
template <typename LT, int PER>
__global__ __launch_bounds__(256, 4) void verify_pick_kernel(
    const LT* __restrict__ target, RowStrides ts, const LT* __restrict__ base, RowStrides bs,
    const uint16_t* __restrict__ E, const uint16_t* __restrict__ W2,
    const int32_t* __restrict__ anchor, const int32_t* __restrict__ tok,
    const double* __restrict__ stats,
    const int32_t* __restrict__ len, const int32_t* __restrict__ n_accept,
    int32_t* __restrict__ y, int R, int gamma, int V, int r, float inv_temp, uint64_t seed,
    uint32_t round, int n_vt, VerifyWs ws, const uint16_t* __restrict__ S)
{
    __shared__ PickScratch sh;
    __shared__ __attribute__((aligned(16))) uint16_t e_row[kRankMax];
    const int n = blockIdx.x;
    const int tid = threadIdx.x;
    const int l = clamp_len(len, n, gamma);
    const int m = min(max(n_accept[n], 0), l);
    const int slot = ws.resid_slot[n];
    const double u = uniform24(seed, round, (uint32_t)n, (uint32_t)m, 2u);
    const Itl itL = fold_itl(inv_temp);

    if (slot >= 0) {   // workgroup-uniform
        const Part* rp = ws.resid_part + (int64_t)slot * n_vt;
        double w[PER];
        double ls = 0.0;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int t = tid * PER + i;
            w[i] = (t < n_vt) ? rp[t].s : 0.0;
            ls += w[i];
        }
        const double rsum = block_sum256(ls, sh);
        if (rsum > 0.0) {
            const double tgt = u * rsum;
            double before;
            const int tsel = block_locate<PER>(w, tgt, &before, sh, 0);
            // the draft row's logits over the chosen tile, rebuilt as the residual
            // pass computed them, and the target row's
            const int prev = prev_token(anchor, tok, n, gamma, m, V);
            const LT* drow = base + (int64_t)n * bs.rs + (int64_t)m * bs.ps;
            const LT* trow = target + (int64_t)n * ts.rs + (int64_t)m * ts.ps;
            const int v = tsel * kVocabTile + tid;
            const float xb = (v < V) ? Logit<LT>::at(drow, v) : -INFINITY;
            const float xt = (v < V) ? Logit<LT>::at(trow, v) : -INFINITY;
            // the rows' statistics exactly as the residual pass used them
            const float Md = (float)stats[2 * ((int64_t)n * gamma + m)];
            const float invZd = (float)(1.0 / stats[2 * ((int64_t)n * gamma + m) + 1]);
            const float Mt = ws.row_m[n];
            const float invZt = (float)(1.0 / ws.row_z[n]);
            if (tid < kRankMax / 8) {
                // the draft law's bias row: E[x_{m-1}] (Markov head) or S[n, m]
                const uint16_t* er = S ? S + ((int64_t)n * gamma + m) * r
                                       : (prev >= 0 ? E + (int64_t)prev * r : nullptr);
                const int kk = 8 * tid;
                uint4 ev = make_uint4(0, 0, 0, 0);
                if (er && kk < r) ev = *reinterpret_cast<const uint4*>(er + kk);
                *reinterpret_cast<uint4*>(e_row + kk) = ev;
            }
            const float zd = tile_logit(W2, V, r, tsel * kVocabTile, e_row, xb, sh);
            double rho[1] = {(v < V) ? resid_w(wexp(xt - Mt, itL), invZt, wexp(zd - Md, itL), invZd) : 0.0};
            double b2;
            const int loc = block_locate<1>(rho, tgt - before, &b2, sh, 1);
            if (tid == 0) y[n] = tsel * kVocabTile + loc;
            return;
        }
    }
    // bonus draw from target row l, or the zero-residual fallback from row m
    const int row_j = (slot >= 0) ? m : l;
    const Part* pp = ws.rowpart + ((int64_t)n * (gamma + 1) + row_j) * n_vt;
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
    const double tgt = u * Z;
    double before;
    const int tsel = block_locate<PER>(w, tgt, &before, sh, 0);
    const LT* trow = target + (int64_t)n * ts.rs + (int64_t)row_j * ts.ps;
    const int v = tsel * kVocabTile + tid;
    // verify_rows' own weights: relative to the tile maximum, moved onto M
    const float m_t = pp[tsel].m;
    const float mref = (m_t == -INFINITY) ? 0.0f : m_t;
    double e1[1] = {(v < V) ? (double)wexp(Logit<LT>::at(trow, v) - mref, itL) * rescale64(m_t, M, inv_temp)
                            : 0.0};
    double b2;
    const int loc = block_locate<1>(e1, tgt - before, &b2, sh, 1);
    if (tid == 0) y[n] = tsel * kVocabTile + loc;
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
size_t verify_workspace_bytes(int R, int gamma, int V)
{
    size_t total = 0;
    carve(nullptr, R, gamma, V, &total);
    return total;
}

const unsigned* verify_error_word(const void* ws, int R, int gamma, int V)
{
    return carve(const_cast<void*>(ws), R, gamma, V, nullptr).run_ctl;
}

template <bool GREEDY>
static void launch_accept(const int32_t* anchor, int V, const int32_t* tok, const float* q,
                          const int32_t* len, int8_t* accept, int32_t* n_accept, int32_t* y,
                          float* p, int R, int gamma, float it, uint64_t seed, uint32_t round,
                          int n_vt, const VerifyWs& ws, hipStream_t s, int run_n_t, int rnn)
{
    const int np = 4 * ((n_vt + kSpanTiles - 1) / kSpanTiles);
    const int per = (np + kWave - 1) / kWave;     // <= 4 for V <= kVocabMax
#define DSP_ACCEPT(P)                                                                          \
    hipLaunchKernelGGL((verify_accept_kernel<GREEDY, P>), dim3(R), dim3(256), 0, s, anchor, V, \
                       tok, q, len, accept, n_accept, y, p, R, gamma, it, seed, round, n_vt, ws,  \
                       run_n_t, rnn)
    if (per <= 1) DSP_ACCEPT(1);
    else if (per <= 2) DSP_ACCEPT(2);
    else if (per <= 4) DSP_ACCEPT(4);
    else if (per <= 8) DSP_ACCEPT(8);
    else if (per <= 16) DSP_ACCEPT(16);
    else DSP_ACCEPT(32);
#undef DSP_ACCEPT
}

template <typename LT, int PER>
static void launch_vpick(const LT* target, RowStrides ts, const LT* base, RowStrides bs,
                         const uint16_t* E, const uint16_t* W2,
                         const int32_t* anchor, const int32_t* tok, const double* stats,
                         const int32_t* len, const int32_t* n_accept, int32_t* y, int R, int gamma,
                         int V, int r, float it, uint64_t seed, uint32_t round, int n_vt,
                         const VerifyWs& ws, const uint16_t* S, hipStream_t s)
{
    hipLaunchKernelGGL((verify_pick_kernel<LT, PER>), dim3(R), dim3(256), 0, s, target, ts, base, bs,
                       E, W2,
                       anchor, tok, stats, len, n_accept, y, R, gamma, V, r, it, seed, round, n_vt,
                       ws, S);
}

template <int TU>
static hipError_t launch_resid_t(const ResidArgs& ra, int G, int ncu, hipStream_t s, bool* launched)
{
    *launched = false;
    static std::atomic<int> occ{-1};
    if (occ.load(std::memory_order_relaxed) < 0) {
        int o = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, resid_run_kernel<TU>, 256, 0) != hipSuccess)
            o = 0;
        occ.store(o, std::memory_order_relaxed);
    }
    if (G > occ.load(std::memory_order_relaxed) * ncu) return hipSuccess;
    // an ordinary launch with every workgroup resident at once (at most one per
    // CU, and the kernel admits exactly one), as for draft_run_kernel
    hipLaunchKernelGGL((resid_run_kernel<TU>), dim3(G), dim3(256), 0, s, ra);
    const hipError_t e = hipGetLastError();
    if (e == hipSuccess) *launched = true;
    return e;
}

template <typename LT>
static hipError_t launch_verify_t(const LT* target, RowStrides ts, const LT* base, RowStrides bs,
                                  int path, bool give_up, const uint16_t* E,
                                  const uint16_t* W2, const int32_t* anchor, const int32_t* tok,
                                  const float* q, const double* stats, const int32_t* len,
                                  int8_t* accept, int32_t* n_accept, int32_t* y, float* p, int R,
                                  int gamma, int V, int r, float temperature, uint64_t seed,
                                  uint32_t round, void* ws_raw, const uint16_t* S, hipStream_t s)
{
    const VerifyWs ws = carve(ws_raw, R, gamma, V, nullptr);
    const int rnn = S ? 1 : 0;
    const int n_vt = (V + kVocabTile - 1) / kVocabTile;
    const bool greedy = (temperature == 0.0f);
    const float it = greedy ? 1.0f : 1.0f / temperature;
    const int spans = (n_vt + kSpanTiles - 1) / kSpanTiles;
    const int64_t items = (int64_t)R * spans;   // verify_rows: (request, span) items
    const dim3 g1((unsigned)items);
    if (path == kPathPersistent && !std::is_same<LT, uint16_t>::value) return hipErrorNotSupported;
    if (greedy) {
        if (rows_vec(ts, V, Logit<LT>::kVecAlign))
            hipLaunchKernelGGL((verify_rows_kernel<LT, true, true>), g1, dim3(256), 0, s, target, ts, tok, len,
                               R, gamma, V, it, n_vt, ws, 0u);
        else
            hipLaunchKernelGGL((verify_rows_kernel<LT, true, false>), g1, dim3(256), 0, s, target, ts, tok,
                               len, R, gamma, V, it, n_vt, ws, 0u);
        launch_accept<true>(anchor, V, tok, q, len, accept, n_accept, y, p, R, gamma, it, seed,
                            round, n_vt, ws, s, 0, rnn);
        return hipGetLastError();
    }
    // the persistent residual launch, where the draft's geometry applies (Markov
    // head only)
    RunGeometry geo{0, 0, 0};
    bool run = false;
    if constexpr (std::is_same<LT, uint16_t>::value)
        run = !S && path != kPathStream && rows_vec(bs, V, 8) && rows_vec(ts, V, 8) && R <= kRunReqMax &&
              run_geometry(V, &geo);
    if (path == kPathPersistent && !run) return hipErrorNotSupported;
    if (rows_vec(ts, V, Logit<LT>::kVecAlign))
        hipLaunchKernelGGL((verify_rows_kernel<LT, false, true>), g1, dim3(256), 0, s, target, ts, tok, len,
                           R, gamma, V, it, n_vt, ws, (run && give_up) ? 1u : 0u);
    else
        hipLaunchKernelGGL((verify_rows_kernel<LT, false, false>), g1, dim3(256), 0, s, target, ts, tok, len,
                           R, gamma, V, it, n_vt, ws, (run && give_up) ? 1u : 0u);
    launch_accept<false>(anchor, V, tok, q, len, accept, n_accept, y, p, R, gamma, it, seed, round,
                         n_vt, ws, s, run ? geo.n_t : 0, rnn);
    if constexpr (std::is_same<LT, uint16_t>::value) {
        if (run) {
            ResidArgs ra{};
            ra.base = base; ra.bs = bs; ra.target = target; ra.ts = ts; ra.E = E; ra.W2 = W2;
            ra.stats = stats; ra.len = len; ra.n_accept = n_accept; ra.y = y;
            ra.R = R; ra.gamma = gamma; ra.V = V; ra.r = r; ra.inv_temp = it; ra.seed = seed;
            ra.round = round; ra.n_t = geo.n_t; ra.n_vt = n_vt;
            ra.count = ws.resid_cnt; ra.list = ws.resid_list; ra.list_m = ws.resid_m;
            ra.list_prev = ws.resid_prev; ra.slot_of = ws.resid_slot; ra.row_m = ws.row_m;
            ra.row_z = ws.row_z; ra.rowpart = ws.rowpart; ra.slots = ws.run_slots; ra.ctl = ws.run_ctl;
            // one workgroup per request where CUs are free beyond the tile
            // workgroups (those past the tiles run phase 1 on empty tiles)
            const int G = std::max((geo.n_t + 3) / 4, std::min(R, geo.ncu));
            bool launched = false;
            hipError_t e = hipSuccess;
            switch (geo.tu) {
            case 1: e = launch_resid_t<1>(ra, G, geo.ncu, s, &launched); break;
            case 2: e = launch_resid_t<2>(ra, G, geo.ncu, s, &launched); break;
            case 3: e = launch_resid_t<3>(ra, G, geo.ncu, s, &launched); break;
            case 4: e = launch_resid_t<4>(ra, G, geo.ncu, s, &launched); break;
            default: e = launch_resid_t<5>(ra, G, geo.ncu, s, &launched); break;
            }
            if (launched || e != hipSuccess) return e;
            if (path == kPathPersistent) return hipErrorNotSupported;
        }
    }
    PassArgs a{};
    a.base = base; a.target = target; a.bs = bs; a.ts = ts;
    a.W2 = W2; a.anchor = anchor; a.tok = tok;
    // bias rows of the queued rejections: E[x] or the states S[n, m]
    a.E = S ? S : E; a.e_rs = r; a.e_rows = S ? R * gamma : V; a.rnn = 0;
    a.list = ws.resid_list; a.list_m = ws.resid_m; a.list_prev = ws.resid_prev;
    a.count = ws.resid_cnt; a.n_accept = n_accept; a.stats = stats;
    a.row_m = ws.row_m; a.row_z = ws.row_z;
    a.R = R; a.gamma = gamma; a.V = V; a.r = r; a.k = 0; a.inv_temp = it;
    a.n_vt = n_vt;
    a.req_per_wg = pass_req_per_wg(R, n_vt);
    a.part = ws.resid_part;
    const dim3 g3(n_vt, (R + a.req_per_wg - 1) / a.req_per_wg);
    const bool vec = rows_vec(bs, V, 8) && rows_vec(ts, V, 8);
    if (std::is_same<LT, uint16_t>::value && vec) {   // bf16 rows of 16-byte words
        hipLaunchKernelGGL(resid_prep_kernel, dim3((unsigned)((R + 255) / 256)), dim3(256), 0, s,
                           ws.resid_list, ws.resid_m, ws.resid_prev, ws.resid_cnt, stats, ws.row_m,
                           ws.row_z, 0, bs, ts, gamma, ws.resid_roff, ws.resid_erow, ws.resid_rst);
        hipLaunchKernelGGL(resid_pass_kernel, g3, dim3(kDpThreads), 0, s, a,
                           ResidRecs{ws.resid_roff, ws.resid_erow, ws.resid_rst});
    } else if (vec) {
        hipLaunchKernelGGL((bias_pass_kernel<LT, kResidual, true>), g3, dim3(256), 0, s, a);
    } else {
        hipLaunchKernelGGL((bias_pass_kernel<LT, kResidual, false>), g3, dim3(256), 0, s, a);
    }
    const int per = (n_vt + 255) / 256;
    if (per <= 1) launch_vpick<LT, 1>(target, ts, base, bs, E, W2, anchor, tok, stats, len, n_accept, y, R, gamma, V, r, it, seed, round, n_vt, ws, S, s);
    else if (per <= 2) launch_vpick<LT, 2>(target, ts, base, bs, E, W2, anchor, tok, stats, len, n_accept, y, R, gamma, V, r, it, seed, round, n_vt, ws, S, s);
    else if (per <= 4) launch_vpick<LT, 4>(target, ts, base, bs, E, W2, anchor, tok, stats, len, n_accept, y, R, gamma, V, r, it, seed, round, n_vt, ws, S, s);
    else launch_vpick<LT, 8>(target, ts, base, bs, E, W2, anchor, tok, stats, len, n_accept, y, R, gamma, V, r, it, seed, round, n_vt, ws, S, s);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Exact acceptance probability of every draft position:
//   alpha[n, k] = sum_v min(q_k(v), p_k(v)) = 1 - sum_v max(0, p_k(v) - q_k(v))
// (page "为什么DSpark 可以加速推理？", section on the mathematics of speculative
// decoding: the total acceptance probability; page "DeepSeek联合北大最新文章DSpark",
// section 2.1: one minus the total-variation distance is the confidence head's
// target).  The target rows' normalisers come first (verify_rows and a per-row
// combine); then the residual pass runs over every (request, position) entry --
// the draft row rebuilt with the draft step's MFMA bias, max(0, p - q) per column
// in fp64 -- and a combine sums each entry's tiles.
// ---------------------------------------------------------------------------
namespace {

struct TvWs {
    VerifyWs v;          // verify_rows' outputs (rowpart, spanpart, zx) and scratch words
    int* lens;           // [R] gamma - 1: verify_rows streams target rows 0 .. gamma-1
    int* count;          // [1] R gamma
    int* list;           // [R gamma] request of each entry
    int* list_m;         // [R gamma] its position
    int* list_prev;      // [R gamma] the token before it (-1: no bias)
    float* row_m;        // [R gamma] target row maximum
    double* row_z;       // [R gamma] target row normaliser
    Part* part;          // [R gamma, n_vt] residual mass per tile
    int64_t* roff;       // [R gamma, 2] records for resid_pass_kernel
    int* erow;           // [R gamma]
    float4* rst;         // [R gamma]
};

inline TvWs carve_tv(void* ws, int R, int gamma, int V, size_t* total)
{
    const size_t n_vt = (size_t)((V + kVocabTile - 1) / kVocabTile);
    const size_t spans = (n_vt + kSpanTiles - 1) / kSpanTiles;
    const size_t N = (size_t)R * gamma;
    char* p = static_cast<char*>(ws);
    size_t off = 0;
    TvWs w{};
    w.v.rowpart = reinterpret_cast<Part*>(p + off);  off += align256((size_t)R * (gamma + 1) * n_vt * sizeof(Part));
    w.v.spanpart = reinterpret_cast<Part*>(p + off); off += align256((size_t)R * (gamma + 1) * 4 * spans * sizeof(Part));
    w.v.zx = reinterpret_cast<float*>(p + off);      off += align256(N * sizeof(float));
    w.v.resid_cnt = reinterpret_cast<int*>(p + off); off += 256;
    w.v.run_ctl = reinterpret_cast<unsigned*>(p + off); off += 256;
    w.lens = reinterpret_cast<int*>(p + off);        off += align256((size_t)R * sizeof(int));
    w.count = reinterpret_cast<int*>(p + off);       off += 256;
    w.list = reinterpret_cast<int*>(p + off);        off += align256(N * sizeof(int));
    w.list_m = reinterpret_cast<int*>(p + off);      off += align256(N * sizeof(int));
    w.list_prev = reinterpret_cast<int*>(p + off);   off += align256(N * sizeof(int));
    w.row_m = reinterpret_cast<float*>(p + off);     off += align256(N * sizeof(float));
    w.row_z = reinterpret_cast<double*>(p + off);    off += align256(N * sizeof(double));
    w.part = reinterpret_cast<Part*>(p + off);       off += align256(N * n_vt * sizeof(Part));
    w.roff = reinterpret_cast<int64_t*>(p + off);    off += align256(N * 2 * sizeof(int64_t));
    w.erow = reinterpret_cast<int*>(p + off);        off += align256(N * sizeof(int));
    w.rst = reinterpret_cast<float4*>(p + off);      off += align256(N * sizeof(float4));
    if (total) *total = off;
    return w;
}

}  // namespace

// one thread per (request, position) entry: the residual pass's queue and the
// row limit that makes verify_rows stream target rows 0 .. gamma - 1
__global__ void tv_prep_kernel(const int32_t* __restrict__ anchor, const int32_t* __restrict__ tok,
                               int R, int gamma, int V, TvWs ws, int rnn)
{
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t N = (int64_t)R * gamma;
    if (e < R) ws.lens[e] = gamma - 1;
    if (e == 0) *ws.count = (int)N;
    if (e >= N) return;
    const int n = (int)(e / gamma), k = (int)(e % gamma);
    const int p = (k == 0) ? anchor[n] : tok[e - 1];
    ws.list[e] = n;
    ws.list_m[e] = k;
    // bias row: the token before the position, or the recurrent state row e
    ws.list_prev[e] = rnn ? (int)e : (p >= 0 && p < V) ? p : -1;
}

// one wave per entry: the target row's (M, Z) from verify_rows' 8-tile partials
template <int PER>
__global__ __launch_bounds__(256) void tv_rowstats_kernel(int R, int gamma, int n_vt, float inv_temp,
                                                          TvWs ws)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t e = (int64_t)blockIdx.x * 4 + wave;
    if (e >= (int64_t)R * gamma) return;
    const int n = (int)(e / gamma), k = (int)(e % gamma);
    const int np = 4 * ((n_vt + kSpanTiles - 1) / kSpanTiles);
    const Part* pp = ws.v.spanpart + ((int64_t)n * (gamma + 1) + k) * np;
    Part pt[PER];
    float M = -INFINITY;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int t = lane * PER + i;
        pt[i] = (t < np) ? pp[t] : Part{-INFINITY, 0, 0.0};
        M = fmaxf(M, pt[i].m);
    }
    M = wave_max_f(M);
    double Z = 0.0;
#pragma unroll
    for (int i = 0; i < PER; ++i) Z += pt[i].s * rescale64(pt[i].m, M, inv_temp);
    Z = wave_sum_d(Z);
    if (lane == 0) {
        ws.row_m[e] = M;
        ws.row_z[e] = Z;
    }
}

// one wave per entry: alpha = 1 - (sum of the tiles' residual mass); lane l adds
// tiles l, l + 64, ..., so that each load reads 64 consecutive partials
template <int PER>
__global__ __launch_bounds__(256) void tv_combine_kernel(int R, int gamma, int n_vt, TvWs ws,
                                                         double* __restrict__ alpha)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t e = (int64_t)blockIdx.x * 4 + wave;
    if (e >= (int64_t)R * gamma) return;
    const Part* pp = ws.part + e * n_vt;
    double s = 0.0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int t = i * kWave + lane;
        if (t < n_vt) s += pp[t].s;
    }
    s = wave_sum_d(s);
    if (lane == 0) alpha[e] = fmin(fmax(1.0 - s, 0.0), 1.0);
}

size_t tv_workspace_bytes(int R, int gamma, int V)
{
    size_t total = 0;
    carve_tv(nullptr, R, gamma, V, &total);
    return total;
}

template <typename LT>
static hipError_t launch_tv_t(const LT* target, RowStrides ts, const LT* base, RowStrides bs,
                              const uint16_t* E, const uint16_t* W2, const int32_t* anchor,
                              const int32_t* tok, const double* stats, double* alpha, int R,
                              int gamma, int V, int r, float temperature, void* ws_raw,
                              const uint16_t* S, hipStream_t s)
{
    const TvWs ws = carve_tv(ws_raw, R, gamma, V, nullptr);
    const int n_vt = (V + kVocabTile - 1) / kVocabTile;
    const float it = 1.0f / temperature;
    const int64_t N = (int64_t)R * gamma;
    hipLaunchKernelGGL(tv_prep_kernel, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, s, anchor, tok,
                       R, gamma, V, ws, S ? 1 : 0);
    const int spans = (n_vt + kSpanTiles - 1) / kSpanTiles;
    const int64_t items = (int64_t)R * spans;
    if (rows_vec(ts, V, Logit<LT>::kVecAlign))
        hipLaunchKernelGGL((verify_rows_kernel<LT, false, true>), dim3((unsigned)items), dim3(256), 0, s,
                           target, ts, tok, ws.lens, R, gamma, V, it, n_vt, ws.v, 0u);
    else
        hipLaunchKernelGGL((verify_rows_kernel<LT, false, false>), dim3((unsigned)items), dim3(256), 0, s,
                           target, ts, tok, ws.lens, R, gamma, V, it, n_vt, ws.v, 0u);
    const int np = 4 * spans;
    const int per = (np + kWave - 1) / kWave;
    const dim3 gw((unsigned)((N + 3) / 4));
#define DSP_TVROW(P) hipLaunchKernelGGL((tv_rowstats_kernel<P>), gw, dim3(256), 0, s, R, gamma, n_vt, it, ws)
    if (per <= 1) DSP_TVROW(1);
    else if (per <= 2) DSP_TVROW(2);
    else if (per <= 4) DSP_TVROW(4);
    else if (per <= 8) DSP_TVROW(8);
    else if (per <= 16) DSP_TVROW(16);
    else DSP_TVROW(32);
#undef DSP_TVROW
    PassArgs a{};
    a.base = base; a.target = target; a.bs = bs; a.ts = ts;
    a.W2 = W2; a.anchor = anchor; a.tok = tok;
    a.E = S ? S : E; a.e_rs = r; a.e_rows = S ? R * gamma : V; a.rnn = 0;
    a.list = ws.list; a.list_m = ws.list_m; a.list_prev = ws.list_prev; a.count = ws.count;
    a.stats = stats; a.row_m = ws.row_m; a.row_z = ws.row_z; a.row_by_entry = 1;
    a.R = R; a.gamma = gamma; a.V = V; a.r = r; a.k = 0; a.inv_temp = it;
    a.n_vt = n_vt;
    a.req_per_wg = pass_req_per_wg((int)N, n_vt);
    a.part = ws.part;
    const dim3 g3(n_vt, (unsigned)((N + a.req_per_wg - 1) / a.req_per_wg));
    const bool vec = rows_vec(bs, V, 8) && rows_vec(ts, V, 8);
    if (std::is_same<LT, uint16_t>::value && vec) {   // bf16 rows of 16-byte words
        hipLaunchKernelGGL(resid_prep_kernel, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, s,
                           ws.list, ws.list_m, ws.list_prev, ws.count, stats, ws.row_m, ws.row_z, 1,
                           bs, ts, gamma, ws.roff, ws.erow, ws.rst);
        hipLaunchKernelGGL(resid_pass_kernel, g3, dim3(kDpThreads), 0, s, a,
                           ResidRecs{ws.roff, ws.erow, ws.rst});
    } else if (vec) {
        hipLaunchKernelGGL((bias_pass_kernel<LT, kResidual, true>), g3, dim3(256), 0, s, a);
    } else {
        hipLaunchKernelGGL((bias_pass_kernel<LT, kResidual, false>), g3, dim3(256), 0, s, a);
    }
    const int pc = (n_vt + kWave - 1) / kWave;
#define DSP_TVC(P) hipLaunchKernelGGL((tv_combine_kernel<P>), gw, dim3(256), 0, s, R, gamma, n_vt, ws, alpha)
    if (pc <= 1) DSP_TVC(1);
    else if (pc <= 2) DSP_TVC(2);
    else if (pc <= 4) DSP_TVC(4);
    else if (pc <= 8) DSP_TVC(8);
    else DSP_TVC(16);
#undef DSP_TVC
    return hipGetLastError();
}

hipError_t launch_tv_accept(const void* target, RowStrides ts, const void* base, RowStrides bs,
                            bool bf16, const uint16_t* E, const uint16_t* W2, const int32_t* anchor,
                            const int32_t* tok, const double* stats, double* alpha, int R, int gamma,
                            int V, int r, float temperature, void* ws, hipStream_t s, const uint16_t* S)
{
    if (bf16)
        return launch_tv_t(static_cast<const uint16_t*>(target), ts, static_cast<const uint16_t*>(base),
                           bs, E, W2, anchor, tok, stats, alpha, R, gamma, V, r, temperature, ws, S, s);
    return launch_tv_t(static_cast<const float*>(target), ts, static_cast<const float*>(base), bs, E,
                       W2, anchor, tok, stats, alpha, R, gamma, V, r, temperature, ws, S, s);
}

hipError_t launch_verify(const void* target, RowStrides ts, const void* base, RowStrides bs,
                         bool bf16, int path, bool give_up, const uint16_t* E,
                         const uint16_t* W2, const int32_t* anchor, const int32_t* tok,
                         const float* q, const double* stats, const int32_t* len, int8_t* accept,
                         int32_t* n_accept, int32_t* y, float* p, int R, int gamma, int V, int r,
                         float temperature, uint64_t seed, uint32_t round, void* ws, hipStream_t s,
                         const uint16_t* S)
{
    if (S && path == kPathPersistent) return hipErrorNotSupported;
    if (bf16)
        return launch_verify_t(static_cast<const uint16_t*>(target), ts,
                               static_cast<const uint16_t*>(base), bs, path, give_up, E, W2, anchor, tok, q, stats,
                               len, accept, n_accept, y, p, R, gamma, V, r, temperature, seed, round,
                               ws, S, s);
    return launch_verify_t(static_cast<const float*>(target), ts, static_cast<const float*>(base), bs,
                           path, give_up, E, W2,
                           anchor, tok, q, stats, len, accept, n_accept, y, p, R, gamma, V, r,
                           temperature, seed, round, ws, S, s);
}

}  // namespace dsp

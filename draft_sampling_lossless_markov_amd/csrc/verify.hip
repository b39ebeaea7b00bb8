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
//   verify_rows     stream each verified target row (r, j <= l_r) once in
//                   8192-wide chunks: online-softmax (or argmax) partials, and
//                   the target logit at the drafted token
//   verify_accept   one wave per request: row normalisers (fp64), p_j(x_j), the
//                   accept tests, the first rejection, greedy corrections; queue
//                   requests that need a residual draw
//   verify_resid    residual mass per (queued request, 256-vocabulary tile); the
//                   draft row is recomputed with the draft kernel's MFMA bias
//   verify_pick     one wave per request: locate the residual tile (or the bonus
//                   / fallback chunk of a target row) and scan it in order
#include "bias_tile.h"
#include "dsp_device.h"
#include "dsp_launch.h"

namespace dsp {

namespace {

struct VerifyWs {
    float2* rowpart;     // [R, gamma+1, n_ch]
    float* zx;           // [R, gamma] target logit at the drafted token
    int* resid_cnt;      // [1]
    int* resid_list;     // [R]
    int* resid_slot;     // [R]
    double* row_z;       // [R] fp64 normaliser of target row n_accept
    float* row_m;        // [R] max logit of target row n_accept
    float* resid_part;   // [R, n_vt]
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

inline VerifyWs carve(void* ws, int R, int gamma, int V, size_t* total)
{
    const size_t n_ch = (size_t)((V + kVerifyChunk - 1) / kVerifyChunk);
    const size_t n_vt = (size_t)((V + kVocabTile - 1) / kVocabTile);
    char* p = static_cast<char*>(ws);
    size_t off = 0;
    VerifyWs w;
    w.rowpart = reinterpret_cast<float2*>(p + off);  off += align256((size_t)R * (gamma + 1) * n_ch * sizeof(float2));
    w.zx = reinterpret_cast<float*>(p + off);        off += align256((size_t)R * gamma * sizeof(float));
    w.resid_cnt = reinterpret_cast<int*>(p + off);   off += align256(sizeof(int));
    w.resid_list = reinterpret_cast<int*>(p + off);  off += align256((size_t)R * sizeof(int));
    w.resid_slot = reinterpret_cast<int*>(p + off);  off += align256((size_t)R * sizeof(int));
    w.row_z = reinterpret_cast<double*>(p + off);    off += align256((size_t)R * sizeof(double));
    w.row_m = reinterpret_cast<float*>(p + off);     off += align256((size_t)R * sizeof(float));
    w.resid_part = reinterpret_cast<float*>(p + off); off += align256((size_t)R * n_vt * sizeof(float));
    if (total) *total = off;
    return w;
}

__device__ __forceinline__ int clamp_len(const int32_t* len, int n, int gamma)
{
    return min(max(len[n], 0), gamma);
}

}  // namespace

// ---------------------------------------------------------------------------
// verify_rows: grid-stride over (request, row, chunk) items; rows past l_r are
// skipped.  256 threads x 32 values per 8192-wide chunk.
// ---------------------------------------------------------------------------
template <typename LT, bool GREEDY>
__global__ __launch_bounds__(256) void verify_rows_kernel(
    const LT* __restrict__ target, const int32_t* __restrict__ tok,
    const int32_t* __restrict__ len, int R, int gamma, int V, float inv_temp, int n_ch,
    VerifyWs ws)
{
    __shared__ float2 red[4];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    if (blockIdx.x == 0 && tid == 0) *ws.resid_cnt = 0;
    const int per_req = (gamma + 1) * n_ch;
    const int64_t total = (int64_t)R * per_req;
    const bool vec_ok = (V % Logit<LT>::kVecAlign) == 0;
    for (int64_t item = blockIdx.x; item < total; item += gridDim.x) {
        const int n = (int)(item / per_req);
        const int rem = (int)(item % per_req);
        const int j = rem / n_ch, ch = rem % n_ch;
        const int l = clamp_len(len, n, gamma);
        if (j > l) continue;
        const LT* row = target + ((int64_t)n * (gamma + 1) + j) * V;
        const int v0 = ch * kVerifyChunk;
        float x[32];
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int v = v0 + it * 2048 + tid * 8;
            const int vend = min(V, v0 + kVerifyChunk);
            if (v + 8 <= vend) {
                Logit<LT>::load8(row, v, V, vec_ok, x + 8 * it);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    x[8 * it + e] = (v + e < vend) ? Logit<LT>::at(row, v + e) : -INFINITY;
            }
        }
        float2 res;
        if constexpr (GREEDY) {
            ArgMax am{-INFINITY, 0x7fffffff};
#pragma unroll
            for (int it = 0; it < 4; ++it)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int v = v0 + it * 2048 + tid * 8 + e;
                    if (v < V) am = argmax_merge(am, ArgMax{x[8 * it + e], v});
                }
            am = wave_argmax(am);
            res = make_float2(am.v, __int_as_float(am.i));
        } else {
            float m = -INFINITY;
#pragma unroll
            for (int e = 0; e < 32; ++e) m = fmaxf(m, x[e]);
            float s = 0.f;
            if (m != -INFINITY) {
#pragma unroll
                for (int e = 0; e < 32; ++e) s += __expf((x[e] - m) * inv_temp);
            }
            res = make_float2(m, s);
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) {
                float2 b;
                b.x = __shfl_xor(res.x, o, kWave);
                b.y = __shfl_xor(res.y, o, kWave);
                res = lse_merge(res, b, inv_temp);
            }
        }
        if (lane == 0) red[wave] = res;
        __syncthreads();
        if (tid == 0) {
            float2 a = red[0];
#pragma unroll
            for (int w = 1; w < 4; ++w) {
                if constexpr (GREEDY) {
                    const ArgMax m = argmax_merge(ArgMax{a.x, __float_as_int(a.y)},
                                                  ArgMax{red[w].x, __float_as_int(red[w].y)});
                    a = make_float2(m.v, __int_as_float(m.i));
                } else {
                    a = lse_merge(a, red[w], inv_temp);
                }
            }
            ws.rowpart[((int64_t)n * (gamma + 1) + j) * n_ch + ch] = a;
            if (!GREEDY && j < l) {
                const int xj = tok[(int64_t)n * gamma + j];
                if (xj >= v0 && xj < min(V, v0 + kVerifyChunk))
                    ws.zx[(int64_t)n * gamma + j] = Logit<LT>::at(row, xj);
            }
        }
        __syncthreads();
    }
}

// Combine the chunk partials of one target row (every lane gets the result).
__device__ __forceinline__ void row_stats(const float2* __restrict__ pp, int n_ch, float it,
                                          int lane, float* M_out, double* Z_out)
{
    float M = -INFINITY;
    for (int c = lane; c < n_ch; c += kWave) M = fmaxf(M, pp[c].x);
    M = wave_max(M);
    double Z = 0.0;
    for (int c = lane; c < n_ch; c += kWave) {
        const float2 p = pp[c];
        if (p.x != -INFINITY) Z += (double)p.y * exp(((double)p.x - (double)M) * (double)it);
    }
    *M_out = M;
    *Z_out = wave_sum(Z);
}

__device__ __forceinline__ ArgMax row_argmax(const float2* __restrict__ pp, int n_ch, int lane)
{
    ArgMax am{-INFINITY, 0x7fffffff};
    for (int c = lane; c < n_ch; c += kWave) am = argmax_merge(am, ArgMax{pp[c].x, __float_as_int(pp[c].y)});
    return wave_argmax(am);
}

// ---------------------------------------------------------------------------
// verify_accept: one wave per request
// ---------------------------------------------------------------------------
template <bool GREEDY>
__global__ __launch_bounds__(256) void verify_accept_kernel(
    const int32_t* __restrict__ tok, const float* __restrict__ q, const int32_t* __restrict__ len,
    int8_t* __restrict__ accept, int32_t* __restrict__ n_accept, int32_t* __restrict__ y,
    float* __restrict__ p_out, int R, int gamma, float inv_temp, uint64_t seed, uint32_t round,
    int n_ch, VerifyWs ws)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n = blockIdx.x * 4 + wave;
    if (n >= R) return;
    const int l = clamp_len(len, n, gamma);
    const float2* rows = ws.rowpart + (int64_t)n * (gamma + 1) * n_ch;
    int nacc = l;
    for (int j = 0; j < l; ++j) {
        const int64_t o = (int64_t)n * gamma + j;
        int acc;
        float pj;
        if constexpr (GREEDY) {
            const ArgMax am = row_argmax(rows + (int64_t)j * n_ch, n_ch, lane);
            acc = (tok[o] == am.i);
            pj = acc ? 1.0f : 0.0f;
        } else {
            float M;
            double Z;
            row_stats(rows + (int64_t)j * n_ch, n_ch, inv_temp, lane, &M, &Z);
            const double p = exp(((double)ws.zx[o] - (double)M) * (double)inv_temp) / Z;
            const double u = uniform24(seed, round, (uint32_t)n, (uint32_t)j, 1u);
            acc = (u * (double)q[o] <= p);
            pj = (float)p;
            if (!acc && nacc == l) { ws.row_m[n] = M; ws.row_z[n] = Z; }
        }
        if (lane == 0) { accept[o] = (int8_t)acc; p_out[o] = pj; }
        if (!acc && nacc == l) nacc = j;
    }
    if (lane == 0) {
        for (int j = l; j < gamma; ++j) {
            accept[(int64_t)n * gamma + j] = -1;
            p_out[(int64_t)n * gamma + j] = 0.0f;
        }
        n_accept[n] = nacc;
    }
    if constexpr (GREEDY) {
        const ArgMax am = row_argmax(rows + (int64_t)nacc * n_ch, n_ch, lane);
        if (lane == 0) y[n] = am.i;
    } else {
        if (lane == 0) {
            if (nacc < l) {
                const int slot = atomicAdd(ws.resid_cnt, 1);
                ws.resid_list[slot] = n;
                ws.resid_slot[n] = slot;
            } else {
                ws.resid_slot[n] = -1;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// verify_resid: residual mass sum_v max(0, p_v - q_v) per (queued request,
// 256-vocabulary tile).  Same workgroup shape and MFMA sequence as the draft
// kernel; requests come from the queue in sub-blocks of 64.
// ---------------------------------------------------------------------------
template <typename LT>
__global__ __launch_bounds__(256) void verify_resid_kernel(
    const LT* __restrict__ target, const LT* __restrict__ base, const uint16_t* __restrict__ E,
    const uint16_t* __restrict__ W2, const int32_t* __restrict__ anchor,
    const int32_t* __restrict__ tok, const float* __restrict__ stats,
    const int32_t* __restrict__ n_accept, int R, int gamma, int V, int r, float inv_temp,
    int n_vt, VerifyWs ws)
{
    __shared__ __attribute__((aligned(16))) uint16_t e_tile[kReqBlock][kRankMax + kERowPad];
    __shared__ float red[4][kReqBlock];
    const int cnt = *ws.resid_cnt;
    const int e0 = blockIdx.y * kReqBlock;
    if (e0 >= cnt) return;   // workgroup-uniform
    const int e_end = min(cnt, e0 + kReqBlock);
    const int vt = blockIdx.x;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int g = lane >> 4, c16 = lane & 15;
    const int v_blk = vt * kVocabTile + wave * 64;
    const int ksteps = (r + kKStep - 1) / kKStep;
    bf16x8 afrag[4][kKSteps];
    load_w2_frags(W2, V, r, v_blk, lane, afrag);

    const int chunks = kRankMax / 8;
    for (int idx = threadIdx.x; idx < kReqBlock * chunks; idx += blockDim.x) {
        const int row = idx / chunks, ch = idx % chunks;
        const int e = e0 + row;
        uint4 u = make_uint4(0, 0, 0, 0);
        if (e < e_end && ch * 8 < r) {
            const int n = ws.resid_list[e];
            const int prev = prev_token(anchor, tok, n, gamma, n_accept[n], V);
            if (prev >= 0) u = *reinterpret_cast<const uint4*>(E + (int64_t)prev * r + ch * 8);
        }
        *reinterpret_cast<uint4*>(&e_tile[row][ch * 8]) = u;
    }
    __syncthreads();

    floatx4 acc[4][4];
#pragma unroll
    for (int tn = 0; tn < 4; ++tn)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[tn][t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
        if (ks < ksteps) {
#pragma unroll
            for (int tn = 0; tn < 4; ++tn) {
                const bf16x8 b = as_bf16x8(
                    *reinterpret_cast<const uint4*>(&e_tile[16 * tn + c16][ks * kKStep + 8 * g]));
#pragma unroll
                for (int t = 0; t < 4; ++t) acc[tn][t] = mfma_bf16(afrag[t][ks], b, acc[tn][t]);
            }
        }
    }

    const bool vec_ok = (V % Logit<LT>::kVecAlign) == 0;
#pragma unroll
    for (int tn = 0; tn < 4; ++tn) {
        const int e = e0 + 16 * tn + c16;
        float sum = 0.f;
        if (e < e_end) {
            const int n = ws.resid_list[e];
            const int m = n_accept[n];
            const LT* drow = base + ((int64_t)n * gamma + m) * V;
            const LT* trow = target + ((int64_t)n * (gamma + 1) + m) * V;
            const float Md = stats[2 * ((int64_t)n * gamma + m)];
            const float invZd = (float)(1.0 / (double)stats[2 * ((int64_t)n * gamma + m) + 1]);
            const float Mt = ws.row_m[n];
            const float invZt = (float)(1.0 / ws.row_z[n]);
            float xd[16], xt[16];
            const int va = v_blk + 8 * g, vb = v_blk + 32 + 8 * g;
            Logit<LT>::load8(drow, va, V, vec_ok && va + 8 <= V, xd);
            Logit<LT>::load8(drow, vb, V, vec_ok && vb + 8 <= V, xd + 8);
            Logit<LT>::load8(trow, va, V, vec_ok && va + 8 <= V, xt);
            Logit<LT>::load8(trow, vb, V, vec_ok && vb + 8 <= V, xt + 8);
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                if (xd[s] == -INFINITY || xt[s] == -INFINITY) continue;
                const float zd = xd[s] + acc[tn][s >> 2][s & 3];
                const float pv = __expf((xt[s] - Mt) * inv_temp) * invZt;
                const float qv = __expf((zd - Md) * inv_temp) * invZd;
                sum += fmaxf(pv - qv, 0.0f);
            }
        }
        sum += __shfl_xor(sum, 16, kWave);
        sum += __shfl_xor(sum, 32, kWave);
        if (g == 0) red[wave][16 * tn + c16] = sum;
    }
    __syncthreads();
    if (threadIdx.x < kReqBlock) {
        const int e = e0 + threadIdx.x;
        if (e < e_end)
            ws.resid_part[(int64_t)e * n_vt + vt] =
                red[0][threadIdx.x] + red[1][threadIdx.x] + red[2][threadIdx.x] + red[3][threadIdx.x];
    }
}

// In-order inverse CDF over a 8192-wide chunk of one target row: 128 consecutive
// values per lane.  Returns the vocabulary index.
template <typename LT>
__device__ int chunk_inverse_cdf(const LT* __restrict__ row, int v0, int V, float M, float it,
                                 double before, double target, int lane)
{
    const int vb = v0 + lane * (kVerifyChunk / kWave);
    const int ve = min(V, vb + kVerifyChunk / kWave);
    double ls = 0.0;
    int last = -1;
    for (int v = vb; v < ve; ++v) {
        const float w = __expf((Logit<LT>::at(row, v) - M) * it);
        ls += (double)w;
        if (w > 0.f) last = v;
    }
    const double incl = wave_incl_scan(ls, lane);
    int hit = 0x7fffffff;
    if (before + incl > target) {
        double cum = before + incl - ls;
        for (int v = vb; v < ve; ++v) {
            cum += (double)__expf((Logit<LT>::at(row, v) - M) * it);
            if (cum > target) { hit = v; break; }
        }
        if (hit == 0x7fffffff) hit = last >= 0 ? last : vb;
    }
    hit = wave_min_i(hit);
    if (hit == 0x7fffffff) hit = wave_max_i(last);
    return hit;
}

// ---------------------------------------------------------------------------
// verify_pick: one wave per request (sampling only)
// ---------------------------------------------------------------------------
template <typename LT>
__global__ __launch_bounds__(256) void verify_pick_kernel(
    const LT* __restrict__ target, const LT* __restrict__ base, const uint16_t* __restrict__ E,
    const uint16_t* __restrict__ W2, const int32_t* __restrict__ anchor,
    const int32_t* __restrict__ tok, const float* __restrict__ stats,
    const int32_t* __restrict__ len, const int32_t* __restrict__ n_accept,
    int32_t* __restrict__ y, int R, int gamma, int V, int r, float inv_temp, uint64_t seed,
    uint32_t round, int n_ch, int n_vt, VerifyWs ws)
{
    __shared__ float lg_s[4][kVocabTile];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n = blockIdx.x * 4 + wave;
    const bool active = n < R;   // wave-uniform
    const int l = active ? clamp_len(len, n, gamma) : 0;
    const int m = active ? n_accept[n] : 0;
    const int slot = active ? ws.resid_slot[n] : -1;
    const double u = uniform24(seed, round, (uint32_t)n, (uint32_t)m, 2u);

    // residual draw: locate the tile of cumulative residual mass u * sum
    double rsum = 0.0, before = 0.0, target_mass = 0.0;
    int tsel = -1;
    if (active && slot >= 0) {
        const float* rp = ws.resid_part + (int64_t)slot * n_vt;
        for (int t = lane; t < n_vt; t += kWave) rsum += (double)rp[t];
        rsum = wave_sum(rsum);
        if (rsum > 0.0) {
            target_mass = u * rsum;
            double run = 0.0, before_last = 0.0;
            int tlast = 0;
            for (int t0 = 0; t0 < n_vt && tsel < 0; t0 += kWave) {
                const int t = t0 + lane;
                const double w = (t < n_vt) ? (double)rp[t] : 0.0;
                const double incl = wave_incl_scan(w, lane) + run;
                const int hit = wave_min_i((incl > target_mass) ? t : 0x7fffffff);
                const int lastpos = wave_max_i((w > 0.0) ? t : -1);
                if (lastpos >= 0) {
                    tlast = lastpos;
                    before_last = __shfl(incl - w, lastpos - t0, kWave);
                }
                if (hit != 0x7fffffff) {
                    tsel = hit;
                    before = __shfl(incl - w, hit - t0, kWave);
                }
                run = __shfl(incl, kWave - 1, kWave);
            }
            if (tsel < 0) { tsel = tlast; before = before_last; }
            const int prev = prev_token(anchor, tok, n, gamma, m, V);
            const LT* drow = base + ((int64_t)n * gamma + m) * V;
            tile_logits<LT>(drow, E, W2, V, r, prev, tsel, lane, lg_s[wave]);
        }
    }
    __syncthreads();
    if (!active) return;
    if (tsel >= 0) {
        const LT* trow = target + ((int64_t)n * (gamma + 1) + m) * V;
        const float Md = stats[2 * ((int64_t)n * gamma + m)];
        const float invZd = (float)(1.0 / (double)stats[2 * ((int64_t)n * gamma + m) + 1]);
        const float Mt = ws.row_m[n];
        const float invZt = (float)(1.0 / ws.row_z[n]);
        float w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int v = tsel * kVocabTile + 4 * lane + e;
            const float zd = lg_s[wave][4 * lane + e];
            w[e] = 0.f;
            if (v < V && zd != -INFINITY) {
                const float pv = __expf((Logit<LT>::at(trow, v) - Mt) * inv_temp) * invZt;
                const float qv = __expf((zd - Md) * inv_temp) * invZd;
                w[e] = fmaxf(pv - qv, 0.0f);
            }
        }
        float wsel;
        const int loc = tile_inverse_cdf_w(w, before, target_mass, lane, &wsel);
        if (lane == 0) y[n] = tsel * kVocabTile + loc;
        return;
    }
    // bonus draw from target row l, or the zero-residual fallback from row m
    const int row_j = (slot >= 0) ? m : l;
    const float2* pp = ws.rowpart + ((int64_t)n * (gamma + 1) + row_j) * n_ch;
    float M;
    double Z;
    row_stats(pp, n_ch, inv_temp, lane, &M, &Z);
    const double tgt = u * Z;
    double run = 0.0, bsel = 0.0, blast = 0.0;
    int csel = -1, clast = 0;
    for (int c0 = 0; c0 < n_ch && csel < 0; c0 += kWave) {
        const int c = c0 + lane;
        double w = 0.0;
        if (c < n_ch) {
            const float2 p = pp[c];
            if (p.x != -INFINITY) w = (double)p.y * exp(((double)p.x - (double)M) * (double)inv_temp);
        }
        const double incl = wave_incl_scan(w, lane) + run;
        const int hit = wave_min_i((incl > tgt) ? c : 0x7fffffff);
        const int lastpos = wave_max_i((w > 0.0) ? c : -1);
        if (lastpos >= 0) { clast = lastpos; blast = __shfl(incl - w, lastpos - c0, kWave); }
        if (hit != 0x7fffffff) { csel = hit; bsel = __shfl(incl - w, hit - c0, kWave); }
        run = __shfl(incl, kWave - 1, kWave);
    }
    if (csel < 0) { csel = clast; bsel = blast; }
    const LT* trow = target + ((int64_t)n * (gamma + 1) + row_j) * V;
    const int v = chunk_inverse_cdf<LT>(trow, csel * kVerifyChunk, V, M, inv_temp, bsel, tgt, lane);
    if (lane == 0) y[n] = v;
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

template <typename LT>
static hipError_t launch_verify_t(const LT* target, const LT* base, const uint16_t* E,
                                  const uint16_t* W2, const int32_t* anchor, const int32_t* tok,
                                  const float* q, const float* stats, const int32_t* len,
                                  int8_t* accept, int32_t* n_accept, int32_t* y, float* p, int R,
                                  int gamma, int V, int r, float temperature, uint64_t seed,
                                  uint32_t round, void* ws_raw, hipStream_t s)
{
    const VerifyWs ws = carve(ws_raw, R, gamma, V, nullptr);
    const int n_ch = (V + kVerifyChunk - 1) / kVerifyChunk;
    const int n_vt = (V + kVocabTile - 1) / kVocabTile;
    const bool greedy = (temperature == 0.0f);
    const float it = greedy ? 1.0f : 1.0f / temperature;
    const int64_t items = (int64_t)R * (gamma + 1) * n_ch;
    const dim3 g1((unsigned)std::min<int64_t>(items, 8192));
    const dim3 g2((R + 3) / 4);
    if (greedy) {
        hipLaunchKernelGGL((verify_rows_kernel<LT, true>), g1, dim3(256), 0, s, target, tok, len,
                           R, gamma, V, it, n_ch, ws);
        hipLaunchKernelGGL((verify_accept_kernel<true>), g2, dim3(256), 0, s, tok, q, len, accept,
                           n_accept, y, p, R, gamma, it, seed, round, n_ch, ws);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((verify_rows_kernel<LT, false>), g1, dim3(256), 0, s, target, tok, len, R,
                       gamma, V, it, n_ch, ws);
    hipLaunchKernelGGL((verify_accept_kernel<false>), g2, dim3(256), 0, s, tok, q, len, accept,
                       n_accept, y, p, R, gamma, it, seed, round, n_ch, ws);
    const dim3 g3(n_vt, (R + kReqBlock - 1) / kReqBlock);
    hipLaunchKernelGGL((verify_resid_kernel<LT>), g3, dim3(256), 0, s, target, base, E, W2, anchor,
                       tok, stats, n_accept, R, gamma, V, r, it, n_vt, ws);
    hipLaunchKernelGGL((verify_pick_kernel<LT>), g2, dim3(256), 0, s, target, base, E, W2, anchor,
                       tok, stats, len, n_accept, y, R, gamma, V, r, it, seed, round, n_ch, n_vt, ws);
    return hipGetLastError();
}

hipError_t launch_verify(const void* target, const void* base, bool bf16, const uint16_t* E,
                         const uint16_t* W2, const int32_t* anchor, const int32_t* tok,
                         const float* q, const float* stats, const int32_t* len, int8_t* accept,
                         int32_t* n_accept, int32_t* y, float* p, int R, int gamma, int V, int r,
                         float temperature, uint64_t seed, uint32_t round, void* ws, hipStream_t s)
{
    if (bf16)
        return launch_verify_t(static_cast<const uint16_t*>(target),
                               static_cast<const uint16_t*>(base), E, W2, anchor, tok, q, stats,
                               len, accept, n_accept, y, p, R, gamma, V, r, temperature, seed, round,
                               ws, s);
    return launch_verify_t(static_cast<const float*>(target), static_cast<const float*>(base), E, W2,
                           anchor, tok, q, stats, len, accept, n_accept, y, p, R, gamma, V, r,
                           temperature, seed, round, ws, s);
}

}  // namespace dsp

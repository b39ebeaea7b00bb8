/*
 * dsp_oracle.c -- plain, slow, single-threaded CPU oracle for the DSpark
 * draft-sampling / confidence / prefix-scheduling / lossless-verification path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path (the
 * HIP library) shares no code, header, table or helper with this file.
 *
 * Arithmetic: fp64 throughout, sequential sums in index order, libm exp/log.
 * Where the method fixes a rounding (the fp32 survival products, the
 * fixed-point expected-acceptance sum) it is written out explicitly below.
 *
 * Sources (DSpark pages):
 *   [P2-SA]  "DSpark.让每一轮计算，多走几步", semi-autoregressive section and its
 *            Markov-head example (base scores 0, 0 plus ln 9 -> 50% to 90%).
 *   [P2-SCH] same page, "写得长，不如验得值" section: survival products
 *            a_j = c_1 x ... x c_j, global descending sort, greedy admission
 *            while the expected output rate rises.
 *   [P2-LL]  same page, lossless section: accept / residual max(p - q, 0) /
 *            bonus token when the whole block is accepted.
 *   [P4-2.1] "DeepSeek联合北大最新文章DSpark", section 2.1 confidence head
 *            c_k = sigma(w^T [h_k; W1[x_{k-1}]]) and sequential temperature
 *            scaling.
 *   [P4-2.2] same page, section 2.2 hardware-aware prefix scheduler:
 *            max over l of Theta = tau * SPS(B), B = sum_r (1 + l_r),
 *            tau = sum_r sum_{j<=l_r} a_{r,j}; greedy sort + early stop.
 *   [P4-SEQ] same page, "第二阶段轻量顺序头": the Markov head injects the
 *            previous token into the next position's distribution through a
 *            low-rank matrix.
 *   [P5-PROOF] "为什么DSpark 可以加速推理？", section "投机解码在数学上会不会
 *            影响最终生成结果": acceptance min(1, p/q), total acceptance
 *            sum min(p, q), residual max(0, p - q) / sum max(0, p - q).
 *   [P1-SEQ] "DeepSeek DSpark：Confidence-Scheduled Speculative Decoding
 *            技术解析", section 四: only the previous token id is passed forward.
 * The random source is Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel
 * random numbers: as easy as 1, 2, 3", SC'11); the pages leave the generator
 * open.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------- */
/* Philox4x32-10 from its published definition.                              */
/* ------------------------------------------------------------------------- */

static void philox_one_round(uint32_t c[4], const uint32_t k[2])
{
    /* Two 32x32->64 products; the S-box mixes high halves with the key. */
    const uint64_t p0 = (uint64_t)0xD2511F53u * (uint64_t)c[0];
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * (uint64_t)c[2];
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    const uint32_t n0 = hi1 ^ c[1] ^ k[0];
    const uint32_t n1 = lo1;
    const uint32_t n2 = hi0 ^ c[3] ^ k[1];
    const uint32_t n3 = lo0;
    c[0] = n0; c[1] = n1; c[2] = n2; c[3] = n3;
}

void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t c[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
    uint32_t k[2] = {key[0], key[1]};
    for (int i = 0; i < 10; ++i) {
        philox_one_round(c, k);
        /* Weyl key schedule: golden ratio and sqrt(3)-1 in 32-bit fixed point. */
        k[0] += 0x9E3779B9u;
        k[1] += 0xBB67AE85u;
    }
    memcpy(out, c, sizeof(c));
}

/* u in [0, 1): top 24 bits of word 0 of Philox(counter = (round, request,
 * position, purpose), key = seed). Exact in fp32 and fp64. */
double orc_uniform(uint64_t seed, uint32_t round, uint32_t req, uint32_t pos, uint32_t purpose)
{
    const uint32_t ctr[4] = {round, req, pos, purpose};
    const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t out[4];
    orc_philox4x32_10(ctr, key, out);
    return (double)(out[0] >> 8) * (1.0 / 16777216.0);
}

enum { PURPOSE_DRAFT = 0, PURPOSE_ACCEPT = 1, PURPOSE_RESAMPLE = 2 };
enum { DT_F32 = 0, DT_BF16 = 1 };

/* ------------------------------------------------------------------------- */
/* Element access                                                            */
/* ------------------------------------------------------------------------- */

static float bf16_to_float(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof(f));
    return f;
}

static float logit_at(const void* p, int dtype, size_t idx)
{
    if (dtype == DT_F32) return ((const float*)p)[idx];
    return bf16_to_float(((const uint16_t*)p)[idx]);
}

/* fp32 unit in the last place of |x| (x finite). */
static double ulp32(float x)
{
    float ax = fabsf(x);
    return (double)nextafterf(ax, INFINITY) - (double)ax;
}

/* ------------------------------------------------------------------------- */
/* Markov head [P4-SEQ], [P2-SA]: biased logits of one draft row.            */
/*   bias_v  = sum_i E[prev, i] * W2(i, v)   (exact-order fp64, one rounding) */
/*   logit_v = fl32(base_v + fl32(bias_v))                                    */
/* W2(i, v) is stored at W2[v * r + i].  A prev outside [0, V) (-1 before   */
/* any token) selects no embedding row: "no Markov bias".                    */
/* absdot[v] (optional) receives sum_i |E[prev,i] * W2(i,v)|, the magnitude   */
/* that bounds any fp32 summation-order difference of the bias.              */
/* ------------------------------------------------------------------------- */

int orc_markov_logits(int V, int r, const void* base_row, int dtype,
                      const uint16_t* E, const uint16_t* W2, int prev,
                      float* logit, double* absdot)
{
    if (V <= 0 || r <= 0) return 1;
    for (int v = 0; v < V; ++v) {
        double s = 0.0, sa = 0.0;
        if (prev >= 0 && prev < V) {
            for (int i = 0; i < r; ++i) {
                const double t = (double)bf16_to_float(E[(size_t)prev * r + i]) *
                                 (double)bf16_to_float(W2[(size_t)v * r + i]);
                s += t;
                sa += fabs(t);
            }
        }
        const float bias = (float)s;
        logit[v] = logit_at(base_row, dtype, (size_t)v) + bias;
        if (absdot) absdot[v] = sa;
    }
    return 0;
}

/* The same logits from an explicit bias row (r bf16 values; NULL: no bias):
 * the Markov head passes E[prev], the recurrent head its state row. */
static void head_logits(int V, int r, const void* base_row, int dtype, const uint16_t* row,
                        const uint16_t* W2, float* logit, double* absdot)
{
    for (int v = 0; v < V; ++v) {
        double s = 0.0, sa = 0.0;
        if (row) {
            for (int i = 0; i < r; ++i) {
                const double t = (double)bf16_to_float(row[i]) *
                                 (double)bf16_to_float(W2[(size_t)v * r + i]);
                s += t;
                sa += fabs(t);
            }
        }
        const float bias = (float)s;
        logit[v] = logit_at(base_row, dtype, (size_t)v) + bias;
        if (absdot) absdot[v] = sa;
    }
}

/* ------------------------------------------------------------------------- */
/* Recurrent sequential head [P4-SEQ] (the pages name an RNN head that keeps */
/* a recurrent state to capture longer dependencies, without its form).      */
/* This library's reading, an Elman recurrence on the Markov head's rank-r   */
/* space:                                                                    */
/*   s_{-1} = 0;  u_k = A s_{k-1} + E[x_{k-1}]  (fp64; no E term when x is   */
/*   outside [0, V));  s_k = bf16(tanh(u_k))  (round to nearest even)        */
/* and the bias of position k is s_k . W2 like the Markov head's E[x_{k-1}]. */
/* A is [r, r] bf16, element (i, j) at A[i r + j] (row i gives output i).    */
/* With A = 0 the head is the Markov head on bf16(tanh(E)).                  */
/* *flag = 1 when some tanh(u_i) lies within 1e-12 (relative) of a bf16      */
/* rounding midpoint (where a differently rounded tanh may round the other   */
/* way).                                                                     */
/* ------------------------------------------------------------------------- */

static uint16_t bf16_rne(double x, int8_t* near)
{
    const float f = (float)x;   /* exact for the tanh values tested: see flag */
    uint32_t u;
    memcpy(&u, &f, sizeof(u));
    /* candidates: truncation and the next bf16 value up in magnitude */
    const uint32_t lo = u & 0xFFFF0000u, hi = lo + 0x10000u;
    float flo, fhi;
    memcpy(&flo, &lo, sizeof(flo));
    memcpy(&fhi, &hi, sizeof(fhi));
    const double dlo = fabs(x - (double)flo), dhi = fabs((double)fhi - x);
    uint32_t pick;
    if (dlo < dhi) pick = lo;
    else if (dhi < dlo) pick = hi;
    else pick = ((lo >> 16) & 1u) ? hi : lo;   /* tie: even mantissa */
    const double mid = 0.5 * ((double)flo + (double)fhi);
    if (near && fabs(x - mid) <= 1e-12 * fabs(x)) *near = 1;
    return (uint16_t)(pick >> 16);
}

int orc_rnn_state(int V, int r, const uint16_t* A, const uint16_t* E, int prev,
                  const uint16_t* s_prev, uint16_t* s_out, int8_t* flag)
{
    if (V <= 0 || r <= 0) return 1;
    int8_t fl = 0;
    for (int i = 0; i < r; ++i) {
        double u = 0.0;
        if (s_prev)
            for (int j = 0; j < r; ++j)
                u += (double)bf16_to_float(A[(size_t)i * r + j]) * (double)bf16_to_float(s_prev[j]);
        if (prev >= 0 && prev < V) u += (double)bf16_to_float(E[(size_t)prev * r + i]);
        s_out[i] = bf16_rne(tanh(u), &fl);
    }
    if (flag) *flag = fl;
    return 0;
}

/* Tempered softmax in fp64: M = max logit, prob_v = exp((logit_v - M) / T) / Z
 * with Z = sum_v exp((logit_v - M) / T).  stats = (M, Z). */
int orc_softmax(int V, const float* logit, double temperature, double* prob, double* stats)
{
    if (V <= 0 || !(temperature > 0.0)) return 1;
    double M = -INFINITY;
    for (int v = 0; v < V; ++v)
        if ((double)logit[v] > M) M = (double)logit[v];
    double Z = 0.0;
    for (int v = 0; v < V; ++v) {
        prob[v] = exp(((double)logit[v] - M) / temperature);
        Z += prob[v];
    }
    for (int v = 0; v < V; ++v) prob[v] /= Z;
    if (stats) { stats[0] = M; stats[1] = Z; }
    return 0;
}

/* Inverse CDF over unnormalised non-negative weights w[0..V):
 *   x = min { v : sum_{i<=v} w_i > u * sum w }.
 * If rounding leaves no such v, the last v with w_v > 0.
 * *near = 1 when u lies within `win` of the normalised CDF on either side of
 * the chosen cell (a decision fp32 rounding elsewhere could flip). */
int orc_inverse_cdf(int V, const double* w, double u, double win, int* near)
{
    double Z = 0.0;
    for (int v = 0; v < V; ++v) Z += w[v];
    const double t = u * Z;
    double cum = 0.0, prev_cum = 0.0;
    int x = -1;
    for (int v = 0; v < V; ++v) {
        prev_cum = cum;
        cum += w[v];
        if (cum > t) { x = v; break; }
    }
    if (x < 0) {
        for (int v = V - 1; v >= 0; --v)
            if (w[v] > 0.0) { x = v; break; }
        if (near) *near = 1;
        return x;
    }
    if (near) {
        const double lo = prev_cum / Z, hi = cum / Z;
        *near = (u - lo < win) || (hi - u < win);
    }
    return x;
}

/* Lowest index of the maximum. */
static int argmax_f32(int V, const float* x)
{
    int best = 0;
    for (int v = 1; v < V; ++v)
        if (x[v] > x[best]) best = v;
    return best;
}

#define SAMPLE_WINDOW 1e-6
#define ACCEPT_WINDOW 1e-6

/* ------------------------------------------------------------------------- */
/* Semi-autoregressive draft [P1-SEQ], [P2-SA], [P4-SEQ].                     */
/* For each request (compact row i, Philox request id req_id[i]) and draft    */
/* position k = 0..gamma-1, sequentially over k:                             */
/*   prev = anchor (k = 0) else x_{k-1}; logits via the Markov head;         */
/*   greedy (temperature == 0): x_k = argmax, q = 1;                         */
/*   sampling: x_k = inverse CDF of softmax(logits / T) at u(seed, round,     */
/*   req, k, purpose 0); q = prob of x_k; stats = (max logit, Z).            */
/* flag[i,k] = 1 when the decision is within rounding reach of a boundary:   */
/*   sampling: u within 1e-6 of the CDF on either side of x_k;               */
/*   greedy: top-2 logit gap within the bias summation bound plus 2 ulp.     */
/* force (optional, [n, gamma]): where force[i,k] >= 0 the chain continues   */
/* from that token instead of its own draw (q and stats are still those of   */
/* this row's law, q = prob of the forced token).  This is how a comparison  */
/* adopts the other side's choice at a flagged decision, so that the later   */
/* positions of the chain stay comparable; flag is computed as usual.        */
/* ------------------------------------------------------------------------- */

/* A (optional): the recurrent head with recurrent matrix A; its states go to */
/* S [n, gamma, r] bf16 and sflag [n, gamma] marks a state with a            */
/* near-midpoint element (orc_rnn_state).                                    */
int orc_draft(int n, int gamma, int V, int r,
              const void* base, int dtype, const uint16_t* E, const uint16_t* W2,
              const int32_t* anchor, const int32_t* req_id,
              double temperature, uint64_t seed, uint32_t round,
              int32_t* tok, double* q, double* stats, int8_t* flag,
              const int32_t* force, const uint16_t* A, uint16_t* S, int8_t* sflag)
{
    if (n < 0 || gamma <= 0 || V <= 0 || r <= 0 || temperature < 0.0) return 1;
    float* logit = (float*)malloc(sizeof(float) * (size_t)V);
    double* absdot = (double*)malloc(sizeof(double) * (size_t)V);
    double* prob = (double*)malloc(sizeof(double) * (size_t)V);
    if (!logit || !absdot || !prob) { free(logit); free(absdot); free(prob); return 2; }
    const int greedy = (temperature == 0.0);
    for (int i = 0; i < n; ++i) {
        int prev = anchor[i];
        for (int k = 0; k < gamma; ++k) {
            const size_t row = ((size_t)i * gamma + k) * (size_t)V;
            const size_t ik = (size_t)i * gamma + k;
            const void* brow = (dtype == DT_F32) ? (const void*)((const float*)base + row)
                                                 : (const void*)((const uint16_t*)base + row);
            if (A) {
                uint16_t* srow = S + ik * (size_t)r;
                orc_rnn_state(V, r, A, E, prev, k > 0 ? srow - r : NULL, srow, &sflag[ik]);
                head_logits(V, r, brow, dtype, srow, W2, logit, absdot);
            } else {
                orc_markov_logits(V, r, brow, dtype, E, W2, prev, logit, absdot);
            }
            int x;
            int8_t fl = 0;
            if (greedy) {
                x = argmax_f32(V, logit);
                /* runner-up */
                int second = -1;
                for (int v = 0; v < V; ++v)
                    if (v != x && (second < 0 || logit[v] > logit[second])) second = v;
                if (second >= 0) {
                    const double gap = (double)logit[x] - (double)logit[second];
                    const double eps = ldexp(1.0, -24);
                    const double bound = 2.0 * ulp32(logit[x]) +
                                         (double)(r + 1) * eps * (absdot[x] + absdot[second]);
                    fl = gap <= bound;
                }
                stats[2 * ik] = (double)logit[x];
                if (force && force[ik] >= 0 && force[ik] < V) x = force[ik];
                q[ik] = 1.0;
                stats[2 * ik + 1] = 0.0;
            } else {
                double st[2];
                orc_softmax(V, logit, temperature, prob, st);
                const double u = orc_uniform(seed, round, (uint32_t)req_id[i], (uint32_t)k,
                                             PURPOSE_DRAFT);
                int near = 0;
                x = orc_inverse_cdf(V, prob, u, SAMPLE_WINDOW, &near);
                fl = (int8_t)near;
                if (force && force[ik] >= 0 && force[ik] < V) x = force[ik];
                q[ik] = prob[x];
                stats[2 * ik] = st[0];
                stats[2 * ik + 1] = st[1];
            }
            tok[ik] = x;
            flag[ik] = fl;
            prev = x;
        }
    }
    free(logit); free(absdot); free(prob);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Confidence head + sequential temperature scaling [P4-2.1].                */
/*   y   = sum_{i<d} w_i h[k,i] + sum_{i<r} w_{d+i} E[prev,i]   (fp64)        */
/*   c_k = 1 / (1 + exp(-(y + offset) / T_k))                                */
/* prev = anchor for k = 0, else x_{k-1}; prev outside [0, V) drops the E   */
/* term.                                                                     */
/* flag = 1 when c lies within 1e-12 (relative) of an fp32 rounding          */
/* midpoint, i.e. fp32 rounding of a differently ordered sum may differ.     */
/* ------------------------------------------------------------------------- */

int orc_confidence(int n, int gamma, int d, int V, int r,
                   const uint16_t* h, const uint16_t* E,
                   const int32_t* anchor, const int32_t* tok,
                   const float* w, const float* T, const float* offset,
                   double* c, int8_t* flag)
{
    if (n < 0 || gamma <= 0 || d < 0 || r <= 0 || V <= 0) return 1;
    for (int i = 0; i < n; ++i) {
        for (int k = 0; k < gamma; ++k) {
            const size_t ik = (size_t)i * gamma + k;
            const int prev = (k == 0) ? anchor[i] : tok[ik - 1];
            double y = 0.0;
            for (int t = 0; t < d; ++t)
                y += (double)w[t] * (double)bf16_to_float(h[ik * (size_t)d + t]);
            if (prev >= 0 && prev < V)
                for (int t = 0; t < r; ++t)
                    y += (double)w[d + t] * (double)bf16_to_float(E[(size_t)prev * r + t]);
            if (offset) y += (double)offset[i];
            const double cc = 1.0 / (1.0 + exp(-y / (double)T[k]));
            c[ik] = cc;
            const float f = (float)cc;
            const double lo = 0.5 * ((double)f + (double)nextafterf(f, -INFINITY));
            const double hi = 0.5 * ((double)f + (double)nextafterf(f, INFINITY));
            const double tol = 1e-12 * fabs(cc);
            flag[ik] = (fabs(cc - lo) <= tol) || (fabs(cc - hi) <= tol);
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Hardware-aware prefix scheduler [P2-SCH], [P4-2.2].                       */
/*   a_{r,j}  = fl32(a_{r,j-1} * c_{r,j}), a_{r,-1} = 1 (left to right)      */
/*   candidates sorted by a descending, then r ascending, then j ascending   */
/*   tau_n    = tau0 + sum of the n best a, each truncated to 2^-48          */
/*              (exact fixed point: equal to the real sum for a >= 2^-25)    */
/*   Theta_n  = fl64(tau_n) * SPS(R + n)                                     */
/*   admit candidates while Theta strictly rises and R + n <= B_max          */
/*   l_r      = admitted candidates of request r; B = R + sum l_r            */
/* mode 0: every position verified, l_r = gamma.                             */
/* ------------------------------------------------------------------------- */

typedef struct { float a; int r, j; } cand_t;

static int cand_cmp(const void* pa, const void* pb)
{
    const cand_t* x = (const cand_t*)pa;
    const cand_t* y = (const cand_t*)pb;
    if (x->a > y->a) return -1;
    if (x->a < y->a) return 1;
    if (x->r != y->r) return x->r < y->r ? -1 : 1;
    if (x->j != y->j) return x->j < y->j ? -1 : 1;
    return 0;
}

int orc_schedule(int R, int gamma, const float* c, const float* sps, int B_max,
                 double tau0, int mode, int32_t* len, float* a, int32_t* B_out,
                 int32_t* n_theta_evals)
{
    /* tau0 < 2^14 keeps tau0 * 2^48 plus the admitted sum (below R gamma 2^48,
     * R gamma <= 2^14) inside 64 bits */
    if (R <= 0 || gamma <= 0 || B_max < R || !(tau0 >= 0.0) || !(tau0 < 16384.0)) return 1;
    if ((int64_t)R * gamma > 16384 && mode != 0) return 1;
    for (int r = 0; r < R; ++r) {
        float prod = 1.0f;
        for (int j = 0; j < gamma; ++j) {
            prod = prod * c[(size_t)r * gamma + j];
            a[(size_t)r * gamma + j] = prod;
        }
    }
    if (mode == 0) {
        for (int r = 0; r < R; ++r) len[r] = gamma;
        *B_out = R * (1 + gamma);
        if (n_theta_evals) *n_theta_evals = 0;
        return 0;
    }
    const size_t N = (size_t)R * gamma;
    cand_t* cs = (cand_t*)malloc(sizeof(cand_t) * N);
    if (!cs) return 2;
    for (int r = 0; r < R; ++r)
        for (int j = 0; j < gamma; ++j) {
            cand_t* t = &cs[(size_t)r * gamma + j];
            t->a = a[(size_t)r * gamma + j]; t->r = r; t->j = j;
        }
    qsort(cs, N, sizeof(cand_t), cand_cmp);

    const double scale = ldexp(1.0, 48);
    uint64_t S = (uint64_t)floor(tau0 * scale);
    double theta_prev = ((double)S / scale) * (double)sps[R - 1];
    for (int r = 0; r < R; ++r) len[r] = 0;
    size_t n = 0;
    int evals = 0;
    while (n < N && (size_t)R + n + 1 <= (size_t)B_max) {
        const uint64_t A = (uint64_t)floor((double)cs[n].a * scale);
        const uint64_t S_next = S + A;
        const double theta = ((double)S_next / scale) * (double)sps[R + n];
        ++evals;
        if (!(theta > theta_prev)) break;
        len[cs[n].r] += 1;
        S = S_next;
        theta_prev = theta;
        ++n;
    }
    *B_out = R + (int32_t)n;
    if (n_theta_evals) *n_theta_evals = evals;
    free(cs);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Lossless verification [P2-LL], [P5-PROOF].                                */
/* Per request with l = len[i]:                                              */
/*   p_j = softmax(target row j / T) for j < l; accept_j iff                 */
/*     sampling: u(seed, round, req, j, purpose 1) <= min(1, p_j(x_j)/q_j)   */
/*     greedy:   x_j == argmax target row j                                  */
/*   n = first j < l that is not accepted, else l                            */
/*   n < l: sampling: y ~ max(0, p_n - q_n) normalised, q_n the full draft   */
/*          row at position n (recomputed through the Markov head); if that  */
/*          mass is zero, y ~ p_n.  greedy: y = argmax target row n          */
/*   n = l: bonus y ~ p_l (target row l); greedy: argmax                     */
/*   both draws use u(seed, round, req, n, purpose 2).                       */
/* accept[i,j] is 1/0 for j < l and -1 for unverified positions.            */
/* flag_acc marks |u - p/q| < 1e-6; flag_y marks a near-boundary draw of y.  */
/* force_acc (optional, [n, gamma]): where force_acc[i,j] is 0 or 1 that     */
/* decision is adopted instead of this side's (a comparison taking the other */
/* side's choice at a flagged accept test); -1 leaves it alone.              */
/* ------------------------------------------------------------------------- */

int orc_verify(int n_req, int gamma, int V, int r,
               const void* target, const void* base, int dtype,
               const uint16_t* E, const uint16_t* W2,
               const int32_t* anchor, const int32_t* tok, const double* q,
               const int32_t* len, const int32_t* req_id,
               double temperature, uint64_t seed, uint32_t round,
               int8_t* accept, int32_t* n_accept, int32_t* y, double* p_out,
               int8_t* flag_acc, int8_t* flag_y, const int8_t* force_acc, const uint16_t* S)
{
    if (n_req < 0 || gamma <= 0 || V <= 0 || r <= 0 || temperature < 0.0) return 1;
    float* tl = (float*)malloc(sizeof(float) * (size_t)V);
    float* dl = (float*)malloc(sizeof(float) * (size_t)V);
    double* pt = (double*)malloc(sizeof(double) * (size_t)V);
    double* pd = (double*)malloc(sizeof(double) * (size_t)V);
    if (!tl || !dl || !pt || !pd) { free(tl); free(dl); free(pt); free(pd); return 2; }
    const int greedy = (temperature == 0.0);
    for (int i = 0; i < n_req; ++i) {
        const int l = len[i];
        if (l < 0 || l > gamma) { free(tl); free(dl); free(pt); free(pd); return 1; }
        const uint32_t rid = (uint32_t)req_id[i];
        int n = l;
        for (int j = 0; j < gamma; ++j) {
            const size_t ij = (size_t)i * gamma + j;
            flag_acc[ij] = 0;
            if (j >= l) { accept[ij] = -1; p_out[ij] = 0.0; continue; }
            const size_t trow = ((size_t)i * (gamma + 1) + j) * (size_t)V;
            for (int v = 0; v < V; ++v) tl[v] = logit_at(target, dtype, trow + v);
            const int x = tok[ij];
            int acc;
            if (greedy) {
                acc = (x == argmax_f32(V, tl));
                p_out[ij] = acc ? 1.0 : 0.0;
            } else {
                orc_softmax(V, tl, temperature, pt, NULL);
                const double px = pt[x];
                const double u = orc_uniform(seed, round, rid, (uint32_t)j, PURPOSE_ACCEPT);
                const double ratio = px / q[ij];
                acc = (u <= (ratio < 1.0 ? ratio : 1.0));
                p_out[ij] = px;
                flag_acc[ij] = fabs(u - ratio) < ACCEPT_WINDOW;
            }
            if (force_acc && (force_acc[ij] == 0 || force_acc[ij] == 1)) acc = force_acc[ij];
            accept[ij] = (int8_t)acc;
            if (!acc && n == l) n = j;
        }
        n_accept[i] = n;
        /* correction (n < l) or bonus (n == l) token from row n */
        const size_t trow = ((size_t)i * (gamma + 1) + n) * (size_t)V;
        for (int v = 0; v < V; ++v) tl[v] = logit_at(target, dtype, trow + v);
        int near = 0;
        if (greedy) {
            y[i] = argmax_f32(V, tl);
        } else {
            const double u = orc_uniform(seed, round, rid, (uint32_t)n, PURPOSE_RESAMPLE);
            orc_softmax(V, tl, temperature, pt, NULL);
            if (n < l) {
                const int prev = (n == 0) ? anchor[i] : tok[(size_t)i * gamma + n - 1];
                const size_t drow = ((size_t)i * gamma + n) * (size_t)V;
                const void* brow = (dtype == DT_F32) ? (const void*)((const float*)base + drow)
                                                     : (const void*)((const uint16_t*)base + drow);
                /* the draft law of position n: Markov row E[prev], or the
                   recurrent head's state row S[i, n] */
                if (S) head_logits(V, r, brow, dtype, S + ((size_t)i * gamma + n) * (size_t)r, W2,
                                   dl, NULL);
                else orc_markov_logits(V, r, brow, dtype, E, W2, prev, dl, NULL);
                orc_softmax(V, dl, temperature, pd, NULL);
                double mass = 0.0;
                for (int v = 0; v < V; ++v) {
                    const double d = pt[v] - pd[v];
                    pd[v] = d > 0.0 ? d : 0.0;
                    mass += pd[v];
                }
                y[i] = (mass > 0.0) ? orc_inverse_cdf(V, pd, u, SAMPLE_WINDOW, &near)
                                    : orc_inverse_cdf(V, pt, u, SAMPLE_WINDOW, &near);
            } else {
                y[i] = orc_inverse_cdf(V, pt, u, SAMPLE_WINDOW, &near);
            }
        }
        flag_y[i] = (int8_t)near;
    }
    free(tl); free(dl); free(pt); free(pd);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Exact acceptance probability of each draft position [P5-PROOF], which is   */
/* also the total-variation target of the confidence head [P4-2.1]:          */
/*   alpha[i,k] = sum_v min(q_k(v), p_k(v)) = 1 - (1/2) sum_v |q_k(v) - p_k(v)| */
/* q_k the draft law at position k (Markov head with prev = anchor for k = 0, */
/* else x_{k-1} = tok[i,k-1]), p_k = softmax(target row k / T).  Both laws in */
/* fp64 from the fp32 logits; sampling temperatures only (T > 0).             */
/* ------------------------------------------------------------------------- */

int orc_tv_accept(int n, int gamma, int V, int r, const void* target, const void* base, int dtype,
                  const uint16_t* E, const uint16_t* W2, const int32_t* anchor,
                  const int32_t* tok, double temperature, double* alpha, const uint16_t* S)
{
    if (n < 0 || gamma <= 0 || V <= 0 || r <= 0 || !(temperature > 0.0)) return 1;
    float* tl = (float*)malloc(sizeof(float) * (size_t)V);
    float* dl = (float*)malloc(sizeof(float) * (size_t)V);
    double* pt = (double*)malloc(sizeof(double) * (size_t)V);
    double* pd = (double*)malloc(sizeof(double) * (size_t)V);
    if (!tl || !dl || !pt || !pd) { free(tl); free(dl); free(pt); free(pd); return 2; }
    for (int i = 0; i < n; ++i) {
        for (int k = 0; k < gamma; ++k) {
            const size_t trow = ((size_t)i * (gamma + 1) + k) * (size_t)V;
            for (int v = 0; v < V; ++v) tl[v] = logit_at(target, dtype, trow + v);
            orc_softmax(V, tl, temperature, pt, NULL);
            const int prev = (k == 0) ? anchor[i] : tok[(size_t)i * gamma + k - 1];
            const size_t drow = ((size_t)i * gamma + k) * (size_t)V;
            const void* brow = (dtype == DT_F32) ? (const void*)((const float*)base + drow)
                                                 : (const void*)((const uint16_t*)base + drow);
            if (S) head_logits(V, r, brow, dtype, S + ((size_t)i * gamma + k) * (size_t)r, W2, dl,
                               NULL);
            else orc_markov_logits(V, r, brow, dtype, E, W2, prev, dl, NULL);
            orc_softmax(V, dl, temperature, pd, NULL);
            double a = 0.0;
            for (int v = 0; v < V; ++v) a += (pd[v] < pt[v]) ? pd[v] : pt[v];
            alpha[(size_t)i * gamma + k] = a;
        }
    }
    free(tl); free(dl); free(pt); free(pd);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Asynchronous scheduler with a capacity barrier ("DeepSeek联合北大最新文章  */
/* DSpark", 挑战2 异步调度与 ZOS 兼容; "DSpark.让每一轮计算，多走几步", the     */
/* causality paragraph of 两个严谨补丁).                                     */
/*   capacity: from the confidences of an earlier round (c_hist), the same   */
/*     survival products, order and Q48 sums as orc_schedule, then the       */
/*     global maximum of Theta_n = tau_n SPS(R + n) over every n with        */
/*     R + n <= B_max and n <= R gamma -- no early stop; the smallest such n */
/*     on ties:  K = argmax_n Theta_n.                                       */
/*   admission: the current survival products (from c) in the same order;    */
/*     the first K candidates are admitted; l_r = admitted candidates of r;  */
/*     B = R + K.                                                            */
/* ------------------------------------------------------------------------- */

static void survival_and_order(int R, int gamma, const float* c, float* a, cand_t* cs)
{
    for (int r = 0; r < R; ++r) {
        float prod = 1.0f;
        for (int j = 0; j < gamma; ++j) {
            prod = prod * c[(size_t)r * gamma + j];
            a[(size_t)r * gamma + j] = prod;
        }
    }
    for (int r = 0; r < R; ++r)
        for (int j = 0; j < gamma; ++j) {
            cand_t* t = &cs[(size_t)r * gamma + j];
            t->a = a[(size_t)r * gamma + j]; t->r = r; t->j = j;
        }
    qsort(cs, (size_t)R * gamma, sizeof(cand_t), cand_cmp);
}

int orc_schedule_async(int R, int gamma, const float* c, const float* c_hist, const float* sps,
                       int B_max, double tau0, int32_t* len, float* a, int32_t* B_out,
                       int32_t* K_out)
{
    if (R <= 0 || gamma <= 0 || B_max < R || !(tau0 >= 0.0) || !(tau0 < 16384.0)) return 1;
    if ((int64_t)R * gamma > 16384) return 1;
    const size_t N = (size_t)R * gamma;
    cand_t* cs = (cand_t*)malloc(sizeof(cand_t) * N);
    float* ah = (float*)malloc(sizeof(float) * N);
    if (!cs || !ah) { free(cs); free(ah); return 2; }
    /* capacity from the earlier round's confidences */
    survival_and_order(R, gamma, c_hist, ah, cs);
    const double scale = ldexp(1.0, 48);
    uint64_t S = (uint64_t)floor(tau0 * scale);
    double best = (double)S / scale * (double)sps[R - 1];
    size_t K = 0;
    const size_t n_max = (N < (size_t)(B_max - R)) ? N : (size_t)(B_max - R);
    for (size_t n = 1; n <= n_max; ++n) {
        S += (uint64_t)floor((double)cs[n - 1].a * scale);
        const double theta = ((double)S / scale) * (double)sps[R + n - 1];
        if (theta > best) { best = theta; K = n; }
    }
    /* admission by the current confidences */
    survival_and_order(R, gamma, c, a, cs);
    for (int r = 0; r < R; ++r) len[r] = 0;
    for (size_t n = 0; n < K; ++n) len[cs[n].r] += 1;
    *B_out = R + (int32_t)K;
    *K_out = (int32_t)K;
    free(cs); free(ah);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Confidence logit [P4-2.1]: the argument of the sigmoid before the         */
/* per-position temperature, y = w . [h_k; E[x_{k-1}]] + offset (fp64).       */
/* ------------------------------------------------------------------------- */

int orc_confidence_logit(int n, int gamma, int d, int V, int r,
                         const uint16_t* h, const uint16_t* E,
                         const int32_t* anchor, const int32_t* tok,
                         const float* w, const float* offset, double* y_out)
{
    if (n < 0 || gamma <= 0 || d < 0 || r <= 0 || V <= 0) return 1;
    for (int i = 0; i < n; ++i) {
        for (int k = 0; k < gamma; ++k) {
            const size_t ik = (size_t)i * gamma + k;
            const int prev = (k == 0) ? anchor[i] : tok[ik - 1];
            double y = 0.0;
            for (int t = 0; t < d; ++t)
                y += (double)w[t] * (double)bf16_to_float(h[ik * (size_t)d + t]);
            if (prev >= 0 && prev < V)
                for (int t = 0; t < r; ++t)
                    y += (double)w[d + t] * (double)bf16_to_float(E[(size_t)prev * r + t]);
            if (offset) y += (double)offset[i];
            y_out[ik] = y;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Sequential temperature scaling [P4-2.1], [P2-SCH] (calibration of the      */
/* cumulative prefix survival on held-out data, position by position from     */
/* left to right).  Reading: sample n of the held-out set carries the raw     */
/* confidence logits z[n, k] and the number of its draft tokens accepted,     */
/* acc[n] (every position verified); s[n, k] = 1 when acc[n] > k, i.e. the    */
/* prefix through position k survived.  With beta_j = 1 / T_j,                */
/*   a[n, k] = prod_{j <= k} sigma(beta_j z[n, j])   (a[n, -1] = 1)           */
/* and T_k, with T_0 .. T_{k-1} already fixed, minimises the binary cross-   */
/* entropy of a[n, k] against s[n, k] over all n:                            */
/*   F_k(beta) = - sum_n [ s ln(a_{k-1} sigma(beta z))                        */
/*                       + (1 - s) ln(1 - a_{k-1} sigma(beta z)) ]            */
/* The minimiser is searched on two grids of G values of beta, each point     */
/* fma(g, step, lo) in fp64: first [1 / t_hi, 1 / t_lo], then the span of the */
/* first grid's best point and its two neighbours; the lowest index wins a    */
/* tie and a NaN objective counts as +inf.  ln a and b = 1 - a are carried    */
/* separately, so that neither is formed by cancellation:                     */
/*   s = 1: -ln(a sigma(x))     = -(ln a + ln sigma(x))                       */
/*   s = 0: -ln(1 - a sigma(x)) = -ln(b + a sigma(-x))                        */
/*   ln sigma(x) = -(max(-x, 0) + log1p(exp(-|x|)))                          */
/* ------------------------------------------------------------------------- */

static double log_sigmoid(double x) { return -(fmax(-x, 0.0) + log1p(exp(-fabs(x)))); }

static double survival_bce(double x, int s, double la, double b)
{
    if (s) return -(la + log_sigmoid(x));
    return -log(b + exp(la + log_sigmoid(-x)));
}

static double sts_objective(int N, int gamma, int k, const float* z, const int32_t* acc,
                            const double* la, const double* b, double beta)
{
    double f = 0.0;
    for (int n = 0; n < N; ++n)
        f += survival_bce(beta * (double)z[(size_t)n * gamma + k], acc[n] > k, la[n], b[n]);
    return f;
}

/* best of G grid points lo + g step; gap = (second best - best) / |best| */
static int sts_grid_argmin(int N, int gamma, int k, const float* z, const int32_t* acc,
                           const double* la, const double* b, int G, double lo, double step,
                           double* f_best, double* gap)
{
    int best = 0;
    double fb = INFINITY, f2 = INFINITY;
    for (int g = 0; g < G; ++g) {
        double f = sts_objective(N, gamma, k, z, acc, la, b, fma((double)g, step, lo));
        if (isnan(f)) f = INFINITY;
        if (f < fb) {
            f2 = fb;
            fb = f;
            best = g;
        } else if (f < f2) {
            f2 = f;
        }
    }
    *f_best = fb;
    *gap = (f2 - fb) / fabs(fb);
    return best;
}

int orc_sts_fit(int N, int gamma, const float* z, const int32_t* acc, double t_lo, double t_hi,
                int G, double* beta_out, double* nll_out, double* gap_out)
{
    if (N <= 0 || gamma <= 0 || G < 2 || !(t_lo > 0.0) || !(t_hi > t_lo)) return 1;
    double* la = (double*)calloc((size_t)N, sizeof(double));
    double* b = (double*)calloc((size_t)N, sizeof(double));
    if (!la || !b) { free(la); free(b); return 2; }
    const double lo1 = 1.0 / t_hi, hi1 = 1.0 / t_lo;
    const double step1 = (hi1 - lo1) / (double)(G - 1);
    for (int k = 0; k < gamma; ++k) {
        double f1, g1gap, f2, g2gap;
        const int g1 = sts_grid_argmin(N, gamma, k, z, acc, la, b, G, lo1, step1, &f1, &g1gap);
        const double lo2 = fma((double)(g1 > 0 ? g1 - 1 : 0), step1, lo1);
        const double hi2 = fma((double)(g1 < G - 1 ? g1 + 1 : G - 1), step1, lo1);
        const double step2 = (hi2 - lo2) / (double)(G - 1);
        const int g2 = sts_grid_argmin(N, gamma, k, z, acc, la, b, G, lo2, step2, &f2, &g2gap);
        const double beta = fma((double)g2, step2, lo2);
        beta_out[k] = beta;
        nll_out[k] = f2;
        gap_out[2 * k] = g1gap;
        gap_out[2 * k + 1] = g2gap;
        /* carry the survival through position k with the fitted temperature */
        for (int n = 0; n < N; ++n) {
            const double x = beta * (double)z[(size_t)n * gamma + k];
            const double la_new = la[n] + log_sigmoid(x);
            b[n] = b[n] + exp(la[n] + log_sigmoid(-x));
            la[n] = la_new;
        }
    }
    free(la);
    free(b);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Expected calibration error of the cumulative survival [P4-2.1] (the page  */
/* reports ECE before and after temperature scaling).  Reading: every pair   */
/* (n, k) is one prediction a[n, k] = prod_{j <= k} sigma(z[n, j] / T_j)      */
/* (T = NULL: T_j = 1) of the outcome s[n, k] = (acc[n] > k); predictions     */
/* fall in M equal-width bins, bin = min(floor(a M), M - 1), and             */
/*   ECE = sum_bins |sum_{bin} (s - a)| / (N gamma)                           */
/* i.e. the bin-size-weighted gap between the bin's accept rate and its mean  */
/* prediction.  sigma(x) = exp(ln sigma(x)).  n_edge counts the predictions   */
/* within 1e-9 of a bin edge (where another rounding may pick the next bin).  */
/* ------------------------------------------------------------------------- */

int orc_ece(int N, int gamma, const float* z, const int32_t* acc, const float* T, int M,
            double* ece, int* n_edge)
{
    if (N <= 0 || gamma <= 0 || M <= 0) return 1;
    double* sa = (double*)calloc((size_t)M, sizeof(double));
    double* ss = (double*)calloc((size_t)M, sizeof(double));
    if (!sa || !ss) { free(sa); free(ss); return 2; }
    int edge = 0;
    for (int n = 0; n < N; ++n) {
        double a = 1.0;
        for (int k = 0; k < gamma; ++k) {
            double x = (double)z[(size_t)n * gamma + k];
            if (T) x = x / (double)T[k];
            a = a * exp(log_sigmoid(x));
            const double aM = a * (double)M;
            int bin = (int)floor(aM);
            if (bin > M - 1) bin = M - 1;
            if (bin < 0) bin = 0;
            if (fabs(aM - nearbyint(aM)) < 1e-9 && aM > 0.5 && aM < M - 0.5) ++edge;
            sa[bin] += a;
            ss[bin] += (acc[n] > k) ? 1.0 : 0.0;
        }
    }
    double e = 0.0;
    for (int m = 0; m < M; ++m) e += fabs(ss[m] - sa[m]);
    *ece = e / ((double)N * (double)gamma);
    *n_edge = edge;
    free(sa);
    free(ss);
    return 0;
}

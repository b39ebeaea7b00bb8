/*
 * dsp.h -- C-ABI of libdsp.so: the per-token hot path of DSpark
 * confidence-scheduled speculative decoding on AMD Instinct MI355X (gfx950).
 *
 * One decode round is
 *     dsp_draft_step(k = 0, n_steps = gamma)       semi-autoregressive draft
 *     dsp_confidence                               confidence head + STS
 *     dsp_schedule                                 hardware-aware prefix scheduler
 *     dsp_verify                                   lossless verification
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is DEVICE memory owned by the caller, row-major with
 *     the last index contiguous and no padding, except the logit tensors (base,
 *     target), whose rows are placed by element strides (below).  The library
 *     never allocates or frees memory; scratch comes from a caller workspace
 *     sized by dsp_workspace_size() and 16-byte aligned (DSP_ERR_WORKSPACE
 *     otherwise; device allocations are).
 *   - Logit rows: element (n, k, v) -- request n, position k, vocabulary id v --
 *     of a logit tensor p with strides (rs, ps) is p[n * rs + k * ps + v]
 *     (strides in elements, >= 0; the vocabulary is contiguous).  A contiguous
 *     [R, gamma, V] tensor has rs = gamma * V, ps = V; a position-major
 *     [gamma, R, V] one has rs = V, ps = R * V.  Every row of the shape must be
 *     readable memory.  Rows stream as 16-byte words when V and both strides
 *     are multiples of 8 elements, otherwise element by element (same results).
 *     Performance note: request strides that are multiples of 2 MiB alias in
 *     HBM on MI355X and cost up to a third of the streaming rate of a draft
 *     step; a position-major base tensor (each draft step reads one contiguous
 *     [R, V] slab) or a row pitch padded off a power of two avoids it.
 *   - Calls are asynchronous and ordered on `stream` (a hipStream_t; NULL is the
 *     default stream).  No call synchronises the host except
 *     dsp_workspace_status(); lengths and batch sizes stay on the device.  Two
 *     calls sharing a workspace must be ordered.  Calls on different streams
 *     with different workspaces may run concurrently only where neither takes a
 *     persistent launch (DSP_PATH_STREAMING, or shapes where DSP_PATH_AUTO does
 *     not apply one): a persistent launch holds one workgroup on every compute
 *     unit and needs all of them resident together, so work beside it can only
 *     delay it, and two persistent launches that overlap can starve each other
 *     until their bounded waits give up.  A wait that gives up leaves that
 *     call's outputs undefined and is reported by dsp_workspace_status().
 *   - bf16 values are passed as their 16-bit patterns (uint16_t).
 *   - Token ids and lengths are int32; V < 2^31.  seed is 64-bit, round 32-bit.
 *   - Randomness: u(seed, round, request, position, purpose) in [0, 1) is the top
 *     24 bits of word 0 of Philox4x32-10 with counter (round, request, position,
 *     purpose) and key (seed low, seed high), divided by 2^24.  Purposes:
 *     0 draft sample, 1 accept test, 2 correction / bonus draw.
 *   - Errors: argument problems return DSP_ERR_INVALID_ARG and shapes outside the
 *     kernels' support DSP_ERR_UNSUPPORTED, both before any HIP call; a workspace
 *     that is too small returns DSP_ERR_WORKSPACE; a failed launch returns
 *     DSP_ERR_HIP.  dsp_last_error() gives a thread-local explanation.  Faults
 *     inside kernels surface at the caller's next synchronisation; a bounded
 *     wait of a persistent launch that gave up is reported as DSP_ERR_TIMEOUT by
 *     dsp_workspace_status().  No C++ exception crosses this boundary.
 *
 * Sizes supported: R >= 1, 1 <= gamma <= 64, 1 <= V <= 524288, 8 <= r <= 256
 * with r % 8 == 0, 0 <= d; the scheduler in mode 1 needs R * gamma <= 16384.
 *
 * ABI version 410: the recurrent sequential head (dsp_draft_step_rnn,
 * dsp_verify_rnn, dsp_tv_accept_rnn), sequential temperature scaling
 * (dsp_confidence_logit, dsp_sts_fit, dsp_ece).
 * 400: DSP_ERR_TIMEOUT and dsp_workspace_status(); the scheduler's
 * tau0 is bounded by 2^14.  (300: dsp_draft_step draws n_steps consecutive
 * positions per call; dsp_draft_step and dsp_verify take flags that select their
 * implementation.  200: element strides.)
 */
#ifndef DSP_H
#define DSP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DSP_OK = 0,
    DSP_ERR_INVALID_ARG = 1,
    DSP_ERR_UNSUPPORTED = 2,
    DSP_ERR_WORKSPACE = 3,
    DSP_ERR_HIP = 4,
    DSP_ERR_TIMEOUT = 5
} dsp_status;

typedef enum { DSP_F32 = 0, DSP_BF16 = 1 } dsp_dtype;

typedef enum {
    DSP_WS_DRAFT = 0,
    DSP_WS_VERIFY = 1,
    DSP_WS_TV = 2,
    DSP_WS_STS = 3,
    DSP_WS_ECE = 4
} dsp_ws_kind;

/* Static text for a status code. */
const char* dsp_status_string(dsp_status s);

/* Detail of the last non-OK status returned on the calling thread ("" if none). */
const char* dsp_last_error(void);

/* Library ABI version (major * 100 + minor). */
int dsp_version(void);

/* Bytes of workspace dsp_draft_step (DSP_WS_DRAFT), dsp_verify (DSP_WS_VERIFY),
 * dsp_tv_accept (DSP_WS_TV), dsp_sts_fit (DSP_WS_STS: R = the number of
 * held-out samples N; V and r are ignored) or dsp_ece (DSP_WS_ECE: a fixed size,
 * every size argument ignored) needs; 0 for invalid sizes. */
size_t dsp_workspace_size(dsp_ws_kind which, int R, int gamma, int V, int r);

/*
 * dsp_workspace_status -- did the last call on this workspace complete every
 * bounded wait?
 *
 * Waits for `stream` (the host blocks), then reads the error word that the last
 * dsp_draft_step (which = DSP_WS_DRAFT) or dsp_verify (DSP_WS_VERIFY) issued with
 * workspace ws wrote: DSP_OK when its waits all completed (and for calls that
 * have none), DSP_ERR_TIMEOUT when a wait of a persistent launch gave up -- the
 * outputs of that call are then undefined (tokens, q, stats, or the correction
 * and bonus tokens) though every kernel ran to its end.  The sizes are the ones
 * of that call; ws and ws_bytes as passed to it.  Undefined before the
 * workspace's first call.  A failing synchronisation returns DSP_ERR_HIP.
 */
dsp_status dsp_workspace_status(dsp_ws_kind which, const void* ws, size_t ws_bytes, int R,
                                int gamma, int V, int r, void* stream);

/*
 * dsp_draft_step -- draft positions k, k+1, ..., k+n_steps-1 for all R requests,
 * in that order (each position's previous token is the one drawn before it).
 *
 * Semi-autoregressive draft with the Markov head (DSpark paper summaries: page
 * "DeepSeek联合北大最新文章DSpark", two-stage design, sequential head: the
 * previous token enters the next position's distribution through a low-rank
 * matrix; page "DSpark.让每一轮计算，多走几步", Markov-head paragraph: a low-rank
 * transition table adds a bias to the vocabulary before each sample; page
 * "DeepSeek DSpark 技术解析" section 四: only the token id is passed forward).
 *
 * For each request n:
 *   prev     = anchor[n] if k == 0 else tok[n, k-1]   (prev outside [0, V): no bias)
 *   logit_v  = base[n, k, v] + sum_i E[prev, i] * W2[v, i]   (fp32)
 *   greedy (temperature == 0): tok[n,k] = argmax_v logit_v (lowest index on
 *     ties), q[n,k] = 1, stats[n,k] = (max logit, 0)
 *   sampling: pi_v proportional to exp((logit_v - M) / temperature), M = max;
 *     tok[n,k] = min{v : sum_{i<=v} pi_i > u(seed, round, n, k, 0)};
 *     q[n,k] = pi of that token; stats[n,k] = (M, Z), Z = sum_v exp((logit_v - M)/T)
 *
 * base   logits (n, k, v) at base[n * base_rs + k * base_ps + v], fp32 or bf16
 *        (dtype): the draft base logits of the backbone, R x gamma rows of V;
 *        positions k .. k+n_steps-1 are read
 * E      [V, r] bf16   Markov embedding; row x is the embedding of token x
 * W2     [V, r] bf16   low-rank output factor stored transposed: W2[v, i] is
 *                      element (i, v) of the r x V matrix
 * anchor [R]  int32    the token the target emitted last (x_{-1})
 * tok    [R, gamma] int32   columns k .. k+n_steps-1 written, column k-1 read (k >= 1)
 * q      [R, gamma] f32     columns k .. k+n_steps-1 written
 * stats  [R, gamma, 2] f64  columns k .. k+n_steps-1 written
 * k, n_steps   0 <= k, 1 <= n_steps, k + n_steps <= gamma
 * flags  implementation, a dsp_path_flags value (the results do not depend on it):
 *        DSP_PATH_AUTO         one persistent launch for every position
 *                              where it applies (bf16 logits in 16-byte rows, R <= 2048
 *                              and a vocabulary whose W2 slice fits on chip: V <= 163840
 *                              for r <= 256 on 256 CUs), W2 read once; two streaming
 *                              launches per position elsewhere, W2 read per position
 *        DSP_PATH_STREAMING    the streaming launches always (for callers sharing the
 *                              GPU with concurrent work: a persistent launch holds one
 *                              workgroup on every CU and relies on all of them being
 *                              resident; work on other streams can only delay it, and
 *                              a wait that outlasts a few seconds gives up, leaving
 *                              the outputs undefined)
 *        DSP_PATH_PERSISTENT   the persistent launch only; where it does not apply
 *                              the call returns DSP_ERR_HIP (hipErrorNotSupported)
 *        optionally or-ed with DSP_FLAG_TEST_GIVE_UP; anything else:
 *        DSP_ERR_INVALID_ARG.  While a persistent launch runs, tok[:, k .. k+n_steps-1] also carries its
 *        progress: the call overwrites those columns (and the workspace) only.
 * ws     >= dsp_workspace_size(DSP_WS_DRAFT, R, gamma, V, r) bytes
 */
typedef enum { DSP_PATH_AUTO = 0, DSP_PATH_STREAMING = 1, DSP_PATH_PERSISTENT = 2 } dsp_path_flags;
/* Test hook, or-ed into flags of dsp_draft_step / dsp_verify: a persistent launch
 * starts as if one of its waits had already given up, so every wait returns at
 * once, every kernel still runs to its end, the outputs are undefined and
 * dsp_workspace_status() reports DSP_ERR_TIMEOUT.  It lets callers test their
 * handling of that report without starving the GPU; calls without a
 * persistent launch ignore it. */
#define DSP_FLAG_TEST_GIVE_UP 0x100u
dsp_status dsp_draft_step(const void* base, dsp_dtype dtype, int64_t base_rs, int64_t base_ps,
                          const uint16_t* E, const uint16_t* W2, const int32_t* anchor, int32_t* tok, float* q,
                          double* stats, int R, int gamma, int V, int r, int k, int n_steps,
                          unsigned flags, float temperature, uint64_t seed, uint32_t round, void* ws,
                          size_t ws_bytes, void* stream);

/*
 * dsp_draft_step_rnn -- dsp_draft_step with the recurrent sequential head.
 *
 * Page "DeepSeek联合北大最新文章DSpark", 第二阶段轻量顺序头: besides the Markov head
 * (previous token only), an RNN head keeps a recurrent state to capture longer
 * dependencies; the page gives no recurrence.  This library's reading, an
 * Elman recurrence on the Markov head's rank-r space:
 *     s[n,-1] = 0
 *     s[n,k]  = bf16(tanh(A s[n,k-1] + E[x_{k-1}]))   (fp64 sum in index order,
 *               no E term for x outside [0, V); one rounding to nearest even)
 *     logit   = base[n,k,:] + s[n,k] . W2^T            (the Markov head's MFMA
 *                                                       bias with s in place of E[x])
 * With A = 0 it is the Markov head on the table bf16(tanh(E)).  Sampling,
 * greedy, Philox counters and outputs as dsp_draft_step.
 *
 * A [r, r] bf16, element (i, j) at A[i r + j]; S [R, gamma, r] bf16 (device):
 * positions k .. k + n_steps - 1 are written, and position k - 1 must hold the
 * state a previous call wrote when k > 0.  R gamma r <= 2^31 - 1.  Streaming
 * launches only: DSP_PATH_PERSISTENT returns DSP_ERR_UNSUPPORTED.  Workspace:
 * dsp_workspace_size(DSP_WS_DRAFT, ...).  Other arguments as dsp_draft_step.
 */
dsp_status dsp_draft_step_rnn(const void* base, dsp_dtype dtype, int64_t base_rs, int64_t base_ps,
                              const uint16_t* E, const uint16_t* W2, const uint16_t* A,
                              const int32_t* anchor, int32_t* tok, float* q, double* stats,
                              uint16_t* S, int R, int gamma, int V, int r, int k, int n_steps,
                              unsigned flags, float temperature, uint64_t seed, uint32_t round,
                              void* ws, size_t ws_bytes, void* stream);

/*
 * dsp_draft_step_noalloc -- dsp_draft_step for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation): the same arguments, the same results bit for bit,
 * without the workspace.  Its scratch is a static array of the library, 16 MiB
 * on each device it runs on, held until the process ends; every call on a
 * device shares it, so calls that overlap on one device (other streams, other
 * threads) race and must be ordered by the caller.  Sizes whose workspace
 * (dsp_workspace_size(DSP_WS_DRAFT, ...)) exceeds 16 MiB return
 * DSP_ERR_WORKSPACE before any HIP call.  No call allocates or frees memory.  A
 * bounded wait that gives up is not reported (dsp_workspace_status needs a
 * workspace); the outputs of such a call are undefined.
 */
dsp_status dsp_draft_step_noalloc(const void* base, dsp_dtype dtype, int64_t base_rs,
                                  int64_t base_ps, const uint16_t* E, const uint16_t* W2,
                                  const int32_t* anchor, int32_t* tok, float* q, double* stats, int R,
                                  int gamma, int V, int r, int k, int n_steps, unsigned flags,
                                  float temperature, uint64_t seed, uint32_t round, void* stream);

/*
 * dsp_confidence -- confidence head with sequential temperature scaling.
 *
 * Page "DeepSeek联合北大最新文章DSpark", section 2.1: c_k is the probability that
 * draft token k is accepted given that every earlier one was; it is a sigmoid of
 * a linear map of [h_k; W1[x_{k-1}]]; temperatures fitted left to right per
 * position calibrate the cumulative survival (the same section, sequential
 * temperature scaling).
 *
 *   y       = sum_{i<d} w[i] h[n,k,i] + sum_{i<r} w[d+i] E[prev,i]   (fp64)
 *   c[n,k]  = 1 / (1 + exp(-(y + offset[n]) / T[k]))   rounded to fp32
 * prev = anchor[n] for k = 0, tok[n, k-1] otherwise (prev outside [0, V) drops the
 * E term).
 *
 * h [R, gamma, d] bf16; E [V, r] bf16; anchor [R]; tok [R, gamma];
 * w [d + r] f32; T [gamma] f32 (> 0); offset [R] f32 or NULL; c [R, gamma] f32.
 */
dsp_status dsp_confidence(const uint16_t* h, const uint16_t* E, const int32_t* anchor,
                          const int32_t* tok, const float* w, const float* T,
                          const float* offset, float* c, int R, int gamma, int d, int V, int r,
                          void* stream);

/*
 * dsp_confidence_logit -- the confidence head's sigmoid argument before the
 * temperatures: y[n,k] = fp32(sum_{i<d} w[i] h[n,k,i] + sum_{i<r} w[d+i] E[prev,i]
 * + offset[n]) with the fp64 sum of dsp_confidence (same arguments without T).
 * These raw logits are what sequential temperature scaling is fitted on.
 */
dsp_status dsp_confidence_logit(const uint16_t* h, const uint16_t* E, const int32_t* anchor,
                                const int32_t* tok, const float* w, const float* offset, float* y,
                                int R, int gamma, int d, int V, int r, void* stream);

/*
 * dsp_sts_fit -- sequential temperature scaling fitted on held-out data.
 *
 * Page "DeepSeek联合北大最新文章DSpark", section 2.1: the raw confidences are
 * overconfident and overestimate the cumulative survival; temperatures are
 * calibrated position by position from left to right on a held-out set.  The
 * page gives no objective.  This library's reading: sample n carries raw logits
 * z[n,k] (dsp_confidence_logit) and n_acc[n], its number of accepted draft tokens
 * in a round that verified every position (0..gamma); s[n,k] = (n_acc[n] > k).
 * With beta_j = 1 / T_j and a[n,k] = prod_{j<=k} sigma(beta_j z[n,j]), T_k (the
 * earlier ones fixed) minimises the binary cross-entropy
 *     F_k(beta) = -sum_n [ s ln a[n,k] + (1 - s) ln(1 - a[n,k]) ]
 * over two grids of 256 betas, each point fma(g, step, lo) in fp64: first
 * [1/t_hi, 1/t_lo], then the span of the first grid's best point and its two
 * neighbours.  The lowest index wins a tie; a NaN objective counts as +inf.
 * fp64 throughout.
 *
 * z [N, gamma] f32; n_acc [N] int32; T [gamma] f32 out (= fp32(1/beta_k));
 * nll [gamma] f64 out (F_k at the fitted beta) or NULL; 0 < t_lo < t_hi finite;
 * ws >= dsp_workspace_size(DSP_WS_STS, N, gamma, 1, 1) bytes, 16-byte aligned
 * (DSP_ERR_WORKSPACE otherwise).  Asynchronous on stream; device memory only.
 */
dsp_status dsp_sts_fit(const float* z, const int32_t* n_acc, int N, int gamma, float t_lo,
                       float t_hi, float* T, double* nll, void* ws, size_t ws_bytes, void* stream);

/*
 * dsp_ece -- expected calibration error of the cumulative survival (the page
 * above reports ECE before and after the temperatures).  Every pair (n, k) is
 * a prediction a[n,k] = prod_{j<=k} sigma(z[n,j] / T_j) (T NULL: T_j = 1) of
 * s[n,k] = (n_acc[n] > k), binned by min(floor(a n_bins), n_bins - 1):
 *     ece = sum_bins |sum_bin (s - a)| / (N gamma)
 * Bin sums are exact integers (a in units of 2^-40), so the result does not
 * depend on the order of the GPU's additions and lies within 2^-40 of the
 * real-number value of these predictions.
 *
 * z [N, gamma] f32; n_acc [N] int32; T [gamma] f32 or NULL; 1 <= n_bins <= 64;
 * N gamma <= 2^23 (DSP_ERR_UNSUPPORTED beyond); ece [1] f64 out (device);
 * ws >= dsp_workspace_size(DSP_WS_ECE, 0, 0, 0, 0) bytes, 16-byte aligned.
 */
dsp_status dsp_ece(const float* z, const int32_t* n_acc, const float* T, int N, int gamma,
                   int n_bins, double* ece, void* ws, size_t ws_bytes, void* stream);

/*
 * dsp_schedule -- hardware-aware prefix scheduler.
 *
 * Page "DeepSeek联合北大最新文章DSpark", section 2.2: choose the verify lengths
 * l_r maximising Theta = tau * SPS(B), B = sum_r (1 + l_r), tau = sum_r
 * sum_{j <= l_r} a_{r,j}, SPS a profiled lookup table; solved by sorting every
 * candidate by survival probability, admitting one by one, stopping as soon as
 * the throughput stops rising.  Survival a_{r,j} = c_{r,1} x ... x c_{r,j}
 * (page "DSpark.让每一轮计算，多走几步", section 写得长，不如验得值).
 *
 *   a[r,j]  = fl32(a[r,j-1] * c[r,j]) left to right
 *   order   : a descending, then r ascending, then j ascending (stable)
 *   tau_n   = tau0 + sum of the n best a, each truncated to a multiple of 2^-48
 *             (exact fixed point, so the sum is independent of evaluation order)
 *   Theta_n = double(tau_n) * SPS(R + n);  admit the n-th candidate while
 *             Theta_n > Theta_{n-1} and R + n <= B_max
 *   len[r]  = admitted candidates of request r;  *B = R + sum_r len[r]
 * mode 0 verifies everything: len[r] = gamma, *B = R (1 + gamma); a still written.
 *
 * c [R, gamma] f32 in [0, 1]; sps [B_max] f32 with sps[B-1] = SPS(B); B_max >= R;
 * 0 <= tau0 < 2^14 (so tau0 2^48 plus the admitted sum fits 64 bits;
 * DSP_ERR_INVALID_ARG otherwise); len [R] int32; a [R, gamma] f32; B [1] int32
 * (all device memory).
 * Runs as one workgroup; mode 1 needs R * gamma <= 16384.
 */
dsp_status dsp_schedule(const float* c, const float* sps, int B_max, double tau0, int mode,
                        int32_t* len, float* a, int32_t* B, int R, int gamma, void* stream);

/*
 * dsp_schedule_async -- the scheduler with a capacity barrier, for engines that
 * must fix a step's batch size before the previous step ends.
 *
 * Page "DeepSeek联合北大最新文章DSpark", 挑战2 (asynchronous scheduling and
 * zero-overhead scheduling): real SPS curves are jagged, so the early stop of
 * dsp_schedule can stop at a local optimum; the verification capacity is instead
 * taken from the confidences of two steps back, the candidates are still ranked
 * by the newest ones, and the capacity barrier lets the search over the old
 * confidences drop the early stop without breaking losslessness (page "DSpark.
 * 让每一轮计算，多走几步", causality paragraph of 两个严谨补丁).
 *
 *   capacity: survival products, order and Q48 sums of dsp_schedule over c_hist;
 *             K = the smallest n in [0, min(R gamma, B_max - R)] with the maximum
 *             Theta_n = (tau0 + sum of the n best) * SPS(R + n) -- no early stop
 *   admission: a = survival products of c (written out), the same order; the
 *             first K candidates admitted; len[r] = admitted candidates of r;
 *             *B = R + K; *K = K
 * c, c_hist [R, gamma] f32 in [0, 1] (c_hist: the same requests' confidences of
 * an earlier round, e.g. two steps back); sps, B_max, tau0 as for dsp_schedule;
 * len [R], a [R, gamma], B [1], K [1] (device memory).  One workgroup;
 * R * gamma <= 16384.
 */
dsp_status dsp_schedule_async(const float* c, const float* c_hist, const float* sps, int B_max,
                              double tau0, int32_t* len, float* a, int32_t* B, int32_t* K, int R,
                              int gamma, void* stream);

/*
 * dsp_verify -- lossless verification of the scheduled prefixes.
 *
 * Accept rule, residual and bonus token: page "DSpark.让每一轮计算，多走几步",
 * lossless section (keep the accepted prefix, one correction token after the
 * first rejection, one extra token when everything passed; greedy mode accepts
 * only an identical choice); page "为什么DSpark 可以加速推理？", section on the
 * mathematics of speculative decoding (acceptance min(1, p/q), residual
 * max(0, p - q) normalised).
 *
 * For each request n with l = len[n] (0 <= l <= gamma):
 *   p_j = softmax(target[n, j, :] / temperature), j = 0..l
 *   j < l, sampling: accept[n,j] = u(seed, round, n, j, 1) <= min(1, p_j(x_j)/q[n,j])
 *          greedy (temperature == 0): accept[n,j] = (x_j == argmax target[n,j,:])
 *   n_accept[n] = first j < l with accept 0, else l
 *   y[n]: if n_accept < l: sampling draws from max(0, p_m - q_m) normalised,
 *         m = n_accept, q_m the full draft row at position m recomputed from base,
 *         E, W2 and stats[n, m] (from p_m if that mass is zero); greedy: argmax
 *         of target row m.  If n_accept == l: a draw from p_l (greedy: argmax).
 *         Draws use u(seed, round, n, n_accept, 2) and the inverse-CDF rule of
 *         dsp_draft_step.
 *   accept[n,j] = -1 and p[n,j] = 0 for j >= l; p[n,j] = p_j(x_j) for j < l
 *   (greedy: 1 if accepted else 0).
 *
 * target logits (n, j, v), j = 0..gamma, at target[n * target_rs + j * target_ps
 * + v] and base (n, k, v) at base[n * base_rs + k * base_ps + v], one dtype;
 * E, W2 as for dsp_draft_step; anchor [R]; tok, q [R, gamma] and stats
 * [R, gamma, 2] (f64) as
 * written by dsp_draft_step; len [R]; outputs accept [R, gamma] int8,
 * n_accept [R] int32, y [R] int32, p [R, gamma] f32.
 * flags: a dsp_path_flags value for the residual draws (sampling; the results do
 * not depend on it): DSP_PATH_AUTO draws them in one persistent launch
 * that holds the W2 slice on chip where the draft's does (see dsp_draft_step), with
 * a streaming pass and a pick launch elsewhere; DSP_PATH_STREAMING always the latter;
 * DSP_PATH_PERSISTENT the former only (DSP_ERR_HIP, hipErrorNotSupported, where it
 * does not apply; greedy verification draws no residual and ignores it),
 * optionally or-ed with DSP_FLAG_TEST_GIVE_UP.
 * ws >= dsp_workspace_size(DSP_WS_VERIFY, R, gamma, V, r) bytes.
 */
dsp_status dsp_verify(const void* target, int64_t target_rs, int64_t target_ps, const void* base,
                      int64_t base_rs, int64_t base_ps, dsp_dtype dtype, const uint16_t* E,
                      const uint16_t* W2, const int32_t* anchor, const int32_t* tok,
                      const float* q, const double* stats, const int32_t* len, int8_t* accept,
                      int32_t* n_accept, int32_t* y, float* p, int R, int gamma, int V, int r,
                      unsigned flags, float temperature, uint64_t seed, uint32_t round, void* ws,
                      size_t ws_bytes, void* stream);

/*
 * dsp_verify_rnn -- dsp_verify after dsp_draft_step_rnn: at a rejection the
 * draft law of position m (whose max(0, p - q) the correction draws from) takes
 * the state row S[n, m] as its bias row instead of E[x_{m-1}].  S [R, gamma, r]
 * bf16 as dsp_draft_step_rnn wrote it; R gamma r <= 2^31 - 1; streaming
 * launches only (DSP_PATH_PERSISTENT: DSP_ERR_UNSUPPORTED).  Other arguments,
 * workspace and results as dsp_verify.
 */
dsp_status dsp_verify_rnn(const void* target, int64_t target_rs, int64_t target_ps, const void* base,
                          int64_t base_rs, int64_t base_ps, dsp_dtype dtype, const uint16_t* E,
                          const uint16_t* W2, const uint16_t* S, const int32_t* anchor,
                          const int32_t* tok, const float* q, const double* stats, const int32_t* len,
                          int8_t* accept, int32_t* n_accept, int32_t* y, float* p, int R, int gamma,
                          int V, int r, unsigned flags, float temperature, uint64_t seed,
                          uint32_t round, void* ws, size_t ws_bytes, void* stream);

/*
 * dsp_tv_accept -- the exact acceptance probability of every draft position.
 *
 * Page "为什么DSpark 可以加速推理？", section on the mathematics of speculative
 * decoding: a draft token x ~ q is accepted with probability min(1, p(x)/q(x)),
 * so the total acceptance probability of a position is sum_v min(q(v), p(v));
 * page "DeepSeek联合北大最新文章DSpark", section 2.1: the confidence head is trained
 * towards one minus the total-variation distance between the draft and target
 * laws, the same quantity.  For each request n and position k < gamma:
 *   q_k  = the draft law of dsp_draft_step at k (prev = anchor for k = 0, else
 *          tok[n, k-1]; base row k plus the Markov bias, / temperature)
 *   p_k  = softmax(target[n, k, :] / temperature)
 *   alpha[n, k] = sum_v min(q_k(v), p_k(v)) = 1 - sum_v max(0, p_k(v) - q_k(v))
 * computed as the latter (fp32 weights, fp64 differences and sums), clamped to
 * [0, 1].  The arguments are those of dsp_verify: stats [R, gamma, 2] (f64) as
 * written by dsp_draft_step give q_k's (M, Z); tok [R, gamma] its tokens; alpha
 * [R, gamma] f64 (device memory).  temperature > 0 (DSP_ERR_INVALID_ARG
 * otherwise).  ws >= dsp_workspace_size(DSP_WS_TV, R, gamma, V, r) bytes.
 * Streams each target row twice (its normaliser first) and each base row once.
 */
dsp_status dsp_tv_accept(const void* target, int64_t target_rs, int64_t target_ps, const void* base,
                         int64_t base_rs, int64_t base_ps, dsp_dtype dtype, const uint16_t* E,
                         const uint16_t* W2, const int32_t* anchor, const int32_t* tok,
                         const double* stats, double* alpha, int R, int gamma, int V, int r,
                         float temperature, void* ws, size_t ws_bytes, void* stream);

/*
 * dsp_tv_accept_rnn -- dsp_tv_accept for the recurrent head: the draft law of
 * position k takes the state row S[n, k] (dsp_draft_step_rnn) as its bias row.
 * R gamma r <= 2^31 - 1; other arguments as dsp_tv_accept.
 */
dsp_status dsp_tv_accept_rnn(const void* target, int64_t target_rs, int64_t target_ps,
                             const void* base, int64_t base_rs, int64_t base_ps, dsp_dtype dtype,
                             const uint16_t* E, const uint16_t* W2, const uint16_t* S,
                             const int32_t* anchor, const int32_t* tok, const double* stats,
                             double* alpha, int R, int gamma, int V, int r, float temperature,
                             void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DSP_H */

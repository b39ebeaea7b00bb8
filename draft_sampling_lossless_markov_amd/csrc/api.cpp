// api.cpp -- the C-ABI entry points of libdsp.so (declared in include/dsp.h).
//
// Every argument is validated on the host before any HIP call, so argument
// errors are reported without touching a device; kernels are then launched on
// the caller's stream.  No exception leaves this file.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "dsp.h"
#include "dsp_launch.h"

namespace {

thread_local char g_err[512] = "";

dsp_status fail(dsp_status s, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

dsp_status ok()
{
    g_err[0] = '\0';
    return DSP_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

dsp_status hip_status(hipError_t e, const char* what)
{
    if (e != hipSuccess) return fail(DSP_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

// strides of a logit tensor argument
dsp_status check_strides(const char* fn, const char* name, int64_t rs, int64_t ps)
{
    if (rs < 0 || ps < 0)
        return fail(DSP_ERR_INVALID_ARG, "%s: %s strides must be >= 0 (got %lld, %lld)", fn, name,
                    (long long)rs, (long long)ps);
    return DSP_OK;
}

// shapes shared by the Markov-head calls
dsp_status check_markov(int R, int gamma, int V, int r)
{
    if (R <= 0) return fail(DSP_ERR_INVALID_ARG, "R must be >= 1 (got %d)", R);
    if (gamma <= 0) return fail(DSP_ERR_INVALID_ARG, "gamma must be >= 1 (got %d)", gamma);
    if (V <= 0) return fail(DSP_ERR_INVALID_ARG, "V must be >= 1 (got %d)", V);
    if (r <= 0) return fail(DSP_ERR_INVALID_ARG, "r must be >= 1 (got %d)", r);
    if (gamma > dsp::kGammaMax)
        return fail(DSP_ERR_UNSUPPORTED, "gamma = %d exceeds the supported maximum %d", gamma,
                    dsp::kGammaMax);
    if (V > dsp::kVocabMax)
        return fail(DSP_ERR_UNSUPPORTED, "V = %d exceeds the supported maximum %d", V, dsp::kVocabMax);
    if (r > 256 || (r % 8) != 0)
        return fail(DSP_ERR_UNSUPPORTED, "r = %d: the bias kernels need r %% 8 == 0 and r <= 256", r);
    if ((int64_t)R * (gamma + 1) > (int64_t)INT32_MAX / 2)
        return fail(DSP_ERR_UNSUPPORTED, "R * (gamma + 1) too large");
    return DSP_OK;
}

static_assert(DSP_PATH_AUTO == dsp::kPathAuto && DSP_PATH_STREAMING == dsp::kPathStream &&
                  DSP_PATH_PERSISTENT == dsp::kPathPersistent,
              "path codes");

// a dsp_path_flags value, optionally with the give-up test hook
bool known_path(unsigned f)
{
    const unsigned p = f & ~DSP_FLAG_TEST_GIVE_UP;
    return p == DSP_PATH_AUTO || p == DSP_PATH_STREAMING || p == DSP_PATH_PERSISTENT;
}

int path_of(unsigned f) { return (int)(f & ~DSP_FLAG_TEST_GIVE_UP); }
bool give_up_of(unsigned f) { return (f & DSP_FLAG_TEST_GIVE_UP) != 0u; }

// the arguments dsp_draft_step and dsp_draft_step_noalloc share
dsp_status check_draft(const char* fn, const void* base, dsp_dtype dtype, int64_t base_rs,
                       int64_t base_ps, const uint16_t* E, const uint16_t* W2, const int32_t* anchor,
                       int32_t* tok, float* q, double* stats, int R, int gamma, int V, int r, int k,
                       int n_steps, unsigned flags, float temperature)
{
    if (!base || !E || !W2 || !anchor || !tok || !q || !stats)
        return fail(DSP_ERR_INVALID_ARG, "%s: null pointer argument", fn);
    if (dtype != DSP_F32 && dtype != DSP_BF16)
        return fail(DSP_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)dtype);
    dsp_status st = check_markov(R, gamma, V, r);
    if (st != DSP_OK) return st;
    if (k < 0 || k >= gamma)
        return fail(DSP_ERR_INVALID_ARG, "%s: k = %d outside [0, gamma)", fn, k);
    if (!known_path(flags))
        return fail(DSP_ERR_INVALID_ARG, "%s: unknown flags %u", fn, flags);
    if (n_steps < 1 || n_steps > gamma - k)
        return fail(DSP_ERR_INVALID_ARG, "%s: n_steps = %d outside [1, gamma - k] (k = %d)", fn,
                    n_steps, k);
    st = check_strides(fn, "base", base_rs, base_ps);
    if (st != DSP_OK) return st;
    if (!(temperature >= 0.0f) || std::isinf(temperature))
        return fail(DSP_ERR_INVALID_ARG, "%s: temperature must be finite and >= 0", fn);
    if (!aligned16(base) || !aligned16(E) || !aligned16(W2))
        return fail(DSP_ERR_INVALID_ARG, "%s: base, E and W2 must be 16-byte aligned", fn);
    return DSP_OK;
}

}  // namespace

namespace {
dsp_status verify_impl(const void* target, int64_t target_rs, int64_t target_ps, const void* base,
                       int64_t base_rs, int64_t base_ps, dsp_dtype dtype, const uint16_t* E,
                       const uint16_t* W2, const int32_t* anchor, const int32_t* tok,
                       const float* q, const double* stats, const int32_t* len, int8_t* accept,
                       int32_t* n_accept, int32_t* y, float* p, int R, int gamma, int V, int r,
                       unsigned flags, float temperature, uint64_t seed, uint32_t round, void* ws,
                       size_t ws_bytes, void* stream, const uint16_t* S);
}  // namespace

extern "C" {

const char* dsp_status_string(dsp_status s)
{
    switch (s) {
    case DSP_OK: return "DSP_OK";
    case DSP_ERR_INVALID_ARG: return "DSP_ERR_INVALID_ARG";
    case DSP_ERR_UNSUPPORTED: return "DSP_ERR_UNSUPPORTED";
    case DSP_ERR_WORKSPACE: return "DSP_ERR_WORKSPACE";
    case DSP_ERR_HIP: return "DSP_ERR_HIP";
    case DSP_ERR_TIMEOUT: return "DSP_ERR_TIMEOUT";
    }
    return "DSP_ERR_UNKNOWN";
}

const char* dsp_last_error(void) { return g_err; }

int dsp_version(void) { return 410; }

size_t dsp_workspace_size(dsp_ws_kind which, int R, int gamma, int V, int r)
{
    if (which == DSP_WS_STS) return (R > 0 && gamma > 0) ? dsp::sts_workspace_bytes(R) : 0;
    if (which == DSP_WS_ECE) return dsp::ece_workspace_bytes();
    if (R <= 0 || gamma <= 0 || V <= 0 || r <= 0) return 0;
    if (which == DSP_WS_DRAFT) return dsp::draft_workspace_bytes(R, V);
    if (which == DSP_WS_VERIFY) return dsp::verify_workspace_bytes(R, gamma, V);
    if (which == DSP_WS_TV) return dsp::tv_workspace_bytes(R, gamma, V);
    return 0;
}

dsp_status dsp_workspace_status(dsp_ws_kind which, const void* ws, size_t ws_bytes, int R,
                                int gamma, int V, int r, void* stream)
{
    if (which != DSP_WS_DRAFT && which != DSP_WS_VERIFY)
        return fail(DSP_ERR_INVALID_ARG, "dsp_workspace_status: unknown workspace kind %d", (int)which);
    if (!ws) return fail(DSP_ERR_INVALID_ARG, "dsp_workspace_status: null workspace");
    dsp_status st = check_markov(R, gamma, V, r);
    if (st != DSP_OK) return st;
    const size_t need = which == DSP_WS_DRAFT ? dsp::draft_workspace_bytes(R, V)
                                              : dsp::verify_workspace_bytes(R, gamma, V);
    if (ws_bytes < need)
        return fail(DSP_ERR_WORKSPACE, "dsp_workspace_status: workspace of %zu bytes, %zu needed",
                    ws_bytes, need);
    const unsigned* word = which == DSP_WS_DRAFT ? dsp::draft_error_word(ws, R, V)
                                                 : dsp::verify_error_word(ws, R, gamma, V);
    unsigned v = 0;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(&v, word, sizeof(v), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_status(e, "dsp_workspace_status");
    if (v != 0u)
        return fail(DSP_ERR_TIMEOUT,
                    "a bounded wait of the last persistent launch on this workspace gave up; "
                    "its outputs are undefined");
    return ok();
}

dsp_status dsp_draft_step(const void* base, dsp_dtype dtype, int64_t base_rs, int64_t base_ps,
                          const uint16_t* E, const uint16_t* W2, const int32_t* anchor, int32_t* tok, float* q,
                          double* stats, int R, int gamma, int V, int r, int k, int n_steps,
                          unsigned flags, float temperature, uint64_t seed, uint32_t round,
                          void* ws, size_t ws_bytes, void* stream)
{
    dsp_status st = check_draft("dsp_draft_step", base, dtype, base_rs, base_ps, E, W2, anchor, tok,
                                q, stats, R, gamma, V, r, k, n_steps, flags, temperature);
    if (st != DSP_OK) return st;
    const size_t need = dsp::draft_workspace_bytes(R, V);
    if (!ws || ws_bytes < need)
        return fail(DSP_ERR_WORKSPACE, "dsp_draft_step: workspace of %zu bytes, %zu needed",
                    ws_bytes, need);
    if (!aligned16(ws))
        return fail(DSP_ERR_WORKSPACE, "dsp_draft_step: the workspace must be 16-byte aligned");
    return hip_status(dsp::launch_draft_step(base, dsp::RowStrides{base_rs, base_ps},
                                             dtype == DSP_BF16, E, W2, anchor, tok, q,
                                             stats, R, gamma, V, r, k, n_steps, path_of(flags),
                                             give_up_of(flags), temperature,
                                             seed, round,
                                             ws, static_cast<hipStream_t>(stream)),
                      "dsp_draft_step launch");
}

dsp_status dsp_draft_step_rnn(const void* base, dsp_dtype dtype, int64_t base_rs, int64_t base_ps,
                              const uint16_t* E, const uint16_t* W2, const uint16_t* A,
                              const int32_t* anchor, int32_t* tok, float* q, double* stats,
                              uint16_t* S, int R, int gamma, int V, int r, int k, int n_steps,
                              unsigned flags, float temperature, uint64_t seed, uint32_t round,
                              void* ws, size_t ws_bytes, void* stream)
{
    dsp_status st = check_draft("dsp_draft_step_rnn", base, dtype, base_rs, base_ps, E, W2, anchor,
                                tok, q, stats, R, gamma, V, r, k, n_steps, flags, temperature);
    if (st != DSP_OK) return st;
    if (!A || !S) return fail(DSP_ERR_INVALID_ARG, "dsp_draft_step_rnn: null A or S");
    if (!aligned16(A) || !aligned16(S))
        return fail(DSP_ERR_INVALID_ARG, "dsp_draft_step_rnn: A and S must be 16-byte aligned");
    if ((int64_t)R * gamma * r > dsp::kRnnMaxStateElems)
        return fail(DSP_ERR_UNSUPPORTED, "dsp_draft_step_rnn: R * gamma * r exceeds 2^31 - 1");
    if (path_of(flags) == DSP_PATH_PERSISTENT)
        return fail(DSP_ERR_UNSUPPORTED, "dsp_draft_step_rnn: the recurrent head runs the streaming path only");
    const size_t need = dsp::draft_workspace_bytes(R, V);
    if (!ws || ws_bytes < need)
        return fail(DSP_ERR_WORKSPACE, "dsp_draft_step_rnn: workspace of %zu bytes, %zu needed",
                    ws_bytes, need);
    if (!aligned16(ws))
        return fail(DSP_ERR_WORKSPACE, "dsp_draft_step_rnn: the workspace must be 16-byte aligned");
    return hip_status(dsp::launch_draft_step(base, dsp::RowStrides{base_rs, base_ps},
                                             dtype == DSP_BF16, E, W2, anchor, tok, q, stats, R, gamma,
                                             V, r, k, n_steps, path_of(flags), give_up_of(flags),
                                             temperature, seed, round, ws,
                                             static_cast<hipStream_t>(stream), A, S),
                      "dsp_draft_step_rnn launch");
}

dsp_status dsp_draft_step_noalloc(const void* base, dsp_dtype dtype, int64_t base_rs,
                                  int64_t base_ps, const uint16_t* E, const uint16_t* W2,
                                  const int32_t* anchor, int32_t* tok, float* q, double* stats, int R,
                                  int gamma, int V, int r, int k, int n_steps, unsigned flags,
                                  float temperature, uint64_t seed, uint32_t round, void* stream)
{
    dsp_status st = check_draft("dsp_draft_step_noalloc", base, dtype, base_rs, base_ps, E, W2,
                                anchor, tok, q, stats, R, gamma, V, r, k, n_steps, flags, temperature);
    if (st != DSP_OK) return st;
    const size_t need = dsp::draft_workspace_bytes(R, V);
    if (need > dsp::kStaticScratchBytes)
        return fail(DSP_ERR_WORKSPACE,
                    "dsp_draft_step_noalloc: these sizes need %zu bytes of scratch, more than the "
                    "static %zu",
                    need, dsp::kStaticScratchBytes);
    void* ws = nullptr;
    const hipError_t e = dsp::static_scratch(&ws);
    if (e != hipSuccess) return hip_status(e, "dsp_draft_step_noalloc: static scratch address");
    return hip_status(dsp::launch_draft_step(base, dsp::RowStrides{base_rs, base_ps},
                                             dtype == DSP_BF16, E, W2, anchor, tok, q,
                                             stats, R, gamma, V, r, k, n_steps, path_of(flags),
                                             give_up_of(flags), temperature, seed, round, ws,
                                             static_cast<hipStream_t>(stream)),
                      "dsp_draft_step_noalloc launch");
}

dsp_status dsp_confidence(const uint16_t* h, const uint16_t* E, const int32_t* anchor,
                          const int32_t* tok, const float* w, const float* T,
                          const float* offset, float* c, int R, int gamma, int d, int V, int r,
                          void* stream)
{
    if (!E || !anchor || !tok || !w || !T || !c || (!h && d > 0))
        return fail(DSP_ERR_INVALID_ARG, "dsp_confidence: null pointer argument");
    if (R <= 0 || gamma <= 0 || V <= 0 || r <= 0 || d < 0)
        return fail(DSP_ERR_INVALID_ARG, "dsp_confidence: bad sizes R=%d gamma=%d d=%d V=%d r=%d",
                    R, gamma, d, V, r);
    if ((int64_t)R * gamma > (int64_t)INT32_MAX / 2)
        return fail(DSP_ERR_UNSUPPORTED, "dsp_confidence: R * gamma too large");
    if ((h && !aligned16(h)) || !aligned16(w))
        return fail(DSP_ERR_INVALID_ARG, "dsp_confidence: h and w must be 16-byte aligned");
    return hip_status(dsp::launch_confidence(h, E, anchor, tok, w, T, offset, c, R, gamma, d, V,
                                             r, static_cast<hipStream_t>(stream)),
                      "dsp_confidence launch");
}

dsp_status dsp_confidence_logit(const uint16_t* h, const uint16_t* E, const int32_t* anchor,
                                const int32_t* tok, const float* w, const float* offset, float* y,
                                int R, int gamma, int d, int V, int r, void* stream)
{
    if (!E || !anchor || !tok || !w || !y || (!h && d > 0))
        return fail(DSP_ERR_INVALID_ARG, "dsp_confidence_logit: null pointer argument");
    if (R <= 0 || gamma <= 0 || V <= 0 || r <= 0 || d < 0)
        return fail(DSP_ERR_INVALID_ARG, "dsp_confidence_logit: bad sizes R=%d gamma=%d d=%d V=%d r=%d",
                    R, gamma, d, V, r);
    if ((int64_t)R * gamma > (int64_t)INT32_MAX / 2)
        return fail(DSP_ERR_UNSUPPORTED, "dsp_confidence_logit: R * gamma too large");
    if ((h && !aligned16(h)) || !aligned16(w))
        return fail(DSP_ERR_INVALID_ARG, "dsp_confidence_logit: h and w must be 16-byte aligned");
    return hip_status(dsp::launch_confidence(h, E, anchor, tok, w, nullptr, offset, y, R, gamma, d,
                                             V, r, static_cast<hipStream_t>(stream)),
                      "dsp_confidence_logit launch");
}

dsp_status dsp_sts_fit(const float* z, const int32_t* n_acc, int N, int gamma, float t_lo,
                       float t_hi, float* T, double* nll, void* ws, size_t ws_bytes, void* stream)
{
    if (!z || !n_acc || !T || !ws)
        return fail(DSP_ERR_INVALID_ARG, "dsp_sts_fit: null pointer argument");
    if (N <= 0 || gamma <= 0)
        return fail(DSP_ERR_INVALID_ARG, "dsp_sts_fit: bad sizes N=%d gamma=%d", N, gamma);
    if ((int64_t)N * gamma > (int64_t)INT32_MAX / 2)
        return fail(DSP_ERR_UNSUPPORTED, "dsp_sts_fit: N * gamma too large");
    if (!(t_lo > 0.0f) || !(t_hi > t_lo) || !std::isfinite(t_hi))
        return fail(DSP_ERR_INVALID_ARG, "dsp_sts_fit: need 0 < t_lo < t_hi < inf (got %g, %g)",
                    (double)t_lo, (double)t_hi);
    const size_t need = dsp::sts_workspace_bytes(N);
    if (ws_bytes < need || !aligned16(ws))
        return fail(DSP_ERR_WORKSPACE, "dsp_sts_fit: workspace of %zu bytes (16-byte aligned), %zu needed",
                    ws_bytes, need);
    return hip_status(dsp::launch_sts_fit(z, n_acc, N, gamma, (double)t_lo, (double)t_hi, T, nll, ws,
                                          static_cast<hipStream_t>(stream)),
                      "dsp_sts_fit launch");
}

dsp_status dsp_ece(const float* z, const int32_t* n_acc, const float* T, int N, int gamma,
                   int n_bins, double* ece, void* ws, size_t ws_bytes, void* stream)
{
    if (!z || !n_acc || !ece || !ws)
        return fail(DSP_ERR_INVALID_ARG, "dsp_ece: null pointer argument");
    if (N <= 0 || gamma <= 0 || n_bins <= 0)
        return fail(DSP_ERR_INVALID_ARG, "dsp_ece: bad sizes N=%d gamma=%d n_bins=%d", N, gamma, n_bins);
    if (n_bins > dsp::kEceMaxBins)
        return fail(DSP_ERR_UNSUPPORTED, "dsp_ece: n_bins = %d exceeds %d", n_bins, dsp::kEceMaxBins);
    if ((int64_t)N * gamma > dsp::kEceMaxPredictions)
        return fail(DSP_ERR_UNSUPPORTED, "dsp_ece: N * gamma = %lld exceeds 2^23",
                    (long long)N * gamma);
    const size_t need = dsp::ece_workspace_bytes();
    if (ws_bytes < need || !aligned16(ws))
        return fail(DSP_ERR_WORKSPACE, "dsp_ece: workspace of %zu bytes (16-byte aligned), %zu needed",
                    ws_bytes, need);
    return hip_status(dsp::launch_ece(z, n_acc, T, N, gamma, n_bins, ece, ws,
                                      static_cast<hipStream_t>(stream)),
                      "dsp_ece launch");
}

dsp_status dsp_schedule(const float* c, const float* sps, int B_max, double tau0, int mode,
                        int32_t* len, float* a, int32_t* B, int R, int gamma, void* stream)
{
    if (!c || !len || !a || !B || (mode != 0 && !sps))
        return fail(DSP_ERR_INVALID_ARG, "dsp_schedule: null pointer argument");
    if (R <= 0 || gamma <= 0)
        return fail(DSP_ERR_INVALID_ARG, "dsp_schedule: bad sizes R=%d gamma=%d", R, gamma);
    if (mode != 0 && mode != 1)
        return fail(DSP_ERR_INVALID_ARG, "dsp_schedule: mode must be 0 or 1 (got %d)", mode);
    if (mode == 1 && B_max < R)
        return fail(DSP_ERR_INVALID_ARG, "dsp_schedule: B_max = %d < R = %d", B_max, R);
    // tau0 2^48 plus the admitted sum (below R gamma 2^48 <= 2^62) must fit 64 bits
    if (!(tau0 >= 0.0) || !(tau0 < 16384.0))
        return fail(DSP_ERR_INVALID_ARG, "dsp_schedule: tau0 must be in [0, 2^14)");
    if (mode == 1 && (int64_t)R * gamma > dsp::kSchedMaxCand)
        return fail(DSP_ERR_UNSUPPORTED, "dsp_schedule: R * gamma = %lld exceeds %d",
                    (long long)R * gamma, dsp::kSchedMaxCand);
    const uint64_t S0 = (uint64_t)std::floor(tau0 * 281474976710656.0);
    return hip_status(dsp::launch_schedule(c, sps, B_max, S0, mode, len, a, B, R, gamma,
                                           static_cast<hipStream_t>(stream)),
                      "dsp_schedule launch");
}

dsp_status dsp_verify(const void* target, int64_t target_rs, int64_t target_ps, const void* base,
                      int64_t base_rs, int64_t base_ps, dsp_dtype dtype, const uint16_t* E,
                      const uint16_t* W2, const int32_t* anchor, const int32_t* tok,
                      const float* q, const double* stats, const int32_t* len, int8_t* accept,
                      int32_t* n_accept, int32_t* y, float* p, int R, int gamma, int V, int r,
                      unsigned flags, float temperature, uint64_t seed, uint32_t round, void* ws,
                      size_t ws_bytes, void* stream)
{
    return verify_impl(target, target_rs, target_ps, base, base_rs, base_ps, dtype, E, W2, anchor, tok,
                       q, stats, len, accept, n_accept, y, p, R, gamma, V, r, flags, temperature, seed,
                       round, ws, ws_bytes, stream, nullptr);
}

dsp_status dsp_verify_rnn(const void* target, int64_t target_rs, int64_t target_ps, const void* base,
                          int64_t base_rs, int64_t base_ps, dsp_dtype dtype, const uint16_t* E,
                          const uint16_t* W2, const uint16_t* S, const int32_t* anchor,
                          const int32_t* tok, const float* q, const double* stats, const int32_t* len,
                          int8_t* accept, int32_t* n_accept, int32_t* y, float* p, int R, int gamma,
                          int V, int r, unsigned flags, float temperature, uint64_t seed,
                          uint32_t round, void* ws, size_t ws_bytes, void* stream)
{
    if (!S) return fail(DSP_ERR_INVALID_ARG, "dsp_verify_rnn: null S");
    if (!aligned16(S)) return fail(DSP_ERR_INVALID_ARG, "dsp_verify_rnn: S must be 16-byte aligned");
    if ((int64_t)R * gamma * r > dsp::kRnnMaxStateElems)
        return fail(DSP_ERR_UNSUPPORTED, "dsp_verify_rnn: R * gamma * r exceeds 2^31 - 1");
    if (path_of(flags) == DSP_PATH_PERSISTENT)
        return fail(DSP_ERR_UNSUPPORTED, "dsp_verify_rnn: the recurrent head runs the streaming path only");
    return verify_impl(target, target_rs, target_ps, base, base_rs, base_ps, dtype, E, W2, anchor, tok,
                       q, stats, len, accept, n_accept, y, p, R, gamma, V, r, flags, temperature, seed,
                       round, ws, ws_bytes, stream, S);
}

}  // extern "C"

namespace {

dsp_status verify_impl(const void* target, int64_t target_rs, int64_t target_ps, const void* base,
                       int64_t base_rs, int64_t base_ps, dsp_dtype dtype, const uint16_t* E,
                       const uint16_t* W2, const int32_t* anchor, const int32_t* tok,
                       const float* q, const double* stats, const int32_t* len, int8_t* accept,
                       int32_t* n_accept, int32_t* y, float* p, int R, int gamma, int V, int r,
                       unsigned flags, float temperature, uint64_t seed, uint32_t round, void* ws,
                       size_t ws_bytes, void* stream, const uint16_t* S)
{
    if (!target || !base || !E || !W2 || !anchor || !tok || !q || !stats || !len || !accept ||
        !n_accept || !y || !p)
        return fail(DSP_ERR_INVALID_ARG, "dsp_verify: null pointer argument");
    if (dtype != DSP_F32 && dtype != DSP_BF16)
        return fail(DSP_ERR_INVALID_ARG, "dsp_verify: unknown dtype %d", (int)dtype);
    dsp_status st = check_markov(R, gamma, V, r);
    if (st != DSP_OK) return st;
    if (!(temperature >= 0.0f) || std::isinf(temperature))
        return fail(DSP_ERR_INVALID_ARG, "dsp_verify: temperature must be finite and >= 0");
    if (!known_path(flags)) return fail(DSP_ERR_INVALID_ARG, "dsp_verify: unknown flags %u", flags);
    st = check_strides("dsp_verify", "target", target_rs, target_ps);
    if (st != DSP_OK) return st;
    st = check_strides("dsp_verify", "base", base_rs, base_ps);
    if (st != DSP_OK) return st;
    if (!aligned16(target) || !aligned16(base) || !aligned16(E) || !aligned16(W2))
        return fail(DSP_ERR_INVALID_ARG, "dsp_verify: target, base, E and W2 must be 16-byte aligned");
    const size_t need = dsp::verify_workspace_bytes(R, gamma, V);
    if (!ws || ws_bytes < need)
        return fail(DSP_ERR_WORKSPACE, "dsp_verify: workspace of %zu bytes, %zu needed", ws_bytes,
                    need);
    if (!aligned16(ws))
        return fail(DSP_ERR_WORKSPACE, "dsp_verify: the workspace must be 16-byte aligned");
    return hip_status(dsp::launch_verify(target, dsp::RowStrides{target_rs, target_ps}, base,
                                         dsp::RowStrides{base_rs, base_ps}, dtype == DSP_BF16,
                                         path_of(flags), give_up_of(flags), E,
                                         W2, anchor, tok, q,
                                         stats, len, accept, n_accept, y, p, R, gamma, V, r,
                                         temperature, seed, round, ws,
                                         static_cast<hipStream_t>(stream), S),
                      "dsp_verify launch");
}

}  // namespace

namespace {

dsp_status tv_impl(const void* target, int64_t target_rs, int64_t target_ps, const void* base,
                   int64_t base_rs, int64_t base_ps, dsp_dtype dtype, const uint16_t* E,
                   const uint16_t* W2, const int32_t* anchor, const int32_t* tok, const double* stats,
                   double* alpha, int R, int gamma, int V, int r, float temperature, void* ws,
                   size_t ws_bytes, void* stream, const uint16_t* S);

}  // namespace

extern "C" dsp_status dsp_tv_accept(const void* target, int64_t target_rs, int64_t target_ps,
                                    const void* base, int64_t base_rs, int64_t base_ps,
                                    dsp_dtype dtype, const uint16_t* E, const uint16_t* W2,
                                    const int32_t* anchor, const int32_t* tok, const double* stats,
                                    double* alpha, int R, int gamma, int V, int r, float temperature,
                                    void* ws, size_t ws_bytes, void* stream)
{
    return tv_impl(target, target_rs, target_ps, base, base_rs, base_ps, dtype, E, W2, anchor, tok,
                   stats, alpha, R, gamma, V, r, temperature, ws, ws_bytes, stream, nullptr);
}

extern "C" dsp_status dsp_tv_accept_rnn(const void* target, int64_t target_rs, int64_t target_ps,
                                        const void* base, int64_t base_rs, int64_t base_ps,
                                        dsp_dtype dtype, const uint16_t* E, const uint16_t* W2,
                                        const uint16_t* S, const int32_t* anchor, const int32_t* tok,
                                        const double* stats, double* alpha, int R, int gamma, int V,
                                        int r, float temperature, void* ws, size_t ws_bytes,
                                        void* stream)
{
    if (!S) return fail(DSP_ERR_INVALID_ARG, "dsp_tv_accept_rnn: null S");
    if (!aligned16(S)) return fail(DSP_ERR_INVALID_ARG, "dsp_tv_accept_rnn: S must be 16-byte aligned");
    if ((int64_t)R * gamma * r > dsp::kRnnMaxStateElems)
        return fail(DSP_ERR_UNSUPPORTED, "dsp_tv_accept_rnn: R * gamma * r exceeds 2^31 - 1");
    return tv_impl(target, target_rs, target_ps, base, base_rs, base_ps, dtype, E, W2, anchor, tok,
                   stats, alpha, R, gamma, V, r, temperature, ws, ws_bytes, stream, S);
}

namespace {

dsp_status tv_impl(const void* target, int64_t target_rs, int64_t target_ps, const void* base,
                   int64_t base_rs, int64_t base_ps, dsp_dtype dtype, const uint16_t* E,
                   const uint16_t* W2, const int32_t* anchor, const int32_t* tok, const double* stats,
                   double* alpha, int R, int gamma, int V, int r, float temperature, void* ws,
                   size_t ws_bytes, void* stream, const uint16_t* S)
{
    if (!target || !base || !E || !W2 || !anchor || !tok || !stats || !alpha)
        return fail(DSP_ERR_INVALID_ARG, "dsp_tv_accept: null pointer argument");
    if (dtype != DSP_F32 && dtype != DSP_BF16)
        return fail(DSP_ERR_INVALID_ARG, "dsp_tv_accept: unknown dtype %d", (int)dtype);
    dsp_status st = check_markov(R, gamma, V, r);
    if (st != DSP_OK) return st;
    if ((int64_t)R * gamma > (int64_t)INT32_MAX / 4)
        return fail(DSP_ERR_UNSUPPORTED, "dsp_tv_accept: R * gamma too large");
    if (!(temperature > 0.0f) || std::isinf(temperature))
        return fail(DSP_ERR_INVALID_ARG, "dsp_tv_accept: temperature must be finite and > 0");
    st = check_strides("dsp_tv_accept", "target", target_rs, target_ps);
    if (st != DSP_OK) return st;
    st = check_strides("dsp_tv_accept", "base", base_rs, base_ps);
    if (st != DSP_OK) return st;
    if (!aligned16(target) || !aligned16(base) || !aligned16(E) || !aligned16(W2))
        return fail(DSP_ERR_INVALID_ARG, "dsp_tv_accept: target, base, E and W2 must be 16-byte aligned");
    const size_t need = dsp::tv_workspace_bytes(R, gamma, V);
    if (!ws || ws_bytes < need)
        return fail(DSP_ERR_WORKSPACE, "dsp_tv_accept: workspace of %zu bytes, %zu needed", ws_bytes,
                    need);
    if (!aligned16(ws))
        return fail(DSP_ERR_WORKSPACE, "dsp_tv_accept: the workspace must be 16-byte aligned");
    return hip_status(dsp::launch_tv_accept(target, dsp::RowStrides{target_rs, target_ps}, base,
                                            dsp::RowStrides{base_rs, base_ps}, dtype == DSP_BF16, E, W2,
                                            anchor, tok, stats, alpha, R, gamma, V, r, temperature,
                                            ws, static_cast<hipStream_t>(stream), S),
                      "dsp_tv_accept launch");
}

}  // namespace

extern "C" dsp_status dsp_schedule_async(const float* c, const float* c_hist, const float* sps,
                                         int B_max, double tau0, int32_t* len, float* a, int32_t* B,
                                         int32_t* K, int R, int gamma, void* stream)
{
    if (!c || !c_hist || !sps || !len || !a || !B || !K)
        return fail(DSP_ERR_INVALID_ARG, "dsp_schedule_async: null pointer argument");
    if (R <= 0 || gamma <= 0)
        return fail(DSP_ERR_INVALID_ARG, "dsp_schedule_async: bad sizes R=%d gamma=%d", R, gamma);
    if (B_max < R)
        return fail(DSP_ERR_INVALID_ARG, "dsp_schedule_async: B_max = %d < R = %d", B_max, R);
    if (!(tau0 >= 0.0) || !(tau0 < 16384.0))
        return fail(DSP_ERR_INVALID_ARG, "dsp_schedule_async: tau0 must be in [0, 2^14)");
    if ((int64_t)R * gamma > dsp::kSchedMaxCand)
        return fail(DSP_ERR_UNSUPPORTED, "dsp_schedule_async: R * gamma = %lld exceeds %d",
                    (long long)R * gamma, dsp::kSchedMaxCand);
    const uint64_t S0 = (uint64_t)std::floor(tau0 * 281474976710656.0);
    return hip_status(dsp::launch_schedule_async(c, c_hist, sps, B_max, S0, len, a, B, K, R, gamma,
                                                 static_cast<hipStream_t>(stream)),
                      "dsp_schedule_async launch");
}

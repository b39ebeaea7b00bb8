// dsp_launch.h -- host-side launchers of the gfx950 kernels (internal to libdsp).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsp {

constexpr int kSchedMaxCand = 16384;   // R * gamma limit of the one-workgroup scheduler
constexpr int kGammaMax = 64;
constexpr int kVocabMax = 2048 * 256;  // pick workgroups hold up to 8 tiles per thread

// Element strides of a logit tensor: element (n, k, v) of request n, position k
// is p[n * rs + k * ps + v]; the vocabulary is contiguous.
struct RowStrides {
    int64_t rs;   // between requests
    int64_t ps;   // between positions
};

// True when every row starts on a 16-byte boundary of a 16-byte-aligned tensor
// (align = elements per 16 bytes) and a row is whole 8-element chunks.
__host__ __device__ inline bool rows_vec(RowStrides s, int V, int align)
{
    return (V % 8) == 0 && (s.rs % align) == 0 && (s.ps % align) == 0;
}

size_t draft_workspace_bytes(int R, int V);

// Bytes of the per-device static scratch that dsp_draft_step_noalloc uses as its
// workspace, and its device address on the current device (looked up once per
// device with hipGetSymbolAddress).
constexpr size_t kStaticScratchBytes = (size_t)16 << 20;
hipError_t static_scratch(void** ptr);
size_t verify_workspace_bytes(int R, int gamma, int V);
// the error word of a workspace: nonzero when a bounded wait of the last call
// on it gave up
const unsigned* draft_error_word(const void* ws, int R, int V);
const unsigned* verify_error_word(const void* ws, int R, int gamma, int V);
int pass_req_per_wg(int count_max, int n_vt);

// implementation paths of the draft and the residual draws: automatic
// (persistent where it fits), streaming only, persistent only
// (hipErrorNotSupported where it does not fit)
constexpr int kPathAuto = 0;
constexpr int kPathStream = 1;
constexpr int kPathPersistent = 2;

// Geometry of a persistent launch for vocabulary V on the current device:
// units per wave (0: none fits), tiles, compute units; false when none fits.
struct RunGeometry {
    int tu, n_t, ncu;
};
bool run_geometry(int V, RunGeometry* g);

hipError_t launch_draft_step(const void* base, RowStrides bs, bool bf16, const uint16_t* E,
                             const uint16_t* W2,
                             const int32_t* anchor, int32_t* tok, float* q, double* stats, int R,
                             int gamma, int V, int r, int k, int n_steps, int path,
                             bool give_up, float temperature, uint64_t seed, uint32_t round,
                             void* ws, hipStream_t s, const uint16_t* A = nullptr,
                             uint16_t* S = nullptr);
// (A, S non-null: the recurrent head with matrix A [r, r] and states S [R, gamma, r],
// streaming launches only.)

hipError_t launch_confidence(const uint16_t* h, const uint16_t* E, const int32_t* anchor,
                             const int32_t* tok, const float* w, const float* T,
                             const float* offset, float* c, int R, int gamma, int d, int V, int r,
                             hipStream_t s);

// Sequential temperature scaling: candidates per grid stage, most sample chunks of
// one objective launch; calibration-error bins.
constexpr int kStsGrid = 256;
constexpr int kStsMaxChunks = 1024;
constexpr int kEceMaxBins = 64;
constexpr int64_t kEceMaxPredictions = (int64_t)1 << 23;   // exact 2^-40 bin sums fit 64 bits
size_t sts_workspace_bytes(int N);
size_t ece_workspace_bytes();
hipError_t launch_sts_fit(const float* z, const int32_t* acc, int N, int gamma, double t_lo,
                          double t_hi, float* T, double* nll, void* ws, hipStream_t s);
hipError_t launch_ece(const float* z, const int32_t* nacc, const float* T, int N, int gamma, int M,
                      double* ece, void* ws, hipStream_t s);

hipError_t launch_schedule(const float* c, const float* sps, int B_max, uint64_t S0, int mode,
                           int32_t* len, float* a, int32_t* B, int R, int gamma, hipStream_t s);

size_t tv_workspace_bytes(int R, int gamma, int V);
hipError_t launch_tv_accept(const void* target, RowStrides ts, const void* base, RowStrides bs,
                            bool bf16, const uint16_t* E, const uint16_t* W2, const int32_t* anchor,
                            const int32_t* tok, const double* stats, double* alpha, int R, int gamma,
                            int V, int r, float temperature, void* ws, hipStream_t s,
                            const uint16_t* S = nullptr);

hipError_t launch_schedule_async(const float* c, const float* c_hist, const float* sps, int B_max,
                                 uint64_t S0, int32_t* len, float* a, int32_t* B, int32_t* K, int R,
                                 int gamma, hipStream_t s);

hipError_t launch_verify(const void* target, RowStrides ts, const void* base, RowStrides bs,
                         bool bf16, int path, bool give_up, const uint16_t* E,
                         const uint16_t* W2, const int32_t* anchor, const int32_t* tok,
                         const float* q, const double* stats, const int32_t* len, int8_t* accept,
                         int32_t* n_accept, int32_t* y, float* p, int R, int gamma, int V, int r,
                         float temperature, uint64_t seed, uint32_t round, void* ws,
                         hipStream_t s, const uint16_t* S = nullptr);
// (S non-null: the recurrent head's states [R, gamma, r] give the draft law at a
// rejection; the residual draws run the streaming passes.)

// Largest R gamma r for the recurrent head (its state rows are indexed with
// 32-bit offsets).
constexpr int64_t kRnnMaxStateElems = ((int64_t)1 << 31) - 1;

}  // namespace dsp

// draft_pass.h -- shared pieces of the software-pipelined streaming passes (gfx950):
// the W2 fragment layout and its staging through swizzled LDS, raw buffer
// resources with hardware range checks, and the launch-time check that a call
// fits their 32-bit offsets.  The draft pass (draft_pass_wide.h, two workgroups
// per CU) and the residual pass (resid_pass.h, eight waves) build on them.
//
// A pass holds its workgroup's W2 tile in registers as MFMA A fragments and
// streams request blocks of 32: a block's base logits and embedding rows are
// read a whole row segment per group of lanes (per-lane reads of 16 bytes from
// 32 rows turn every lane into its own cache access and half-line request, and
// a pass then runs at the L1's limit of requests in flight) and reach the MFMA
// layout through LDS.  Every logit is the sum of the same MFMA sequence
// (k-steps 0..15 from zero) and the base logit, as in bias_pass_kernel and the
// picks' tile rebuild.
#pragma once

#include "tile_pass.h"

namespace dsp {

constexpr int kDpWaves = 8;                 // waves per workgroup of the residual pass
constexpr int kDpThreads = 64 * kDpWaves;
constexpr int kDpRing = 2;                  // blocks of logit words held in registers

// Vocabulary offset (within the wave's 32 columns) of MFMA row i: output
// register j of lane l is row 8 (j / 4) + 4 (l / 32) + j % 4, which this maps
// to column 16 (l / 32) + j.
__device__ __forceinline__ int dp_arow(int i) { return 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3); }

// slot of 16-byte word c of staged W2 row rho: each 16-lane phase of a fragment
// read (rows dp_arow(i) of one half) meets 16 distinct bank groups, and a row's
// words stay a permutation of its slots
__device__ __forceinline__ int dp_slot(int rho, int c) { return c ^ ((rho & 15) ^ (((rho >> 4) & 1) << 3)); }

// The A fragments of wave w of eight (32 columns each): W2 rows
// v0 + 32 w + dp_arow(i), k-steps 0..15.  Each 64-row quarter of the 256-row tile
// is read contiguously into LDS; waves 2 q and 2 q + 1 then read their fragments
// from quarter q.
template <class Lds>   // an LDS union whose member w2 is [2][64][kRankMax / 8] words
__device__ __forceinline__ void dp_stage_w2(const uint16_t* __restrict__ W2, int V, int r, int v0,
                                            Lds& L, bf16x8 (&a)[kKSteps])
{
    constexpr int kWordsRow = kRankMax / 8;                  // 32 words of 16 bytes
    constexpr int kPer = 64 * kWordsRow / kDpThreads;        // 4 words per quarter
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    uint4 cur[kPer], nxt[kPer];
    auto fetch = [&](int q, uint4* u) {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int f = i * kDpThreads + tid, rho = f / kWordsRow, c = f % kWordsRow;
            const int v = v0 + 64 * q + rho;
            u[i] = (v < V && 8 * c < r)
                       ? *reinterpret_cast<const uint4*>(W2 + (int64_t)v * r + 8 * c)
                       : make_uint4(0, 0, 0, 0);
        }
    };
    fetch(0, cur);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        if (q + 1 < 4) fetch(q + 1, nxt);
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int f = i * kDpThreads + tid, rho = f / kWordsRow, c = f % kWordsRow;
            L.w2[q & 1][rho][dp_slot(rho, c)] = cur[i];
        }
        lds_barrier();
        if ((wave >> 1) == q) {
            const int rho = 32 * (wave & 1) + dp_arow(lane & 31), h = lane >> 5;
#pragma unroll
            for (int ks = 0; ks < kKSteps; ++ks) a[ks] = as_bf16x8(L.w2[q & 1][rho][dp_slot(rho, 2 * ks + h)]);
        }
#pragma unroll
        for (int i = 0; i < kPer; ++i) cur[i] = nxt[i];
    }
    lds_barrier();   // the buffers are reused for the embedding tiles
}

// Raw buffer resources: a base in scalar registers, a 32-bit byte offset per
// lane and a range the hardware checks -- a load at or past the range returns
// zeros, a store there is dropped.  Rows past the end, bias rows that select
// none and idle lanes thus take offsets out of range instead of address masks
// and branches, and the per-block address arithmetic of the logit words is
// scalar.  Every range here stays below 2^31 bytes (dp_offsets_fit), so
// kBufOut lies outside all of them.
typedef __amdgpu_buffer_rsrc_t BufRsrc;
constexpr int kBufWord3 = 0x00020000;       // raw access, 32-bit data format
constexpr uint32_t kBufOut = 0x80000000u;

__device__ __forceinline__ BufRsrc buf_rsrc(const void* p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, kBufWord3);
}

// 16-byte loads: kBufNt streams (the logit words, read once)
constexpr int kBufNt = 2;
template <int AUX>
__device__ __forceinline__ uint4 buf_load16(BufRsrc r, uint32_t off)
{
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// the maximum of three values without the quieting of signalling NaNs that
// fmaxf adds to operands it did not compute itself (values read back from LDS)
__device__ __forceinline__ float max3_lds(float a, float b, float c)
{
    float d;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
    return d;
}

// Whether a call's tensors fit the pass's 32-bit offsets: the 32 rows of a
// block of logit words, and the bias table, whose row index and row stride in
// bytes also have to fit the 24-bit multiply and whose offsets (row e_rows
// included, the out-of-range row) stay below 2^31 bytes.
__host__ __device__ inline bool dp_offsets_fit(RowStrides bs, int64_t e_rows, int64_t e_rs, int r)
{
    const int64_t lim = (int64_t)1 << 31, lim24 = (int64_t)1 << 24;
    return bs.rs >= 0 && bs.ps >= 0 && (kPassBlock * bs.rs + kVocabTile) * 2 < lim &&
           e_rows < lim24 && e_rs >= r && e_rs * 2 < lim24 && e_rows * e_rs * 2 < lim;
}

}  // namespace dsp

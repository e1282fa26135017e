// Internal declarations shared by the C-ABI layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dspk {

constexpr int kWave = 64;          // CDNA wavefront width
constexpr int kWavesPerWG = 4;     // waves per workgroup in the projection kernels
constexpr int kTilesPerWave = 4;   // 16-column MFMA tiles per wave
constexpr int kBlockCols = 16 * kTilesPerWave;          // columns per wave (64)
constexpr int kWGCols = kBlockCols * kWavesPerWG;       // columns per workgroup (256)
constexpr int kSbChunk = 40;       // K groups of scales/biases a wave stages in LDS at a time
constexpr int kMaxHeadK = 8192;    // largest hidden size of the vocabulary head
constexpr int kMaxGrouped = 4;
constexpr int kMaxRows = 32;

// One weight of a (possibly grouped) projection launch, with its work split.
//   A wave owns 64 output columns and one K range ("split") of a weight; the
//   four waves of a workgroup take four neighbouring column blocks of the same
//   split, so they read the same activation rows.  With splits > 1, each split
//   publishes its partial sums and the last workgroup of a 256-column group to
//   arrive adds them in split order.
struct GemmProblem {
    const void *codes;        // packed codes (bits 4/8) or bf16 weights (bits 16)
    const uint16_t *scales;   // fp16 [n][k/64]
    const uint16_t *biases;   // fp16 [n][k/64]
    void *y;                  // output [m][ldy]
    float *partial;           // workspace: [splits][m][n] fp32 (splits > 1)
    uint32_t *counters;       // workspace: [ncg] arrival counters (splits > 1)
    int64_t ldy;
    int32_t n, k;
    int32_t ncg;              // 256-column groups: ceil(n / 256)
    int32_t splits;           // K ranges per column group
    int32_t split_groups;     // K groups per split (the last may be shorter)
    int32_t wg_begin;         // first workgroup of this problem in the grid
};

struct GemmLaunch {
    GemmProblem p[kMaxGrouped];
    const uint16_t *x;        // bf16 rows [m][ldx]
    int64_t ldx;
    int32_t count;
    int32_t m;
    int32_t y_bf16;           // store y as bf16 instead of fp32
    // vocabulary-head epilogue (argmax kernel only)
    int32_t *argmax;
    float *logits;
    int64_t ldl;
    unsigned long long *keys; // workspace: [workgroups][kMaxRows] per-workgroup row maxima
    uint32_t *done;           // workspace: arrival counter
};

// Work split of one weight (host side).
struct GemmPlan {
    int32_t ncg, splits, split_groups;
    size_t ws_bytes;          // workspace this weight needs (0 when splits == 1)
};
GemmPlan plan_gemm(int32_t n, int32_t k, int32_t m, bool single_split);
size_t lmhead_workspace_bytes(int32_t v);

hipError_t launch_qgemm(const GemmLaunch &L, int bits, int grid, hipStream_t s);
hipError_t launch_lmhead(const GemmLaunch &L, int bits, int grid, hipStream_t s);

// Acceptance kernels.
hipError_t launch_accept_greedy(const int32_t *t, const int32_t *d, int32_t b, int32_t m_rows,
                                int32_t *accept_len, int32_t *committed, hipStream_t s);

constexpr int kSampleChunk = 4096;   // logits per workgroup in the sampling kernels
size_t sample_workspace_bytes(int32_t v, int32_t m_rows);
hipError_t launch_accept_sample(const float *z, int64_t ldz, const float *q, int64_t ldq,
                                const int32_t *d, const float *u, int32_t m_rows, int32_t v,
                                float temperature, int32_t *accept_len, int32_t *committed,
                                void *ws, hipStream_t s);

}  // namespace dspk

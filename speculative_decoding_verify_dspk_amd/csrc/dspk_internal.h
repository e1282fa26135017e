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
constexpr int kMaxGrouped = 4;
constexpr int kMaxRows = 32;

// Work of a projection launch is a list of quads: (weight, 64-column block,
// four consecutive K stages), one stage per wave of a workgroup.  Quads are
// numbered weight by weight, block by block, K first, and each workgroup of
// the persistent grid takes one contiguous range of them ("stream-K"), so
// every workgroup streams the same number of weight bytes.  A block whose
// quads straddle workgroups is finished by the last of them to arrive, adding
// the pieces in workgroup order.  Grouped weights share k, bits and rows.
struct GemmProblem {
    const void *codes;        // packed codes (bits 4/8) or bf16 weights (bits 16)
    const uint16_t *scales;   // fp16 [n][k/64]
    const uint16_t *biases;   // fp16 [n][k/64]
    void *y;                  // output [m][ldy]
    int64_t ldy;
    int32_t n;
    int32_t cg_begin;         // first block of this weight in the launch
};

struct GemmLaunch {
    GemmProblem p[kMaxGrouped];
    const uint16_t *x;        // bf16 rows [m][ldx]
    int64_t ldx;
    int32_t count;
    int32_t m;
    int32_t k;
    int32_t nst;              // K stages per block
    int32_t nq;               // quads per block: ceil(nst / 4)
    int32_t quads;            // quads of the launch
    int32_t total_cg;         // blocks of the launch
    int32_t y_bf16;           // store y as bf16 instead of fp32
    // workspace
    uint32_t *counters;       // [total_cg][4] arrival counters of split blocks
    float *partial;           // [grid][2][4][MT][64][4] partial sums of split blocks
    // vocabulary-head epilogue (argmax kernel only)
    int32_t *argmax;
    float *logits;
    int64_t ldl;
    unsigned long long *keys; // [grid][kMaxRows] per-workgroup row maxima
    uint32_t *done;           // arrival counter over workgroups
};

// Launch plan of one (possibly grouped) projection call (host side).
struct GemmPlan {
    int32_t nst, nq, quads, grid, total_cg;
    bool fits;                // quads * grid < 2^31 (the kernel's index range)
    size_t off_counters, off_keys, off_partial, ws_bytes;
};
// K elements of one wave's stage for a weight format
int stage_k(int bits);
GemmPlan plan_gemm(int count, const int32_t *n, int32_t k, int32_t m, int bits, bool argmax);
int device_cus();

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

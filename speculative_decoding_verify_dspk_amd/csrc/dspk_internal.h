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

// Tiled weight layout (the format every projection kernel reads; written by
// dspk_qweight_pack).  A weight is cut into units of 64 output columns times
// tile_k(bits) K elements, stored unit after unit, K fastest within a
// 64-column block, blocks in column order.  A unit is tile_code_slots(bits)
// slots of 1 KiB (one 16-byte piece per lane of a wave, in the MFMA operand
// order of that lane) -- 8 for 4/8-bit and bf16, 4 for 2-bit, 6 for 3-bit --
// followed, for quantised formats, by the scale/bias dwords of its groups
// (16 columns x tile_k/64 groups x 4 tiles).  2- and 3-bit units span four
// groups like 4-bit ones, so a lane's activation registers stay those of
// the 4-bit kernel.
constexpr int tile_k(int bits) { return bits == 16 ? 64 : bits == 8 ? 128 : 256; }
constexpr int tile_groups(int bits) { return tile_k(bits) / 64; }
constexpr int tile_code_slots(int bits) { return bits == 2 ? 4 : bits == 3 ? 6 : 8; }
constexpr int tile_unit_bytes(int bits) {
    return 1024 * tile_code_slots(bits) + (bits == 16 ? 0 : 256 * tile_groups(bits));
}
constexpr bool supported_bits(int bits) { return bits == 2 || bits == 3 || bits == 4 || bits == 8 || bits == 16; }
size_t tiled_bytes(int32_t n, int32_t k, int bits);
hipError_t launch_pack(int32_t n, int32_t k, int bits, const void *codes, const uint16_t *scales,
                       const uint16_t *biases, void *tiles, hipStream_t s);

// Register-ring depth (units in flight per wave) and workgroups per CU of the
// projection kernel, by weight format, 16-row tiles and kind (head or
// projection), as measured on MI355X:
//  * 8-bit and bf16, <= 16 rows: heads a 2-deep ring at two workgroups per
//    CU (<= 244 VGPRs, no scratch; no ring at three per CU: head 77 -> 83
//    us).  8-bit projections no ring at two per CU (Qwen3-4B layer 63.5 ->
//    61.9 us, 27B-shaped layer 105.7 -> 102.5 us against the 2-deep ring).
//  * 2/3/4-bit, <= 16 rows: their units span four groups, and a 2-deep ring
//    spills (100-260 B/lane); with no ring they fit three workgroups per CU
//    without scratch: 9B-shaped 4-bit layer 103 -> 83 us, head 88 -> 80 us.
//  * 17..32 rows (twice the activation and accumulator registers): no ring,
//    two workgroups per CU for projections (27B-shaped layer 138 -> 120 us
//    against a 2-deep ring at one per CU); the head, whose workgroups stream
//    many units each, no ring at three per CU (27B-shaped head 197 -> 162
//    us); 2/3/4-bit heads keep a 2-deep ring at one per CU.
constexpr int kernel_depth(int bits, int mt, bool argmax) {
    return mt == 1 ? (bits <= 4 || (bits == 8 && !argmax) ? 1 : 2) : (argmax && bits <= 4 ? 2 : 1);
}
constexpr int kernel_occ(int bits, int mt, bool argmax) {
    return mt == 1 ? (bits <= 4 ? 3 : 2) : (!argmax ? 2 : bits >= 8 ? 3 : 1);
}

// Work of a projection launch is a list of quads: (weight, 64-column block,
// four consecutive units), one unit per wave of a workgroup.  Quads are
// numbered weight by weight, block by block, K first, and each workgroup of
// the persistent grid takes one contiguous range of them ("stream-K"), so
// every workgroup streams the same number of weight bytes -- and, with the
// tiled layout, one contiguous run of memory.  A block whose quads straddle
// workgroups is finished by the last of them to arrive, adding the pieces in
// workgroup order.  Grouped weights share k, bits and rows.
struct GemmProblem {
    const void *tiles;        // tiled weight (tiled_bytes(n, k, bits) bytes)
    void *y;                  // output [m][ldy]
    int64_t ldy;
    int32_t n;
    int32_t cg_begin;         // first block of this weight in the launch
};

struct GemmLaunch {
    GemmProblem p[kMaxGrouped];
    const uint16_t *x;        // bf16 rows, chunk-major [k/8][ldx][8]
    int64_t ldx;
    int32_t count;
    int32_t m;
    int32_t k;
    int32_t nst;              // units per block: ceil(k / tile_k)
    int32_t nq;               // quads per block: ceil(nst / 4)
    int32_t quads;            // quads of the launch
    int32_t total_cg;         // blocks of the launch
    int32_t y_bf16;           // store y as bf16 instead of fp32
    // workspace
    int32_t pairs;            // > 0: workgroups b and b + pairs share a CU (weighted split), else 0
    uint32_t *counters;       // [total_cg][4] arrival counters of split blocks
    float *partial;           // [grid][2][4][MT][64][4] partial sums of split blocks
    // vocabulary-head epilogue (argmax kernel only)
    int32_t *argmax;
    float *logits;
    int64_t ldl;
    unsigned long long *keys; // [kMaxRows] row maxima over the grid (atomic max; cleared by the last workgroup)
    // optional greedy acceptance on the ids (head only; accept_len == NULL: none)
    const int32_t *draft;     // [acc_b][acc_rows - 1]
    int32_t acc_b, acc_rows;  // acc_b * acc_rows == m
    int32_t *accept_len;      // [acc_b]
    int32_t *committed;       // [acc_b][acc_rows]
    uint32_t *done;           // arrival counter over workgroups
};

// One prefill projection (many rows, row-major activations).
struct PrefillArgs {
    const void *tiles;        // tiled weight
    int32_t n, k, nst;        // columns, inputs, units per 64-column block
    int32_t nblocks;          // 64-column blocks
    const uint16_t *x;        // bf16 rows [m][ldx]
    int64_t ldx;
    int32_t m;
    void *y;                  // [m][ldy], fp32 or bf16
    int64_t ldy;
    int32_t y_bf16;
};
hipError_t launch_prefill(const PrefillArgs &a, int bits, hipStream_t s);

// Launch plan of one (possibly grouped) projection call (host side).
struct GemmPlan {
    int32_t nst, nq, quads, grid, total_cg;
    int32_t pairs;            // see GemmLaunch::pairs
    bool fits;                // quads * grid < 2^31 (the kernel's index range)
    size_t off_counters, off_keys, off_partial, ws_bytes;
};
GemmPlan plan_gemm(int count, const int32_t *n, int32_t k, int32_t m, int bits, bool argmax);
int device_cus();

hipError_t launch_qgemm(const GemmLaunch &L, int bits, int grid, hipStream_t s);
hipError_t launch_lmhead(const GemmLaunch &L, int bits, int grid, hipStream_t s);

// Acceptance kernels.
hipError_t launch_accept_greedy(const int32_t *t, const int32_t *d, int32_t b, int32_t m_rows,
                                int32_t *accept_len, int32_t *committed, hipStream_t s);

constexpr int kSampleChunk = 4096;   // logits per workgroup in the sampling kernels
size_t sample_workspace_bytes(int32_t v, int32_t m_rows);
struct SampleParams {
    const float *z;
    int64_t ldz;
    const float *q;
    int64_t ldq;
    const int32_t *d;
    const float *u;
    int32_t m_rows, v;
    float temperature;
    int32_t top_k;            // 0: off
    float top_p;              // 1: off
    float presence, frequency;
    const int32_t *counts;    // or NULL
    int32_t *accept_len, *committed;
    void *ws;
};
hipError_t launch_accept_sample(const SampleParams &p, hipStream_t s);

}  // namespace dspk

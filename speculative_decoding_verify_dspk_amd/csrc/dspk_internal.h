// Internal declarations shared by the C-ABI layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime_api.h>
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
//    against a 2-deep ring at one per CU) and for the 8-bit head (170
//    VGPRs; against three per CU, 27B-shaped head at 17 / 24 / 32 rows
//    173-178 / 188-190 / 201 -> 170-171 / 178-180 / 186-187 us, Qwen3-8B-
//    shaped 139-141 / 149-150 / 161 -> 139-141 / 143-144 / 149 us; a
//    2-deep ring there spills 388 B/lane); the bf16 head no ring at three
//    per CU; 2/3/4-bit heads keep a 2-deep ring at one per CU.
constexpr int kernel_depth(int bits, int mt, bool argmax) {
    return mt == 1 ? (bits <= 4 || (bits == 8 && !argmax) ? 1 : 2) : (argmax && bits <= 4 ? 2 : 1);
}
constexpr int kernel_occ(int bits, int mt, bool argmax) {
    return mt == 1 ? (bits <= 4 ? 3 : 2) : (!argmax || bits == 8 ? 2 : bits > 8 ? 3 : 1);
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
    const uint16_t *x;        // bf16 rows, row-major [m][ldx] (ldx % 8 == 0, 16-byte aligned)
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
    float *partial;           // [grid][2][4][MT][64][4] partial sums of split blocks (MT: this launch's row tiles)
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
    int32_t block_rows;       // rows per workgroup: 64 or 128
    int32_t ks;               // K splits; > 1 needs the two regions below
    float *part;              // partial tiles [tile][wave][split][row tile][column tile][2][64][2]
    uint32_t *ctr;            // arrival counters [tile][wave], zero between calls
};
hipError_t launch_prefill(const PrefillArgs &a, int bits, hipStream_t s);

// Launch plan of one (possibly grouped) projection call (host side).
//
// Workspace of the projection and head kernels, at offsets that depend on
// nothing but the device's CU count, so that one buffer can serve any
// sequence of projection and head calls ordered on one stream:
//   [0, 256)            head arrival counter (reset by the head's last workgroup)
//   [256, 512)          row keys of the head argmax, kMaxRows x 8 B (reset likewise)
//   [512, 512 + P)      partial sums of split blocks, P = partial_region_bytes():
//                       every piece is written before it is read, so stale
//                       contents are harmless
//   [512 + P, ...)      arrival counters, 4 per 64-column block of the call
//                       (each reset by the last arrival of its block)
// Every completed call leaves the counters, keys and arrival word at zero.
constexpr int kMaxOcc = 3;          // most workgroups per CU of any kernel_occ()
constexpr size_t kWsHead = 512;     // arrival counter + row keys
static_assert(kernel_occ(2, 1, true) <= kMaxOcc && kernel_occ(8, 1, true) <= kMaxOcc &&
                  kernel_occ(8, 2, true) <= kMaxOcc && kernel_occ(2, 2, true) <= kMaxOcc &&
                  kernel_occ(8, 1, false) <= kMaxOcc && kernel_occ(8, 2, false) <= kMaxOcc &&
                  kernel_occ(2, 1, false) <= kMaxOcc && kernel_occ(2, 2, false) <= kMaxOcc,
              "the partial-sum region is sized for kMaxOcc workgroups per CU");
// bytes of the partial-sum region: [grid][2 sides][4 waves][MT <= 2][64 lanes][4 floats]
constexpr size_t partial_region_bytes(int cus) {
    return (size_t)kMaxOcc * (size_t)cus * 2 * kWavesPerWG * 2 * kWave * 16;
}
// How a projection launch is decomposed (head launches are always stream-K):
//   kStreamK: persistent workgroups over contiguous quad ranges (qgemm.hip);
//   kSlab:    one workgroup per 16-column tile over the whole K (slab.hip),
//             for launches whose tiles all fit on the device at once;
//   kDot:     the slab decomposition with the K reduction on the vector ALUs
//             (v_dot2_f32_bf16) instead of the matrix cores: 8-bit weights,
//             at most kDotMaxRows rows (other calls fall back to kAuto).
// kAuto picks by shape; the others force a decomposition (measurement, tests).
enum Variant : int { kAuto = 0, kStreamK = 1, kSlab = 2, kDot = 3 };
constexpr int kDotMaxRows = 4;
// Slab kernels: 8-bit and bf16 weights at up to kSlabLdsMaxRows rows stage
// the activations in LDS; other calls keep them in registers.  kAuto takes
// the slab kernel for 8-bit and bf16 calls of at most kSlabLdsMaxRows rows
// when the weights one CU streams for its tiles (tiles per CU x 16 x k) are
// at most kSlabAutoWeights and, at 9..16 rows, k <= kSlabAutoMaxKWide and the
// tiles fill at least three quarters of the CUs' last round.  A CU's tiles
// share one workgroup and one staged copy of x.  Launch times, slab vs
// stream-K, 8-bit, HIP events over back-to-back launches, 8 / 9 / 12 / 16 rows:
//   9B gate/up   (1536 tiles, k 4096)  20.2 / 21.4 / 20.6 / 21.8 vs 23.9 / 24.0 / 24.3 / 24.9 us
//   Qwen3-4B gate/up (1216, k 2560)    12.5 / 12.7 / 13.0 / 13.7 vs 17.7 / 17.6 / 17.9 / 18.6
//   27B o        (320 tiles, k 5120)   10.4 / 10.6 / 11.2 / 12.1 vs 11.4 / 11.4 / 11.5 / 11.7
//   Qwen3-4B down (160, k 9728)        12.0 / 12.0 / 12.8 / 14.0 vs 12.9 / 12.9 / 13.0 / 13.0
//   9B down      (256 tiles, k 12288)  15.5 / 15.3 / 16.4 / 17.6 vs 14.5 / 14.4 / 14.4 / 15.2
//   27B gate/up  (2176 tiles, k 5120)  46.0 / 47.0 / 50.1 / 56.1 vs 40.8 / 41.1 / 42.0 / 43.4
//   27B down     (320 tiles, k 17408)  28.1 / 28.8 / 30.9 / 34.1 vs 22.2 / 22.2 / 22.5 / 23.6
// (the 27B gate/up, 8.5 tiles per CU, runs in two rounds; at 1..8 rows the
// 9B gate/up as eight resident 2-wave tiles per CU had measured 24.2-25.6 us
// against stream-K's 26.9-27.5, bf16 34.3-34.8 against 40.2-40.5 us).
constexpr int kSlabLdsMaxRows = 16;
constexpr int64_t kSlabAutoWeights = 400 * 1024;
constexpr int32_t kSlabAutoMaxKWide = 5120;
int projection_variant();               // the process-wide setting (DSPK_VARIANT, or the setter)
int set_projection_variant(int v);      // previous setting, or -1 if v is not a Variant

struct GemmPlan {
    int32_t nst, nq, quads, grid, total_cg;
    int32_t slab_waves;       // > 0: slab kernel with this many waves per 16-column tile (4 * total_cg tiles)
    int32_t dot;              // with slab_waves: the dot-product form of the slab kernel
    int32_t pairs;            // see GemmLaunch::pairs
    bool fits;                // quads * grid < 2^31 (the kernel's index range)
    size_t off_counters, off_keys, off_partial, ws_bytes;
};
GemmPlan plan_gemm(int count, const int32_t *n, int32_t k, int32_t m, int bits, bool argmax);
// the same plan for a given CU count (host tests)
GemmPlan plan_gemm_cus(int count, const int32_t *n, int32_t k, int32_t m, int bits, bool argmax, int cus);
int device_cus();

hipError_t launch_qgemm(const GemmLaunch &L, int bits, int grid, hipStream_t s);
hipError_t launch_qgemm_slab(const GemmLaunch &L, int bits, int waves, hipStream_t s);
hipError_t launch_qgemm_dot(const GemmLaunch &L, int waves, hipStream_t s);   // 8-bit, m <= kDotMaxRows

// Device address of this GPU's file-scope scratch array (the workspace of the
// allocation-free projection call), fetched once per device; the first call on
// a device also enqueues the clearing of its counters on `s`.  The array serves
// calls of up to kScratchMaxBlocks 64-column blocks on up to kScratchCus CUs.
constexpr int kScratchCus = 256;
constexpr int64_t kScratchMaxBlocks = 4096;          // 262144 columns per call
hipError_t static_scratch(void **ptr, hipStream_t s);
size_t static_scratch_bytes();
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

// Host-side planning of the verify-pass launches: workgroup counts, the
// stream-K split of a projection, workspace offsets and buffer sizes.  No
// kernel code lives here, so the argument checks and plans of the C ABI can be
// built and exercised on a host without a GPU (with sanitizers).
#include <hip/hip_runtime_api.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>

#include "dspk_internal.h"
#include "prefill_plan.h"
#include "sample_layout.h"

namespace dspk {

int device_cus() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        cached[dev] = cus;
    }
    return cached[dev];
}

namespace {
int variant_from_env() {
    const char *e = getenv("DSPK_VARIANT");
    if (e == nullptr || strcmp(e, "auto") == 0) return kAuto;
    if (strcmp(e, "streamk") == 0) return kStreamK;
    if (strcmp(e, "slab") == 0) return kSlab;
    if (strcmp(e, "dot") == 0) return kDot;
    return kAuto;
}
std::atomic<int> g_variant{-1};
}  // namespace

int projection_variant() {
    int v = g_variant.load(std::memory_order_relaxed);
    if (v < 0) {
        int expected = -1;
        g_variant.compare_exchange_strong(expected, variant_from_env());
        v = g_variant.load(std::memory_order_relaxed);
    }
    return v;
}

int set_projection_variant(int v) {
    if (v != kAuto && v != kStreamK && v != kSlab && v != kDot) return -1;
    const int prev = projection_variant();
    g_variant.store(v, std::memory_order_relaxed);
    return prev;
}

// Waves per tile of the slab kernel for `slabs` tiles, or 0 when the tiles
// would not all be resident at once (a slab launch then takes 4 waves per
// tile and runs its tiles in more than one round).  At most 128 VGPRs per
// lane, a CU holds 16 waves: one tile of 16, two of 8, four of 4, five of 3
// or eight of 2; the most waves per tile that still fit all tiles are taken,
// for the most loads in flight per tile.  (Resident 3- or 2-wave tiles
// rather than a second round of 4-wave ones: Qwen3-4B-
// shaped gate/up, 4.75 tiles per CU, 18.4-19.7 -> 15.4-17.0 us at 1-8 rows;
// 9B-shaped gate/up, 6 tiles per CU, once the automatic choice takes it,
// 26.9-27.5 -> 24.2-25.6 us at 1-4 rows and bf16 40.2-40.5 -> 34.3-34.8 us.)
static int slab_waves_for(int64_t slabs, int cus) {
    if (slabs <= cus) return 16;
    if (slabs <= 2 * (int64_t)cus) return 8;
    if (slabs <= 4 * (int64_t)cus) return 4;
    if (slabs <= 5 * (int64_t)cus) return 3;
    if (slabs <= 8 * (int64_t)cus) return 2;
    return 0;
}

// The automatic choice: the slab kernel with activations in LDS (8-bit and
// bf16, at most 16 rows) when the weights a CU streams for its share of the
// tiles stay small -- it saves the stream-K kernel's split-block exchange and
// most of its small loads, but a CU given two long tiles (or many) streams
// them alone at the end.  Above 8 rows the staged activations grow with the
// rows and with K (a CU stages them once for all its tiles, but a long K
// still costs), and a launch whose CUs hold uneven tile counts waits for the
// fuller ones, so the slab is kept there only for K <= 5120 and tiles that
// fill at least three quarters of the CUs' last round.  Limits from launch
// durations of the 4B-, 9B- and 27B-shaped layers at 1, 8, 9, 12 and 16 rows
// (8-bit and bf16).
static bool slab_pays(int bits, int m, int64_t slabs, int32_t k, int cus) {
    if (!(bits == 8 || bits == 16) || m > kSlabLdsMaxRows) return false;
    const int64_t per_cu = (slabs + cus - 1) / cus;               // tiles per CU
    const int64_t weights = per_cu * 16 * (int64_t)k;             // weights one CU streams
    if (weights > kSlabAutoWeights) return false;
    return m <= 8 || (k <= kSlabAutoMaxKWide && (per_cu == 1 || 4 * slabs >= 3 * (int64_t)cus * per_cu));
}

GemmPlan plan_gemm_cus(int count, const int32_t *n, int32_t k, int32_t m, int bits, bool argmax, int cus) {
    GemmPlan p{};
    p.nst = (k + tile_k(bits) - 1) / tile_k(bits);
    p.nq = (p.nst + kWavesPerWG - 1) / kWavesPerWG;
    int64_t blocks = 0;
    for (int i = 0; i < count; ++i) blocks += (n[i] + kBlockCols - 1) / kBlockCols;
    p.total_cg = (int32_t)blocks;
    const int64_t quads = blocks * p.nq;
    const int mt = m <= 16 ? 1 : 2;
    // OCC workgroups per CU; never more workgroups than quads
    const int64_t slots = (int64_t)kernel_occ(bits, mt, argmax) * cus;
    const int64_t grid = quads < slots ? quads : slots;
    p.grid = grid < 1 ? 1 : (int32_t)grid;
    // a full grid of two workgroups per CU runs as CU pairs (weighted split)
    p.pairs = (kernel_occ(bits, mt, argmax) == 2 && p.grid == 2 * cus) ? cus : 0;
    // the kernel splits quads with 32-bit products
    p.fits = quads * p.grid < ((int64_t)1 << 31);
    p.quads = p.fits ? (int32_t)quads : 0;
    p.slab_waves = 0;
    p.dot = 0;
    if (!argmax) {
        int v = projection_variant();
        if (v == kDot && !(bits == 8 && m <= kDotMaxRows)) v = kAuto;
        const int64_t slabs = 4 * blocks;
        if (v == kSlab || v == kDot)
            p.slab_waves = slab_waves_for(slabs, cus) > 0 ? slab_waves_for(slabs, cus) : 4;
        else if (v == kAuto && slab_pays(bits, m, slabs, k, cus))
            p.slab_waves = slab_waves_for(slabs, cus) > 0 ? slab_waves_for(slabs, cus) : 4;
        if (slabs > 0x7fffffff) p.slab_waves = 0;
        p.dot = (v == kDot && p.slab_waves > 0) ? 1 : 0;
    }
    // fixed offsets (see the workspace layout in dspk_internal.h)
    p.off_keys = 256;
    p.off_partial = kWsHead;
    p.off_counters = kWsHead + partial_region_bytes(cus);
    p.ws_bytes = (p.off_counters + (size_t)blocks * kWavesPerWG * 4 + 255) / 256 * 256;
    return p;
}

GemmPlan plan_gemm(int count, const int32_t *n, int32_t k, int32_t m, int bits, bool argmax) {
    return plan_gemm_cus(count, n, k, m, bits, argmax, device_cus());
}

// Rows per prefill workgroup.  Where the 128-row workgroups would not cover
// every CU the 64-row ones are taken (the Qwen3-4B-shaped k and v projections
// over 2048 rows: 128 workgroups, 49-60 -> 33-41 us in 2/3/4/8-bit, 50 -> 42-44
// us in bf16).  Otherwise each CU is taken to run ceil(workgroups / CUs) of
// them, at 16 time units per 128-row workgroup and, for the 64-row ones whose
// decoded weights serve half as many rows, 9 units (2- and 4-bit) or 11 (3-
// and 8-bit, whose decoding costs more per weight); the shorter estimate
// wins, 128 rows on a tie.  bf16 keeps 128-row blocks there: its 64-row
// blocks issue twice the weight loads per matrix instruction and ran 15-40%
// slower per row.  (Units fitted to rocprof durations of the seven
// Qwen3-4B-shaped projections over 2048 rows with each block forced; the o
// and down projections, 320 128-row workgroups, 108 -> 99 and 238 -> 224 us
// in 2-bit, 119 -> 105 and 265 -> 231 us in 4-bit.)
int prefill_block_rows(int32_t m, int32_t nblocks, int bits, int cus) {
    const int64_t cols = ((int64_t)nblocks + 1) / 2;
    const int64_t w128 = ((int64_t)m + 127) / 128 * cols, w64 = ((int64_t)m + 63) / 64 * cols;
    if (w128 <= cus) return 64;
    if (bits == 16) return 128;
    const int64_t c128 = 16 * ((w128 + cus - 1) / cus);
    const int64_t c64 = (bits == 3 || bits == 8 ? 11 : 9) * ((w64 + cus - 1) / cus);
    return c64 < c128 ? 64 : 128;
}

namespace {
std::atomic<int> g_prefill_rows{0};   // 0: automatic, else 64 or 128
}  // namespace

int set_prefill_block_rows(int rows) {
    if (rows != 0 && rows != 64 && rows != 128) return -1;
    return g_prefill_rows.exchange(rows, std::memory_order_relaxed);
}

int prefill_rows_for(int32_t m, int32_t nblocks, int bits) {
    const int r = g_prefill_rows.load(std::memory_order_relaxed);
    return r != 0 ? r : prefill_block_rows(m, nblocks, bits, device_cus());
}

// A launch with fewer workgroups than the CUs hold at once leaves CUs idle or
// running one workgroup alone for the whole launch (the Qwen3-4B-shaped o and
// down projections over 2048 rows: 320 128-row workgroups for 512 slots).
// Splitting K into ks ranges, each workgroup summing one and the last of a
// tile's ks workgroups adding their partial tiles in split order, makes ks
// times as many shorter workgroups.  The estimate is ceil(ks wgs / slots)
// rounds of nst / ks units; the split with the lowest one is taken when it
// promises at least 30% over the single partial round, and every split keeps
// at least eight units (shorter ones did not pay for their pipeline start
// and exchange: the 4-bit o projection, 16 units, 91-93 us as 64-row blocks
// against 97-98 us as 128-row blocks split three ways; the 4-bit k and v,
// 10 units, 32-33 us either way).
int prefill_splits(int64_t wgs, int32_t nst, int occ, int cus) {
    const int64_t slots = (int64_t)occ * cus;
    if (wgs >= slots) return 1;
    int best = 1;
    int64_t best_rounds = 7, best_ks = 10;        // rounds / ks to beat: 0.7
    for (int ks = 2; ks <= 4 && 8 * ks <= nst; ++ks) {
        const int64_t rounds = (wgs * ks + slots - 1) / slots;
        if (rounds * best_ks < best_rounds * ks) {
            best = ks;
            best_rounds = rounds;
            best_ks = ks;
        }
    }
    return best;
}

PrefillPlan prefill_plan(int32_t m, int32_t nblocks, int32_t nst, int bits, bool may_split) {
    PrefillPlan p{};
    p.rows = prefill_rows_for(m, nblocks, bits);
    // With a workspace, a 128-row grid that covers the CUs but not two per CU
    // splits K rather than halving the rows, where the split pays: the 2- and
    // 4-bit down projections (320 128-row blocks, 38 units) 200-202 -> 184-186
    // us.  Grids that do not cover the CUs keep 64-row blocks (k and v: 35-37
    // us at 64 rows, 49-54 us split four ways at 128).
    const int cus = device_cus();
    if (may_split && g_prefill_rows.load(std::memory_order_relaxed) == 0) {
        const int64_t w128 = ((int64_t)m + 127) / 128 * (((int64_t)nblocks + 1) / 2);
        if (w128 > cus && w128 < 2 * (int64_t)cus && prefill_splits(w128, nst, 2, cus) > 1) p.rows = 128;
    }
    const int64_t tiles = ((int64_t)m + p.rows - 1) / p.rows * (((int64_t)nblocks + 1) / 2);
    // two workgroups per CU (64 KiB of LDS, 184-256 VGPRs).  bf16 fits
    // three at 128 rows, but its 512-workgroup q launch already runs as a
    // full grid (65-67 us unsplit, 85 us split three ways), so it is planned
    // as two as well
    p.ks = may_split ? prefill_splits(tiles, nst, 2, cus) : 1;
    if (p.ks > 1) {
        // the counters of the largest launch that splits (fewer than two
        // blocks per CU, four waves each) at a fixed place, so that calls
        // of any shape sharing one buffer find them zero: a region sized
        // by this call's blocks would overlap the partials of a call with
        // fewer blocks
        p.off_part = ((size_t)2 * cus * 4 * sizeof(uint32_t) + 255) / 256 * 256;
        // per wave and split: (rows / 32) x 4 tiles of 64 lanes x 16 bytes
        p.ws_bytes = p.off_part + (size_t)tiles * 4 * p.ks * (p.rows / 32) * 4 * 1024;
    }
    return p;
}

size_t tiled_bytes(int32_t n, int32_t k, int bits) {
    if (n < 1 || k < 64 || k % 64 || !supported_bits(bits)) return 0;
    const size_t nb = ((size_t)n + 63) / 64, nst = ((size_t)k + tile_k(bits) - 1) / tile_k(bits);
    return nb * nst * (size_t)tile_unit_bytes(bits);
}

size_t sample_workspace_bytes(int32_t v, int32_t m_rows) { return sample_ws_layout(m_rows, v).total; }

}  // namespace dspk

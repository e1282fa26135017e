// Host-only check of the C ABI layer, built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_host_sanitize.py.
//
// It links the library's host sources (argument checks, launch plans,
// workspace carving, cap policy) with recorders in place of the kernel
// launches and of the two HIP runtime queries they make, so no GPU and no
// device memory are involved: every pointer handed to an entry point is a
// made-up, suitably aligned address that nothing dereferences.  For each
// accepted call the recorder checks that everything the kernels would touch
// in the workspace lies inside the caller's buffer and that the regions do
// not overlap; rejected calls must leave a message.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "dspk.h"
#include "dspk_internal.h"
#include "prefill_plan.h"
#include "sample_layout.h"

static int g_fail = 0;
#define CHECK(c)                                                                   \
    do {                                                                           \
        if (!(c)) {                                                                \
            fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c); \
            ++g_fail;                                                              \
        }                                                                          \
    } while (0)

static const int kCus = 256;

// ------------------------------------------------------------------ recorders
static int g_prefill_splits = 0;    // prefill launches that split K
static uintptr_t g_ws = 0;
static size_t g_ws_bytes = 0;
static int g_launches = 0;

static bool inside(const void *p, size_t bytes) {
    const uintptr_t a = (uintptr_t)p;
    return a >= g_ws && a + bytes <= g_ws + g_ws_bytes && a + bytes >= a;
}

static void check_gemm(const dspk::GemmLaunch &L, int bits, int grid, bool head) {
    ++g_launches;
    CHECK(grid >= 1 && grid <= dspk::kMaxOcc * kCus);
    CHECK(L.quads >= grid);
    CHECK((long long)L.quads * grid < (1ll << 31));
    CHECK(L.pairs == 0 || (L.pairs == kCus && grid == 2 * kCus));
    CHECK(L.nq == (L.nst + 3) / 4 && L.nst == (L.k + dspk::tile_k(bits) - 1) / dspk::tile_k(bits));
    CHECK(L.m >= 1 && L.m <= dspk::kMaxRows);
    CHECK(L.count >= 1 && L.count <= dspk::kMaxGrouped);
    int cg = 0;
    for (int i = 0; i < L.count; ++i) {
        CHECK(L.p[i].cg_begin == cg);
        cg += (L.p[i].n + 63) / 64;
    }
    CHECK(cg == L.total_cg && L.quads == L.total_cg * L.nq);
    const int mt = L.m <= 16 ? 1 : 2;
    const size_t partial = (size_t)grid * 2 * 4 * mt * 64 * 16;
    const size_t counters = (size_t)L.total_cg * 4 * 4;
    CHECK(inside(L.partial, partial));
    CHECK(inside(L.counters, counters));
    // regions: [0, 512) head words, partial sums, counters -- disjoint
    CHECK((uintptr_t)L.partial >= g_ws + 512);
    CHECK((uintptr_t)L.partial + partial <= (uintptr_t)L.counters);
    // offsets do not depend on the call
    CHECK((uintptr_t)L.partial == g_ws + 512);
    CHECK((uintptr_t)L.counters == g_ws + 512 + dspk::partial_region_bytes(kCus));
    if (head) {
        CHECK((uintptr_t)L.done == g_ws);
        CHECK((uintptr_t)L.keys == g_ws + 256 && inside(L.keys, dspk::kMaxRows * 8));
        CHECK(L.argmax != nullptr);
        if (L.accept_len != nullptr) CHECK(L.acc_b * L.acc_rows == L.m);
    }
}

namespace dspk {
hipError_t launch_qgemm(const GemmLaunch &L, int bits, int grid, hipStream_t) {
    check_gemm(L, bits, grid, false);
    return hipSuccess;
}
hipError_t launch_lmhead(const GemmLaunch &L, int bits, int grid, hipStream_t) {
    check_gemm(L, bits, grid, true);
    return hipSuccess;
}
hipError_t launch_qgemm_slab(const GemmLaunch &L, int bits, int waves, hipStream_t) {
    ++g_launches;
    CHECK(waves == 2 || waves == 3 || waves == 4 || waves == 8 || waves == 16);
    CHECK(L.m >= 1 && L.m <= kMaxRows && L.count >= 1 && L.count <= kMaxGrouped);
    CHECK(L.nst == (L.k + tile_k(bits) - 1) / tile_k(bits));
    // with the automatic choice every tile of the call is resident at once
    if (projection_variant() == kAuto) {
        CHECK((bits == 8 || bits == 16) && L.m <= kSlabLdsMaxRows);
        const int64_t per_cu = (4 * (int64_t)L.total_cg + 255) / 256;
        CHECK(per_cu * 16 * L.k <= kSlabAutoWeights);
    }
    return hipSuccess;
}
hipError_t launch_qgemm_dot(const GemmLaunch &L, int waves, hipStream_t) {
    ++g_launches;
    CHECK(waves == 2 || waves == 3 || waves == 4 || waves == 8 || waves == 16);
    CHECK(L.m >= 1 && L.m <= kDotMaxRows);
    return hipSuccess;
}
hipError_t launch_prefill(const PrefillArgs &a, int bits, hipStream_t) {
    ++g_launches;
    CHECK(supported_bits(bits) && a.m >= 1 && a.ldx >= a.k && a.ldy >= a.n);
    CHECK(a.nblocks == (a.n + 63) / 64 && a.nst == (a.k + tile_k(bits) - 1) / tile_k(bits));
    CHECK(a.block_rows == 64 || a.block_rows == 128);
    CHECK(a.ks >= 1 && a.ks <= 4);
    if (a.ks > 1) {
        // counters, then the partial tiles, inside the caller's buffer
        const int64_t tiles = (int64_t)(a.m + a.block_rows - 1) / a.block_rows * ((a.nblocks + 1) / 2);
        CHECK(2 * a.ks <= a.nst);
        CHECK((uintptr_t)a.ctr == g_ws && inside(a.ctr, (size_t)tiles * 4 * 4));
        CHECK(inside(a.part, (size_t)tiles * 4 * a.ks * (a.block_rows / 32) * 4 * 1024));
        CHECK((uintptr_t)a.part >= (uintptr_t)a.ctr + (uintptr_t)tiles * 16 && (uintptr_t)a.part % 256 == 0);
        // the partials start at a place that does not depend on the call
        CHECK((uintptr_t)a.part == g_ws + (2 * kCus * 16 + 255) / 256 * 256);
        ++g_prefill_splits;
    } else {
        CHECK(a.part == nullptr && a.ctr == nullptr);
    }
    return hipSuccess;
}
hipError_t launch_pack(int32_t n, int32_t k, int bits, const void *, const uint16_t *, const uint16_t *, void *,
                       hipStream_t) {
    ++g_launches;
    CHECK(n >= 1 && k % 64 == 0 && supported_bits(bits));
    return hipSuccess;
}
hipError_t launch_accept_greedy(const int32_t *t, const int32_t *, int32_t b, int32_t m_rows, int32_t *a, int32_t *c,
                                hipStream_t) {
    ++g_launches;
    CHECK(t != nullptr && a != nullptr && c != nullptr && b >= 1 && m_rows >= 1 && m_rows <= kMaxRows);
    return hipSuccess;
}
hipError_t launch_accept_sample(const SampleParams &p, hipStream_t) {
    ++g_launches;
    const SampleWsLayout L = sample_ws_layout(p.m_rows, p.v);
    CHECK((uintptr_t)p.ws == g_ws && L.total <= g_ws_bytes);
    const size_t offs[] = {256, L.stats, L.flags, L.qmax, L.mass, L.trunc, L.pcnt, L.pmass, L.bin1, L.total};
    for (size_t i = 1; i < sizeof offs / sizeof offs[0]; ++i) CHECK(offs[i] >= offs[i - 1] && offs[i] % 256 == 0);
    CHECK(p.temperature > 0.f && p.m_rows >= 2 && p.v >= 1);
    return hipSuccess;
}
// the allocation-free entry point's scratch: a made-up device address
static const uintptr_t kScratchAddr = 0x7d0000000000ull;
hipError_t static_scratch(void **ptr, hipStream_t) {
    *ptr = (void *)kScratchAddr;
    g_ws = kScratchAddr;
    g_ws_bytes = static_scratch_bytes();
    return hipSuccess;
}
size_t static_scratch_bytes() { return kWsHead + partial_region_bytes(kScratchCus) + kScratchMaxBlocks * 16; }
}  // namespace dspk

// The only HIP runtime calls of the host sources: a device with kCus CUs.
extern "C" hipError_t hipGetDevice(int *d) {
    *d = 0;
    return hipSuccess;
}
extern "C" hipError_t hipDeviceGetAttribute(int *v, hipDeviceAttribute_t, int) {
    *v = kCus;
    return hipSuccess;
}
extern "C" const char *hipGetErrorString(hipError_t) { return "recorded launch"; }

// ---------------------------------------------------------------- helpers
static void *fake(uintptr_t a) { return (void *)a; }
static const uintptr_t X = 0x7f0000000000ull, Y = 0x7f1000000000ull, W = 0x7f2000000000ull;

static dspk_tiled_weight tiled(int n, int k, int bits) {
    dspk_tiled_weight d;
    d.n = n;
    d.k = k;
    d.bits = bits;
    d.group = 64;
    d.tiles = fake(W);
    return d;
}

static void use_ws(size_t bytes) {
    g_ws = 0x7e0000000000ull;
    g_ws_bytes = bytes;
}

static void expect_error(int rc, int code) {
    CHECK(rc == code);
    CHECK(strlen(dspk_last_error()) > 0);
}

// ------------------------------------------------------------------- checks
static void projections() {
    const int ns[] = {1, 37, 64, 65, 1000, 1024, 2560, 4096, 9728, 17408, 151936};
    const int ks[] = {64, 128, 320, 2560, 4096, 4160, 9728, 17408};
    const int bitsv[] = {2, 3, 4, 8, 16};
    for (int n : ns)
        for (int k : ks)
            for (int bits : bitsv)
                for (int m = 1; m <= 32; m += (m < 4 ? 1 : 5)) {
                    dspk_tiled_weight w = tiled(n, k, bits);
                    const size_t need = dspk_qgemm_workspace_bytes(n, k, m);
                    CHECK(need > 0 && need % 256 == 0);
                    CHECK(need == dspk_qgemm_workspace_bytes(n, 64, 1));       // shape-independent offsets
                    use_ws(need);
                    int rc = dspk_qgemm_verify(&w, (const uint16_t *)fake(X), k + 8 * (m % 3), m, fake(Y), m & 1,
                                               n + (m % 2), fake(g_ws), need, nullptr);
                    CHECK(rc == DSPK_OK);
                    expect_error(dspk_qgemm_verify(&w, (const uint16_t *)fake(X), k, m, fake(Y), 0, n, fake(g_ws),
                                                   need - 1, nullptr),
                                 DSPK_EINVAL);
                    // the head over the same matrix, with the fused acceptance at m = b * rows
                    const size_t hneed = dspk_lmhead_workspace_bytes(n, m);
                    CHECK(hneed == need);
                    use_ws(hneed);
                    rc = dspk_lmhead_argmax(&w, (const uint16_t *)fake(X), k, m, (int32_t *)fake(Y), nullptr, 0,
                                            fake(g_ws), hneed, nullptr);
                    CHECK(rc == DSPK_OK);
                    if (m % 2 == 0) {
                        rc = dspk_lmhead_argmax_accept_greedy(&w, (const uint16_t *)fake(X), k, 2, m / 2,
                                                              (int32_t *)fake(Y), (float *)fake(Y + 4096), n,
                                                              (const int32_t *)fake(X), (int32_t *)fake(Y),
                                                              (int32_t *)fake(Y + 256), fake(g_ws), hneed, nullptr);
                        CHECK(rc == DSPK_OK);
                    }
                }
    // grouped: the sum of the single sizes is enough
    const int qkv[] = {4096, 1024, 1024, 512};
    for (int count = 1; count <= 4; ++count)
        for (int m : {1, 8, 16, 17, 32}) {
            dspk_tiled_weight ws[4];
            void *ys[4];
            int64_t ld[4];
            size_t need = 0;
            for (int i = 0; i < count; ++i) {
                ws[i] = tiled(qkv[i], 2560, 8);
                ys[i] = fake(Y + (uintptr_t)i * 0x100000);
                ld[i] = qkv[i];
                need += dspk_qgemm_workspace_bytes(qkv[i], 2560, m);
            }
            use_ws(need);
            CHECK(dspk_qgemm_verify_grouped(count, ws, (const uint16_t *)fake(X), 2560, m, ys, 0, ld, fake(g_ws),
                                            need, nullptr) == DSPK_OK);
        }
}

static void noalloc() {
    // the same plans and carving as the workspace call, on the library's array
    const int qkv[] = {4096, 1024, 1024};
    dspk_tiled_weight ws[3];
    void *ys[3];
    int64_t ld[3];
    for (int i = 0; i < 3; ++i) {
        ws[i] = tiled(qkv[i], 2560, 8);
        ys[i] = fake(Y + (uintptr_t)i * 0x100000);
        ld[i] = qkv[i];
    }
    for (int m : {1, 8, 16, 17, 32})
        CHECK(dspk_qgemm_verify_grouped_noalloc(3, ws, (const uint16_t *)fake(X), 2560, m, ys, 0, ld, nullptr) ==
              DSPK_OK);
    // the largest call that fits: 4096 blocks; one block more is refused
    dspk_tiled_weight big = tiled(4096 * 64, 512, 8);
    int64_t bl = 4096 * 64;
    void *by = fake(Y);
    CHECK(dspk_qgemm_verify_grouped_noalloc(1, &big, (const uint16_t *)fake(X), 512, 4, &by, 0, &bl, nullptr) ==
          DSPK_OK);
    big.n += 1;
    bl += 1;
    const int before = g_launches;
    expect_error(dspk_qgemm_verify_grouped_noalloc(1, &big, (const uint16_t *)fake(X), 512, 4, &by, 0, &bl, nullptr),
                 DSPK_EUNSUPPORTED);
    CHECK(g_launches == before);
    // argument errors are those of the grouped call
    expect_error(dspk_qgemm_verify_grouped_noalloc(0, ws, (const uint16_t *)fake(X), 2560, 4, ys, 0, ld, nullptr),
                 DSPK_EINVAL);
    expect_error(dspk_qgemm_verify_grouped_noalloc(3, ws, (const uint16_t *)fake(X), 2560, 40, ys, 0, ld, nullptr),
                 DSPK_EINVAL);
}

static void variants() {
    // every forced decomposition plans and launches for every format and width
    for (int v : {DSPK_VARIANT_STREAMK, DSPK_VARIANT_SLAB, DSPK_VARIANT_DOT, DSPK_VARIANT_AUTO}) {
        CHECK(dspk_set_projection_variant(v) >= 0);
        for (int bits : {2, 3, 4, 8, 16})
            for (int m : {1, 3, 4, 5, 16, 17, 32})
                for (int n : {37, 2560, 19456, 151936}) {
                    dspk_tiled_weight w = tiled(n, 2560, bits);
                    const size_t need = dspk_qgemm_workspace_bytes(n, 2560, m);
                    use_ws(need);
                    CHECK(dspk_qgemm_verify(&w, (const uint16_t *)fake(X), 2560, m, fake(Y), 0, n, fake(g_ws), need,
                                            nullptr) == DSPK_OK);
                }
    }
    expect_error(dspk_set_projection_variant(7), DSPK_EINVAL);
    CHECK(dspk_set_projection_variant(DSPK_VARIANT_AUTO) == DSPK_VARIANT_AUTO);
}

static void rejections() {
    dspk_tiled_weight w = tiled(64, 128, 8);
    const size_t need = dspk_qgemm_workspace_bytes(64, 128, 32);
    use_ws(need);
    const uint16_t *x = (const uint16_t *)fake(X);
    expect_error(dspk_qgemm_verify(&w, x, 128, 0, fake(Y), 0, 64, fake(g_ws), need, nullptr), DSPK_EINVAL);
    expect_error(dspk_qgemm_verify(&w, x, 128, 33, fake(Y), 0, 64, fake(g_ws), need, nullptr), DSPK_EINVAL);
    expect_error(dspk_qgemm_verify(&w, x, 120, 4, fake(Y), 0, 64, fake(g_ws), need, nullptr), DSPK_EINVAL);
    expect_error(dspk_qgemm_verify(&w, x, 132, 4, fake(Y), 0, 64, fake(g_ws), need, nullptr), DSPK_EINVAL);
    expect_error(dspk_qgemm_verify(&w, x + 4, 128, 4, fake(Y), 0, 64, fake(g_ws), need, nullptr), DSPK_EINVAL);
    expect_error(dspk_qgemm_verify(&w, x, (int64_t)1 << 26, 32, fake(Y), 0, 64, fake(g_ws), need, nullptr),
                 DSPK_EUNSUPPORTED);
    expect_error(dspk_qgemm_verify(&w, x, 128, 4, fake(Y), 0, 63, fake(g_ws), need, nullptr), DSPK_EINVAL);
    expect_error(dspk_qgemm_verify(&w, x, 128, 4, fake(Y), 0, 64, fake(g_ws + 16), need, nullptr), DSPK_EINVAL);
    expect_error(dspk_qgemm_verify(nullptr, x, 128, 4, fake(Y), 0, 64, fake(g_ws), need, nullptr), DSPK_EINVAL);
    dspk_tiled_weight bad = tiled(64, 128, 5);
    expect_error(dspk_qgemm_verify(&bad, x, 128, 4, fake(Y), 0, 64, fake(g_ws), need, nullptr), DSPK_EUNSUPPORTED);
    bad = tiled(64, 100, 8);
    expect_error(dspk_qgemm_verify(&bad, x, 128, 4, fake(Y), 0, 64, fake(g_ws), need, nullptr), DSPK_EINVAL);
    CHECK(dspk_qgemm_workspace_bytes(0, 64, 1) == 0 && dspk_qgemm_workspace_bytes(64, 64, 33) == 0);
    CHECK(dspk_lmhead_workspace_bytes(0, 1) == 0 && dspk_tiled_bytes(64, 100, 8) == 0);
    expect_error(dspk_accept_greedy((const int32_t *)fake(X), nullptr, 1, 4, (int32_t *)fake(Y),
                                    (int32_t *)fake(Y), nullptr),
                 DSPK_EINVAL);
    CHECK(dspk_accept_greedy((const int32_t *)fake(X), (const int32_t *)fake(X), 3, 6, (int32_t *)fake(Y),
                             (int32_t *)fake(Y), nullptr) == DSPK_OK);
}

static void packing_and_prefill() {
    for (int bits : {2, 3, 4, 8, 16}) {
        dspk_qweight q;
        q.n = 130;
        q.k = 320;
        q.bits = bits;
        q.group = 64;
        q.codes = fake(X);
        q.scales = bits == 16 ? nullptr : (const uint16_t *)fake(X + 0x100000);
        q.biases = bits == 16 ? nullptr : (const uint16_t *)fake(X + 0x200000);
        const size_t tb = dspk_tiled_bytes(130, 320, bits);
        CHECK(tb > 0);
        CHECK(dspk_qweight_pack(&q, fake(W), tb, nullptr) == DSPK_OK);
        expect_error(dspk_qweight_pack(&q, fake(W), tb - 1, nullptr), DSPK_EINVAL);
        dspk_tiled_weight w = tiled(130, 320, bits);
        CHECK(dspk_qgemm_prefill(&w, (const uint16_t *)fake(X), 320, 2048, fake(Y), 0, 130, nullptr, 0, nullptr) ==
              DSPK_OK);
        expect_error(dspk_qgemm_prefill(&w, (const uint16_t *)fake(X), 316, 2048, fake(Y), 0, 130, nullptr, 0, nullptr),
                     DSPK_EINVAL);
    }
    // prefill with a workspace: shapes whose launches split K and one that
    // does not; a short or misaligned buffer is refused
    for (int bits : {2, 3, 4, 8, 16})
        for (int n : {130, 2560, 9728})
            for (int m : {1, 300, 2048}) {
                const int k = 4096;
                const size_t need = dspk_prefill_workspace_bytes(n, k, m, bits);
                dspk_tiled_weight w = tiled(n, k, bits);
                use_ws(need > 0 ? need : 256);
                const int before = g_prefill_splits;
                CHECK(dspk_qgemm_prefill(&w, (const uint16_t *)fake(X), k, m, fake(Y), 0, n, fake(g_ws), need,
                                         nullptr) == DSPK_OK);
                CHECK((g_prefill_splits > before) == (need > 0));
                if (need > 0) {
                    expect_error(dspk_qgemm_prefill(&w, (const uint16_t *)fake(X), k, m, fake(Y), 0, n, fake(g_ws),
                                                    need - 1, nullptr),
                                 DSPK_EINVAL);
                    expect_error(dspk_qgemm_prefill(&w, (const uint16_t *)fake(X), k, m, fake(Y), 0, n,
                                                    fake(g_ws + 16), need, nullptr),
                                 DSPK_EINVAL);
                }
            }
}

// The prefill row block: Qwen3-4B-shaped projections over 2048 rows on 256
// CUs, a one-row call, and the override.
static void prefill_blocks() {
    for (int bits : {2, 3, 4, 8, 16}) {
        CHECK(dspk::prefill_block_rows(2048, 64, bits, 256) == 128);    // q, 4096 columns: two per CU
        CHECK(dspk::prefill_block_rows(2048, 16, bits, 256) == 64);     // k, v, 1024: 128 workgroups
        CHECK(dspk::prefill_block_rows(2048, 152, bits, 256) == 128);   // gate, up, 9728
        CHECK(dspk::prefill_block_rows(1, 1, bits, 256) == 64);
        // o, down, 2560: 320 128-row workgroups load the CUs unevenly
        CHECK(dspk::prefill_block_rows(2048, 40, bits, 256) == (bits == 2 || bits == 4 ? 64 : 128));
    }
    // K splits: o and down (320 workgroups of 128 rows, 512 slots) three,
    // k and v at 64 rows (256 workgroups) two, full grids none
    CHECK(dspk::prefill_splits(320, 32, 2, 256) == 3);
    CHECK(dspk::prefill_splits(320, 76, 2, 256) == 3);
    CHECK(dspk::prefill_splits(256, 20, 2, 256) == 2);
    CHECK(dspk::prefill_splits(512, 20, 2, 256) == 1);
    CHECK(dspk::prefill_splits(1216, 20, 2, 256) == 1);
    CHECK(dspk::prefill_splits(256, 10, 2, 256) == 1);    // 4-bit k/v: splits would be under 8 units
    CHECK(dspk::prefill_splits(320, 16, 2, 256) == 1);    // 4-bit o at 128 rows: likewise
    CHECK(dspk::prefill_splits(320, 38, 2, 256) == 3);    // 4-bit down
    for (int bits : {2, 3, 4, 8, 16}) {
        const int32_t ku = dspk::tile_k(bits);
        CHECK(dspk::prefill_plan(2048, 64, 2560 / ku, bits, true).ks == 1);      // q: a full grid
        CHECK(dspk::prefill_plan(2048, 40, 4096 / ku, bits, false).ks == 1);     // no workspace
        // down with a workspace: 128-row blocks, K split three ways
        const dspk::PrefillPlan pd = dspk::prefill_plan(2048, 40, 9728 / ku, bits, true);
        CHECK(pd.rows == 128 && pd.ks == 3 && pd.ws_bytes > pd.off_part);
        // o and k/v: split where each split keeps 8 units (8-bit and bf16)
        const dspk::PrefillPlan po = dspk::prefill_plan(2048, 40, 4096 / ku, bits, true);
        const dspk::PrefillPlan pk = dspk::prefill_plan(2048, 16, 2560 / ku, bits, true);
        if (bits >= 8) {
            CHECK(po.rows == 128 && po.ks == 3);
            CHECK(pk.rows == 64 && pk.ks == 2);
        } else {
            CHECK(po.ks == 1 && pk.ks == 1 && pk.rows == 64);
        }
    }
    CHECK(dspk_set_prefill_block_rows(128) == 0);
    CHECK(dspk::prefill_rows_for(2048, 16, 8) == 128);
    CHECK(dspk_set_prefill_block_rows(64) == 128);
    CHECK(dspk::prefill_rows_for(2048, 64, 8) == 64);
    expect_error(dspk_set_prefill_block_rows(96), DSPK_EINVAL);
    CHECK(dspk_set_prefill_block_rows(0) == 64);
    CHECK(dspk::prefill_rows_for(2048, 16, 8) == 64);
}

static void sampling() {
    for (int v : {1, 100, 4096, 4097, 151936})
        for (int rows : {2, 6, 17, 32}) {
            const size_t need = dspk_sample_workspace_bytes(v, rows);
            CHECK(need >= 256);
            use_ws(need);
            const float *f = (const float *)fake(X);
            CHECK(dspk_accept_sample(f, v, f, v, (const int32_t *)fake(X), f, rows, v, 1.0f, (int32_t *)fake(Y),
                                     (int32_t *)fake(Y), fake(g_ws), need, nullptr) == DSPK_OK);
            dspk_sample_params sp = {0.7f, 50, 0.9f, 0.5f, 0.1f};
            CHECK(dspk_accept_sample_ex(f, v, f, v, (const int32_t *)fake(X), f, rows, v, &sp,
                                        (const int32_t *)fake(X), (int32_t *)fake(Y), (int32_t *)fake(Y),
                                        fake(g_ws), need, nullptr) == DSPK_OK);
            sp.top_p = 0.f;
            expect_error(dspk_accept_sample_ex(f, v, f, v, (const int32_t *)fake(X), f, rows, v, &sp, nullptr,
                                               (int32_t *)fake(Y), (int32_t *)fake(Y), fake(g_ws), need, nullptr),
                         DSPK_EINVAL);
            expect_error(dspk_accept_sample(f, v, f, v, (const int32_t *)fake(X), f, rows, v, 0.f,
                                            (int32_t *)fake(Y), (int32_t *)fake(Y), fake(g_ws), need, nullptr),
                         DSPK_EINVAL);
        }
}

static void policy() {
    unsigned s = 12345u;
    auto rnd = [&]() {
        s = s * 1103515245u + 12345u;
        return (double)((s >> 8) & 0xffffff) / (double)(1 << 24);
    };
    for (int trial = 0; trial < 2000; ++trial) {
        const int n = 1 + trial % DSPK_MAX_ROWS;
        double vu[DSPK_MAX_ROWS], du[DSPK_MAX_ROWS];
        for (int i = 0; i < n; ++i) {
            vu[i] = 50.0 + 200.0 * rnd();
            du[i] = 10.0 * rnd();
        }
        double rate = -1.0;
        const int cap = dspk_choose_cap(vu, trial % 2 ? du : nullptr, n, rnd(), &rate);
        CHECK(cap >= 0 && cap < n && rate > 0.0 && isfinite(rate));
        dspk_cap_controller ctl;
        CHECK(dspk_cap_init(&ctl, vu, du, n, 0.9, 0.5, 8, n > 1 ? 1 : 0) == (n > 1 ? DSPK_OK : DSPK_EINVAL));
        if (n > 1)
            for (int r = 0; r < 50; ++r) {
                const int c = dspk_cap_next(&ctl);
                CHECK(c >= 0 && c < n);
                CHECK(dspk_cap_observe(&ctl, c, c == 0 ? 0 : (int)(rnd() * (c + 1)) % (c + 1)) == DSPK_OK);
                const double a = dspk_cap_alpha(&ctl);
                CHECK(a >= 0.0 && a <= 1.0);
            }
    }
    double bad[2] = {1.0, NAN};
    CHECK(dspk_choose_cap(bad, nullptr, 2, 0.5, nullptr) == DSPK_EINVAL);
    CHECK(dspk_choose_cap(bad, nullptr, 0, 0.5, nullptr) == DSPK_EINVAL);
}

int main() {
    projections();
    noalloc();
    variants();
    rejections();
    packing_and_prefill();
    prefill_blocks();
    sampling();
    policy();
    if (g_fail) {
        fprintf(stderr, "host check: %d failures\n", g_fail);
        return 1;
    }
    printf("host check ok: %d recorded launches\n", g_launches);
    return 0;
}

// C ABI of the verify-pass library: argument checks, work planning and
// launches.  Every entry point validates everything it can see on the host
// before enqueuing anything; nothing here allocates, frees or synchronises.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <string>

#include "../../include/dspk.h"
#include "dspk_internal.h"
#include "prefill_plan.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int ok() {
    g_err.clear();
    return DSPK_OK;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

int check_shape(int32_t n, int32_t k, int32_t bits, int32_t group, const char *who) {
    if (!dspk::supported_bits(bits))
        return fail(DSPK_EUNSUPPORTED, "%s: bits=%d (supported: 2, 3, 4, 8, 16)", who, bits);
    if (group != DSPK_GROUP) return fail(DSPK_EUNSUPPORTED, "%s: group=%d (must be 64)", who, group);
    if (n < 1) return fail(DSPK_EINVAL, "%s: n=%d must be >= 1", who, n);
    if (k < DSPK_GROUP || k % DSPK_GROUP) return fail(DSPK_EINVAL, "%s: k=%d must be a positive multiple of 64", who, k);
    return DSPK_OK;
}

// A weight in the interchange layout (input of the packing call).
int check_weight(const dspk_qweight *w, const char *who) {
    if (w == nullptr) return fail(DSPK_EINVAL, "%s: weight descriptor is NULL", who);
    int rc = check_shape(w->n, w->k, w->bits, w->group, who);
    if (rc) return rc;
    if (w->codes == nullptr || !aligned(w->codes, 16))
        return fail(DSPK_EINVAL, "%s: codes must be a non-NULL 16-byte aligned device pointer", who);
    if (w->bits == 16) {
        if (w->scales != nullptr || w->biases != nullptr)
            return fail(DSPK_EINVAL, "%s: bf16 weights take no scales or biases", who);
    } else {
        if (w->scales == nullptr || w->biases == nullptr)
            return fail(DSPK_EINVAL, "%s: scales and biases are required for bits=%d", who, w->bits);
        if (!aligned(w->scales, 2) || !aligned(w->biases, 2))
            return fail(DSPK_EINVAL, "%s: scales and biases must be 2-byte aligned", who);
    }
    return DSPK_OK;
}

// A weight in the tiled layout (what the projection kernels read).
int check_tiled(const dspk_tiled_weight *w, const char *who) {
    if (w == nullptr) return fail(DSPK_EINVAL, "%s: weight descriptor is NULL", who);
    int rc = check_shape(w->n, w->k, w->bits, w->group, who);
    if (rc) return rc;
    if (w->tiles == nullptr || !aligned(w->tiles, 256))
        return fail(DSPK_EINVAL, "%s: tiles must be a non-NULL 256-byte aligned device pointer", who);
    return DSPK_OK;
}

// Activations are row-major bf16 [m][ldx]: ldx >= k, ldx % 8 == 0 and a
// 16-byte aligned base, so every 8-element piece a lane loads is aligned.
int check_rows(const uint16_t *x, int64_t ldx, int32_t m, int32_t k, const char *who) {
    if (m < 1 || m > DSPK_MAX_ROWS) return fail(DSPK_EINVAL, "%s: m=%d out of 1..%d", who, m, DSPK_MAX_ROWS);
    if (x == nullptr || !aligned(x, 16))
        return fail(DSPK_EINVAL, "%s: activations must be a non-NULL 16-byte aligned device pointer", who);
    if (ldx < k || ldx % 8)
        return fail(DSPK_EINVAL, "%s: ldx=%lld must be >= k=%d and a multiple of 8", who, (long long)ldx, k);
    if ((int64_t)m * ldx * 2 >= ((int64_t)1 << 31))
        return fail(DSPK_EUNSUPPORTED, "%s: activation rows span 2 GiB or more (m * ldx * 2 >= 2^31)", who);
    return DSPK_OK;
}

int launch_result(hipError_t e, const char *who) {
    if (e != hipSuccess) return fail(DSPK_EDEVICE, "%s: launch failed: %s", who, hipGetErrorString(e));
    return ok();
}

void fill_plan(dspk::GemmLaunch &L, const dspk::GemmPlan &pl, const uint16_t *x, int64_t ldx, int32_t m,
               int32_t k) {
    L.x = x;
    L.ldx = ldx;
    L.m = m;
    L.k = k;
    L.nst = pl.nst;
    L.nq = pl.nq;
    L.quads = pl.quads;
    L.total_cg = pl.total_cg;
    L.pairs = pl.pairs;
}

int qgemm_common(int32_t count, const dspk_tiled_weight *w, const uint16_t *x, int64_t ldx, int32_t m,
                 void *const *y, int32_t y_dtype, const int64_t *ldy, void *workspace, size_t ws_bytes,
                 void *stream, const char *who) {
    if (count < 1 || count > DSPK_MAX_GROUPED)
        return fail(DSPK_EINVAL, "%s: count=%d out of 1..%d", who, count, DSPK_MAX_GROUPED);
    if (w == nullptr || y == nullptr || ldy == nullptr) return fail(DSPK_EINVAL, "%s: NULL array argument", who);
    if (y_dtype != DSPK_F32 && y_dtype != DSPK_BF16)
        return fail(DSPK_EINVAL, "%s: y_dtype=%d (DSPK_F32 or DSPK_BF16)", who, y_dtype);
    for (int i = 0; i < count; ++i) {
        int rc = check_tiled(&w[i], who);
        if (rc) return rc;
        if (w[i].k != w[0].k || w[i].bits != w[0].bits)
            return fail(DSPK_EINVAL, "%s: grouped weights must share k and bits", who);
        if (y[i] == nullptr || !aligned(y[i], 4)) return fail(DSPK_EINVAL, "%s: y[%d] NULL or misaligned", who, i);
        if (ldy[i] < w[i].n) return fail(DSPK_EINVAL, "%s: ldy[%d]=%lld < n=%d", who, i, (long long)ldy[i], w[i].n);
    }
    int rc = check_rows(x, ldx, m, w[0].k, who);
    if (rc) return rc;

    int32_t ns[DSPK_MAX_GROUPED];
    for (int i = 0; i < count; ++i) ns[i] = w[i].n;
    const dspk::GemmPlan pl = dspk::plan_gemm(count, ns, w[0].k, m, w[0].bits, false);
    if (!pl.fits) return fail(DSPK_EUNSUPPORTED, "%s: weights too large for one launch", who);
    if (workspace == nullptr || !aligned(workspace, 256))
        return fail(DSPK_EINVAL, "%s: workspace of %zu bytes required (256-byte aligned)", who, pl.ws_bytes);
    if (ws_bytes < pl.ws_bytes)
        return fail(DSPK_EINVAL, "%s: workspace %zu bytes < %zu required", who, ws_bytes, pl.ws_bytes);

    dspk::GemmLaunch L{};
    fill_plan(L, pl, x, ldx, m, w[0].k);
    L.count = count;
    L.y_bf16 = y_dtype == DSPK_BF16;
    L.counters = (uint32_t *)((char *)workspace + pl.off_counters);
    L.partial = (float *)((char *)workspace + pl.off_partial);
    int cg = 0;
    for (int i = 0; i < count; ++i) {
        dspk::GemmProblem &P = L.p[i];
        P.tiles = w[i].tiles;
        P.y = y[i];
        P.ldy = ldy[i];
        P.n = w[i].n;
        P.cg_begin = cg;
        cg += (w[i].n + dspk::kBlockCols - 1) / dspk::kBlockCols;
    }
    if (pl.slab_waves > 0 && pl.dot)
        return launch_result(dspk::launch_qgemm_dot(L, pl.slab_waves, (hipStream_t)stream), who);
    if (pl.slab_waves > 0)
        return launch_result(dspk::launch_qgemm_slab(L, w[0].bits, pl.slab_waves, (hipStream_t)stream), who);
    return launch_result(dspk::launch_qgemm(L, w[0].bits, pl.grid, (hipStream_t)stream), who);
}

}  // namespace

extern "C" {

int dspk_version(void) { return 300; }

int dspk_set_projection_variant(int32_t variant) {
    const int prev = dspk::set_projection_variant(variant);
    if (prev < 0)
        return fail(DSPK_EINVAL, "dspk_set_projection_variant: variant=%d (0 auto, 1 stream-K, 2 slab, 3 dot)",
                    variant);
    return prev;
}

int dspk_set_prefill_block_rows(int32_t rows) {
    const int prev = dspk::set_prefill_block_rows(rows);
    if (prev < 0) return fail(DSPK_EINVAL, "dspk_set_prefill_block_rows: rows=%d (0 automatic, 64 or 128)", rows);
    return prev;
}

const char *dspk_last_error(void) { return g_err.c_str(); }

size_t dspk_prefill_workspace_bytes(int32_t n, int32_t k, int32_t m, int32_t bits) {
    if (n < 1 || k < 64 || k % 64 || m < 1 || !dspk::supported_bits(bits)) return 0;
    const int32_t nst = (k + dspk::tile_k(bits) - 1) / dspk::tile_k(bits);
    return dspk::prefill_plan(m, (n + dspk::kBlockCols - 1) / dspk::kBlockCols, nst, bits, true).ws_bytes;
}

int dspk_qgemm_prefill(const dspk_tiled_weight *w, const uint16_t *x, int64_t ldx, int32_t m, void *y,
                       int32_t y_dtype, int64_t ldy, void *workspace, size_t workspace_bytes, void *stream) {
    const char *who = "dspk_qgemm_prefill";
    int rc = check_tiled(w, who);
    if (rc) return rc;
    if (m < 1) return fail(DSPK_EINVAL, "%s: m=%d must be >= 1", who, m);
    if (x == nullptr || !aligned(x, 16)) return fail(DSPK_EINVAL, "%s: x must be a 16-byte aligned device pointer", who);
    if (ldx < w->k || ldx % 8) return fail(DSPK_EINVAL, "%s: ldx=%lld must be >= k and a multiple of 8", who,
                                          (long long)ldx);
    if (y_dtype != DSPK_F32 && y_dtype != DSPK_BF16) return fail(DSPK_EINVAL, "%s: bad y_dtype", who);
    if (y == nullptr || !aligned(y, y_dtype == DSPK_F32 ? 4 : 2) || ldy < w->n)
        return fail(DSPK_EINVAL, "%s: y must be aligned with ldy >= n", who);
    dspk::PrefillArgs A;
    A.tiles = w->tiles;
    A.n = w->n;
    A.k = w->k;
    A.nst = (w->k + dspk::tile_k(w->bits) - 1) / dspk::tile_k(w->bits);
    A.nblocks = (w->n + dspk::kBlockCols - 1) / dspk::kBlockCols;
    if ((A.nblocks + 1) / 2 > 65535) return fail(DSPK_EINVAL, "%s: n=%d too large for one launch", who, w->n);
    A.x = x;
    A.ldx = ldx;
    A.m = m;
    A.y = y;
    A.ldy = ldy;
    A.y_bf16 = y_dtype == DSPK_BF16;
    if (workspace != nullptr && !aligned(workspace, 256))
        return fail(DSPK_EINVAL, "%s: workspace must be 256-byte aligned", who);
    const dspk::PrefillPlan pl = dspk::prefill_plan(m, A.nblocks, A.nst, w->bits, workspace != nullptr);
    if (pl.ks > 1 && workspace_bytes < pl.ws_bytes)
        return fail(DSPK_EINVAL, "%s: workspace of %zu bytes, %zu needed (dspk_prefill_workspace_bytes)", who,
                    workspace_bytes, pl.ws_bytes);
    A.block_rows = pl.rows;
    A.ks = pl.ks;
    A.ctr = pl.ks > 1 ? (uint32_t *)workspace : nullptr;
    A.part = pl.ks > 1 ? (float *)((char *)workspace + pl.off_part) : nullptr;
    return launch_result(dspk::launch_prefill(A, w->bits, (hipStream_t)stream), who);
}

size_t dspk_tiled_bytes(int32_t n, int32_t k, int32_t bits) { return dspk::tiled_bytes(n, k, bits); }

int dspk_qweight_pack(const dspk_qweight *w, void *tiles, size_t tiles_bytes, void *stream) {
    const char *who = "dspk_qweight_pack";
    int rc = check_weight(w, who);
    if (rc) return rc;
    const size_t need = dspk::tiled_bytes(w->n, w->k, w->bits);
    if (tiles == nullptr || !aligned(tiles, 256))
        return fail(DSPK_EINVAL, "%s: tiles must be a non-NULL 256-byte aligned device pointer", who);
    if (tiles_bytes < need) return fail(DSPK_EINVAL, "%s: tiles %zu bytes < %zu required", who, tiles_bytes, need);
    return launch_result(dspk::launch_pack(w->n, w->k, w->bits, w->codes, w->scales, w->biases, tiles,
                                           (hipStream_t)stream),
                         who);
}

size_t dspk_qgemm_workspace_bytes(int32_t n, int32_t k, int32_t m) {
    if (n < 1 || k < DSPK_GROUP || k % DSPK_GROUP || m < 1 || m > DSPK_MAX_ROWS) return 0;
    // offsets are fixed (the partial-sum region is sized for the largest
    // grid), so the size depends on n only and serves every width and format
    return dspk::plan_gemm(1, &n, k, m, 8, false).ws_bytes;
}

int dspk_qgemm_verify(const dspk_tiled_weight *w, const uint16_t *x, int64_t ldx, int32_t m, void *y,
                      int32_t y_dtype, int64_t ldy, void *workspace, size_t ws_bytes, void *stream) {
    void *ys[1] = {y};
    int64_t lds[1] = {ldy};
    return qgemm_common(1, w, x, ldx, m, ys, y_dtype, lds, workspace, ws_bytes, stream, "dspk_qgemm_verify");
}

int dspk_qgemm_verify_grouped(int32_t count, const dspk_tiled_weight *w, const uint16_t *x, int64_t ldx, int32_t m,
                              void *const *y, int32_t y_dtype, const int64_t *ldy, void *workspace,
                              size_t ws_bytes, void *stream) {
    return qgemm_common(count, w, x, ldx, m, y, y_dtype, ldy, workspace, ws_bytes, stream,
                        "dspk_qgemm_verify_grouped");
}

int dspk_qgemm_verify_grouped_noalloc(int32_t count, const dspk_tiled_weight *w, const uint16_t *x, int64_t ldx,
                                      int32_t m, void *const *y, int32_t y_dtype, const int64_t *ldy,
                                      void *stream) {
    const char *who = "dspk_qgemm_verify_grouped_noalloc";
    // the size check first (before any device work), then the scratch
    if (count >= 1 && count <= DSPK_MAX_GROUPED && w != nullptr) {
        int32_t ns[DSPK_MAX_GROUPED];
        bool shapes_ok = true;
        int64_t blocks = 0;
        for (int i = 0; i < count; ++i) {
            if (w[i].n < 1 || w[i].k < DSPK_GROUP || w[i].k % DSPK_GROUP || !dspk::supported_bits(w[i].bits))
                shapes_ok = false;
            ns[i] = w[i].n;
            blocks += ((int64_t)w[i].n + 63) / 64;
        }
        if (shapes_ok && m >= 1 && m <= DSPK_MAX_ROWS) {
            const size_t need = dspk::plan_gemm(count, ns, w[0].k, m, w[0].bits, false).ws_bytes;
            if (blocks > dspk::kScratchMaxBlocks || need > dspk::static_scratch_bytes())
                return fail(DSPK_EUNSUPPORTED, "%s: call needs %zu bytes of scratch, more than the %zu this "
                            "entry point holds (too many columns for one allocation-free call)",
                            who, need, dspk::static_scratch_bytes());
        }
    }
    void *ptr = nullptr;
    const hipError_t e = dspk::static_scratch(&ptr, (hipStream_t)stream);
    if (e != hipSuccess) return fail(DSPK_EDEVICE, "%s: scratch set-up failed: %s", who, hipGetErrorString(e));
    return qgemm_common(count, w, x, ldx, m, y, y_dtype, ldy, ptr, dspk::static_scratch_bytes(), stream, who);
}

size_t dspk_lmhead_workspace_bytes(int32_t v, int32_t m) {
    if (v < 1 || m < 1 || m > DSPK_MAX_ROWS) return 0;
    return dspk::plan_gemm(1, &v, DSPK_GROUP, m, 8, true).ws_bytes;
}

static int lmhead_common(const char *who, const dspk_tiled_weight *w, const uint16_t *h, int64_t ldh, int32_t m,
                         int32_t *argmax, float *logits, int64_t ldl, const int32_t *draft_ids, int32_t b,
                         int32_t m_rows, int32_t *accept_len, int32_t *committed, void *workspace, size_t ws_bytes,
                         void *stream) {
    int rc = check_tiled(w, who);
    if (rc) return rc;
    rc = check_rows(h, ldh, m, w->k, who);
    if (rc) return rc;
    if (argmax == nullptr || !aligned(argmax, 4)) return fail(DSPK_EINVAL, "%s: argmax NULL or misaligned", who);
    if (logits != nullptr && (!aligned(logits, 4) || ldl < w->n))
        return fail(DSPK_EINVAL, "%s: logits misaligned or ldl=%lld < v=%d", who, (long long)ldl, w->n);
    if (workspace == nullptr || !aligned(workspace, 256) || ws_bytes < dspk_lmhead_workspace_bytes(w->n, m))
        return fail(DSPK_EINVAL, "%s: workspace of %zu bytes required (256-byte aligned)", who,
                    dspk_lmhead_workspace_bytes(w->n, m));
    const dspk::GemmPlan pl = dspk::plan_gemm(1, &w->n, w->k, m, w->bits, true);
    if (!pl.fits) return fail(DSPK_EUNSUPPORTED, "%s: vocabulary head too large for one launch", who);
    if (ws_bytes < pl.ws_bytes)
        return fail(DSPK_EINVAL, "%s: workspace %zu bytes < %zu required", who, ws_bytes, pl.ws_bytes);
    dspk::GemmLaunch L{};
    fill_plan(L, pl, h, ldh, m, w->k);
    L.count = 1;
    L.done = (uint32_t *)workspace;
    L.counters = (uint32_t *)((char *)workspace + pl.off_counters);
    L.keys = (unsigned long long *)((char *)workspace + pl.off_keys);
    L.partial = (float *)((char *)workspace + pl.off_partial);
    L.argmax = argmax;
    L.logits = logits;
    L.ldl = ldl;
    L.draft = draft_ids;
    L.acc_b = b;
    L.acc_rows = m_rows;
    L.accept_len = accept_len;
    L.committed = committed;
    dspk::GemmProblem &P = L.p[0];
    P.tiles = w->tiles;
    P.n = w->n;
    P.cg_begin = 0;
    return launch_result(dspk::launch_lmhead(L, w->bits, pl.grid, (hipStream_t)stream), who);
}

int dspk_lmhead_argmax(const dspk_tiled_weight *w, const uint16_t *h, int64_t ldh, int32_t m, int32_t *argmax,
                       float *logits, int64_t ldl, void *workspace, size_t ws_bytes, void *stream) {
    return lmhead_common("dspk_lmhead_argmax", w, h, ldh, m, argmax, logits, ldl, nullptr, 0, 0, nullptr, nullptr,
                         workspace, ws_bytes, stream);
}

int dspk_lmhead_argmax_accept_greedy(const dspk_tiled_weight *w, const uint16_t *h, int64_t ldh, int32_t b,
                                     int32_t m_rows, int32_t *argmax, float *logits, int64_t ldl,
                                     const int32_t *draft_ids, int32_t *accept_len, int32_t *committed,
                                     void *workspace, size_t ws_bytes, void *stream) {
    const char *who = "dspk_lmhead_argmax_accept_greedy";
    if (b < 1 || m_rows < 1 || m_rows > DSPK_MAX_ROWS || (int64_t)b * m_rows > DSPK_MAX_ROWS)
        return fail(DSPK_EINVAL, "%s: b=%d x m_rows=%d must be 1..%d rows", who, b, m_rows, DSPK_MAX_ROWS);
    if (accept_len == nullptr || committed == nullptr || !aligned(accept_len, 4) || !aligned(committed, 4))
        return fail(DSPK_EINVAL, "%s: accept_len or committed NULL or misaligned", who);
    if (m_rows > 1 && (draft_ids == nullptr || !aligned(draft_ids, 4)))
        return fail(DSPK_EINVAL, "%s: draft_ids NULL or misaligned", who);
    return lmhead_common(who, w, h, ldh, b * m_rows, argmax, logits, ldl, draft_ids, b, m_rows, accept_len,
                         committed, workspace, ws_bytes, stream);
}

int dspk_accept_greedy(const int32_t *target_ids, const int32_t *draft_ids, int32_t b, int32_t m_rows,
                       int32_t *accept_len, int32_t *committed, void *stream) {
    const char *who = "dspk_accept_greedy";
    if (b < 1) return fail(DSPK_EINVAL, "%s: b=%d must be >= 1", who, b);
    if (m_rows < 1 || m_rows > DSPK_MAX_ROWS)
        return fail(DSPK_EINVAL, "%s: m_rows=%d out of 1..%d", who, m_rows, DSPK_MAX_ROWS);
    if (target_ids == nullptr || accept_len == nullptr || committed == nullptr)
        return fail(DSPK_EINVAL, "%s: NULL pointer", who);
    if (m_rows > 1 && draft_ids == nullptr) return fail(DSPK_EINVAL, "%s: draft_ids is NULL", who);
    return launch_result(
        dspk::launch_accept_greedy(target_ids, draft_ids, b, m_rows, accept_len, committed, (hipStream_t)stream),
        who);
}

size_t dspk_sample_workspace_bytes(int32_t v, int32_t m_rows) {
    if (v < 1 || m_rows < 1) return 0;
    return dspk::sample_workspace_bytes(v, m_rows);
}

static int accept_sample_common(const char *who, const float *logits, int64_t ldz, const float *q, int64_t ldq,
                                const int32_t *draft_ids, const float *uniforms, int32_t m_rows, int32_t v,
                                const dspk_sample_params &sp, const int32_t *counts, int32_t *accept_len,
                                int32_t *committed, void *workspace, size_t ws_bytes, void *stream) {
    if (m_rows < 2 || m_rows > DSPK_MAX_ROWS)
        return fail(DSPK_EINVAL, "%s: m_rows=%d out of 2..%d", who, m_rows, DSPK_MAX_ROWS);
    if (v < 1) return fail(DSPK_EINVAL, "%s: v=%d must be >= 1", who, v);
    if (!(sp.temperature > 0.f) || !isfinite(sp.temperature))
        return fail(DSPK_EINVAL, "%s: temperature must be finite and > 0", who);
    if (sp.top_k < 0) return fail(DSPK_EINVAL, "%s: top_k=%d must be >= 0", who, sp.top_k);
    if (!(sp.top_p > 0.f && sp.top_p <= 1.f)) return fail(DSPK_EINVAL, "%s: top_p must be in (0, 1]", who);
    if (!isfinite(sp.presence_penalty) || !isfinite(sp.frequency_penalty))
        return fail(DSPK_EINVAL, "%s: penalties must be finite", who);
    if (logits == nullptr || q == nullptr || draft_ids == nullptr || uniforms == nullptr || accept_len == nullptr ||
        committed == nullptr)
        return fail(DSPK_EINVAL, "%s: NULL pointer", who);
    if (!aligned(logits, 4) || !aligned(q, 4) || !aligned(counts, 4))
        return fail(DSPK_EINVAL, "%s: misaligned logits, q or counts", who);
    if (ldz < v || ldq < v) return fail(DSPK_EINVAL, "%s: ldz/ldq must be >= v", who);
    const size_t need = dspk_sample_workspace_bytes(v, m_rows);
    if (workspace == nullptr || !aligned(workspace, 256) || ws_bytes < need)
        return fail(DSPK_EINVAL, "%s: workspace of %zu bytes required (256-byte aligned)", who, need);
    dspk::SampleParams P;
    P.z = logits;
    P.ldz = ldz;
    P.q = q;
    P.ldq = ldq;
    P.d = draft_ids;
    P.u = uniforms;
    P.m_rows = m_rows;
    P.v = v;
    P.temperature = sp.temperature;
    P.top_k = sp.top_k;
    P.top_p = sp.top_p;
    P.presence = sp.presence_penalty;
    P.frequency = sp.frequency_penalty;
    P.counts = counts;
    P.accept_len = accept_len;
    P.committed = committed;
    P.ws = workspace;
    return launch_result(dspk::launch_accept_sample(P, (hipStream_t)stream), who);
}

int dspk_accept_sample(const float *logits, int64_t ldz, const float *q, int64_t ldq, const int32_t *draft_ids,
                       const float *uniforms, int32_t m_rows, int32_t v, float temperature, int32_t *accept_len,
                       int32_t *committed, void *workspace, size_t ws_bytes, void *stream) {
    dspk_sample_params sp;
    sp.temperature = temperature;
    sp.top_k = 0;
    sp.top_p = 1.f;
    sp.presence_penalty = 0.f;
    sp.frequency_penalty = 0.f;
    return accept_sample_common("dspk_accept_sample", logits, ldz, q, ldq, draft_ids, uniforms, m_rows, v, sp,
                                nullptr, accept_len, committed, workspace, ws_bytes, stream);
}

int dspk_accept_sample_ex(const float *logits, int64_t ldz, const float *q, int64_t ldq, const int32_t *draft_ids,
                          const float *uniforms, int32_t m_rows, int32_t v, const dspk_sample_params *params,
                          const int32_t *counts, int32_t *accept_len, int32_t *committed, void *workspace,
                          size_t ws_bytes, void *stream) {
    const char *who = "dspk_accept_sample_ex";
    if (params == nullptr) return fail(DSPK_EINVAL, "%s: params is NULL", who);
    return accept_sample_common(who, logits, ldz, q, ldq, draft_ids, uniforms, m_rows, v, *params, counts,
                                accept_len, committed, workspace, ws_bytes, stream);
}

}  // extern "C"

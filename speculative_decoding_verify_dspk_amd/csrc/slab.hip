// Verify-pass projection for launches with few output columns: each
// 16-column tile ("slab") over the whole K range is the work of W waves of
// one workgroup, for gfx950 (MI355X).
//
// What is computed is the projection of qgemm.hip, y[i][c] = sum_r x[i][r] *
// (s[c][r/64] * q[c][r] + b[c][r/64]) ("mlx-dspark" wiki summary, sections
// "Architecture" and "Key techniques": one pass over all verify rows, each
// weight group dequantised once and reused for every row).
//
// Why a second decomposition: the stream-K kernel splits K between
// workgroups so that every CU streams, and a block split between workgroups
// is completed by the last of them to arrive -- three serial device-scope
// round trips (partial stores, arrival ticket, piece loads) at the end of the
// launch.  For the small launches of a decoder layer (2560-column o and down,
// 6144-column q/k/v) that exchange and the cold start are most of the launch.
// Here W waves own one 16-column MFMA tile of one 64-column block: they take
// the block's K units round-robin (unit w, w + W, ...), each wave streams
// only its tile's code slots of each unit (2 KiB of the 8 KiB, plus the
// tile's scale/bias dwords), and the W partial tiles are added in LDS in
// wave order.  No workspace, no cross-workgroup traffic, results
// deterministic (the order of every sum is fixed by the shapes).  The host
// picks W (16, 8, 4, 3 or 2 waves) so that all tiles are resident at once
// where they fit (up to 1, 2, 4, 5 or 8 tiles per CU); with more tiles than
// that it takes 4 waves and the rest run as a second round, which its
// automatic choice only accepts while the weights per CU stay small.  The
// register-staged kernel runs one tile per workgroup; the LDS-staged one
// puts a CU's whole share of tiles in one workgroup (see there).
//
// The arithmetic per group is that of the stream-K kernel: exact-product bf16
// MFMAs on the codes (8-bit codes, or 128 + q below 8 bits) and on a ones
// operand for the row sums of x, then one fp32 scale/bias update.
#include <hip/hip_runtime.h>

#include "decode.h"
#include "dspk_internal.h"

namespace dspk {
namespace {

using namespace dec;

// code slots of one 16-column tile t within a unit (see pack.hip):
//   8-bit : 4 g + t (g = 0, 1)        4-bit : 4 p + t (p = 0, 1)
//   bf16  : 4 h + t (h = 0, 1)        2-bit : t
//   3-bit : t (low planes) and 4 + t / 2 (high bits of tiles t & ~1, t | 1)
constexpr int tile_slots(int bits) { return bits == 2 ? 1 : 2; }
__device__ __forceinline__ int slot_of(int bits, int s, int t) {
    return bits == 2 ? t : bits == 3 ? (s == 0 ? t : 4 + (t >> 1)) : 4 * s + t;
}

// units in flight per wave (register ring), within 128 VGPRs (four waves per SIMD)
constexpr int slab_depth(int bits, int mt) {
    return mt == 2 ? (bits == 16 ? 2 : 1) : (bits == 16 ? 4 : bits == 8 ? 3 : bits == 3 ? 1 : 2);
}

__device__ __forceinline__ u32x4 load_nt(const unsigned char *p) {
    return __builtin_nontemporal_load((const u32x4 *)p);
}
__device__ __forceinline__ u32x4 load16(const unsigned char *p) { return *(const u32x4 *)p; }
__device__ __forceinline__ uint32_t load4(const unsigned char *p) { return *(const uint32_t *)p; }

__device__ __forceinline__ void wait_vm_all() {
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));     // vmcnt(0)
    asm volatile("" ::: "memory");
}

// result stores hidden from the compiler's count of outstanding memory
// operations (see qgemm.hip)
__device__ __forceinline__ void st_global_f32(float *p, float v) {
    asm volatile("global_store_dword %0, %1, off" ::"v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ void st_global_u16(uint16_t *p, uint32_t v) {
    asm volatile("global_store_short %0, %1, off" ::"v"(p), "v"(v) : "memory");
}

// Every W runs at most four waves per SIMD (16 per CU): the plan assumes
// floor(16 / W) tiles of W waves per CU.
//
// The register ring of a wave's n units: requests run DEPTH - 1 units ahead
// of the computation.  The steady-state loop issues without a condition, so
// the compiler's own count of outstanding loads places each wait just before
// its slot is used; the last 2 DEPTH - 2 steps are unrolled with guarded
// requests, so no unit is requested twice (a wave here has only a few units,
// and a repeated request would be a large share of its traffic).  Slots are
// compile-time indices throughout (a run-time index would put the ring in
// scratch memory).
template <int DEPTH, typename Slot, typename Issue, typename Compute>
__device__ __forceinline__ void run_ring(int n, Slot (&ring)[DEPTH], Issue &&issue, Compute &&compute) {
#pragma unroll
    for (int s = 0; s < DEPTH - 1; ++s)
        if (s < n) issue(s, ring[s]);
    int i = 0;
    for (; i + 2 * DEPTH - 1 <= n; i += DEPTH) {
#pragma unroll
        for (int s = 0; s < DEPTH; ++s) {
            issue(i + s + DEPTH - 1, ring[(s + DEPTH - 1) % DEPTH]);
            compute(i + s, ring[s]);
        }
    }
#pragma unroll
    for (int s = 0; s < 2 * DEPTH - 2; ++s)
        if (i + s < n) {
            if (i + s + DEPTH - 1 < n) issue(i + s + DEPTH - 1, ring[(s + DEPTH - 1) % DEPTH]);
            compute(i + s, ring[s % DEPTH]);
        }
}

template <int BITS, int MT, int W>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(4))) void qgemm_slab_kernel(
    const GemmLaunch L) {
    using C = Cfg<BITS>;
    constexpr int DEPTH = slab_depth(BITS, MT);
    constexpr int TS = tile_slots(BITS);
    __shared__ f32x4 red[W][MT][kWave];

    (void)L;
    const GemmLaunch *KL = (const GemmLaunch *)__builtin_amdgcn_kernarg_segment_ptr();
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 15, j = lane >> 4;
    const int gb = (int)blockIdx.x >> 2, t = (int)blockIdx.x & 3;   // global block, tile
    int pi = 0;
#pragma unroll
    for (int i = 1; i < kMaxGrouped; ++i)
        if (i < KL->count && gb >= KL->p[i].cg_begin) pi = i;
    const GemmProblem &P = KL->p[pi];
    const int cb = gb - P.cg_begin;
    if (cb * kBlockCols + 16 * t >= P.n) return;        // a tile wholly past n (the whole workgroup)
    const int NST = KL->nst, K = KL->k, G = K >> 6, M = KL->m;
    const unsigned char *const base = (const unsigned char *)P.tiles + (size_t)cb * NST * C::UNIT;

    // activations: row-major [m][ldx] bf16; lane (c, j) reads row 16*mt + c
    // (clamped to the last row) at K offset 16*j + 8*h of each group: a
    // wave-uniform byte offset per (unit, group, half) plus this lane offset
    const uint32_t LDXB = (uint32_t)KL->ldx * 2u;
    const unsigned char *const xbase = (const unsigned char *)KL->x;
    uint32_t xlane[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) xlane[mt] = (uint32_t)min(16 * mt + c, M - 1) * LDXB + 32u * (uint32_t)j;

    struct Slot {
        u32x4 w[TS];
        uint32_t sb[C::SBQ > 0 ? C::SBQ : 1];
        u32x4 a[C::GS][MT][2];
    };
    Slot ring[DEPTH];

    // this wave's units: w, w + W, ...
    const int nsteps = w < NST ? (NST - 1 - w) / W + 1 : 0;
    auto issue = [&](int i, Slot &s) __attribute__((always_inline)) {
        const int st = w + i * W;
        const unsigned char *ub = base + (size_t)st * C::UNIT;
#pragma unroll
        for (int q = 0; q < TS; ++q) s.w[q] = load_nt(ub + slot_of(BITS, q, t) * 1024 + 16 * lane);
        // dword (group g, tile t) of column c: scale (low half), bias (high half)
#pragma unroll
        for (int g = 0; g < C::SBQ; ++g) s.sb[g] = load4(ub + C::SBOFF + c * (16 * C::SBQ) + 16 * g + 4 * t);
        const int ng = min(C::GS, G - st * C::GS);     // groups of a short last unit; the rest re-read it
#pragma unroll
        for (int g = 0; g < C::GS; ++g)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int chunk = st * (C::KU / 8) + 8 * min(g, ng - 1) + h;
                const unsigned char *xs = xbase + (uint32_t)__builtin_amdgcn_readfirstlane((int)(chunk * 16));
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) s.a[g][mt][h] = load16(xs + xlane[mt]);
            }
    };

    f32x4 y[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) y[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int i, const Slot &s) __attribute__((always_inline)) {
        const int st = w + i * W;
        const int ng = min(C::GS, G - st * C::GS);
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        const bf16x8 ones = as_bf16x8(u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});
#pragma unroll
        for (int g = 0; g < C::GS; ++g) {
            if (g >= ng) break;
            bf16x8 a0[MT], a1[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                if constexpr (BITS == 4) {
                    a0[mt] = as_bf16x8(perm_x_for4(s.a[g][mt][0]));
                    a1[mt] = as_bf16x8(perm_x_for4(s.a[g][mt][1]));
                } else if constexpr (BITS == 2 || BITS == 3) {
                    u32x4 p0, p1;
                    perm_x_for2(s.a[g][mt][0], s.a[g][mt][1], p0, p1);
                    a0[mt] = as_bf16x8(p0);
                    a1[mt] = as_bf16x8(p1);
                } else {
                    a0[mt] = as_bf16x8(s.a[g][mt][0]);
                    a1[mt] = as_bf16x8(s.a[g][mt][1]);
                }
            }
            if constexpr (BITS == 16) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    y[mt] = mfma(a0[mt], as_bf16x8(s.w[0]), y[mt]);
                    y[mt] = mfma(a1[mt], as_bf16x8(s.w[1]), y[mt]);
                }
            } else {
                bf16x8 b0, b1;
                if constexpr (BITS == 8) {
                    const u32x4 qv = s.w[g];
                    b0 = codes8_to_bf16(qv[0], qv[1]);
                    b1 = codes8_to_bf16(qv[2], qv[3]);
                } else if constexpr (BITS == 2) {
                    codes2_to_bf16(s.w[0][g], b0, b1);
                } else if constexpr (BITS == 3) {
                    // high-bit dword 2 (t % 2) + g / 2; t is not a compile-time
                    // constant, so select rather than index the register vector
                    const uint32_t hd = (t & 1) ? s.w[1][2 + (g >> 1)] : s.w[1][g >> 1];
                    codes3_to_bf16(s.w[0][g], hd >> (8 * (g & 1)), b0, b1);
                } else {
                    const u32x4 qv = s.w[g >> 1];
                    b0 = codes4_to_bf16(qv[2 * (g & 1)]);
                    b1 = codes4_to_bf16(qv[2 * (g & 1) + 1]);
                }
                const uint32_t sbd = s.sb[g];
                const float sc = h2f(sbd & 0xffffu);
                float bi = h2f(sbd >> 16);
                if constexpr (BITS <= 4) bi = fmaf(-128.f, sc, bi);   // codes carry +128
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    f32x4 xs = mfma(a0[mt], ones, zero);
                    xs = mfma(a1[mt], ones, xs);
                    f32x4 acc = mfma(a0[mt], b0, zero);
                    acc = mfma(a1[mt], b1, acc);
#pragma unroll
                    for (int r4 = 0; r4 < 4; ++r4) y[mt][r4] = fmaf(sc, acc[r4], fmaf(bi, xs[r4], y[mt][r4]));
                }
            }
        }
    };

    run_ring<DEPTH>(nsteps, ring, issue, compute);

    // the W partial tiles, added in wave order
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) red[w][mt][lane] = y[mt];
    __syncthreads();
    if (w != 0) return;
    const int n = cb * kBlockCols + 16 * t + c;
    if (n >= P.n) return;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        f32x4 z = red[0][mt][lane];
#pragma unroll
        for (int q = 1; q < W; ++q) z += red[q][mt][lane];
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const int m = 16 * mt + 4 * j + r4;
            if (m < M) {
                if (KL->y_bf16)
                    st_global_u16((uint16_t *)P.y + (int64_t)m * P.ldy + n, f2bf16(z[r4]));
                else
                    st_global_f32((float *)P.y + (int64_t)m * P.ldy + n, z[r4]);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// The slab kernel with the activations staged in LDS (8-bit and bf16 weights,
// at most 16 rows).  In the kernel above every wave loads its own activation
// pieces for every unit: one 16-column tile per load, against four in the
// stream-K kernel, so at 8 and more rows those small loads outnumber the
// weight loads and set the launch time (measured on the 2560 x 4096 and
// 2560 x 9728 launches: with constant activations the kernel ran 2 and 4.7 us
// faster).  Here the W waves walk K in lockstep steps of W units (wave w takes
// unit i W + w of step i, as above); the K chunk of x a step needs (m rows x
// W units) is loaded by all threads with full-line 16-byte loads one step
// ahead, written to one of two LDS buffers, and read by the waves with
// ds_read_b128.  Per step: issue the next chunk's loads, then the weights DEPTH
// - 1 steps ahead (in that order: a wait for the chunk then leaves the newer
// weight requests in flight), compute from LDS, store the next chunk, barrier.
// A workgroup may hold T tiles (T W waves, T = blockDim.x / 64 W, consecutive
// tiles of the launch): every tile walks the same K steps, so one staged
// chunk serves all of them, and a CU given T tiles stages each chunk once
// instead of T times.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// v_dot2_f32_bf16: c + a.x * b.x + a.y * b.y (bf16 pairs, products exact in fp32)
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

constexpr int kLdsPad = 8;        // bf16 per staged row: a 16-byte pad keeps the 16 rows of a read off one bank group
constexpr int lds_slab_depth(int bits) { return bits == 16 ? 4 : 2; }

//
// MR > 0 selects the dot-product form (8-bit weights, at most MR rows): the
// same decomposition, weight stream and staged activations, with the K
// reduction on the vector ALUs instead of the matrix cores.  Lane (c, j) holds
// the 16 codes of column c at K offsets 16 j .. 16 j + 15 of a group; they
// become eight exact bf16 pairs, and for each row the lane forms
// d = sum_e x_e q_e and sx = sum_e x_e with v_dot2_f32_bf16, then
// y += s d + b sx.  The four lanes of a column (j = 0..3) are added with two
// cross-lane exchanges, then the waves in LDS, both in a fixed order.  The
// host uses it only when forced: it exists to measure where the matrix cores
// stop paying for padded rows.
template <int BITS, int W, int MR>
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(4))) void qgemm_slab_lds_kernel(
    const GemmLaunch L) {
    using C = Cfg<BITS>;
    static_assert(BITS == 8 || BITS == 16, "activations in LDS: 8-bit and bf16 units only");
    static_assert(MR == 0 || BITS == 8, "the dot-product form is 8-bit only");
    constexpr int DEPTH = lds_slab_depth(BITS);
    constexpr int CK = W * C::KU;                      // K elements per step
    constexpr int ROWP = CK + kLdsPad;                 // staged row pitch (bf16)
    constexpr int PPT = (16 * CK / 8) / (64 * W);      // 16-byte pieces per thread at one tile per workgroup
    // the two chunk buffers; after the last step the same LDS holds the
    // waves' partial tiles (at most 16 waves)
    constexpr int XS = 2 * 16 * ROWP > 16 * kWave * 8 ? 2 * 16 * ROWP : 16 * kWave * 8;
    __shared__ __attribute__((aligned(16))) uint16_t xs[XS];
    f32x4 *const red = (f32x4 *)xs;

    (void)L;
    const GemmLaunch *KL = (const GemmLaunch *)__builtin_amdgcn_kernarg_segment_ptr();
    const int tid = threadIdx.x, lane = tid & 63;
    const int NT = (int)blockDim.x;                     // 64 W T threads
    const int wt = __builtin_amdgcn_readfirstlane(tid >> 6);     // wave in the workgroup
    const int tt = wt / W, w = wt - W * tt;             // its tile in the workgroup, its wave in the tile
    const int c = lane & 15, j = lane >> 4;
    const int tile = (int)blockIdx.x * (NT / (64 * W)) + tt;
    const int gb = tile >> 2, t = tile & 3;
    int pi = 0;
#pragma unroll
    for (int i = 1; i < kMaxGrouped; ++i)
        if (i < KL->count && gb >= KL->p[i].cg_begin) pi = i;
    const GemmProblem &P = KL->p[pi];
    const int cb = gb - P.cg_begin;
    // a tile past the last column still stages and meets every barrier
    const bool active = cb * kBlockCols + 16 * t < P.n;
    const int NST = KL->nst, K = KL->k, G = K >> 6, M = KL->m;
    const int NSTEP = (NST + W - 1) / W;
    // a tile past the last column streams block 0, tile 0 of its problem
    // instead (never used): the weight requests stay unconditional, so the
    // compiler's count of outstanding loads still places each wait
    const int tl = active ? t : 0;
    const unsigned char *const base = (const unsigned char *)P.tiles + (size_t)(active ? cb : 0) * NST * C::UNIT;
    const uint16_t *const xg = KL->x;
    const int64_t ldx = KL->ldx;

    // staging: thread tid copies 8 elements at column col0 of rows r0, r0 +
    // RPP, ... (a pass of the workgroup covers RPP whole rows, RPP = NT / CPR
    // = 512 T / KU); rows past m and columns past k are zero, rows past the
    // 16 staged ones are skipped
    constexpr int CPR = CK / 8;                        // 16-byte pieces per staged row
    static_assert((64 * W) % CPR == 0 && PPT * (64 * W / CPR) == 16, "passes of whole rows cover the 16 rows");
    const int RPP = NT / CPR;
    const int r0 = tid / CPR, col0 = 8 * (tid % CPR);
    const uint16_t *const xt = xg + (int64_t)r0 * ldx + col0;
    u32x4 stg[PPT];
    auto stage_load = [&](int i) __attribute__((always_inline)) {
        const bool kin = i * CK + col0 < K;
#pragma unroll
        for (int q = 0; q < PPT; ++q)
            stg[q] = (r0 + RPP * q < M && kin) ? *(const u32x4 *)(xt + (int64_t)(RPP * q) * ldx + i * CK)
                                               : u32x4{0u, 0u, 0u, 0u};
    };
    uint16_t *const xsl = xs + r0 * ROWP + col0;
    auto stage_store = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < PPT; ++q)
            if (r0 + RPP * q < 16) *(u32x4 *)(xsl + buf * (16 * ROWP) + RPP * q * ROWP) = stg[q];
    };

    struct Slot {
        u32x4 w[2];
        uint32_t sb[C::SBQ > 0 ? C::SBQ : 1];
    };
    Slot ring[DEPTH];
    // the unit of step i for this wave (past the last unit: repeat it; only
    // the final step can be past the end, and its compute is skipped)
    auto issue = [&](int i, Slot &s) __attribute__((always_inline)) {
        const int st = min(w + i * W, NST - 1);
        const unsigned char *ub = base + (size_t)st * C::UNIT;
#pragma unroll
        for (int q = 0; q < 2; ++q) s.w[q] = load_nt(ub + (4 * q + tl) * 1024 + 16 * lane);
#pragma unroll
        for (int g = 0; g < C::SBQ; ++g) s.sb[g] = load4(ub + C::SBOFF + c * (16 * C::SBQ) + 16 * g + 4 * tl);
    };
    f32x4 y = {0.f, 0.f, 0.f, 0.f};
    float yd[MR > 0 ? MR : 1];
#pragma unroll
    for (int r = 0; r < (MR > 0 ? MR : 1); ++r) yd[r] = 0.f;
    const int xrow = min(c, M - 1);
    auto compute = [&](int i, const Slot &s, int buf) __attribute__((always_inline)) {
        const int st = w + i * W;
        if (!active || st >= NST) return;
        const int ng = min(C::GS, G - st * C::GS);
        if constexpr (MR > 0) {
            const uint32_t ONES = 0x3f803f80u;          // two bf16 ones
#pragma unroll
            for (int g = 0; g < C::GS; ++g) {
                if (g >= ng) break;
                const u32x4 qv = s.w[g];
                const u32x4 q0 = __builtin_bit_cast(u32x4, codes8_to_bf16(qv[0], qv[1]));   // codes 0..7, pairs
                const u32x4 q1 = __builtin_bit_cast(u32x4, codes8_to_bf16(qv[2], qv[3]));   // codes 8..15
                const float sc = h2f(s.sb[g] & 0xffffu), bi = h2f(s.sb[g] >> 16);
#pragma unroll
                for (int r = 0; r < MR; ++r) {
                    // rows past m are staged as zeros: they add nothing and are not stored
                    const uint16_t *xp = &xs[buf * (16 * ROWP) + r * ROWP + w * C::KU + 64 * g + 16 * j];
                    const u32x4 xa = *(const u32x4 *)xp, xb = *(const u32x4 *)(xp + 8);
                    float d = 0.f, sx = 0.f;
#pragma unroll
                    for (int p = 0; p < 4; ++p) {
                        d = dot2(xa[p], q0[p], d);
                        sx = dot2(xa[p], ONES, sx);
                    }
#pragma unroll
                    for (int p = 0; p < 4; ++p) {
                        d = dot2(xb[p], q1[p], d);
                        sx = dot2(xb[p], ONES, sx);
                    }
                    yd[r] = fmaf(sc, d, fmaf(bi, sx, yd[r]));
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            return;
        }
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        const bf16x8 ones = as_bf16x8(u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});
        const uint16_t *xr = &xs[buf * (16 * ROWP) + xrow * ROWP + w * C::KU + 16 * j];
#pragma unroll
        for (int g = 0; g < C::GS; ++g) {
            if (g >= ng) break;
            const bf16x8 a0 = as_bf16x8(*(const u32x4 *)(xr + 64 * g));
            const bf16x8 a1 = as_bf16x8(*(const u32x4 *)(xr + 64 * g + 8));
            if constexpr (BITS == 16) {
                y = mfma(a0, as_bf16x8(s.w[0]), y);
                y = mfma(a1, as_bf16x8(s.w[1]), y);
            } else {
                const u32x4 qv = s.w[g];
                const bf16x8 b0 = codes8_to_bf16(qv[0], qv[1]);
                const bf16x8 b1 = codes8_to_bf16(qv[2], qv[3]);
                const float sc = h2f(s.sb[g] & 0xffffu), bi = h2f(s.sb[g] >> 16);
                f32x4 xsum = mfma(a0, ones, zero);
                xsum = mfma(a1, ones, xsum);
                f32x4 acc = mfma(a0, b0, zero);
                acc = mfma(a1, b1, acc);
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) y[r4] = fmaf(sc, acc[r4], fmaf(bi, xsum[r4], y[r4]));
            }
            // one group at a time: otherwise the scheduler converts the codes
            // of several steps up front and runs out of registers
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto lds_barrier = [&]() __attribute__((always_inline)) {
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };
    // one step; `guarded`: the tail, where requests past the end are skipped
    auto step = [&](int i, Slot &cur, Slot &nxt, bool guarded) __attribute__((always_inline)) {
        if (i + 1 < NSTEP) stage_load(i + 1);
        if (!guarded || i + DEPTH - 1 < NSTEP) issue(i + DEPTH - 1, nxt);
        compute(i, cur, i & 1);
        if (i + 1 < NSTEP) stage_store((i + 1) & 1);
        lds_barrier();
    };

    stage_load(0);
    stage_store(0);
#pragma unroll
    for (int s = 0; s < DEPTH - 1; ++s)
        if (s < NSTEP) issue(s, ring[s]);
    lds_barrier();
    int i = 0;
    for (; i + 2 * DEPTH - 1 <= NSTEP; i += DEPTH) {
#pragma unroll
        for (int s = 0; s < DEPTH; ++s) step(i + s, ring[s], ring[(s + DEPTH - 1) % DEPTH], false);
    }
#pragma unroll
    for (int s = 0; s < 2 * DEPTH - 2; ++s)
        if (i + s < NSTEP) step(i + s, ring[s % DEPTH], ring[(s + DEPTH - 1) % DEPTH], true);
    wait_vm_all();                     // a final-step request past the last unit has landed

    const int n = cb * kBlockCols + 16 * t + c;
    if constexpr (MR > 0) {
        // the four K quarters of a column (lanes c, c + 16, c + 32, c + 48), then the waves
        float *redf = (float *)red;
#pragma unroll
        for (int r = 0; r < MR; ++r) {
            yd[r] += __shfl_xor(yd[r], 16);
            yd[r] += __shfl_xor(yd[r], 32);
            if (j == 0) redf[(wt * MR + r) * 16 + c] = yd[r];
        }
        __syncthreads();
        if (!active || w != 0 || j != 0 || n >= P.n) return;
#pragma unroll
        for (int r = 0; r < MR; ++r) {
            if (r >= M) break;
            float z = redf[(W * tt * MR + r) * 16 + c];
#pragma unroll
            for (int q = 1; q < W; ++q) z += redf[((W * tt + q) * MR + r) * 16 + c];
            if (KL->y_bf16)
                st_global_u16((uint16_t *)P.y + (int64_t)r * P.ldy + n, f2bf16(z));
            else
                st_global_f32((float *)P.y + (int64_t)r * P.ldy + n, z);
        }
        return;
    }
    red[wt * kWave + lane] = y;
    __syncthreads();
    if (!active || w != 0) return;
    if (n >= P.n) return;
    f32x4 z = red[W * tt * kWave + lane];
#pragma unroll
    for (int q = 1; q < W; ++q) z += red[(W * tt + q) * kWave + lane];
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
        const int m = 4 * j + r4;
        if (m < M) {
            if (KL->y_bf16)
                st_global_u16((uint16_t *)P.y + (int64_t)m * P.ldy + n, f2bf16(z[r4]));
            else
                st_global_f32((float *)P.y + (int64_t)m * P.ldy + n, z[r4]);
        }
    }
}

template <int BITS, int MT>
hipError_t launch_w(const GemmLaunch &L, int waves, hipStream_t s) {
    const dim3 grid((unsigned)(4 * L.total_cg));
    switch (waves) {
        case 16: hipLaunchKernelGGL((qgemm_slab_kernel<BITS, MT, 16>), grid, dim3(1024), 0, s, L); break;
        case 8: hipLaunchKernelGGL((qgemm_slab_kernel<BITS, MT, 8>), grid, dim3(512), 0, s, L); break;
        case 4: hipLaunchKernelGGL((qgemm_slab_kernel<BITS, MT, 4>), grid, dim3(256), 0, s, L); break;
        case 3: hipLaunchKernelGGL((qgemm_slab_kernel<BITS, MT, 3>), grid, dim3(192), 0, s, L); break;
        case 2: hipLaunchKernelGGL((qgemm_slab_kernel<BITS, MT, 2>), grid, dim3(128), 0, s, L); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// Tiles per workgroup of the LDS-staged slab kernel: a CU's whole share
// ceil(tiles / CUs) in one workgroup of T W <= 16 waves (one workgroup per
// CU), so that the CU stages each chunk of x once; 1 where the share does not
// fit (the tiles then run in more than one round).
int lds_tiles_per_workgroup(int64_t tiles, int waves, int cus) {
    const int64_t share = (tiles + cus - 1) / cus;
    return share >= 1 && share * waves <= 16 ? (int)share : 1;
}

template <int BITS, int MR = 0>
hipError_t launch_lds_w(const GemmLaunch &L, int waves, hipStream_t s) {
    const int64_t tiles = 4 * (int64_t)L.total_cg;
    const int T = lds_tiles_per_workgroup(tiles, waves, device_cus());
    const dim3 grid((unsigned)((tiles + T - 1) / T)), block((unsigned)(64 * waves * T));
    switch (waves) {
        case 16: hipLaunchKernelGGL((qgemm_slab_lds_kernel<BITS, 16, MR>), grid, block, 0, s, L); break;
        case 8: hipLaunchKernelGGL((qgemm_slab_lds_kernel<BITS, 8, MR>), grid, block, 0, s, L); break;
        case 4: hipLaunchKernelGGL((qgemm_slab_lds_kernel<BITS, 4, MR>), grid, block, 0, s, L); break;
        case 3: hipLaunchKernelGGL((qgemm_slab_lds_kernel<BITS, 3, MR>), grid, block, 0, s, L); break;
        case 2: hipLaunchKernelGGL((qgemm_slab_lds_kernel<BITS, 2, MR>), grid, block, 0, s, L); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int BITS>
hipError_t launch_bits(const GemmLaunch &L, int waves, hipStream_t s) {
    if constexpr (BITS == 8 || BITS == 16)
        if (L.m <= 16) return launch_lds_w<BITS>(L, waves, s);
    return L.m <= 16 ? launch_w<BITS, 1>(L, waves, s) : launch_w<BITS, 2>(L, waves, s);
}

}  // namespace

hipError_t launch_qgemm_dot(const GemmLaunch &L, int waves, hipStream_t s) {
    if (L.m <= 1) return launch_lds_w<8, 1>(L, waves, s);
    if (L.m <= 2) return launch_lds_w<8, 2>(L, waves, s);
    if (L.m <= 4) return launch_lds_w<8, 4>(L, waves, s);
    return hipErrorInvalidValue;
}

hipError_t launch_qgemm_slab(const GemmLaunch &L, int bits, int waves, hipStream_t s) {
    switch (bits) {
        case 2: return launch_bits<2>(L, waves, s);
        case 3: return launch_bits<3>(L, waves, s);
        case 4: return launch_bits<4>(L, waves, s);
        case 8: return launch_bits<8>(L, waves, s);
        case 16: return launch_bits<16>(L, waves, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace dspk

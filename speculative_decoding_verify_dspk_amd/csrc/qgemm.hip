// Verify-pass projections through affine group-quantised weights, and the
// vocabulary head fused with the row argmax, for gfx950 (MI355X).
//
// What is computed: y[i][c] = sum_r x[i][r] * (s[c][r/64] * q[c][r] + b[c][r/64])
// for the M = anchor + drafts rows i ("mlx-dspark" wiki summary, sections
// "Architecture" and "Key techniques": one target pass over all rows, each
// weight group dequantised once and reused for every row).
//
// How (MI355X-first, not the pages' Metal kernel):
// * The weights are the only large stream.  They are read in the library's
//   tiled layout (pack.hip): units of 64 columns x one K slice, 8 KiB of codes
//   plus their scale/bias dwords, already in the order in which each lane
//   feeds the matrix cores.  A wave loads a unit straight into registers with
//   eight fully coalesced 1 KiB global_load_dwordx4 (non-temporal) plus one
//   16-byte scale/bias load per group, DEPTH units deep (kernel_depth), so a workgroup's
//   four waves read one contiguous 35 KiB run per step and the whole launch
//   sweeps memory in order.  Nothing passes through LDS on the way in.
// * The group is the MFMA contraction unit.  Codes 0..255 (and 128+q for
//   4-bit) are exact in bf16 and the rows are bf16, so
//     sum_{r in group} x*w = s * sum x*q + b * sum x
//   is formed from two exact-product bf16 MFMAs (v_mfma_f32_16x16x32_bf16,
//   fp32 accumulation) plus a per-group fp32 scale/bias update.  The row sums
//   of x per group come from the same MFMA against a ones operand.  No
//   dequantised weight is ever rounded.
// * M rows pad to 16 (MT = 1) or 32 (MT = 2) MFMA rows; the weight fragment is
//   converted once and multiplied into every row tile, so the weight bytes per
//   call do not depend on M.
// * Work unit of a workgroup = a "quad": one 64-column block times four
//   consecutive units, one per wave.  Persistent workgroups (OCC per CU) take
//   contiguous ranges of the quads of the whole launch (stream-K over
//   workgroups), so small and large weights alike keep every CU streaming;
//   the two workgroups that share a CU split one range unevenly (see
//   range_begin).  A block inside one range is summed by its four waves
//   through LDS in wave order without a workgroup barrier; a block split
//   between workgroups (the first or last piece of a range) is summed
//   through LDS per piece and completed by the last workgroup to arrive,
//   which adds the pieces in workgroup order.  Results do not depend on
//   scheduling.  Pieces and arrival counters move through device-scope
//   atomic accesses, so no cache flush is needed.
// * Head: row maxima fold into one 64-bit key per row by atomic max; the
//   last workgroup writes the ids (and, on request, runs the greedy
//   acceptance on them).
#include <hip/hip_runtime.h>

#include "decode.h"
#include "dspk_internal.h"

namespace dspk {
namespace {

using namespace dec;

constexpr int NT = kTilesPerWave;
constexpr uint32_t kSlots = 2;      // whole-block sums in flight per workgroup

// Total order used for the argmax: larger value first, NaN above everything,
// -0 equal to +0, then the smaller column.  0 is below every real key.
__device__ __forceinline__ unsigned long long argmax_key(float v, int col) {
    uint32_t u = __float_as_uint(v);
    if (v != v) {
        u = 0xffffffffu;
    } else {
        if (u == 0x80000000u) u = 0u;
        u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    }
    return ((unsigned long long)u << 32) | (unsigned long long)(0xffffffffu - (uint32_t)col);
}

// 16-column tiles posted per pass of the in-workgroup sum
constexpr int CTILES = kTilesPerWave;

// Workgroup barrier for LDS traffic only: it does not wait for this wave's
// outstanding global loads (the next units stay in flight across it).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ f32x4 lds_get(const f32x4 *__restrict__ p) { return *p; }
__device__ __forceinline__ void lds_put(f32x4 *__restrict__ p, f32x4 v) { *p = v; }

// Wait until every vector memory access of this wave has completed.
__device__ __forceinline__ void wait_vm_all() {
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));     // vmcnt(0); expcnt, lgkmcnt not waited
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ u32x4 load_nt(const unsigned char *p) {
    return __builtin_nontemporal_load((const u32x4 *)p);
}
__device__ __forceinline__ u32x4 load16(const unsigned char *p) { return *(const u32x4 *)p; }

// Result stores as asm: the compiler's count of outstanding memory operations
// treats pending stores as out of order with the loads and would then wait for
// every load in flight at the next use of a loaded register.  Hidden from it,
// the stores only make its own waits longer than needed (never shorter); the
// stores themselves need no wait inside the kernel.
__device__ __forceinline__ void st_global_f32(float *p, float v) {
    asm volatile("global_store_dword %0, %1, off" ::"v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ void st_global_u16(uint16_t *p, uint32_t v) {
    asm volatile("global_store_short %0, %1, off" ::"v"(p), "v"(v) : "memory");
}

// A lane's four partial sums of one 16-row tile as two device-scope 64-bit
// accesses, laid out [half][lane][2] so that each wave-wide access covers
// 512 contiguous bytes (four scattered 4-byte stores per lane wrote 13.6 MB
// of counted HBM writes per head launch).
__device__ __forceinline__ void store_pair4(float *tile, int lane, f32x4 v) {
    unsigned long long *q = (unsigned long long *)tile;
    const unsigned long long lo = (unsigned long long)__float_as_uint(v[0]) |
                                  ((unsigned long long)__float_as_uint(v[1]) << 32);
    const unsigned long long hi = (unsigned long long)__float_as_uint(v[2]) |
                                  ((unsigned long long)__float_as_uint(v[3]) << 32);
    __hip_atomic_store(q + lane, lo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(q + kWave + lane, hi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ f32x4 load_pair4(const float *tile, int lane) {
    unsigned long long *q = (unsigned long long *)tile;
    const unsigned long long lo = __hip_atomic_load(q + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned long long hi = __hip_atomic_load(q + kWave + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return f32x4{__uint_as_float((uint32_t)lo), __uint_as_float((uint32_t)(lo >> 32)), __uint_as_float((uint32_t)hi),
                 __uint_as_float((uint32_t)(hi >> 32))};
}


// First quad of workgroup v when `quads` are split over `groups` workgroups
// (quads * groups < 2^31 is checked on the host).
__device__ __forceinline__ int quad_begin(int quads, int groups, int v) {
    return (int)(((uint32_t)quads * (uint32_t)v) / (uint32_t)groups);
}
// workgroup whose quad range contains quad q (every range is non-empty)
__device__ __forceinline__ int quad_owner(int quads, int groups, int q) {
    return (int)(((uint32_t)(q + 1) * (uint32_t)groups + (uint32_t)quads - 1u) / (uint32_t)quads) - 1;
}

// Two workgroups per CU: the dispatcher places workgroups b and b + pairs on
// one CU, and the one dispatched first (b) is served ahead of the other by the
// memory pipeline, so with equal shares the later one finishes well after it
// (measured: 58 vs 70 us medians on the 151936 x 2560 head) and runs its tail
// at half the CU's loads in flight.  Each CU's pair therefore gets one equal
// range, which the earlier workgroup splits kLeadNum / kLeadDen : rest with
// the later one.  Ranks number the workgroups in memory order (pair p: ranks
// 2p, 2p + 1); with pairs == 0 the split is plain equal.
constexpr uint32_t kLeadNum = 10, kLeadDen = 16;   // swept 8..12 sixteenths on the head: 10 fastest
// The earlier workgroup takes max(ceil(n / 2), floor(n * f)) of a pair's n
// quads: rounding down alone would hand the later one the larger piece of a
// short range (n = 3: 1 and 2).  A pair's range has n >= 2 quads (quads >=
// grid), and both terms lie in [1, n - 1] for n >= 2 when 1/2 <= f < 1, so
// both pieces are non-empty.
static_assert(2 * kLeadNum >= kLeadDen && kLeadNum < kLeadDen,
              "a pair's range of >= 2 quads must give both workgroups a non-empty piece");
// A pair whose range spans at least four blocks (nq quads each) moves the
// split point to the nearest block boundary inside the range: then neither
// workgroup has a split piece there (no cross-workgroup exchange, no ring
// drain), at a cost of at most half a block in the balance (head 75 -> 74 us).
__device__ __forceinline__ int split_point(int a, int b, int nq) {
    const uint32_t n = (uint32_t)(b - a);
    const uint32_t lead = (n * kLeadNum) / kLeadDen, half = (n + 1) / 2;
    const int sp = a + (int)(lead > half ? lead : half);
    if ((int)n >= 4 * nq) {
        const int al = ((sp + nq / 2) / nq) * nq;
        if (al > a && al < b) return al;
    }
    return sp;
}
__device__ __forceinline__ int range_begin(int quads, int grid, int pairs, int rank, int nq) {
    if (pairs == 0) return quad_begin(quads, grid, rank);
    const int p = rank >> 1;
    const int a = quad_begin(quads, pairs, p);
    if ((rank & 1) == 0) return a;
    return split_point(a, quad_begin(quads, pairs, p + 1), nq);
}
__device__ __forceinline__ int range_owner(int quads, int grid, int pairs, int q, int nq) {
    if (pairs == 0) return quad_owner(quads, grid, q);
    const int p = quad_owner(quads, pairs, q);
    const int s = split_point(quad_begin(quads, pairs, p), quad_begin(quads, pairs, p + 1), nq);
    return 2 * p + (q >= s ? 1 : 0);
}

__device__ __forceinline__ unsigned long long umax64(unsigned long long a, unsigned long long b) {
    return a > b ? a : b;
}

template <int BITS, int MT, bool ARGMAX>
__global__ __launch_bounds__(256, kernel_occ(BITS, MT, ARGMAX)) void qgemm_kernel(const GemmLaunch L) {
    using C = Cfg<BITS>;
    constexpr int DEPTH = kernel_depth(BITS, MT, ARGMAX);
    // LDS slots for whole-block sums: two, unless that would keep the
    // kernel's workgroups per CU from fitting in the 160 KiB of LDS
    constexpr uint32_t SL = kernel_occ(BITS, MT, ARGMAX) * (2 * 16 * MT + 16) < 160 ? kSlots : 1;
    constexpr int XB = MT == 1 ? 8 : 4;        // partial sums in flight when completing a split block
    // In-workgroup sum (each wave posts CTILES of its 16-column tiles per
    // pass, one 16-row tile at a time); after the main loop the same bytes
    // hold the argmax reduction.
    __shared__ union {
        f32x4 cbuf[kWavesPerWG][CTILES][kWave];
        struct {
            unsigned long long red[kWavesPerWG][kMaxRows];
            int flag;
        } tail;
    } sh;
    auto &cbuf = sh.cbuf;
    // Whole-block sums without a workgroup barrier: each wave posts its four
    // tiles into a slot and counts itself in with an LDS atomic; the fourth
    // wave to arrive adds the posts in wave order and finishes the block.
    // A slot word holds (use << 3) | arrivals; a wave waits for the slot's
    // previous use to be finished (use advanced) before posting into it.
    __shared__ f32x4 slots[SL][kWavesPerWG][NT][MT][kWave];
    __shared__ uint32_t slot_word[SL];
    auto &red = sh.tail.red;
    int &s_flag = sh.tail.flag;

    // Every field is read in place from the kernel-argument segment (scalar
    // loads): the problem table is indexed at run time, and a by-value copy
    // captured by the lambdas below would be spilled to scratch.
    (void)L;
    const GemmLaunch *KL = (const GemmLaunch *)__builtin_amdgcn_kernarg_segment_ptr();
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 15, j = lane >> 4;
    const int GRID = gridDim.x;
    const int PAIRS = KL->pairs;
    // rank of this workgroup in memory order (indexes its range and its
    // partial-sum slots)
    const int bid = PAIRS == 0 ? (int)blockIdx.x
                               : ((int)blockIdx.x < PAIRS ? 2 * (int)blockIdx.x : 2 * ((int)blockIdx.x - PAIRS) + 1);
    const int QU = KL->quads;                 // quads of the launch
    const int NQ = KL->nq;                    // quads per block
    const int NST = KL->nst;                  // units per block
    const int LASTW = NST - 4 * (NQ - 1);     // waves with a unit in a block's last quad (1..4)
    const int K = KL->k;
    const int G = K >> 6;
    const int Q0 = range_begin(QU, GRID, PAIRS, bid, NQ), Q1 = range_begin(QU, GRID, PAIRS, bid + 1, NQ);
    const int M = KL->m;
    if (tid < (int)SL) slot_word[tid] = 0u;
    __syncthreads();

    // global block -> weight index
    auto weight_of = [&](int gb) __attribute__((always_inline)) {
        int pi = 0;
#pragma unroll
        for (int i = 1; i < kMaxGrouped; ++i)
            if (i < KL->count && gb >= KL->p[i].cg_begin) pi = i;
        return pi;
    };

    // This wave's quads in [Q0, Q1), walked with (quad, block, index in block).
    // A quad is skipped only when it is the last of its block and this wave
    // has no unit in it; when NQ == 1 that holds for all of them, and the
    // wave has no unit at all.
    struct Cur {
        int q, gb, qi;
    };
    const bool skips_last = w >= LASTW;
    auto advance = [&](Cur &u) __attribute__((always_inline)) {
        ++u.q;
        if (++u.qi == NQ) { u.qi = 0; ++u.gb; }
        if (skips_last && u.qi == NQ - 1) { ++u.q; u.qi = 0; ++u.gb; }
    };
    const int nsteps = (NQ == 1 && skips_last)
                           ? 0
                           : (Q1 - Q0) - (skips_last ? (Q1 / NQ - Q0 / NQ) : 0);

    // One ring slot: a unit's eight code pieces and scale/bias dwords of this
    // lane, and the matching activation fragments.
    struct Slot {
        u32x4 w[C::NS];
        u32x4 sb[C::SBQ > 0 ? C::SBQ : 1];
        u32x4 a[C::GS][MT][2];
    };
    Slot ring[DEPTH];

    // Base of the block the requests are in (wave-uniform), refreshed when
    // they move to a new block.
    int ib_gb = -1;
    const unsigned char *ib_base = nullptr;
    // activations: row-major [m][ldx] bf16.  Lane (c, j) reads the 16-byte
    // piece of row 16*mt + c (clamped to the last row) at K offset 16*j + 8*h
    // of each group: a wave-uniform byte offset per (unit, group, half) plus
    // this fixed lane offset.  The two halves of a group read the two halves
    // of the same 64-byte span of each row, so the second load hits L1.
    const uint32_t LDXB = (uint32_t)KL->ldx * 2u;
    const unsigned char *const xbase = (const unsigned char *)KL->x;
    uint32_t xlane[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) xlane[mt] = (uint32_t)min(16 * mt + c, M - 1) * LDXB + 32u * (uint32_t)j;

    // Request this wave's unit of quad u and its activation fragments into
    // slot s.  Lane (c, j) takes 16 bytes of each 1 KiB code slot and the
    // dwords of its column c; units are contiguous, so a quad is one run.
    auto issue = [&](const Cur &u, Slot &s) __attribute__((always_inline)) {
        if (u.gb != ib_gb) {
            ib_gb = u.gb;
            const GemmProblem &P = KL->p[weight_of(u.gb)];
            ib_base = (const unsigned char *)P.tiles + (size_t)(u.gb - P.cg_begin) * NST * C::UNIT;
        }
        const int st = 4 * u.qi + w;
        const unsigned char *ub = ib_base + (size_t)st * C::UNIT;
#pragma unroll
        for (int i = 0; i < C::NS; ++i) s.w[i] = load_nt(ub + i * 1024 + 16 * lane);
#pragma unroll
        for (int q = 0; q < C::SBQ; ++q) s.sb[q] = load16(ub + C::SBOFF + c * (16 * C::SBQ) + 16 * q);
        // lane (c, j) takes row 16*mt + c, K offsets 64*g + 16*j (+8): a
        // wave-uniform byte offset per (g, h) plus a fixed lane offset.  The
        // groups past the end of K (a short last unit) re-read the last one,
        // so no load reaches past a row's k entries.
        const int ng = min(C::GS, G - st * C::GS);
#pragma unroll
        for (int g = 0; g < C::GS; ++g)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int chunk = st * (C::KU / 8) + 8 * min(g, ng - 1) + h;   // 8-element chunk of the row
                const uint32_t off = (uint32_t)chunk * 16u;
                const unsigned char *xs = xbase + (uint32_t)__builtin_amdgcn_readfirstlane((int)off);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) s.a[g][mt][h] = load16(xs + xlane[mt]);
            }
    };

    f32x4 y[NT][MT];
    auto zero_y = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) y[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    };

    // MFMA work of this wave's unit of quad u, from slot s
    auto compute = [&](const Cur &u, const Slot &s) __attribute__((always_inline)) {
        const int st = 4 * u.qi + w;
        const int ng = min(C::GS, G - st * C::GS);      // groups of a short last unit
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
                // slot h*4 + t: bf16 weights of K offsets 16*j + 8*h of tile t
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const bf16x8 b0 = as_bf16x8(s.w[t]);
                    const bf16x8 b1 = as_bf16x8(s.w[4 + t]);
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) {
                        y[t][mt] = mfma(a0[mt], b0, y[t][mt]);
                        y[t][mt] = mfma(a1[mt], b1, y[t][mt]);
                    }
                }
            } else {
                f32x4 xs[MT];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    xs[mt] = mfma(a0[mt], ones, zero);
                    xs[mt] = mfma(a1[mt], ones, xs[mt]);
                }
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    bf16x8 b0, b1;
                    if constexpr (BITS == 8) {
                        // slot g*4 + t: the 16 codes of K offsets 64*g + 16*j
                        const u32x4 qv = s.w[4 * g + t];
                        b0 = codes8_to_bf16(qv[0], qv[1]);
                        b1 = codes8_to_bf16(qv[2], qv[3]);
                    } else if constexpr (BITS == 2) {
                        // slot t, dword g
                        codes2_to_bf16(s.w[t][g], b0, b1);
                    } else if constexpr (BITS == 3) {
                        // low planes: slot t, dword g; high bits: slot 4 + t/2,
                        // dword 2*(t%2) + g/2, byte lanes 8*(g%2) of each half
                        const uint32_t hd = s.w[4 + (t >> 1)][2 * (t & 1) + (g >> 1)];
                        codes3_to_bf16(s.w[t][g], hd >> (8 * (g & 1)), b0, b1);
                    } else {
                        // slot (g/2)*4 + t: groups 2*(g/2) and 2*(g/2)+1, 8 bytes each
                        const u32x4 qv = s.w[4 * (g >> 1) + t];
                        b0 = codes4_to_bf16(qv[2 * (g & 1)]);
                        b1 = codes4_to_bf16(qv[2 * (g & 1) + 1]);
                    }
                    // dword t of load g: scale (low half) and bias (high half)
                    const uint32_t sbd = s.sb[g][t];
                    const float sc = h2f(sbd & 0xffffu);
                    float bi = h2f(sbd >> 16);
                    if constexpr (BITS <= 4) bi = fmaf(-128.f, sc, bi);   // codes carry +128
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) {
                        f32x4 acc = mfma(a0[mt], b0, zero);
                        acc = mfma(a1[mt], b1, acc);
#pragma unroll
                        for (int r4 = 0; r4 < 4; ++r4)
                            y[t][mt][r4] = fmaf(sc, acc[r4], fmaf(bi, xs[mt][r4], y[t][mt][r4]));
                    }
                    // one tile at a time: the scheduler would otherwise convert
                    // every tile's codes up front and run out of registers
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
    };

    // running row maxima (value, column) of the tiles this wave finished
    unsigned long long wbest[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) wbest[mt][r4] = 0ull;

    // Final values of this wave's tile (columns 16*w .. 16*w+15 of block cb):
    // store them, or fold them into the argmax.
    auto finish_tile = [&](int pi, int cb, int t, const f32x4 (&z)[MT]) __attribute__((always_inline)) {
        const GemmProblem &P = KL->p[pi];
        const int n = cb * kBlockCols + 16 * t + c;
        const int N = P.n;
        if (n >= N) return;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int m = 16 * mt + 4 * j + r4;
                const float v = z[mt][r4];
                if constexpr (!ARGMAX) {
                    if (m < M) {
                        if (KL->y_bf16)
                            st_global_u16((uint16_t *)P.y + (int64_t)m * P.ldy + n, f2bf16(v));
                        else
                            st_global_f32((float *)P.y + (int64_t)m * P.ldy + n, v);
                    }
                } else {
                    wbest[mt][r4] = umax64(wbest[mt][r4], argmax_key(v, n));
                    if (KL->logits != nullptr && m < M) st_global_f32(KL->logits + (int64_t)m * KL->ldl + n, v);
                }
            }
    };

    // End of the workgroup's piece [a, b) of one block: add the four waves'
    // sums through LDS in wave order (wave w keeps tile w), then finish the
    // tile, or hand the piece to the last workgroup that works on the block.
    uint32_t seq = 0;     // whole blocks closed so far (the same count in every wave)
    auto close_piece = [&](int a, int b) __attribute__((always_inline)) {
        const int gb = a / NQ;
        const int pi = weight_of(gb);
        const int cb = gb - KL->p[pi].cg_begin;
        if (a == gb * NQ && b == gb * NQ + NQ) {
            const uint32_t sl = seq % SL, use = seq / SL;
            ++seq;
            // the slot's previous use has been read out (its last wave moved
            // it on); waves are at most SL blocks apart, so this ends.
            // The bound only guards against a broken invariant: a wave never
            // spins forever (results would then be wrong, not the GPU hung).
            for (int spin = 0; spin < (1 << 20); ++spin) {
                if ((__hip_atomic_load(&slot_word[sl], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >> 3) == use)
                    break;
                __builtin_amdgcn_s_sleep(1);
            }
            asm volatile("" ::: "memory");
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) lds_put(&slots[sl][w][t][mt][lane], y[t][mt]);
            // LDS operations of a wave complete in order: the posts land before the count
            __builtin_amdgcn_s_waitcnt(0xc07f);           // lgkmcnt(0) only
            asm volatile("" ::: "memory");
            // one arrival per wave: a single lane counts the wave in
            uint32_t old = 0;
            if (lane == 0)
                old = __hip_atomic_fetch_add(&slot_word[sl], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            old = (uint32_t)__builtin_amdgcn_readfirstlane((int)old);
            if ((old & 7u) != kWavesPerWG - 1) return;
            asm volatile("" ::: "memory");
            // one tile at a time (few registers next to the ring)
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                f32x4 zt[MT];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    zt[mt] = lds_get(&slots[sl][0][t][mt][lane]);
#pragma unroll
                    for (int q = 1; q < kWavesPerWG; ++q) zt[mt] += lds_get(&slots[sl][q][t][mt][lane]);
                }
                finish_tile(pi, cb, t, zt);
            }
            __builtin_amdgcn_s_waitcnt(0xc07f);           // every read of the slot is done
            asm volatile("" ::: "memory");
            if (lane == 0)
                __hip_atomic_store(&slot_word[sl], (use + 1) << 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            return;
        }
        f32x4 z[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
            for (int t0 = 0; t0 < NT; t0 += CTILES) {
                lds_barrier();                           // the previous sum has been read
#pragma unroll
                for (int t = 0; t < CTILES; ++t) lds_put(&cbuf[w][t][lane], y[t0 + t][mt]);
                lds_barrier();
                if (w >= t0 && w < t0 + CTILES) {
                    z[mt] = lds_get(&cbuf[0][w - t0][lane]);
#pragma unroll
                    for (int q = 1; q < kWavesPerWG; ++q) z[mt] += lds_get(&cbuf[q][w - t0][lane]);
                }
            }
        }
        const int bq0 = gb * NQ, bq1 = bq0 + NQ;
        // publish: slot 0 for the workgroup's first piece, 1 for its last
        const int side = a == Q0 ? 0 : 1;
        float *mine = KL->partial + (((int64_t)bid * 2 + side) * kWavesPerWG + w) * (MT * kWave * 4);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) store_pair4(mine + mt * kWave * 4, lane, z[mt]);
        wait_vm_all();
        const int wf = range_owner(QU, GRID, PAIRS, bq0, NQ), wl = range_owner(QU, GRID, PAIRS, bq1 - 1, NQ);
        uint32_t ticket = 0;
        uint32_t *ctr = KL->counters + (int64_t)gb * kWavesPerWG + w;
        if (lane == 0) ticket = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ticket = __shfl(ticket, 0);
        if (ticket != (uint32_t)(wl - wf)) return;
        // Last arrival: the pieces in workgroup order, XB pieces in
        // flight (few: the ring's registers are live here).  Every workgroup after wf starts inside the block (its piece
        // is its first, slot 0); wf's piece is its first only if its range
        // starts at the block start.
        const int wf_side = range_begin(QU, GRID, PAIRS, wf, NQ) >= bq0 ? 0 : 1;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) z[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int v0 = wf; v0 <= wl; v0 += XB) {
            f32x4 part[XB][MT];
#pragma unroll
            for (int i = 0; i < XB; ++i) {
                const int v = min(v0 + i, wl);
                const int sl = v == wf ? wf_side : 0;
                const float *src = KL->partial + (((int64_t)v * 2 + sl) * kWavesPerWG + w) * (MT * kWave * 4);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) part[i][mt] = load_pair4(src + mt * kWave * 4, lane);
            }
            // every loaded value is consumed (a duplicate past wl adds zero), so
            // no load of this batch is left pending
#pragma unroll
            for (int i = 0; i < XB; ++i) {
                const bool real = v0 + i <= wl;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const f32x4 p = real ? part[i][mt] : f32x4{0.f, 0.f, 0.f, 0.f};
                    z[mt] = (v0 + i == wf) ? p : z[mt] + p;
                }
            }
        }
        if (lane == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        finish_tile(pi, cb, w, z);
    };

    // Pieces not yet closed start at `open`; close every piece that ends at or
    // before quad `lim`.  All four waves close the same pieces in the same
    // order, so their barriers match.
    int open = Q0;
    auto close_until = [&](int lim) __attribute__((always_inline)) {
        while (open < Q1) {
            const int end = min((open / NQ + 1) * NQ, Q1);
            if (end > lim) break;
            close_piece(open, end);
            zero_y();
            open = end;
        }
    };

    zero_y();
    // First quad of this wave: Q0, or the next one if Q0 is skipped.
    Cur cu{Q0, Q0 / NQ, Q0 % NQ};
    if (skips_last && cu.qi == NQ - 1 && NQ > 1) advance(cu);
    close_until(nsteps > 0 ? cu.q : Q1);
    if (nsteps > 0) {
        // Requests run DEPTH - 1 units ahead of the computation; past this
        // wave's last unit they repeat it, so that every step makes the same
        // requests.  Units land in registers: the compiler's own count of
        // outstanding loads places each wait just before a slot is used.
        Cur iu = cu;
        int issued = 0;
        auto issue_next = [&](Slot &sl) __attribute__((always_inline)) {
            issue(iu, sl);
            if (++issued < nsteps) advance(iu);
        };
#pragma unroll
        for (int s = 0; s < DEPTH - 1; ++s) issue_next(ring[s]);
        // one step: request DEPTH - 1 ahead, compute this unit, close the
        // pieces that end before the next one
        auto step = [&](int slot, int nslot) __attribute__((always_inline)) {
            issue_next(ring[nslot]);
            compute(cu, ring[slot]);
            Cur nu = cu;
            advance(nu);
            close_until(nu.q);
            cu = nu;
        };
        // unrolled by DEPTH so that every ring slot is a constant in each step
        int i = 0;
        for (; i + DEPTH <= nsteps; i += DEPTH) {
#pragma unroll
            for (int s = 0; s < DEPTH; ++s) step(s, (s + DEPTH - 1) % DEPTH);
        }
#pragma unroll
        for (int s = 0; s < DEPTH - 1; ++s)
            if (i + s < nsteps) step(s, (s + DEPTH - 1) % DEPTH);
    }
    close_until(Q1);
    wait_vm_all();                      // the unused requests past the last unit have landed

    if constexpr (ARGMAX) {
        // row maxima: over the wave's columns, the workgroup's waves, then the grid
        __syncthreads();                // the last in-workgroup sum has been read
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                unsigned long long b = wbest[mt][r4];
#pragma unroll
                for (int off = 1; off < 16; off <<= 1) b = umax64(b, __shfl_xor(b, off));
                if (c == 0) red[w][16 * mt + 4 * j + r4] = b;
            }
        __syncthreads();
        // The grid's row maxima accumulate in one key per row with 64-bit
        // atomic max (exact and order-free, so deterministic); the last
        // workgroup reads them, writes the ids and clears the keys.
        if (tid < M) {
            unsigned long long b = red[0][tid];
#pragma unroll
            for (int qq = 1; qq < kWavesPerWG; ++qq) b = umax64(b, red[qq][tid]);
            __hip_atomic_fetch_max(&KL->keys[tid], b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        wait_vm_all();
        __syncthreads();
        if (tid == 0)
            s_flag = __hip_atomic_fetch_add(KL->done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                     gridDim.x - 1;
        __syncthreads();
        if (!s_flag) return;
        if (tid < M) {
            const unsigned long long b = __hip_atomic_load(&KL->keys[tid], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const int32_t id = (int32_t)(0xffffffffu - (uint32_t)(b & 0xffffffffull));
            KL->argmax[tid] = id;
            __hip_atomic_store(&KL->keys[tid], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            red[0][tid] = (unsigned long long)(uint32_t)id;
        }
        if (KL->accept_len != nullptr) {
            // Greedy acceptance of each request's drafts against these ids
            // (the same rule as accept_greedy_kernel): drafts are accepted
            // while they equal the target's token of the same row, then the
            // target's token of the first mismatching row (or of the last
            // row) is committed.
            __syncthreads();
            const int R = KL->acc_rows;
            for (int r = tid; r < KL->acc_b; r += 256) {
                const int32_t *dr = KL->draft + (int64_t)r * (R - 1);
                int32_t *cr = KL->committed + (int64_t)r * R;
                auto t_of = [&](int j) { return (int32_t)(uint32_t)red[0][r * R + j]; };
                int a = 0;
                while (a < R - 1 && dr[a] == t_of(a)) {
                    cr[a] = dr[a];
                    ++a;
                }
                cr[a] = t_of(a);
                for (int i = a + 1; i < R; ++i) cr[i] = -1;
                KL->accept_len[r] = a + 1;
            }
        }
        if (tid == 0) __hip_atomic_store(KL->done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

template <int BITS, bool ARGMAX>
hipError_t launch_cfg(const GemmLaunch &L, int grid, hipStream_t s) {
    if (L.m <= 16)
        hipLaunchKernelGGL((qgemm_kernel<BITS, 1, ARGMAX>), dim3(grid), dim3(256), 0, s, L);
    else
        hipLaunchKernelGGL((qgemm_kernel<BITS, 2, ARGMAX>), dim3(grid), dim3(256), 0, s, L);
    return hipGetLastError();
}

template <bool ARGMAX>
hipError_t launch_any(const GemmLaunch &L, int bits, int grid, hipStream_t s) {
    switch (bits) {
        case 2: return launch_cfg<2, ARGMAX>(L, grid, s);
        case 3: return launch_cfg<3, ARGMAX>(L, grid, s);
        case 4: return launch_cfg<4, ARGMAX>(L, grid, s);
        case 8: return launch_cfg<8, ARGMAX>(L, grid, s);
        case 16: return launch_cfg<16, ARGMAX>(L, grid, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_qgemm(const GemmLaunch &L, int bits, int grid, hipStream_t s) {
    return launch_any<false>(L, bits, grid, s);
}

hipError_t launch_lmhead(const GemmLaunch &L, int bits, int grid, hipStream_t s) {
    return launch_any<true>(L, bits, grid, s);
}

}  // namespace dspk

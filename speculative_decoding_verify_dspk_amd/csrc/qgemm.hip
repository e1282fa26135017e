// Verify-pass projections through affine group-quantised weights, and the
// vocabulary head fused with the row argmax, for gfx950 (MI355X).
//
// What is computed: y[i][c] = sum_r x[i][r] * (s[c][r/64] * q[c][r] + b[c][r/64])
// for the M = anchor + drafts rows i ("mlx-dspark" wiki summary, sections
// "Architecture" and "Key techniques": one target pass over all rows, each
// weight group dequantised once and reused for every row).
//
// How (MI355X-first, not the pages' Metal kernel):
// * The weights are the only large stream.  They move HBM -> LDS with
//   direct-to-LDS loads (global_load_lds_dwordx4, non-temporal), whole 16-byte
//   chunks of 64 weight rows per instruction, into a double-buffered stage per
//   wave, XOR-swizzled so the MFMA-order reads (ds_read_b128) are free of bank
//   conflicts.  The per-group fp16 scale/bias pairs ride the same path
//   (4- or 2-byte direct loads).  The stage's activation fragments
//   (L2-resident) come into registers alongside.  Each wave requests its next
//   stage before it waits for the current one, so two stages are in flight
//   while it waits and one while it computes.
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
// * Work unit = a "quad": one 64-column block times four consecutive K stages,
//   one stage per wave of a four-wave workgroup, so the workgroup reads four
//   adjacent chunks of the same 64 rows at once.  One persistent workgroup per
//   CU takes an equal contiguous range of the quads of the whole launch
//   (stream-K over workgroups), so small and large weights alike keep every CU
//   streaming.  At the end of each block piece the four waves add their
//   partial sums through LDS (fixed order), each wave keeping one 16-column
//   tile; a block split between workgroups is completed by the last of them to
//   arrive, which adds the pieces in workgroup order.  Results do not depend
//   on scheduling.  Pieces and arrival counters move through device-scope
//   atomic accesses, so no cache flush is needed.
#include "dspk_internal.h"

namespace dspk {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int NT = kTilesPerWave;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ float h2f(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// high halves of two floats holding small integers -> one dword of two bf16 (exact)
__device__ __forceinline__ uint32_t pack_hi16(float lo, float hi) {
    return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// eight 8-bit codes (two dwords, LSB first) -> eight exact bf16 values, same order
__device__ __forceinline__ bf16x8 codes8_to_bf16(uint32_t w0, uint32_t w1) {
    u32x4 r;
    r[0] = pack_hi16((float)(w0 & 0xffu), (float)((w0 >> 8) & 0xffu));
    r[1] = pack_hi16((float)((w0 >> 16) & 0xffu), (float)(w0 >> 24));
    r[2] = pack_hi16((float)(w1 & 0xffu), (float)((w1 >> 8) & 0xffu));
    r[3] = pack_hi16((float)((w1 >> 16) & 0xffu), (float)(w1 >> 24));
    return as_bf16x8(r);
}

// eight 4-bit codes (one dword) -> bf16 values 128 + q in the order
// q0,q4,q1,q5,q2,q6,q3,q7 (0x4300 is bf16 128.0; q fills the low mantissa bits)
__device__ __forceinline__ bf16x8 codes4_to_bf16(uint32_t w) {
    u32x4 r;
    r[0] = (w & 0x000F000Fu) | 0x43004300u;
    r[1] = ((w >> 4) & 0x000F000Fu) | 0x43004300u;
    r[2] = ((w >> 8) & 0x000F000Fu) | 0x43004300u;
    r[3] = ((w >> 12) & 0x000F000Fu) | 0x43004300u;
    return as_bf16x8(r);
}

// eight bf16 activations reordered to match codes4_to_bf16
__device__ __forceinline__ u32x4 perm_x_for4(u32x4 x) {
    u32x4 r;
    r[0] = __builtin_amdgcn_perm(x[2], x[0], 0x05040100u);
    r[1] = __builtin_amdgcn_perm(x[2], x[0], 0x07060302u);
    r[2] = __builtin_amdgcn_perm(x[3], x[1], 0x05040100u);
    r[3] = __builtin_amdgcn_perm(x[3], x[1], 0x07060302u);
    return r;
}

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint16_t f2bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

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

// Stage geometry.  A stage is one wave's share of a quad: 64 weight rows times
// KS = 128 K elements (64 for bf16 weights), SB bytes per row; GS = 64-wide K
// groups per stage.  The stage's scale and bias halves (group-major arrays,
// so the 64 columns of one group are 128 contiguous bytes) come with 2-byte
// direct loads, one per group and array, each landing in a 4-byte LDS slot.
//
// OCC workgroups share a CU.  DEPTH = stages of a wave's LDS ring: a wave
// requests stage i + DEPTH - 1 before it waits for stage i, so DEPTH stages
// are in flight while it waits and DEPTH - 1 while it computes.
#ifndef DSPK_OCC
#define DSPK_OCC 1
#endif
#ifndef DSPK_DEPTH
#define DSPK_DEPTH 4
#endif
constexpr int OCC = DSPK_OCC;
constexpr int DEPTH = DSPK_DEPTH;
// 16-column tiles posted per pass of the in-workgroup sum
constexpr int CTILES = OCC == 1 ? kTilesPerWave : kTilesPerWave / 2;

template <int BITS>
struct Cfg {
    static constexpr int KS = BITS == 16 ? 64 : 128;            // K per stage
    static constexpr int SB = KS * BITS / 8;                    // bytes of a weight row per stage
    static constexpr int GS = KS / 64;                          // groups per stage
    static constexpr int LPR = SB / 16;                         // 16-byte chunks per weight row
    static constexpr int RPI = 1024 / SB;                       // weight rows per load instruction
    static constexpr int NDMA = 64 / RPI;                       // weight load instructions per stage
    static constexpr int B_BYTES = kBlockCols * SB;             // one wave's weights per stage
    static constexpr int SB_LOADS = BITS == 16 ? 0 : GS;        // loads per array (scales, biases)
    static constexpr int SBP_BYTES = 2 * SB_LOADS * 256;        // [scales g][biases g] x 64 lanes x 4 bytes
    static constexpr int WAVE_STAGE = B_BYTES + SBP_BYTES;
    static constexpr int RING = DEPTH * kWavesPerWG * WAVE_STAGE;
    static_assert(RING + kWavesPerWG * CTILES * kWave * 16 <= 163840 / OCC, "LDS budget per workgroup");
};

template <int LPR>
__device__ __forceinline__ int swz(int row) {                 // chunk XOR key of a weight row
    return (row / (16 / LPR)) & (LPR - 1);
}

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void dma16(const void *g, lds_void *l) {
    __builtin_amdgcn_global_load_lds(g, l, 16, 0, 2 /* non-temporal */);
}
__device__ __forceinline__ void dma4(const void *g, lds_void *l) {
    __builtin_amdgcn_global_load_lds(g, l, 4, 0, 0);
}
__device__ __forceinline__ void dma2(const void *g, lds_void *l) {
    __builtin_amdgcn_global_load_lds(g, l, 2, 0, 0);
}

// Wait until at most N of this wave's vector memory operations are pending
// (they retire in issue order).  The builtin keeps the compiler's own count
// of outstanding loads in step (so it adds no waits of its own for data that
// this wait already covers); the empty asm keeps every memory access on its
// side of the wait.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
    asm volatile("" ::: "memory");
}
__device__ __forceinline__ void wait_vm_all() { wait_vm<0>(); }

// Workgroup barrier for LDS traffic only: it does not wait for this wave's
// outstanding global loads (the next stage stays in flight across it).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// LDS accesses through restrict-qualified parameters: once inlined they carry
// alias-scope information, which tells the compiler that they do not touch
// the stage buffers that direct-to-LDS loads are filling (it would otherwise
// wait for those loads).  The stage a wave reads has always landed already:
// the explicit wait_vm before every compute guarantees it.
__device__ __forceinline__ f32x4 lds_get(const f32x4 *__restrict__ p) { return *p; }
__device__ __forceinline__ void lds_put(f32x4 *__restrict__ p, f32x4 v) { *p = v; }

// The scale/bias dwords of one stage for this lane's four columns, read with
// one asm block that also waits for them.  Plain reads would be merged into
// ds_read2 instructions, which drop the alias-scope information and make the
// compiler wait for every load in flight; hidden from it, they need no such
// wait (the stage has landed already), only the LDS wait inside the block.
// lds = LDS byte address of this lane's first column; dword k of the result
// is the word at lds + 256 * (k / 4) + 64 * (k % 4).
__device__ __forceinline__ void lds_read_8x(uint32_t lds, uint32_t (&v)[8]) {
    asm volatile(
        "ds_read_b32 %0, %8\n\t"
        "ds_read_b32 %1, %8 offset:64\n\t"
        "ds_read_b32 %2, %8 offset:128\n\t"
        "ds_read_b32 %3, %8 offset:192\n\t"
        "ds_read_b32 %4, %8 offset:256\n\t"
        "ds_read_b32 %5, %8 offset:320\n\t"
        "ds_read_b32 %6, %8 offset:384\n\t"
        "ds_read_b32 %7, %8 offset:448\n\t"
        "s_waitcnt lgkmcnt(0)"
        // early-clobber outputs: none may share the address register
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]),
          "=&v"(v[7])
        : "v"(lds)
        : "memory");
}

// The weight fragments of one stage for this lane, read with one asm block
// that also waits for them (same reason as lds_read_8x: the compiler would
// otherwise wait for the direct-to-LDS loads in flight).  For two lane
// addresses a0, a1 and the four 16-column tiles t: v[h][t] = LDS[a_h + S*t].
template <int S>
__device__ __forceinline__ void lds_read_b128_2x4(uint32_t a0, uint32_t a1, u32x4 (&v)[2][4]) {
    asm volatile(
        "ds_read_b128 %0, %8\n\t"
        "ds_read_b128 %1, %8 offset:%10\n\t"
        "ds_read_b128 %2, %8 offset:%11\n\t"
        "ds_read_b128 %3, %8 offset:%12\n\t"
        "ds_read_b128 %4, %9\n\t"
        "ds_read_b128 %5, %9 offset:%10\n\t"
        "ds_read_b128 %6, %9 offset:%11\n\t"
        "ds_read_b128 %7, %9 offset:%12\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0][0]), "=&v"(v[0][1]), "=&v"(v[0][2]), "=&v"(v[0][3]), "=&v"(v[1][0]), "=&v"(v[1][1]),
          "=&v"(v[1][2]), "=&v"(v[1][3])
        : "v"(a0), "v"(a1), "n"(S), "n"(2 * S), "n"(3 * S)
        : "memory");
}
template <int S>
__device__ __forceinline__ void lds_read_b64_2x4(uint32_t a0, uint32_t a1, u32x2 (&v)[2][4]) {
    asm volatile(
        "ds_read_b64 %0, %8\n\t"
        "ds_read_b64 %1, %8 offset:%10\n\t"
        "ds_read_b64 %2, %8 offset:%11\n\t"
        "ds_read_b64 %3, %8 offset:%12\n\t"
        "ds_read_b64 %4, %9\n\t"
        "ds_read_b64 %5, %9 offset:%10\n\t"
        "ds_read_b64 %6, %9 offset:%11\n\t"
        "ds_read_b64 %7, %9 offset:%12\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0][0]), "=&v"(v[0][1]), "=&v"(v[0][2]), "=&v"(v[0][3]), "=&v"(v[1][0]), "=&v"(v[1][1]),
          "=&v"(v[1][2]), "=&v"(v[1][3])
        : "v"(a0), "v"(a1), "n"(S), "n"(2 * S), "n"(3 * S)
        : "memory");
}

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

__device__ __forceinline__ void store_agent(float *p, float v) {
    __hip_atomic_store((uint32_t *)p, __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_agent(const float *p) {
    return __uint_as_float(__hip_atomic_load((uint32_t *)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
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

__device__ __forceinline__ unsigned long long umax64(unsigned long long a, unsigned long long b) {
    return a > b ? a : b;
}

template <int BITS, int MT, bool ARGMAX>
__global__ __launch_bounds__(256, OCC) void qgemm_kernel(const GemmLaunch L) {
    using C = Cfg<BITS>;
    constexpr int SB = C::SB;
    // ring of DEPTH stage buffers per wave: [slot][wave][weights | scales | biases]
    __shared__ __attribute__((aligned(16))) unsigned char ring[C::RING];
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
    const int bid = blockIdx.x;
    const int GRID = gridDim.x;
    const int QU = KL->quads;                 // quads of the launch
    const int NQ = KL->nq;                    // quads per block
    const int NST = KL->nst;                  // stages per block
    const int LASTW = NST - 4 * (NQ - 1);     // waves with a stage in a block's last quad (1..4)
    const int K = KL->k;
    const int G = K >> 6;
    const int64_t rowbytes = (int64_t)K * BITS / 8;
    const int Q0 = quad_begin(QU, GRID, bid), Q1 = quad_begin(QU, GRID, bid + 1);
    const int M = KL->m;
    unsigned char *const myring = ring + w * C::WAVE_STAGE;   // + slot * (4 * WAVE_STAGE)

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
    // has no stage in it; when NQ == 1 that holds for all of them, and the
    // wave has no stage at all.
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

    u32x4 act[DEPTH][C::GS][MT][2];       // one set per ring slot

    // Request state, refreshed when the requests move to a new block: the
    // weight's base pointers and each lane's 32-bit byte offsets of its rows
    // (rows past n repeat the last one); a weight holds < 4 GiB of codes.
    int ib_gb = -1;
    const unsigned char *ib_codes = nullptr;
    const uint16_t *ib_scales = nullptr, *ib_biases = nullptr;
    int ib_n = 1;
    uint32_t ib_row[C::NDMA];
    int ib_col = 0;             // this lane's column for the scale/bias loads
    uint32_t ch16[C::NDMA];     // 16 * (swizzled chunk) of each weight load of this lane
#pragma unroll
    for (int i = 0; i < C::NDMA; ++i) {
        const int r = i * C::RPI + lane / C::LPR;
        ch16[i] = 16u * (uint32_t)((lane % C::LPR) ^ swz<C::LPR>(r));
    }
    // activations: chunk-major [k/8][ldm][8]; this lane's rows
    const int LDM = (int)KL->ldx;
    int xrowoff[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) xrowoff[mt] = 8 * min(16 * mt + c, M - 1);

    // Request this wave's stage of quad u into ring slot `slot`: 64 weight rows
    // and their scale/bias halves, straight into LDS.  Chunks past the end of
    // K (a short last stage) re-read valid data, so every load is
    // unconditional.
    auto issue = [&](const Cur &u, int slot) __attribute__((always_inline)) {
        if (u.gb != ib_gb) {
            ib_gb = u.gb;
            const int pi = weight_of(u.gb);
            const GemmProblem &P = KL->p[pi];
            const int n0 = (u.gb - P.cg_begin) * kBlockCols;
            ib_codes = (const unsigned char *)P.codes;
            ib_scales = P.scales;
            ib_biases = P.biases;
#pragma unroll
            for (int i = 0; i < C::NDMA; ++i) {
                const int r = i * C::RPI + lane / C::LPR;
                ib_row[i] = (uint32_t)min(n0 + r, P.n - 1) * (uint32_t)rowbytes;
            }
            ib_col = min(n0 + lane, P.n - 1);
            ib_n = P.n;
        }
        const int st = 4 * u.qi + w;
        unsigned char *Bw = myring + slot * (kWavesPerWG * C::WAVE_STAGE);
        const uint32_t kb = (uint32_t)st * SB;
        // chunks past the row end (a short last stage) re-read its last 16 bytes
#pragma unroll
        for (int i = 0; i < C::NDMA; ++i) {
            const uint32_t off = min(kb + ch16[i], (uint32_t)rowbytes - 16u);
            dma16(ib_codes + (ib_row[i] + off), (lds_void *)(Bw + i * 1024));
        }
        if constexpr (BITS != 16) {
            const int g0 = st * C::GS;
            unsigned char *S = Bw + C::B_BYTES;
#pragma unroll
            for (int g = 0; g < C::GS; ++g) {
                const int64_t o = (int64_t)min(g0 + g, G - 1) * ib_n + ib_col;
                dma2(ib_scales + o, (lds_void *)(S + 256 * g));
                dma2(ib_biases + o, (lds_void *)(S + 256 * (C::GS + g)));
            }
        }
    };
    // The activations of this wave's stage of quad u (L2-resident), requested
    // with its weights: lane (c, j) takes row 16*mt + c, K offsets
    // 64*g + 16*j (+8).
    auto load_act = [&](const Cur &u, u32x4 (&a)[C::GS][MT][2]) __attribute__((always_inline)) {
        const int st = 4 * u.qi + w;
        const int last = K / 8 - 1;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
            for (int g = 0; g < C::GS; ++g) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int chunk = min(st * (C::KS / 8) + 8 * g + 2 * j + h, last);
                    a[g][mt][h] = *(const u32x4 *)(KL->x + ((uint32_t)chunk * (uint32_t)LDM * 8u + xrowoff[mt]));
                }
            }
        }
    };
    // vector memory instructions of one issue()
    constexpr int ISSUE_OPS = C::NDMA + 2 * C::SB_LOADS + 2 * MT * C::GS;
    constexpr int AHEAD_OPS = (DEPTH - 1) * ISSUE_OPS;
    static_assert(AHEAD_OPS < 64, "the stages in flight must fit the vmcnt range");

    f32x4 y[NT][MT];
    auto zero_y = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) y[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    };

    // MFMA work of this wave's stage of quad u, from ring slot `slot`
    auto compute = [&](const Cur &u, const unsigned char *__restrict__ Bw, const u32x4 (&act)[C::GS][MT][2])
        __attribute__((always_inline)) {
        const int st = 4 * u.qi + w;
        const int ng = min(C::GS, G - st * C::GS);
        // scale/bias words of columns 16*t + c: [load][t], scales first
        uint32_t sbw[BITS == 16 ? 1 : 2 * C::SB_LOADS][NT];
        if constexpr (BITS != 16) {
            const uint32_t base = (uint32_t)(uintptr_t)(lds_void *)(Bw + C::B_BYTES) + 4 * c;
#pragma unroll
            for (int h = 0; h < C::SB_LOADS; ++h) {
                uint32_t v[8];
                lds_read_8x(base + 512 * h, v);     // loads 2h and 2h+1 of the region
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    sbw[2 * h][t] = v[t];
                    sbw[2 * h + 1][t] = v[4 + t];
                }
            }
        }
        // this lane's weight fragments of the stage: [g or chunk][t]; a tile's
        // rows are 16 * SB bytes apart and the chunk swizzle of rows 16*t + c
        // does not depend on t
        const uint32_t lbase = (uint32_t)(uintptr_t)(lds_void *)Bw + (uint32_t)c * SB;
        u32x4 wq[2][4];
        u32x2 wq4[2][4];
        if constexpr (BITS == 8) {
            const int sw = swz<C::LPR>(c);
            lds_read_b128_2x4<16 * SB>(lbase + 16 * ((4 * 0 + j) ^ sw), lbase + 16 * ((4 * 1 + j) ^ sw), wq);
        } else if constexpr (BITS == 16) {
            const int sw = swz<C::LPR>(c);
            lds_read_b128_2x4<16 * SB>(lbase + 16 * ((2 * j) ^ sw), lbase + 16 * ((2 * j + 1) ^ sw), wq);
        } else {
            const int sw = swz<C::LPR>(c);
            lds_read_b64_2x4<16 * SB>(lbase + 16 * ((0 + (j >> 1)) ^ sw) + 8 * (j & 1),
                                      lbase + 16 * ((2 + (j >> 1)) ^ sw) + 8 * (j & 1), wq4);
        }
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        const bf16x8 ones = as_bf16x8(u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});
#pragma unroll
        for (int g = 0; g < C::GS; ++g) {
            if (g >= ng) break;
            bf16x8 a0[MT], a1[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                if constexpr (BITS == 4) {
                    a0[mt] = as_bf16x8(perm_x_for4(act[g][mt][0]));
                    a1[mt] = as_bf16x8(perm_x_for4(act[g][mt][1]));
                } else {
                    a0[mt] = as_bf16x8(act[g][mt][0]);
                    a1[mt] = as_bf16x8(act[g][mt][1]);
                }
            }
            if constexpr (BITS == 16) {
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const bf16x8 b0 = as_bf16x8(wq[0][t]);
                    const bf16x8 b1 = as_bf16x8(wq[1][t]);
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
                        const u32x4 qv = wq[g][t];
                        b0 = codes8_to_bf16(qv[0], qv[1]);
                        b1 = codes8_to_bf16(qv[2], qv[3]);
                    } else {
                        const u32x2 qv = wq4[g][t];
                        b0 = codes4_to_bf16(qv[0]);
                        b1 = codes4_to_bf16(qv[1]);
                    }
                    const uint32_t sh = sbw[g][t] & 0xffffu;
                    const uint32_t bh = sbw[C::GS + g][t] & 0xffffu;
                    const float sc = h2f(sh);
                    float bi = h2f(bh);
                    if constexpr (BITS == 4) bi = fmaf(-128.f, sc, bi);   // codes carry +128
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) {
                        f32x4 acc = mfma(a0[mt], b0, zero);
                        acc = mfma(a1[mt], b1, acc);
#pragma unroll
                        for (int r4 = 0; r4 < 4; ++r4)
                            y[t][mt][r4] = fmaf(sc, acc[r4], fmaf(bi, xs[mt][r4], y[t][mt][r4]));
                    }
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
    auto finish_tile = [&](int pi, int cb, const f32x4 (&z)[MT]) __attribute__((always_inline)) {
        const GemmProblem &P = KL->p[pi];
        const int n = cb * kBlockCols + 16 * w + c;
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
    auto close_piece = [&](int a, int b) __attribute__((always_inline)) {
        const int gb = a / NQ;
        const int pi = weight_of(gb);
        const int cb = gb - KL->p[pi].cg_begin;
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
        if (a == bq0 && b == bq1) {
            finish_tile(pi, cb, z);
            return;
        }
        // publish: slot 0 for the workgroup's first piece, 1 for its last
        const int side = a == Q0 ? 0 : 1;
        float *mine = KL->partial + (((int64_t)bid * 2 + side) * kWavesPerWG + w) * (MT * kWave * 4);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) store_agent(mine + (mt * kWave + lane) * 4 + r4, z[mt][r4]);
        wait_vm_all();
        const int wf = quad_owner(QU, GRID, bq0), wl = quad_owner(QU, GRID, bq1 - 1);
        uint32_t ticket = 0;
        uint32_t *ctr = KL->counters + (int64_t)gb * kWavesPerWG + w;
        if (lane == 0) ticket = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ticket = __shfl(ticket, 0);
        if (ticket != (uint32_t)(wl - wf)) return;
        // Last arrival: the pieces in workgroup order, eight requests in
        // flight.  Every workgroup after wf starts inside the block (its piece
        // is its first, slot 0); wf's piece is its first only if its range
        // starts at the block start.
        const int wf_side = quad_begin(QU, GRID, wf) >= bq0 ? 0 : 1;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) z[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int v0 = wf; v0 <= wl; v0 += 8) {
            f32x4 part[8][MT];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int v = min(v0 + i, wl);
                const int sl = v == wf ? wf_side : 0;
                const float *src = KL->partial + (((int64_t)v * 2 + sl) * kWavesPerWG + w) * (MT * kWave * 4);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int r4 = 0; r4 < 4; ++r4) part[i][mt][r4] = load_agent(src + (mt * kWave + lane) * 4 + r4);
            }
            // every loaded value is consumed (a duplicate past wl adds zero), so
            // no load of this batch is left pending
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const bool real = v0 + i <= wl;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const f32x4 p = real ? part[i][mt] : f32x4{0.f, 0.f, 0.f, 0.f};
                    z[mt] = (v0 + i == wf) ? p : z[mt] + p;
                }
            }
        }
        if (lane == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        finish_tile(pi, cb, z);
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
        // Requests run DEPTH - 1 stages ahead of the computation; past this
        // wave's last stage they repeat it, so that every step makes the same
        // requests and the waits stay positional.
        // nothing of this wave is in flight here (the compiler's count of
        // outstanding loads starts the loop from the same state every time)
        wait_vm<0>();
        Cur iu = cu;
        int issued = 0;
        auto issue_next = [&](int slot, u32x4 (&a)[C::GS][MT][2]) __attribute__((always_inline)) {
            issue(iu, slot);
            load_act(iu, a);
            if (++issued < nsteps) advance(iu);
        };
#pragma unroll
        for (int s = 0; s < DEPTH - 1; ++s) issue_next(s, act[s]);
        // one stage: request DEPTH - 1 ahead, wait for this one, compute it,
        // close the pieces that end before the next one
        auto step = [&](int slot, int nslot) __attribute__((always_inline)) {
            issue_next(nslot, act[nslot]);
            wait_vm<AHEAD_OPS>();       // everything older than the last DEPTH - 1 requests has landed
            compute(cu, myring + slot * (kWavesPerWG * C::WAVE_STAGE), act[slot]);
            Cur nu = cu;
            advance(nu);
            close_until(nu.q);
            cu = nu;
        };
        // unrolled by DEPTH so that every ring slot and activation set is a
        // constant in each step
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
    wait_vm_all();                      // no load into LDS outlives the workgroup

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
        if (tid < M) {
            unsigned long long b = red[0][tid];
#pragma unroll
            for (int qq = 1; qq < kWavesPerWG; ++qq) b = umax64(b, red[qq][tid]);
            __hip_atomic_store(&KL->keys[(int64_t)bid * kMaxRows + tid], b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        wait_vm_all();
        __syncthreads();
        if (tid == 0)
            s_flag = __hip_atomic_fetch_add(KL->done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                     gridDim.x - 1;
        __syncthreads();
        if (!s_flag) return;
        // last workgroup: maximum over all workgroups, 8 rows at a time
        const int nwg = gridDim.x;
        for (int m0 = 0; m0 < M; m0 += 8) {
            unsigned long long b8[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) b8[i] = 0ull;
            for (int g = tid; g < nwg; g += 256) {
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    if (m0 + i < M)
                        b8[i] = umax64(b8[i], __hip_atomic_load(&KL->keys[(int64_t)g * kMaxRows + m0 + i],
                                                                __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
            }
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) b8[i] = umax64(b8[i], __shfl_xor(b8[i], off));
            __syncthreads();
            if (lane == 0) {
#pragma unroll
                for (int i = 0; i < 8; ++i) red[w][i] = b8[i];
            }
            __syncthreads();
            if (tid < 8 && m0 + tid < M) {
                unsigned long long b = red[0][tid];
#pragma unroll
                for (int qq = 1; qq < kWavesPerWG; ++qq) b = umax64(b, red[qq][tid]);
                KL->argmax[m0 + tid] = (int32_t)(0xffffffffu - (uint32_t)(b & 0xffffffffull));
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
        case 4: return launch_cfg<4, ARGMAX>(L, grid, s);
        case 8: return launch_cfg<8, ARGMAX>(L, grid, s);
        case 16: return launch_cfg<16, ARGMAX>(L, grid, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

// K elements per stage
int stage_k(int bits) { return bits == 16 ? 64 : 128; }

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

GemmPlan plan_gemm(int count, const int32_t *n, int32_t k, int32_t m, int bits, bool argmax) {
    GemmPlan p{};
    p.nst = (k + stage_k(bits) - 1) / stage_k(bits);
    p.nq = (p.nst + kWavesPerWG - 1) / kWavesPerWG;
    int64_t blocks = 0;
    for (int i = 0; i < count; ++i) blocks += (n[i] + kBlockCols - 1) / kBlockCols;
    p.total_cg = (int32_t)blocks;
    const int64_t quads = blocks * p.nq;
    // OCC workgroups per CU; never more workgroups than quads
    const int64_t slots = (int64_t)OCC * device_cus();
    const int64_t grid = quads < slots ? quads : slots;
    p.grid = grid < 1 ? 1 : (int32_t)grid;
    // the kernel splits quads with 32-bit products and addresses each weight
    // with 32-bit byte offsets
    int64_t nmax = 0;
    for (int i = 0; i < count; ++i) nmax = n[i] > nmax ? n[i] : nmax;
    p.fits = quads * p.grid < ((int64_t)1 << 31) && nmax * ((int64_t)k * bits / 8) < ((int64_t)1 << 32);
    p.quads = p.fits ? (int32_t)quads : 0;
    const int mt = m <= 16 ? 1 : 2;
    size_t off = 256;                                   // [0, 256): argmax arrival counter
    p.off_counters = off;
    off += ((size_t)blocks * kWavesPerWG * 4 + 255) / 256 * 256;
    p.off_keys = off;
    if (argmax) off += (size_t)p.grid * kMaxRows * 8;
    off = (off + 255) / 256 * 256;
    p.off_partial = off;
    off += (size_t)p.grid * 2 * kWavesPerWG * mt * kWave * 16;
    p.ws_bytes = (off + 255) / 256 * 256;
    return p;
}

hipError_t launch_qgemm(const GemmLaunch &L, int bits, int grid, hipStream_t s) {
    return launch_any<false>(L, bits, grid, s);
}

hipError_t launch_lmhead(const GemmLaunch &L, int bits, int grid, hipStream_t s) {
    return launch_any<true>(L, bits, grid, s);
}

}  // namespace dspk

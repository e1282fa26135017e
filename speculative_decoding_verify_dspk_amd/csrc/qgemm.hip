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
//   direct-to-LDS loads (global_load_lds_dwordx4, non-temporal), 256 (or 128)
//   contiguous bytes of a weight row per load instruction -- the access width
//   at which HBM3E delivers its best rate -- into a double-buffered LDS stage,
//   with an XOR swizzle so that the MFMA-order reads (ds_read_b128) are free of
//   bank conflicts.  The stage's activation fragments (L2-resident) and
//   scale/bias pairs come into registers alongside and are first touched
//   after the stage wait, so the only waits are the explicit ones at the
//   stage boundary.
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
// * One persistent workgroup of four independent waves per CU; every wave
//   takes an equal, contiguous share of the (weight, 64-column block, K stage)
//   units of the whole launch (stream-K), so small and large weights alike
//   keep every CU streaming and no wave waits for another in the main loop.
//   A block split between waves is completed by the last of them to arrive,
//   which adds the pieces in wave order: results do not depend on scheduling.
//   Pieces and arrival counters move through device-scope atomic accesses, so
//   no cache flush is needed.
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

// Stage geometry per weight format.  SB = weight bytes of one row per stage
// (256, or 128 for 4-bit codes to keep the activation registers in budget);
// GS = 64-wide K groups per stage.  Each wave owns two LDS stage buffers
// (its 64 weight rows + their fp16 scale/bias pairs); the activations of a
// stage travel through registers.
template <int BITS, int MT>
struct Cfg {
    static constexpr int SB = BITS == 4 ? 128 : 256;
    static constexpr int GS = SB / (8 * BITS);                  // 64 * BITS / 8 bytes per group
    static constexpr int KS = 64 * GS;                          // K per stage
    static constexpr int LPR = SB / 16;                         // 16-byte chunks per weight row
    static constexpr int B_BYTES = kBlockCols * SB;             // one wave's weights per stage
    static constexpr int SBP_BYTES = BITS == 16 ? 0 : kBlockCols * GS * 4;
    static constexpr int WAVE_STAGE = B_BYTES + SBP_BYTES;
    static constexpr int STAGE = kWavesPerWG * WAVE_STAGE;      // one buffer of the workgroup
    static_assert(2 * STAGE <= 155648, "two stages must fit the LDS");
};

__device__ __forceinline__ int swz(int row, int lpr) {      // chunk XOR key of a weight row
    return lpr == 16 ? (row & 15) : ((row >> 1) & 7);
}

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void dma16(const void *g, lds_void *l) {
    __builtin_amdgcn_global_load_lds(g, l, 16, 0, 2 /* non-temporal */);
}

__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ void store_agent(float *p, float v) {
    __hip_atomic_store((uint32_t *)p, __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_agent(const float *p) {
    return __uint_as_float(__hip_atomic_load((uint32_t *)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

__device__ __forceinline__ int unit_begin(int units, int waves, int v) {
    return (int)(((int64_t)units * v) / waves);
}
// wave whose unit range contains unit u
__device__ __forceinline__ int unit_owner(int units, int waves, int u) {
    return (int)((((int64_t)u + 1) * waves + units - 1) / units) - 1;
}

__device__ __forceinline__ unsigned long long umax64(unsigned long long a, unsigned long long b) {
    return a > b ? a : b;
}

// SBV: scale/bias rows are read 8 bytes (4 groups) at a time -- K a multiple
// of 256 and 8-byte aligned arrays; otherwise one 2-byte load per group.
template <int BITS, int MT, bool ARGMAX, bool SBV>
__global__ __launch_bounds__(256, 1) void qgemm_kernel(const GemmLaunch L) {
    using C = Cfg<BITS, MT>;
    // two stage buffers as distinct objects: with the loop unrolled by two the
    // compiler can tell the in-flight loads from the reads (no extra waits)
    __shared__ __attribute__((aligned(16))) unsigned char lds0[C::STAGE];
    __shared__ __attribute__((aligned(16))) unsigned char lds1[C::STAGE];
    __shared__ unsigned long long red[kWavesPerWG][kMaxRows];
    __shared__ int s_flag;

    // Every field is read in place from the kernel-argument segment (scalar
    // loads): the problem table is indexed at run time, and a by-value copy
    // captured by the lambdas below would be spilled to scratch.
    (void)L;
    const GemmLaunch *KL = (const GemmLaunch *)__builtin_amdgcn_kernarg_segment_ptr();
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 15, j = lane >> 4;
    const int bid = blockIdx.x;
    const int NW = gridDim.x * kWavesPerWG;        // waves of the grid
    const int wid = bid * kWavesPerWG + w;         // this wave
    const int U = KL->units;
    const int u0 = unit_begin(U, NW, wid), u1 = unit_begin(U, NW, wid + 1);
    const int M = KL->m;

    // unit -> (weight, block, stage); all wave-uniform
    auto decode = [&](int u, int &pi, int &cb, int &st) __attribute__((always_inline)) {
        pi = 0;
#pragma unroll
        for (int i = 1; i < kMaxGrouped; ++i)
            if (i < KL->count && u >= KL->p[i].u_begin) pi = i;
        const int local = u - KL->p[pi].u_begin;
        cb = local / KL->p[pi].nst;
        st = local - cb * KL->p[pi].nst;
    };

    // scale/bias halves of the next stage (lane = column) and its activation
    // fragments travel through registers; they are used only after the
    // stage wait, so nothing waits on them earlier
    uint32_t s16[C::GS], b16[C::GS];   // 2-byte path: one half each
    u32x2 svec, bvec;                  // 8-byte path (4 groups): raw dwords
    u32x4 actA[C::GS][MT][2], actB[C::GS][MT][2];

    // Request stage u: this wave's 64 weight rows into LDS buffer `base`,
    // the rows' activations into `act`, the scale/bias pairs into s16/b16.
    // Chunks past the end of K (a short last stage) re-read valid data, so
    // every load is unconditional.
    auto issue = [&](int u, unsigned char *base, u32x4 (&act)[C::GS][MT][2]) __attribute__((always_inline)) {
        int pi, cb, st;
        decode(u, pi, cb, st);
        const GemmProblem &P = KL->p[pi];
        const int G = P.k >> 6;
        const int64_t rowbytes = (int64_t)P.k * BITS / 8;
        const int n0 = cb * kBlockCols;
        unsigned char *Bw = base + w * C::WAVE_STAGE;
        // weights: instruction i covers rows i*RPI .. i*RPI+RPI-1
        constexpr int RPI = 1024 / C::SB;
        const int64_t kb = (int64_t)st * C::SB;
#pragma unroll
        for (int i = 0; i < 64 / RPI; ++i) {
            const int r = i * RPI + lane / C::LPR;
            const int n = min(n0 + r, P.n - 1);
            const int chunk = (lane % C::LPR) ^ swz(r, C::LPR);
            const int64_t off = min(kb + 16 * chunk, rowbytes - 16);
            dma16((const unsigned char *)P.codes + (int64_t)n * rowbytes + off, (lds_void *)(Bw + i * 1024));
        }
        // activations: lane (c, j) takes row 16*mt + c, K offsets 64*g + 16*j (+8)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const uint16_t *xr = KL->x + (int64_t)min(16 * mt + c, M - 1) * KL->ldx;
#pragma unroll
            for (int g = 0; g < C::GS; ++g) {
                const int64_t k0 = min((int64_t)st * C::KS + 64 * g + 16 * j, (int64_t)P.k - 16);
                act[g][mt][0] = *(const u32x4 *)(xr + k0);
                act[g][mt][1] = *(const u32x4 *)(xr + k0 + 8);
            }
        }
        // scale/bias pairs of this wave's 64 columns
        if constexpr (BITS != 16) {
            const int n = min(n0 + lane, P.n - 1);
            const int g0 = st * C::GS;
            const int64_t o = (int64_t)n * G + g0;
            if constexpr (SBV && C::GS == 4) {
                svec = *(const u32x2 *)(P.scales + o);   // 8-byte aligned: G % 4 == 0
                bvec = *(const u32x2 *)(P.biases + o);
            } else {
#pragma unroll
                for (int g = 0; g < C::GS; ++g) {
                    const int gg = min(g0 + g, G - 1);
                    s16[g] = P.scales[(int64_t)n * G + gg];
                    b16[g] = P.biases[(int64_t)n * G + gg];
                }
            }
        }
    };

    f32x4 y[NT][MT];
    auto zero_y = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) y[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    };

    // MFMA work of one stage: weights from LDS buffer `base`, activations `act`
    auto compute = [&](int pi, int st, const unsigned char *base, const u32x4 (&act)[C::GS][MT][2])
        __attribute__((always_inline)) {
        const GemmProblem &P = KL->p[pi];
        const int G = P.k >> 6;
        const unsigned char *Bw = base + w * C::WAVE_STAGE;
        const uint32_t *SBw = (const uint32_t *)(Bw + C::B_BYTES);
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
                    const int r = 16 * t + c;
                    const int ch = 8 * g + 2 * j;
                    const unsigned char *row = Bw + r * C::SB;
                    const bf16x8 b0 = as_bf16x8(*(const u32x4 *)(row + 16 * (ch ^ swz(r, C::LPR))));
                    const bf16x8 b1 = as_bf16x8(*(const u32x4 *)(row + 16 * ((ch + 1) ^ swz(r, C::LPR))));
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
                    const int r = 16 * t + c;
                    const unsigned char *row = Bw + r * C::SB;
                    bf16x8 b0, b1;
                    if constexpr (BITS == 8) {
                        const u32x4 q = *(const u32x4 *)(row + 16 * ((4 * g + j) ^ swz(r, C::LPR)));
                        b0 = codes8_to_bf16(q[0], q[1]);
                        b1 = codes8_to_bf16(q[2], q[3]);
                    } else {
                        const int ch = 2 * g + (j >> 1);
                        const u32x2 q = *(const u32x2 *)(row + 16 * (ch ^ swz(r, C::LPR)) + 8 * (j & 1));
                        b0 = codes4_to_bf16(q[0]);
                        b1 = codes4_to_bf16(q[1]);
                    }
                    const uint32_t sv = SBw[g * kBlockCols + r];
                    const float sc = h2f(sv & 0xffffu);
                    float bi = h2f(sv >> 16);
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

    // running row maxima (value, column) of the blocks this wave finished
    unsigned long long wbest[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) wbest[mt][r4] = 0ull;

    // Final values of a whole block: store them, or fold them into the argmax.
    auto finish_block = [&](int pi, int cb) __attribute__((always_inline)) {
        const GemmProblem &P = KL->p[pi];
        const int n0 = cb * kBlockCols;
        const int N = P.n;
        if constexpr (!ARGMAX) {
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int r4 = 0; r4 < 4; ++r4) {
                        const int m = 16 * mt + 4 * j + r4, n = n0 + 16 * t + c;
                        if (m < M && n < N) {
                            if (KL->y_bf16)
                                ((uint16_t *)P.y)[(int64_t)m * P.ldy + n] = f2bf16(y[t][mt][r4]);
                            else
                                ((float *)P.y)[(int64_t)m * P.ldy + n] = y[t][mt][r4];
                        }
                    }
        } else {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int m = 16 * mt + 4 * j + r4;
#pragma unroll
                    for (int t = 0; t < NT; ++t) {
                        const int n = n0 + 16 * t + c;
                        const float v = y[t][mt][r4];
                        if (n < N) {
                            wbest[mt][r4] = umax64(wbest[mt][r4], argmax_key(v, n));
                            if (KL->logits != nullptr && m < M) KL->logits[(int64_t)m * KL->ldl + n] = v;
                        }
                    }
                }
        }
    };

    // End of a piece (this wave's consecutive stages of one block).
    auto finish_piece = [&](int pi, int cb, int piece_u0, int piece_u1) __attribute__((always_inline)) {
        const GemmProblem &P = KL->p[pi];
        const int bu0 = P.u_begin + cb * P.nst, bu1 = bu0 + P.nst;
        if (piece_u0 == bu0 && piece_u1 == bu1) {
            finish_block(pi, cb);
            return;
        }
        // publish this piece: slot 0 if it is the wave's first piece, else slot 1
        const int slot = piece_u0 == u0 ? 0 : 1;
        float *mine = KL->partial + ((int64_t)wid * 2 + slot) * M * kBlockCols;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int m = 16 * mt + 4 * j + r4;
                    if (m < M) store_agent(mine + m * kBlockCols + 16 * t + c, y[t][mt][r4]);
                }
        wait_vm_all();
        const int wf = unit_owner(U, NW, bu0), wl = unit_owner(U, NW, bu1 - 1);
        const int gb = P.cg_begin + cb;
        uint32_t ticket = 0;
        if (lane == 0)
            ticket = __hip_atomic_fetch_add(&KL->counters[gb], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ticket = __shfl(ticket, 0);
        if (ticket != (uint32_t)(wl - wf)) return;
        // last arrival: the pieces in wave order
        for (int v = wf; v <= wl; ++v) {
            const int sl = unit_begin(U, NW, v) >= bu0 ? 0 : 1;
            const float *src = KL->partial + ((int64_t)v * 2 + sl) * M * kBlockCols;
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int r4 = 0; r4 < 4; ++r4) {
                        const int m = 16 * mt + 4 * j + r4;
                        const float x = m < M ? load_agent(src + m * kBlockCols + 16 * t + c) : 0.f;
                        y[t][mt][r4] = v == wf ? x : y[t][mt][r4] + x;
                    }
        }
        if (lane == 0) __hip_atomic_store(&KL->counters[gb], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        finish_block(pi, cb);
    };

    if (u0 < u1) {
        zero_y();
        int piece_u0 = u0;
        // one stage: wait for it, publish its scale/bias pairs, request the next
        // stage into the other buffers, then compute
        auto step = [&](int u, unsigned char *cur, unsigned char *nxt, const u32x4 (&acur)[C::GS][MT][2],
                        u32x4 (&anxt)[C::GS][MT][2]) __attribute__((always_inline)) {
            wait_vm_all();                // this wave's requests for stage u have landed
            if constexpr (BITS != 16) {
                uint32_t *SBw = (uint32_t *)(cur + w * C::WAVE_STAGE + C::B_BYTES);
                if constexpr (SBV && C::GS == 4) {
#pragma unroll
                    for (int g = 0; g < C::GS; ++g)
                        SBw[g * kBlockCols + lane] = __builtin_amdgcn_perm(bvec[g >> 1], svec[g >> 1],
                                                                           (g & 1) ? 0x07060302u : 0x05040100u);
                } else {
#pragma unroll
                    for (int g = 0; g < C::GS; ++g) SBw[g * kBlockCols + lane] = s16[g] | (b16[g] << 16);
                }
            }
            if (u + 1 < u1) issue(u + 1, nxt, anxt);
            int pi, cb, st;
            decode(u, pi, cb, st);
            compute(pi, st, cur, acur);
            if (u + 1 == u1 || st + 1 == KL->p[pi].nst) {
                finish_piece(pi, cb, piece_u0, u + 1);
                zero_y();
                piece_u0 = u + 1;
            }
        };
        issue(u0, lds0, actA);
        for (int u = u0; u < u1; u += 2) {
            step(u, lds0, lds1, actA, actB);
            if (u + 1 < u1) step(u + 1, lds1, lds0, actB, actA);
        }
    }

    if constexpr (ARGMAX) {
        // row maxima: over the wave's columns, the workgroup's waves, then the grid
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
            for (int q = 1; q < kWavesPerWG; ++q) b = umax64(b, red[q][tid]);
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
                for (int q = 1; q < kWavesPerWG; ++q) b = umax64(b, red[q][tid]);
                KL->argmax[m0 + tid] = (int32_t)(0xffffffffu - (uint32_t)(b & 0xffffffffull));
            }
        }
        if (tid == 0) __hip_atomic_store(KL->done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

template <int BITS, bool ARGMAX>
hipError_t launch_bits(const GemmLaunch &L, int grid, hipStream_t s) {
    // 8-byte scale/bias loads: 4 groups per stage, K % 256 == 0, aligned arrays
    bool sbv = BITS != 16 && Cfg<BITS, 1>::GS == 4 && (L.p[0].k % 256) == 0;
    for (int i = 0; i < L.count; ++i)
        sbv = sbv && ((((uintptr_t)L.p[i].scales | (uintptr_t)L.p[i].biases) & 7) == 0);
    if (L.m <= 16) {
        if (sbv)
            hipLaunchKernelGGL((qgemm_kernel<BITS, 1, ARGMAX, true>), dim3(grid), dim3(256), 0, s, L);
        else
            hipLaunchKernelGGL((qgemm_kernel<BITS, 1, ARGMAX, false>), dim3(grid), dim3(256), 0, s, L);
    } else {
        if (sbv)
            hipLaunchKernelGGL((qgemm_kernel<BITS, 2, ARGMAX, true>), dim3(grid), dim3(256), 0, s, L);
        else
            hipLaunchKernelGGL((qgemm_kernel<BITS, 2, ARGMAX, false>), dim3(grid), dim3(256), 0, s, L);
    }
    return hipGetLastError();
}

template <bool ARGMAX>
hipError_t launch_any(const GemmLaunch &L, int bits, int grid, hipStream_t s) {
    switch (bits) {
        case 4: return launch_bits<4, ARGMAX>(L, grid, s);
        case 8: return launch_bits<8, ARGMAX>(L, grid, s);
        case 16: return launch_bits<16, ARGMAX>(L, grid, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

int stage_groups(int bits, int m) {
    const int mt = m <= 16 ? 1 : 2;
    if (bits == 8) return mt == 1 ? Cfg<8, 1>::GS : Cfg<8, 2>::GS;
    if (bits == 4) return mt == 1 ? Cfg<4, 1>::GS : Cfg<4, 2>::GS;
    return mt == 1 ? Cfg<16, 1>::GS : Cfg<16, 2>::GS;
}

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

// One workgroup of four waves per CU; small launches use fewer workgroups so
// that each wave streams at least kMinWaveUnits stages (fewer split blocks).
constexpr int kMinWaveUnits = 2;

GemmPlan plan_gemm(int count, const int32_t *n, int32_t k, int32_t m, int bits, bool argmax) {
    GemmPlan p{};
    const int G = k / 64;
    const int gs = stage_groups(bits, m);
    const int nst = (G + gs - 1) / gs;
    int units = 0, blocks = 0;
    for (int i = 0; i < count; ++i) {
        const int nb = (n[i] + kBlockCols - 1) / kBlockCols;
        units += nb * nst;
        blocks += nb;
    }
    p.units = units;
    p.total_cg = blocks;
    const int want = (units + kWavesPerWG * kMinWaveUnits - 1) / (kWavesPerWG * kMinWaveUnits);
    p.grid = want < device_cus() ? want : device_cus();
    if (p.grid < 1) p.grid = 1;
    size_t off = 256;                                   // [0, 256): argmax arrival counter
    p.off_counters = off;
    off += ((size_t)blocks * 4 + 255) / 256 * 256;
    p.off_keys = off;
    if (argmax) off += (size_t)p.grid * kMaxRows * 8;
    off = (off + 255) / 256 * 256;
    p.off_partial = off;
    off += (size_t)p.grid * kWavesPerWG * 2 * m * kBlockCols * 4;
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

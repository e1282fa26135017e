// Prefill projections: y[i][c] = sum_r x[i][r] * (s[c][r/64] * q[c][r] + b[c][r/64])
// for many rows at once (a prompt's tokens), through the same tiled weights
// the verify kernels stream ("mlx-dspark" wiki summary, "Key techniques":
// each weight group is dequantised once and reused for every row of the
// pass; prefill is the wide-row case of that pass).
//
// With hundreds of rows the work is bound by the matrix cores and the vector
// ALUs, not by HBM, so this kernel is tiled for MFMA reuse rather than for
// streaming:
// * A workgroup computes a 128-row (or 64-row) x 128-column block of y: four
//   waves, each 64 (32) rows -- four (two) 16-row tiles -- x one 64-column
//   weight block (four 16-column tiles), K walked in stages of 128 (a whole
//   8-bit unit, half of a 2/3/4-bit unit, one bf16 unit of 64).  The 64-row
//   block is taken where the 128-row blocks would leave CUs idle or
//   unevenly loaded (few or skinny column blocks); both walk K in the same
//   order, so their results are identical.
// * Activations reach LDS by direct global-to-LDS loads (no staging
//   registers), double-buffered: the next stage is in flight while the
//   current one is computed.  Each wave loads its weight codes straight from
//   the tiled layout into registers, where every lane already holds its own
//   operand bytes, one unit ahead into a second register set.
// * Codes are exact in bf16, so per group and per 16x16 tile
//     sum_{r in group} x*w = s * sum x*q + b * sum x
//   comes from exact-product MFMAs on the codes (fp32 accumulation) plus a
//   per-group scale/bias update, as in the verify kernels; the row sums of x
//   come from an MFMA against a ones operand.  No dequantised weight is
//   rounded.  Each activation operand read from LDS serves the four column
//   tiles, each decoded weight operand the four row tiles.
// * Two workgroups per CU (64 KiB of LDS each, 32 KiB for bf16).  Row blocks
//   vary fastest in the grid, so the workgroups that run together share their
//   weight units in L2.
// * With a caller's workspace, a launch with fewer output blocks than the
//   CUs hold at once splits K into ks contiguous unit ranges (grid z): each
//   workgroup publishes its partial block, counts itself in per wave, and the
//   last of a block's ks arrivals adds the partials in split order and
//   stores y, so the result does not depend on which arrives last.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "decode.h"
#include "dspk_internal.h"
#include "prefill_plan.h"

namespace dspk {
namespace {

using namespace dec;

constexpr int PT = 256;                  // threads per workgroup

// One stage of K: SK = min(KU, 128) (a whole unit, or half of a 256-K
// unit) for the workgroup's PBM = 32 RT rows (RT 16-row tiles per wave),
// unpadded (a row is SK bf16 = CH 16-byte chunks), filled by direct
// global-to-LDS loads.  Such a load writes
// 16 bytes per lane at consecutive LDS addresses, so bank spreading cannot
// come from padding: chunk ch of row R sits at position ch ^ (R & SWM) of
// its row instead, and the load of that position fetches that chunk.  The 16
// rows that one MFMA operand read touches (same chunk, rows R..R+15 with R a
// multiple of 16) then fall on distinct positions.
template <int BITS>
struct SCfg {
    static constexpr int KU = Cfg<BITS>::KU;
    static constexpr int SK = KU < 128 ? KU : 128;          // K per stage
    static constexpr int HALVES = KU / SK;                  // stages per unit
    static constexpr int GH = SK / 64;                      // groups per stage
    static constexpr int NSB = BITS == 16 ? 1 : GH;         // scale/bias loads per lane and stage
    static constexpr int CH = SK / 8;                       // 16-byte chunks per row
    static constexpr int SWM = CH >= 16 ? 15 : CH - 1;      // position swizzle mask
    static constexpr int RPI = 64 / CH;                     // rows per 1 KiB load
    static_assert(HALVES * GH == Cfg<BITS>::GS, "stages must tile the unit's groups");
};
// The row-dependent sizes of a stage with RT 16-row tiles per wave.
template <int BITS, int RT>
struct RCfg {
    static constexpr int PBM = 32 * RT;                     // rows per workgroup
    static constexpr int STAGE = PBM * SCfg<BITS>::SK;      // bf16 per stage
    static constexpr int NI = STAGE / 512;                  // 1 KiB loads per stage (512 bf16)
    static_assert(NI % (PT / 64) == 0, "stage loads must split evenly over the waves");
};
// bf16 index of chunk ch of row R in a stage
template <int BITS>
__device__ __forceinline__ int swz_index(int R, int ch) {
    using S = SCfg<BITS>;
    return R * S::SK + 8 * (ch ^ (R & S::SWM));
}

// One stage's share of a wave: 16 RT rows (RT 16-row tiles r) x one 64-column
// weight block (four 16-column tiles t), K = the unit's groups G0..G1-1 (the
// stage's).  xb: the stage; wv: this wave's code slots of the unit; sbv: its
// scale/bias dwords of the stage's groups; ng: valid groups of the unit.
template <int BITS, int RT, int G0, int G1>
__device__ __forceinline__ void prefill_stage(const uint16_t *__restrict__ xb, const u32x4 (&wv)[Cfg<BITS>::NS],
                                              const u32x4 (&sbv)[SCfg<BITS>::NSB], int ng, int wr, int c, int j,
                                              f32x4 (&y)[RT][4]) {
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const bf16x8 ones = as_bf16x8(u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});
#pragma unroll
    for (int g = G0; g < G1; ++g) {
        if (g >= ng) break;
        // the four column tiles' weight operands of group g
        bf16x8 bw0[4], bw1[4];
        float sc[4], bi[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            if constexpr (BITS == 16) {
                bw0[t] = as_bf16x8(wv[t]);
                bw1[t] = as_bf16x8(wv[4 + t]);
                sc[t] = 1.f;
                bi[t] = 0.f;
            } else {
                if constexpr (BITS == 8) {
                    const u32x4 qv = wv[4 * g + t];
                    bw0[t] = codes8_to_bf16(qv[0], qv[1]);
                    bw1[t] = codes8_to_bf16(qv[2], qv[3]);
                } else if constexpr (BITS == 4) {
                    const u32x4 qv = wv[4 * (g >> 1) + t];
                    bw0[t] = codes4_to_bf16(qv[2 * (g & 1)]);
                    bw1[t] = codes4_to_bf16(qv[2 * (g & 1) + 1]);
                } else if constexpr (BITS == 2) {
                    codes2_to_bf16(wv[t][g], bw0[t], bw1[t]);
                } else {
                    const uint32_t hd = wv[4 + (t >> 1)][2 * (t & 1) + (g >> 1)];
                    codes3_to_bf16(wv[t][g], hd >> (8 * (g & 1)), bw0[t], bw1[t]);
                }
                const uint32_t sbd = sbv[g - G0][t];
                sc[t] = h2f(sbd & 0xffffu);
                bi[t] = h2f(sbd >> 16);
                if constexpr (BITS <= 4) bi[t] = fmaf(-128.f, sc[t], bi[t]);   // codes carry +128
            }
        }
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            // lane (c, j): row 16 (RT wr + r) + c, K offsets 64 g + 16 j + 0..15
            const int R = 16 * (RT * wr + r) + c;
            const u32x4 x0 = *(const u32x4 *)(xb + swz_index<BITS>(R, 8 * (g - G0) + 2 * j));
            const u32x4 x1 = *(const u32x4 *)(xb + swz_index<BITS>(R, 8 * (g - G0) + 2 * j + 1));
            bf16x8 a0, a1;
            if constexpr (BITS == 4) {
                a0 = as_bf16x8(perm_x_for4(x0));
                a1 = as_bf16x8(perm_x_for4(x1));
            } else if constexpr (BITS == 2 || BITS == 3) {
                u32x4 p0, p1;
                perm_x_for2(x0, x1, p0, p1);
                a0 = as_bf16x8(p0);
                a1 = as_bf16x8(p1);
            } else {
                a0 = as_bf16x8(x0);
                a1 = as_bf16x8(x1);
            }
            if constexpr (BITS == 16) {
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    y[r][t] = mfma(a0, bw0[t], y[r][t]);
                    y[r][t] = mfma(a1, bw1[t], y[r][t]);
                }
            } else {
                f32x4 xs = mfma(a0, ones, zero);
                xs = mfma(a1, ones, xs);
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    f32x4 acc = mfma(a0, bw0[t], zero);
                    acc = mfma(a1, bw1[t], acc);
#pragma unroll
                    for (int r4 = 0; r4 < 4; ++r4)
                        y[r][t][r4] = fmaf(sc[t], acc[r4], fmaf(bi[t], xs[r4], y[r][t][r4]));
                }
            }
        }
    }
}

// The activations of K [kb, kb + SK) of this workgroup's rows into a stage,
// by direct global-to-LDS loads (wave w issues loads w, w + 4, ...; load i
// fills bf16 [512 i, 512 i + 512) of the stage, lane l the 8 at 512 i + 8 l).
// Rows past m read row m - 1 and K past k reads K offset 0: those values
// reach only rows that are never stored and groups that are never computed.
template <int BITS, int RT>
__device__ __forceinline__ void prefill_dma_x(const PrefillArgs &A, int row0, int kb, uint16_t *stage, int w,
                                              int lane) {
    using S = SCfg<BITS>;
    const int rl = lane / S::CH, pos = lane % S::CH;
#pragma unroll
    for (int ii = 0; ii < RCfg<BITS, RT>::NI / (PT / 64); ++ii) {
        const int i = w + (PT / 64) * ii;
        const int R = i * S::RPI + rl;
        const int ch = pos ^ (R & S::SWM);
        const int row = min(row0 + R, A.m - 1);
        const int kk = kb + 8 * ch;
        const uint16_t *src = A.x + (int64_t)row * A.ldx + (kk < A.k ? kk : 0);
        __builtin_amdgcn_global_load_lds((const void *)src,
                                         (__attribute__((address_space(3))) void *)(stage + 512 * i), 16, 0, 0);
    }
}
// This wave's code slots of unit u.
template <int BITS>
__device__ __forceinline__ void prefill_fetch_codes(const unsigned char *ub0, int u, int lane,
                                                    u32x4 (&wv)[Cfg<BITS>::NS]) {
    using C = Cfg<BITS>;
    const unsigned char *ub = ub0 + (size_t)u * C::UNIT;
#pragma unroll
    for (int i = 0; i < C::NS; ++i) wv[i] = *(const u32x4 *)(ub + i * 1024 + 16 * lane);
}
// This lane's scale/bias dwords (its column of each of the four tiles) of
// the groups of stage h of unit u.
template <int BITS>
__device__ __forceinline__ void prefill_fetch_sb(const unsigned char *ub0, int u, int h, int c,
                                                 u32x4 (&sbv)[SCfg<BITS>::NSB]) {
    using C = Cfg<BITS>;
    using S = SCfg<BITS>;
    if constexpr (BITS != 16) {
        const unsigned char *ub = ub0 + (size_t)u * C::UNIT + C::SBOFF + c * (16 * C::SBQ);
#pragma unroll
        for (int q = 0; q < S::GH; ++q) sbv[q] = *(const u32x4 *)(ub + 16 * (S::GH * h + q));
    }
}

// K split: a lane's four partial sums of one 16 x 16 tile as two
// device-scope 64-bit accesses, laid out [half][lane][2] (each wave-wide
// access covers 512 contiguous bytes).  Device-scope atomic accesses reach
// the other workgroups of the tile without a cache flush.
__device__ __forceinline__ void part_store(float *tile, int lane, f32x4 v) {
    unsigned long long *q = (unsigned long long *)tile;
    const unsigned long long lo = (unsigned long long)__float_as_uint(v[0]) |
                                  ((unsigned long long)__float_as_uint(v[1]) << 32);
    const unsigned long long hi = (unsigned long long)__float_as_uint(v[2]) |
                                  ((unsigned long long)__float_as_uint(v[3]) << 32);
    __hip_atomic_store(q + lane, lo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(q + 64 + lane, hi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ f32x4 part_load(const float *tile, int lane) {
    unsigned long long *q = (unsigned long long *)tile;
    const unsigned long long lo = __hip_atomic_load(q + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned long long hi = __hip_atomic_load(q + 64 + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return f32x4{__uint_as_float((uint32_t)lo), __uint_as_float((uint32_t)(lo >> 32)), __uint_as_float((uint32_t)hi),
                 __uint_as_float((uint32_t)(hi >> 32))};
}

// Final values of this wave's 16 RT x 64 block of y.
template <int RT>
__device__ __forceinline__ void prefill_store(const PrefillArgs &A, int row0, int wr, int b, int c, int j,
                                              const f32x4 (&y)[RT][4]) {
    // lane (c, j) of tile (r, t) holds rows 4 j .. 4 j + 3, column c
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int col = 64 * b + 16 * t + c;
            if (col >= A.n) continue;
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int row = row0 + 16 * (RT * wr + r) + 4 * j + r4;
                if (row < A.m) {
                    if (A.y_bf16)
                        ((uint16_t *)A.y)[(int64_t)row * A.ldy + col] = f2bf16(y[r][t][r4]);
                    else
                        ((float *)A.y)[(int64_t)row * A.ldy + col] = y[r][t][r4];
                }
            }
        }
}

// Software pipeline over the stages of K: while a workgroup computes one
// stage (from LDS, with its unit's code registers and the stage's
// scale/bias registers), the direct loads of the next stage fill the other
// LDS buffer, its scale/bias dwords a second register set and, at a unit's
// first stage, the next unit's codes a second code set; one barrier per
// stage.  Stages, code sets and scale/bias sets are each two distinct
// arrays used alternately and the loop handles two units per trip, so no
// LDS read of a stage can alias the buffer being filled and no register set
// is ever copied.
template <int BITS, int RT>
__global__ __launch_bounds__(PT, 2) void prefill_kernel(const PrefillArgs A) {
    using C = Cfg<BITS>;
    using S = SCfg<BITS>;
    using R = RCfg<BITS, RT>;
    __shared__ __attribute__((aligned(1024))) uint16_t xs0[R::STAGE];
    __shared__ __attribute__((aligned(1024))) uint16_t xs1[R::STAGE];
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wr = w >> 1, wc = w & 1;
    const int c = lane & 15, j = lane >> 4;
    const int row0 = blockIdx.x * R::PBM;
    const int b = 2 * blockIdx.y + wc;                     // this wave's 64-column block
    const bool has_block = b < A.nblocks;
    const unsigned char *ub0 = (const unsigned char *)A.tiles + (size_t)b * A.nst * C::UNIT;
    // K split blockIdx.z of A.ks: units [U0, U1) of the block's A.nst
    const int ks = A.ks, sp = blockIdx.z;
    const int U0 = (int)((int64_t)A.nst * sp / ks), U1 = (int)((int64_t)A.nst * (sp + 1) / ks);

    f32x4 y[RT][4];
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int t = 0; t < 4; ++t) y[r][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x4 wa[C::NS], wb[C::NS];                 // code sets: even units, odd units
    u32x4 s0[S::NSB], s1[S::NSB];               // scale/bias sets: with stage xs0, with xs1
    prefill_dma_x<BITS, RT>(A, row0, C::KU * U0, xs0, w, lane);
    if (has_block) {
        prefill_fetch_codes<BITS>(ub0, U0, lane, wa);
        prefill_fetch_sb<BITS>(ub0, U0, 0, c, s0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // Stage h of unit u: computed from (cur, scur) with the unit's codes wcur
    // while the next stage fills (nxt, snxt) and, at h = 0, unit u + 1's
    // codes fill wnxt.
    auto stage = [&](auto hc, int u, const uint16_t *cur, uint16_t *nxt, const u32x4 (&wcur)[C::NS],
                     u32x4 (&wnxt)[C::NS], const u32x4 (&scur)[S::NSB], u32x4 (&snxt)[S::NSB])
        __attribute__((always_inline)) {
        constexpr int h = decltype(hc)::value;
        const int nu = h + 1 < S::HALVES ? u : u + 1, nh = h + 1 < S::HALVES ? h + 1 : 0;
        if (nu < U1) {
            prefill_dma_x<BITS, RT>(A, row0, C::KU * nu + S::SK * nh, nxt, w, lane);
            if (has_block) {
                if (h == 0 && u + 1 < U1) prefill_fetch_codes<BITS>(ub0, u + 1, lane, wnxt);
                prefill_fetch_sb<BITS>(ub0, nu, nh, c, snxt);
            }
        }
        if (has_block)
            prefill_stage<BITS, RT, h * S::GH, (h + 1) * S::GH>(cur, wcur, scur,
                                                                min(C::GS, (A.k - C::KU * u) / 64), wr, c, j, y);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    };
    using H0 = std::integral_constant<int, 0>;
    using H1 = std::integral_constant<int, 1>;
    for (int u = U0; u < U1; u += 2) {
        if constexpr (S::HALVES == 1) {
            // one stage per unit: unit u on xs0, unit u + 1 on xs1
            stage(H0{}, u, xs0, xs1, wa, wb, s0, s1);
            if (u + 1 < U1) stage(H0{}, u + 1, xs1, xs0, wb, wa, s1, s0);
        } else {
            // two stages per unit: every unit starts on xs0
            stage(H0{}, u, xs0, xs1, wa, wb, s0, s1);
            stage(H1{}, u, xs1, xs0, wa, wb, s1, s0);
            if (u + 1 < U1) {
                stage(H0{}, u + 1, xs0, xs1, wb, wa, s0, s1);
                stage(H1{}, u + 1, xs1, xs0, wb, wa, s1, s0);
            }
        }
    }
    if (!has_block) return;
    if (ks > 1) {
        // publish this split's partial block, count in; the last of the
        // tile's ks arrivals adds the partials in split order (so the result
        // does not depend on the arrival order) and stores y
        const int64_t tile = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
        constexpr int PW = RT * 4 * 256;                 // floats per wave and split
        float *const pw = A.part + (tile * 4 + w) * ks * PW;
#pragma unroll
        for (int r = 0; r < RT; ++r)
#pragma unroll
            for (int t = 0; t < 4; ++t) part_store(pw + sp * PW + (4 * r + t) * 256, lane, y[r][t]);
        __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));   // vmcnt(0): the partials are performed
        uint32_t *const ctr = A.ctr + tile * 4 + w;
        uint32_t ticket = 0;
        if (lane == 0) ticket = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ticket = __shfl(ticket, 0);
        if (ticket != (uint32_t)(ks - 1)) return;
#pragma unroll
        for (int r = 0; r < RT; ++r)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                f32x4 z = sp == 0 ? y[r][t] : part_load(pw + (4 * r + t) * 256, lane);
                for (int q = 1; q < ks; ++q) z += q == sp ? y[r][t] : part_load(pw + q * PW + (4 * r + t) * 256, lane);
                y[r][t] = z;
            }
        if (lane == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    prefill_store(A, row0, wr, b, c, j, y);
}

template <int RT>
hipError_t launch_rt(const PrefillArgs &A, int bits, hipStream_t s) {
    const dim3 grid((unsigned)((A.m + 32 * RT - 1) / (32 * RT)), (unsigned)((A.nblocks + 1) / 2), (unsigned)A.ks),
        block(PT);
    switch (bits) {
        case 2: hipLaunchKernelGGL((prefill_kernel<2, RT>), grid, block, 0, s, A); break;
        case 3: hipLaunchKernelGGL((prefill_kernel<3, RT>), grid, block, 0, s, A); break;
        case 4: hipLaunchKernelGGL((prefill_kernel<4, RT>), grid, block, 0, s, A); break;
        case 8: hipLaunchKernelGGL((prefill_kernel<8, RT>), grid, block, 0, s, A); break;
        case 16: hipLaunchKernelGGL((prefill_kernel<16, RT>), grid, block, 0, s, A); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}
}  // namespace

hipError_t launch_prefill(const PrefillArgs &A, int bits, hipStream_t s) {
    return A.block_rows == 64 ? launch_rt<2>(A, bits, s) : launch_rt<4>(A, bits, s);
}

}  // namespace dspk

// Prefill projections: y[i][c] = sum_r x[i][r] * (s[c][r/64] * q[c][r] + b[c][r/64])
// for many rows at once (a prompt's tokens), through the same tiled weights
// the verify kernels stream ("mlx-dspark" wiki summary, "Key techniques":
// each weight group is dequantised once and reused for every row of the
// pass; prefill is the wide-row case of that pass).
//
// With hundreds of rows the work is bound by the matrix cores, not by HBM,
// so this kernel is tiled for MFMA reuse rather than for streaming:
// * A workgroup computes a 128-row x 128-column block of y: four waves, each
//   64 rows (four 16-row tiles) x one 64-column weight block (four 16-column
//   tiles), K walked one tiled unit at a time.
// * Per unit the workgroup stages its 128 activation rows into LDS (row-major,
//   rows padded by 16 bytes so the 16 rows one MFMA operand reads fall into
//   different banks); each wave loads its weight unit straight from the tiled
//   layout into registers, where every lane already holds its own operand
//   bytes.
// * Codes are exact in bf16, so per group and per 16x16 tile
//     sum_{r in group} x*w = s * sum x*q + b * sum x
//   comes from exact-product MFMAs on the codes (fp32 accumulation) plus a
//   per-group scale/bias update, as in the verify kernels; the row sums of x
//   come from an MFMA against a ones operand.  No dequantised weight is
//   rounded.  Each activation operand read from LDS serves the four column
//   tiles, each decoded weight operand the four row tiles.
// * Two workgroups per CU (LDS <= 68 KiB each): one stages while the other
//   computes.  Row blocks vary fastest in the grid, so the workgroups that
//   run together share their weight units in L2.
#include <hip/hip_runtime.h>

#include "decode.h"
#include "dspk_internal.h"

namespace dspk {
namespace {

using namespace dec;

constexpr int PBM = 128;                 // rows per workgroup
constexpr int PT = 256;                  // threads per workgroup

template <int BITS>
struct PCfg {
    static constexpr int KU = Cfg<BITS>::KU;
    static constexpr int LDSW = KU + 8;                    // bf16 per staged row (16-byte pad)
    static constexpr int CPT = PBM * KU / 8 / PT;          // 16-byte activation chunks per thread per unit
};

// One unit's share of a wave: 64 rows (four 16-row tiles r) x one 64-column
// weight block (four 16-column tiles t), K = the unit's groups.  xb: the
// unit's staged activations (row-major, LDSW bf16 per row); wv / sbv: this
// wave's code slots and scale/bias dwords of the unit.
template <int BITS>
__device__ __forceinline__ void prefill_unit(const uint16_t *__restrict__ xb, const u32x4 (&wv)[Cfg<BITS>::NS],
                                             const u32x4 (&sbv)[Cfg<BITS>::SBQ > 0 ? Cfg<BITS>::SBQ : 1], int ng,
                                             int wr, int c, int j, f32x4 (&y)[4][4]) {
    using C = Cfg<BITS>;
    using P = PCfg<BITS>;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const bf16x8 ones = as_bf16x8(u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});
#pragma unroll
    for (int g = 0; g < C::GS; ++g) {
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
                const uint32_t sbd = sbv[g][t];
                sc[t] = h2f(sbd & 0xffffu);
                bi[t] = h2f(sbd >> 16);
                if constexpr (BITS <= 4) bi[t] = fmaf(-128.f, sc[t], bi[t]);   // codes carry +128
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            // lane (c, j): row 64 wr + 16 r + c, K offsets 64 g + 16 j + 0..15
            const uint16_t *xp = xb + (64 * wr + 16 * r + c) * P::LDSW + 64 * g + 16 * j;
            const u32x4 x0 = *(const u32x4 *)xp, x1 = *(const u32x4 *)(xp + 8);
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

// Unit u's activations of this workgroup's rows into registers (rows past m
// and K past k read as zero), and their store into a staging buffer.
template <int BITS>
__device__ __forceinline__ void prefill_fetch_x(const PrefillArgs &A, int row0, int u,
                                                u32x4 (&stage)[PCfg<BITS>::CPT]) {
    using C = Cfg<BITS>;
    using P = PCfg<BITS>;
#pragma unroll
    for (int i = 0; i < P::CPT; ++i) {
        const int q = threadIdx.x + PT * i;
        const int r = q / (C::KU / 8), ch = q % (C::KU / 8);
        const int row = row0 + r, kk = C::KU * u + 8 * ch;
        stage[i] = (row < A.m && kk < A.k) ? *(const u32x4 *)(A.x + (int64_t)row * A.ldx + kk)
                                           : u32x4{0u, 0u, 0u, 0u};
    }
}
template <int BITS>
__device__ __forceinline__ void prefill_put_x(uint16_t *xb, const u32x4 (&stage)[PCfg<BITS>::CPT]) {
    using C = Cfg<BITS>;
    using P = PCfg<BITS>;
#pragma unroll
    for (int i = 0; i < P::CPT; ++i) {
        const int q = threadIdx.x + PT * i;
        const int r = q / (C::KU / 8), ch = q % (C::KU / 8);
        *(u32x4 *)(xb + r * P::LDSW + 8 * ch) = stage[i];
    }
}
// This wave's code slots and scale/bias dwords of unit u.
template <int BITS>
__device__ __forceinline__ void prefill_fetch_w(const unsigned char *ub0, int u, int lane, int c,
                                                u32x4 (&wv)[Cfg<BITS>::NS],
                                                u32x4 (&sbv)[Cfg<BITS>::SBQ > 0 ? Cfg<BITS>::SBQ : 1]) {
    using C = Cfg<BITS>;
    const unsigned char *ub = ub0 + (size_t)u * C::UNIT;
#pragma unroll
    for (int i = 0; i < C::NS; ++i) wv[i] = *(const u32x4 *)(ub + i * 1024 + 16 * lane);
#pragma unroll
    for (int q = 0; q < C::SBQ; ++q) sbv[q] = *(const u32x4 *)(ub + C::SBOFF + c * (16 * C::SBQ) + 16 * q);
}

// Final values of this wave's 64 x 64 block of y.
__device__ __forceinline__ void prefill_store(const PrefillArgs &A, int row0, int wr, int b, int c, int j,
                                              const f32x4 (&y)[4][4]) {
    // lane (c, j) of tile (r, t) holds rows 4 j .. 4 j + 3, column c
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int col = 64 * b + 16 * t + c;
            if (col >= A.n) continue;
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int row = row0 + 64 * wr + 16 * r + 4 * j + r4;
                if (row < A.m) {
                    if (A.y_bf16)
                        ((uint16_t *)A.y)[(int64_t)row * A.ldy + col] = f2bf16(y[r][t][r4]);
                    else
                        ((float *)A.y)[(int64_t)row * A.ldy + col] = y[r][t][r4];
                }
            }
        }
}

template <int BITS>
__global__ __launch_bounds__(PT, 2) void prefill_kernel(const PrefillArgs A) {
    using C = Cfg<BITS>;
    using P = PCfg<BITS>;
    __shared__ __attribute__((aligned(16))) uint16_t xt[PBM * P::LDSW];
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wr = w >> 1, wc = w & 1;
    const int c = lane & 15, j = lane >> 4;
    const int row0 = blockIdx.x * PBM;
    const int b = 2 * blockIdx.y + wc;                     // this wave's 64-column block
    const bool has_block = b < A.nblocks;
    const unsigned char *ub0 = (const unsigned char *)A.tiles + (size_t)b * A.nst * C::UNIT;

    f32x4 y[4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int t = 0; t < 4; ++t) y[r][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int u = 0; u < A.nst; ++u) {
        u32x4 stage[P::CPT];
        prefill_fetch_x<BITS>(A, row0, u, stage);
        u32x4 wv[C::NS];
        u32x4 sbv[C::SBQ > 0 ? C::SBQ : 1];
        if (has_block) prefill_fetch_w<BITS>(ub0, u, lane, c, wv, sbv);
        prefill_put_x<BITS>(xt, stage);
        __syncthreads();
        if (has_block) prefill_unit<BITS>(xt, wv, sbv, min(C::GS, (A.k - C::KU * u) / 64), wr, c, j, y);
        __syncthreads();
    }
    if (has_block) prefill_store(A, row0, wr, b, c, j, y);
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs &A, int bits, hipStream_t s) {
    const dim3 grid((unsigned)((A.m + PBM - 1) / PBM), (unsigned)((A.nblocks + 1) / 2)), block(PT);
    switch (bits) {
        case 2: hipLaunchKernelGGL(prefill_kernel<2>, grid, block, 0, s, A); break;
        case 3: hipLaunchKernelGGL(prefill_kernel<3>, grid, block, 0, s, A); break;
        case 4: hipLaunchKernelGGL(prefill_kernel<4>, grid, block, 0, s, A); break;
        case 8: hipLaunchKernelGGL(prefill_kernel<8>, grid, block, 0, s, A); break;
        case 16: hipLaunchKernelGGL(prefill_kernel<16>, grid, block, 0, s, A); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace dspk

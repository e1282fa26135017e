// Verify-pass projections through affine group-quantised weights, and the
// vocabulary head fused with the row argmax, for gfx950 (MI355X).
//
// What is computed: y[i][c] = sum_r x[i][r] * (s[c][r/64] * q[c][r] + b[c][r/64])
// for the M = anchor + drafts rows i ("mlx-dspark" wiki summary, sections
// "Architecture" and "Key techniques": one target pass over all rows, each
// weight group dequantised once and reused for every row).
//
// How (MI355X-first, not the pages' Metal kernel):
// * The weights are the only large stream, so the kernel is HBM-bound for
//   every M <= 32: each lane issues one 16-byte load per 16 codes, a wave
//   covers 64 output columns, and loads run PF groups ahead.
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
// * Four waves of a workgroup take consecutive K ranges of one 64-column block
//   and add their partial sums in LDS in wave order.  Long K is split across
//   workgroups; the last workgroup to arrive adds the partials in split order,
//   so results do not depend on scheduling.
#include "dspk_internal.h"

namespace dspk {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int NT = kTilesPerWave;
constexpr int kSbStride = kBlockCols + 1;       // padded LDS row (dwords) of the scale/bias table
constexpr int kSmemDwords = kMaxWGGroups * kSbStride;

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

template <int BITS, int MT>
struct Slot {
    static constexpr int BQ = BITS == 16 ? 2 : 1;
    u32x4 b[NT][BQ];
    u32x4 a[MT][2];
};

// One wave: 64 columns [n0, n0+64) x groups [g0, g0+ng) of one weight, all rows.
template <int BITS, int MT, int PF>
__device__ __forceinline__ void wave_gemm(const GemmProblem &P, const uint16_t *__restrict__ x,
                                          int64_t ldx, int M, int n0, int g0, int ng, int lg0,
                                          const uint32_t *sb, int lane, f32x4 (&y)[NT][MT]) {
    const int c = lane & 15, j = lane >> 4;
    constexpr int GDW = 64 * BITS / 32;     // dwords per group of one weight row
    constexpr int LDW = GDW / 4;            // dwords per lane per group (4 lanes share a row)
    const int64_t row_dw = (int64_t)P.k * BITS / 32;
    const uint32_t *rows[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int n = min(n0 + 16 * t + c, P.n - 1);   // columns past n read row n-1, never stored
        rows[t] = (const uint32_t *)P.codes + (int64_t)n * row_dw + j * LDW;
    }
    const uint16_t *xr[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int m = min(16 * mt + c, M - 1);          // rows past M repeat row M-1, never stored
        xr[mt] = x + (int64_t)m * ldx + 16 * j;
    }

    auto load = [&](Slot<BITS, MT> &s, int g) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const uint32_t *p = rows[t] + (int64_t)g * GDW;
            if constexpr (BITS == 8) {
                s.b[t][0] = *(const u32x4 *)p;
            } else if constexpr (BITS == 4) {
                const u32x2 v = *(const u32x2 *)p;
                s.b[t][0] = u32x4{v[0], v[1], 0u, 0u};
            } else {
                s.b[t][0] = *(const u32x4 *)p;
                s.b[t][1] = *(const u32x4 *)(p + 4);
            }
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const uint16_t *q = xr[mt] + (int64_t)g * 64;
            s.a[mt][0] = *(const u32x4 *)q;
            s.a[mt][1] = *(const u32x4 *)(q + 8);
        }
    };

    auto compute = [&](const Slot<BITS, MT> &s, int lg) {
        bf16x8 a0[MT], a1[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            if constexpr (BITS == 4) {
                a0[mt] = as_bf16x8(perm_x_for4(s.a[mt][0]));
                a1[mt] = as_bf16x8(perm_x_for4(s.a[mt][1]));
            } else {
                a0[mt] = as_bf16x8(s.a[mt][0]);
                a1[mt] = as_bf16x8(s.a[mt][1]);
            }
        }
        if constexpr (BITS == 16) {
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const bf16x8 b0 = as_bf16x8(s.b[t][0]), b1 = as_bf16x8(s.b[t][1]);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    y[t][mt] = mfma(a0[mt], b0, y[t][mt]);
                    y[t][mt] = mfma(a1[mt], b1, y[t][mt]);
                }
            }
        } else {
            const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
            const bf16x8 ones = as_bf16x8(u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});
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
                    b0 = codes8_to_bf16(s.b[t][0][0], s.b[t][0][1]);
                    b1 = codes8_to_bf16(s.b[t][0][2], s.b[t][0][3]);
                } else {
                    b0 = codes4_to_bf16(s.b[t][0][0]);
                    b1 = codes4_to_bf16(s.b[t][0][1]);
                }
                const uint32_t sbv = sb[lg * kSbStride + 16 * t + c];
                const float sc = h2f(sbv & 0xffffu);
                float bi = h2f(sbv >> 16);
                if constexpr (BITS == 4) bi = fmaf(-128.f, sc, bi);   // codes carry +128
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    f32x4 acc = mfma(a0[mt], b0, zero);
                    acc = mfma(a1[mt], b1, acc);
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        y[t][mt][r] = fmaf(sc, acc[r], fmaf(bi, xs[mt][r], y[t][mt][r]));
                }
            }
        }
    };

    Slot<BITS, MT> buf[PF];
#pragma unroll
    for (int p = 0; p < PF; ++p)
        if (p < ng) load(buf[p], g0 + p);
    int gi = 0;
    for (; gi + 2 * PF <= ng; gi += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            const Slot<BITS, MT> cur = buf[p];
            load(buf[p], g0 + gi + p + PF);
            compute(cur, lg0 + gi + p);
        }
    }
    for (; gi < ng; gi += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            if (gi + p < ng) {
                const Slot<BITS, MT> cur = buf[p];
                if (gi + p + PF < ng) load(buf[p], g0 + gi + p + PF);
                compute(cur, lg0 + gi + p);
            }
        }
    }
}

template <int BITS, int MT, int PF, bool ARGMAX>
__global__ __launch_bounds__(256) void qgemm_kernel(const GemmLaunch L) {
    __shared__ uint32_t smem[kSmemDwords];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int bid = blockIdx.x;
    int pi = 0;
#pragma unroll
    for (int i = 1; i < kMaxGrouped; ++i)
        if (i < L.count && bid >= L.p[i].wg_begin) pi = i;
    const GemmProblem &P = L.p[pi];

    const int local = bid - P.wg_begin;
    const int cb = local / P.splits, split = local - cb * P.splits;
    const int n0 = cb * kBlockCols;
    const int G = P.k >> 6;
    const int wg_groups = P.wave_groups * kWavesPerWG;
    const int wg_g0 = split * wg_groups;
    const int wg_g1 = min(G, wg_g0 + wg_groups);
    const int g0 = min(wg_g1, wg_g0 + w * P.wave_groups);
    const int g1 = min(wg_g1, g0 + P.wave_groups);

    if constexpr (BITS != 16) {
        // scale/bias table of this workgroup: smem[g][col] = s | b << 16
        const int wgn = wg_g1 - wg_g0;
        for (int idx = tid; idx < kBlockCols * wgn; idx += 256) {
            const int col = idx / wgn, g = idx - col * wgn;
            const int n = min(n0 + col, P.n - 1);
            const int64_t off = (int64_t)n * G + wg_g0 + g;
            smem[g * kSbStride + col] = (uint32_t)P.scales[off] | ((uint32_t)P.biases[off] << 16);
        }
        __syncthreads();
    }

    f32x4 y[NT][MT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) y[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    wave_gemm<BITS, MT, PF>(P, L.x, L.ldx, L.m, n0, g0, g1 - g0, g0 - wg_g0, smem, lane, y);

    // waves 1..3 hand their partial sums to wave 0, which adds them in wave order
    __syncthreads();
    float *red = (float *)smem;
    const int c = lane & 15, j = lane >> 4;
    constexpr int RROWS = 16 * MT;
    if (w > 0) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    red[((w - 1) * RROWS + 16 * mt + 4 * j + r) * kBlockCols + 16 * t + c] = y[t][mt][r];
    }
    __syncthreads();
    if (w != 0) return;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float v = y[t][mt][r];
#pragma unroll
                for (int q = 0; q < kWavesPerWG - 1; ++q)
                    v += red[(q * RROWS + 16 * mt + 4 * j + r) * kBlockCols + 16 * t + c];
                y[t][mt][r] = v;
            }

    const int M = L.m, N = P.n;
    if constexpr (ARGMAX) {
        // fused argmax over this block's 64 columns, then across workgroups
        unsigned long long best[MT][4];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = 16 * mt + 4 * j + r;
                unsigned long long b = 0ull;
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const int n = n0 + 16 * t + c;
                    const float v = y[t][mt][r];
                    if (n < N) {
                        const unsigned long long k = argmax_key(v, n);
                        b = k > b ? k : b;
                        if (L.logits != nullptr && m < M) L.logits[(int64_t)m * L.ldl + n] = v;
                    }
                }
#pragma unroll
                for (int off = 1; off < 16; off <<= 1) {
                    const unsigned long long o = __shfl_xor(b, off);
                    b = o > b ? o : b;
                }
                best[mt][r] = b;
            }
        if (c == 0) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = 16 * mt + 4 * j + r;
                    if (m < M) atomicMax(&L.keys[m], best[mt][r]);
                }
        }
        __threadfence();
        uint32_t ticket = 0;
        if (lane == 0) ticket = atomicAdd(L.done, 1u);
        ticket = __shfl(ticket, 0);
        if (ticket == gridDim.x - 1) {
            __threadfence();
            if (lane < M) {
                const unsigned long long k = atomicExch(&L.keys[lane], 0ull);
                L.argmax[lane] = (int32_t)(0xffffffffu - (uint32_t)(k & 0xffffffffull));
            }
            if (lane == 0) atomicExch(L.done, 0u);
        }
    } else {
        auto store = [&](int m, int n, float v) {
            if (L.y_bf16)
                ((uint16_t *)P.y)[(int64_t)m * P.ldy + n] = f2bf16(v);
            else
                ((float *)P.y)[(int64_t)m * P.ldy + n] = v;
        };
        if (P.splits == 1) {
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int m = 16 * mt + 4 * j + r, n = n0 + 16 * t + c;
                        if (m < M && n < N) store(m, n, y[t][mt][r]);
                    }
            return;
        }
        // split K: publish this split's partial sums, the last arrival adds all splits in order
        const int64_t plane = (int64_t)M * N;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = 16 * mt + 4 * j + r, n = n0 + 16 * t + c;
                    if (m < M && n < N) P.partial[split * plane + (int64_t)m * N + n] = y[t][mt][r];
                }
        __threadfence();
        uint32_t ticket = 0;
        if (lane == 0) ticket = atomicAdd(&P.counters[cb], 1u);
        ticket = __shfl(ticket, 0);
        if (ticket != (uint32_t)P.splits - 1) return;
        __threadfence();
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = 16 * mt + 4 * j + r, n = n0 + 16 * t + c;
                    if (m < M && n < N) {
                        const float *p = P.partial + (int64_t)m * N + n;
                        float v = p[0];
                        for (int s = 1; s < P.splits; ++s) v += p[s * plane];
                        store(m, n, v);
                    }
                }
        if (lane == 0) atomicExch(&P.counters[cb], 0u);
    }
}

template <int BITS, bool ARGMAX>
hipError_t launch_bits(const GemmLaunch &L, int grid, hipStream_t s) {
    if (L.m <= 16)
        hipLaunchKernelGGL((qgemm_kernel<BITS, 1, 4, ARGMAX>), dim3(grid), dim3(256), 0, s, L);
    else
        hipLaunchKernelGGL((qgemm_kernel<BITS, 2, 3, ARGMAX>), dim3(grid), dim3(256), 0, s, L);
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

// Work split: aim for about kTargetWaves waves in flight (8 per CU on 256 CUs),
// each streaming at least kMinWaveGroups groups so prologue and reduction stay
// small next to the weight stream.
constexpr int kTargetWaves = 2048;
constexpr int kMinWaveGroups = 4;

GemmPlan plan_gemm(int32_t n, int32_t k, int32_t m, int32_t bits, bool force_single_split) {
    (void)bits;
    GemmPlan p{};
    const int G = k / 64;
    p.ncb = (n + kBlockCols - 1) / kBlockCols;
    int parts = (kTargetWaves + p.ncb - 1) / p.ncb;
    parts = max(parts, min(kWavesPerWG, G));
    parts = min(parts, G);
    int wg = (G + parts - 1) / parts;
    wg = max(wg, min(kMinWaveGroups, (G + kWavesPerWG - 1) / kWavesPerWG));
    wg = min(wg, kMaxWGGroups / kWavesPerWG);
    if (force_single_split) wg = (G + kWavesPerWG - 1) / kWavesPerWG;
    parts = (G + wg - 1) / wg;
    p.wave_groups = wg;
    p.splits = (parts + kWavesPerWG - 1) / kWavesPerWG;
    p.ws_bytes = 0;
    if (p.splits > 1) {
        const size_t ctr = ((size_t)p.ncb * 4 + 255) / 256 * 256;
        p.ws_bytes = ctr + (size_t)p.splits * m * n * 4;
        p.ws_bytes = (p.ws_bytes + 255) / 256 * 256;
    }
    return p;
}

hipError_t launch_qgemm(const GemmLaunch &L, int bits, int grid, hipStream_t s) {
    return launch_any<false>(L, bits, grid, s);
}

hipError_t launch_lmhead(const GemmLaunch &L, int bits, int grid, hipStream_t s) {
    return launch_any<true>(L, bits, grid, s);
}

}  // namespace dspk

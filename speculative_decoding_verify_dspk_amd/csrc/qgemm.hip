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
// * A wave owns 64 output columns over one K range and streams it start to
//   end; the four waves of a workgroup take neighbouring column blocks of the
//   same K range, so their activation loads are served by the CU's L1.  Each
//   wave stages the fp16 scale/bias pairs of its columns in its own LDS slice.
// * When a weight has too few columns to fill the GPU, K is split across
//   workgroups: each split publishes fp32 partial sums with device-coherent
//   stores and the last workgroup of a column group to arrive adds them in
//   split order, so results do not depend on scheduling.  No cache flush is
//   needed: the partials and the arrival counter only move through
//   device-scope atomic accesses.
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

template <int BITS, int MT>
struct Slot {
    static constexpr int BQ = BITS == 16 ? 2 : 1;
    u32x4 b[NT][BQ];
    u32x4 a[MT][2];
};

__device__ __forceinline__ void wait_vm_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ void store_agent(float *p, float v) {
    __hip_atomic_store((uint32_t *)p, __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_agent(const float *p) {
    return __uint_as_float(__hip_atomic_load((uint32_t *)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

// Scale/bias pairs of this wave's 64 columns for groups [gc0, gc0 + gcn) into
// its LDS slice: sb[g][col] = s | b << 16.  Lane = column.
__device__ __forceinline__ void stage_sb(const GemmProblem &P, int n0, int G, int gc0, int gcn, bool vec,
                                         uint32_t *sb, int lane) {
    const int n = min(n0 + lane, P.n - 1);
    const uint16_t *srow = P.scales + (int64_t)n * G + gc0;
    const uint16_t *brow = P.biases + (int64_t)n * G + gc0;
    if (vec) {   // 16-byte loads: 8 groups per load (rows and chunk starts are 16-byte aligned)
        u32x4 sv[kSbChunk / 8], bv[kSbChunk / 8];
#pragma unroll
        for (int i = 0; i < kSbChunk / 8; ++i)
            if (8 * i < gcn) {
                sv[i] = *(const u32x4 *)(srow + 8 * i);
                bv[i] = *(const u32x4 *)(brow + 8 * i);
            }
#pragma unroll
        for (int i = 0; i < kSbChunk / 8; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (8 * i + e < gcn)
                    sb[(8 * i + e) * kBlockCols + lane] =
                        __builtin_amdgcn_perm(bv[i][e >> 1], sv[i][e >> 1], (e & 1) ? 0x07060302u : 0x05040100u);
    } else {
        for (int g = 0; g < gcn; ++g) sb[g * kBlockCols + lane] = (uint32_t)srow[g] | ((uint32_t)brow[g] << 16);
    }
}

// One wave: columns [n0, n0 + 64) x groups [g0, g1) of one weight, all rows.
template <int BITS, int MT, int PF>
__device__ __forceinline__ void wave_unit(const GemmProblem &P, bool sb_vec, const uint16_t *__restrict__ x,
                                          int64_t ldx, int M, int n0, int g0, int g1, uint32_t *sb, int lane,
                                          f32x4 (&y)[NT][MT]) {
    const int c = lane & 15, j = lane >> 4;
    const int G = P.k >> 6;
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
                const uint32_t sbv = sb[lg * kBlockCols + 16 * t + c];
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

    for (int gc0 = g0; gc0 < g1; gc0 += kSbChunk) {
        const int ng = min(kSbChunk, g1 - gc0);
        // Ring of PF slots, each consumed in place and then refilled with the
        // group PF ahead; the first PF groups are requested before the
        // scale/bias staging so their latency overlaps it.
        Slot<BITS, MT> buf[PF];
#pragma unroll
        for (int p = 0; p < PF; ++p)
            if (p < ng) load(buf[p], gc0 + p);
        if constexpr (BITS != 16) stage_sb(P, n0, G, gc0, ng, sb_vec, sb, lane);
        int gi = 0;
        for (; gi + 2 * PF <= ng; gi += PF) {
#pragma unroll
            for (int p = 0; p < PF; ++p) {
                compute(buf[p], gi + p);
                load(buf[p], gc0 + gi + p + PF);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        for (; gi < ng; gi += PF) {
#pragma unroll
            for (int p = 0; p < PF; ++p) {
                if (gi + p < ng) {
                    compute(buf[p], gi + p);
                    if (gi + p + PF < ng) load(buf[p], gc0 + gi + p + PF);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
}

// M <= 16 fits three waves per SIMD (12 per CU) without spills; two row tiles need two.
template <int BITS, int MT, int PF, bool ARGMAX>
__global__ __launch_bounds__(256, MT == 1 ? 3 : 2) void qgemm_kernel(const GemmLaunch L) {
    __shared__ uint32_t sb_all[kWavesPerWG][kSbChunk * kBlockCols];
    __shared__ unsigned long long red[kWavesPerWG][kMaxRows];
    __shared__ int s_last;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar loop control
    const int bid = blockIdx.x;
    int pi = 0;
#pragma unroll
    for (int i = 1; i < kMaxGrouped; ++i)
        if (i < L.count && bid >= L.p[i].wg_begin) pi = i;
    const GemmProblem &P = L.p[pi];

    const int local = bid - P.wg_begin;
    const int S = P.splits;
    const int cg = local / S, split = local - cg * S;
    const int n0 = cg * kWGCols + w * kBlockCols;
    const int M = L.m, N = P.n;
    const bool active = n0 < N;
    const int G = P.k >> 6;
    const int g0 = split * P.split_groups;
    const int g1 = min(G, g0 + P.split_groups);
    const bool sb_vec = ((G & 7) == 0) && ((P.split_groups & 7) == 0) &&
                        ((((uintptr_t)P.scales | (uintptr_t)P.biases) & 15) == 0);

    f32x4 y[NT][MT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) y[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (active) wave_unit<BITS, MT, PF>(P, sb_vec, L.x, L.ldx, M, n0, g0, g1, sb_all[w], lane, y);

    const int c = lane & 15, j = lane >> 4;
    if constexpr (ARGMAX) {
        // best (value, column) per row over this wave's 64 columns ...
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
                for (int r = 0; r < 4; ++r) red[w][16 * mt + 4 * j + r] = best[mt][r];
        }
        __syncthreads();
        // ... then over the workgroup, published for the last workgroup to combine
        if (tid < M) {
            unsigned long long b = red[0][tid];
#pragma unroll
            for (int q = 1; q < kWavesPerWG; ++q) b = red[q][tid] > b ? red[q][tid] : b;
            __hip_atomic_store(&L.keys[(int64_t)bid * kMaxRows + tid], b, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
        wait_vm_stores();
        __syncthreads();
        if (tid == 0)
            s_last = __hip_atomic_fetch_add(L.done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                     gridDim.x - 1;
        __syncthreads();
        if (!s_last) return;
        // last workgroup: maximum over all workgroups' keys, 8 rows at a time
        const int nwg = gridDim.x;
        for (int m0 = 0; m0 < M; m0 += 8) {
            unsigned long long b8[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) b8[i] = 0ull;
            for (int g = tid; g < nwg; g += 256) {
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    if (m0 + i < M) {
                        const unsigned long long k = __hip_atomic_load(&L.keys[(int64_t)g * kMaxRows + m0 + i],
                                                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        b8[i] = k > b8[i] ? k : b8[i];
                    }
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const unsigned long long o = __shfl_xor(b8[i], off);
                    b8[i] = o > b8[i] ? o : b8[i];
                }
            }
            __syncthreads();
            if (lane == 0) {
#pragma unroll
                for (int i = 0; i < 8; ++i) red[w][i] = b8[i];
            }
            __syncthreads();
            if (tid < 8 && m0 + tid < M) {
                unsigned long long b = red[0][tid];
#pragma unroll
                for (int q = 1; q < kWavesPerWG; ++q) b = red[q][tid] > b ? red[q][tid] : b;
                L.argmax[m0 + tid] = (int32_t)(0xffffffffu - (uint32_t)(b & 0xffffffffull));
            }
        }
        if (tid == 0) __hip_atomic_store(L.done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
        auto store = [&](int m, int n, float v) {
            if (L.y_bf16)
                ((uint16_t *)P.y)[(int64_t)m * P.ldy + n] = f2bf16(v);
            else
                ((float *)P.y)[(int64_t)m * P.ldy + n] = v;
        };
        if (S == 1) {
            if (!active) return;
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
        // split K: publish this split's partial sums; the last arrival adds all splits in order
        const int64_t plane = (int64_t)M * N;
        if (active) {
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int m = 16 * mt + 4 * j + r, n = n0 + 16 * t + c;
                        if (m < M && n < N) store_agent(P.partial + split * plane + (int64_t)m * N + n, y[t][mt][r]);
                    }
        }
        wait_vm_stores();
        __syncthreads();
        if (tid == 0)
            s_last = __hip_atomic_fetch_add(&P.counters[cg], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                     (uint32_t)S - 1;
        __syncthreads();
        if (!s_last) return;
        if (active) {
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int m = 16 * mt + 4 * j + r, n = n0 + 16 * t + c;
                        if (m < M && n < N) {
                            const float *p = P.partial + (int64_t)m * N + n;
                            float v = load_agent(p);
                            for (int s2 = 1; s2 < S; ++s2) v += load_agent(p + s2 * plane);
                            store(m, n, v);
                        }
                    }
        }
        if (tid == 0) __hip_atomic_store(&P.counters[cg], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

template <int BITS, bool ARGMAX>
hipError_t launch_bits(const GemmLaunch &L, int grid, hipStream_t s) {
    if (L.m <= 16)
        hipLaunchKernelGGL((qgemm_kernel<BITS, 1, 3, ARGMAX>), dim3(grid), dim3(256), 0, s, L);
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

// Work split.  A weight with few columns is split along K so that about
// kTargetWaves waves stream it, each over at least kMinSplitGroups groups
// (multiples of 8 groups keep the scale/bias rows 16-byte aligned).
#ifndef DSPK_TARGET_WAVES
#define DSPK_TARGET_WAVES 2048
#endif
#ifndef DSPK_MIN_SPLIT_GROUPS
#define DSPK_MIN_SPLIT_GROUPS 16
#endif
constexpr int kTargetWaves = DSPK_TARGET_WAVES;
constexpr int kMinSplitGroups = DSPK_MIN_SPLIT_GROUPS;

GemmPlan plan_gemm(int32_t n, int32_t k, int32_t m, bool single_split) {
    GemmPlan p{};
    const int G = k / 64;
    p.ncg = (n + kWGCols - 1) / kWGCols;
    const int wave_cols = (n + kBlockCols - 1) / kBlockCols;
    int splits = 1;
    if (!single_split) {
        splits = (kTargetWaves + wave_cols - 1) / wave_cols;
        splits = max(1, min(splits, G / kMinSplitGroups));
    }
    int sg = (G + splits - 1) / splits;
    if (splits > 1) sg = (sg + 7) / 8 * 8;
    p.split_groups = sg;
    p.splits = (G + sg - 1) / sg;
    p.ws_bytes = 0;
    if (p.splits > 1) {
        const size_t ctr = ((size_t)p.ncg * 4 + 255) / 256 * 256;
        p.ws_bytes = ctr + ((size_t)p.splits * m * n * 4 + 255) / 256 * 256;
    }
    return p;
}

size_t lmhead_workspace_bytes(int32_t v) {
    const size_t nwg = ((size_t)v + kWGCols - 1) / kWGCols;
    return 256 + nwg * kMaxRows * 8;
}

hipError_t launch_qgemm(const GemmLaunch &L, int bits, int grid, hipStream_t s) {
    return launch_any<false>(L, bits, grid, s);
}

hipError_t launch_lmhead(const GemmLaunch &L, int bits, int grid, hipStream_t s) {
    return launch_any<true>(L, bits, grid, s);
}

}  // namespace dspk

// Conversion of a weight from its interchange layout (packed codes and
// row-major fp16 scales/biases per 64-wide K group) into the tiled layout the
// projection kernels stream.  Run once per weight, when it is loaded; codes
// keep their values (3-bit codes are split into a 2-bit and a 1-bit plane)
// and fp16 bit patterns are copied unchanged.
//
// Interchange codes: each row one LSB-first bit stream in uint32 words, code
// r at stream bits bits*r .. bits*r + bits-1 (32/bits codes per word for 2,
// 4 and 8 bits; 3-bit codes may straddle words).
//
// Tiled layout, for a weight of n columns (output features) and k inputs:
//   KU = 128 (8-bit), 256 (2/3/4-bit), 64 (bf16) K elements per unit;
//   S = 8 code slots per unit (4 for 2-bit, 6 for 3-bit);
//   NST = ceil(k / KU) units per 64-column block, NB = ceil(n / 64) blocks;
//   unit (b, u) starts at byte ((b * NST) + u) * UNIT, UNIT = 1024 S + 256 KU/64
//   for quantised formats and 8192 for bf16.
// Inside a unit, slot i (0..S-1) is 1 KiB: 16 bytes for each lane l = c + 16 j
// (c = l % 16, j = l / 16) of a wave, holding for column n = 64 b + 16 t + c
// the codes of K = KU u + 64 g + 16 j + e, e = 0..15 ("the lane's 16 codes of
// group g"):
//   8-bit : i = 4 g + t, one byte per code;
//   4-bit : i = 4 p + t, 8 bytes for group 2p then 8 for group 2p+1 (nibble e
//           of the 8 bytes = code e);
//   2-bit : i = t, dword g = the 16 codes, code e in bits 2e..2e+1;
//   3-bit : i = t, dword g = the low two bits of the 16 codes, code e's in bits
//           2e..2e+1; i = 4 + t/2, dword 2 (t % 2) + p = the high bits of
//           groups 2p (A) and 2p+1 (B): bit e of A's codes 0..7 at bit e, of
//           B's at 8 + e, A's codes 8..15 at 16 + e - 8, B's at 24 + e - 8;
//   bf16  : i = 4 h + t, the 8 weights of K = KU u + 16 j + 8 h + 0..7.
// Quantised formats then hold, at byte 1024 S + 16 * KU/64 * c + 16 g + 4 t,
// the dword (scale | bias << 16) of group KU/64 * u + g of column
// 64 b + 16 t + c.  Columns past n and K past k hold zeros (code 0, scale 0,
// bias 0).
#include <hip/hip_runtime.h>

#include "dspk_internal.h"

namespace dspk {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// The lane's 16 codes of group g (K = k0 .. k0 + 15, k0 a multiple of 16) of
// row col, as an integer of 16 * BITS bits; zero past the weight.
template <int BITS>
__device__ inline unsigned long long lane_codes(const unsigned char *codes, size_t rowbytes, int n, int k, int col,
                                                int k0) {
    if (col >= n || k0 >= k) return 0ull;
    const unsigned char *p = codes + (size_t)col * rowbytes + (size_t)k0 * BITS / 8;   // byte aligned: 16 * BITS bits
    unsigned long long v = 0;
#pragma unroll
    for (int i = 0; i < 2 * BITS; ++i) v |= (unsigned long long)p[i] << (8 * i);
    return v;
}

// One workgroup of 64 threads per unit.
template <int BITS>
__global__ __launch_bounds__(64) void pack_kernel(int32_t n, int32_t k, const unsigned char *__restrict__ codes,
                                                  const uint16_t *__restrict__ scales,
                                                  const uint16_t *__restrict__ biases, unsigned char *__restrict__ tiles,
                                                  int32_t nst) {
    constexpr int KU = tile_k(BITS), GS = tile_groups(BITS), UNIT = tile_unit_bytes(BITS);
    constexpr int S = tile_code_slots(BITS);
    const int lane = threadIdx.x, c = lane & 15, j = lane >> 4;
    const int b = blockIdx.x / nst, u = blockIdx.x % nst;
    const size_t rowbytes = (size_t)k * BITS / 8;
    unsigned char *dst = tiles + (size_t)blockIdx.x * UNIT;
    if constexpr (BITS == 2 || BITS == 3) {
        // low planes (2-bit: the codes) of tile t in slot t; 3-bit high planes
        // of tiles 2s', 2s'+1 in slot 4 + s'
        uint32_t hi[4][2] = {};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int col = 64 * b + 16 * t + c;
            u32x4 v;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const unsigned long long q = lane_codes<BITS>(codes, rowbytes, n, k, col, KU * u + 64 * g + 16 * j);
                uint32_t lo = 0, h = 0;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const uint32_t code = (uint32_t)(q >> (BITS * e)) & ((1u << BITS) - 1u);
                    lo |= (code & 3u) << (2 * e);
                    h |= (code >> 2) << e;
                }
                v[g] = lo;
                if (BITS == 3) {
                    // group g = 2p + r: its codes 0..7 at bits 8r + e, 8..15 at 16 + 8r + e - 8
                    const int p = g >> 1, r = g & 1;
                    hi[t][p] |= ((h & 0xffu) << (8 * r)) | ((h >> 8) << (16 + 8 * r));
                }
            }
            *(u32x4 *)(dst + 1024 * t + 16 * lane) = v;
        }
        if (BITS == 3) {
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                const u32x4 v = {hi[2 * s2][0], hi[2 * s2][1], hi[2 * s2 + 1][0], hi[2 * s2 + 1][1]};
                *(u32x4 *)(dst + 1024 * (4 + s2) + 16 * lane) = v;
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int t = i & 3, hi = i >> 2;
            const int col = 64 * b + 16 * t + c;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (BITS == 8) {
                const int k0 = KU * u + 64 * hi + 16 * j;
                if (col < n && k0 < k) v = *(const u32x4 *)(codes + col * rowbytes + k0);
            } else if (BITS == 4) {
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const int k0 = KU * u + 64 * (2 * hi + half) + 16 * j;
                    if (col < n && k0 < k) {
                        const u32x2 p = *(const u32x2 *)(codes + col * rowbytes + k0 / 2);
                        v[2 * half] = p[0];
                        v[2 * half + 1] = p[1];
                    }
                }
            } else {
                const int k0 = KU * u + 16 * j + 8 * hi;
                if (col < n && k0 < k) v = *(const u32x4 *)(codes + col * rowbytes + 2 * k0);
            }
            *(u32x4 *)(dst + 1024 * i + 16 * lane) = v;
        }
    }
    if (BITS != 16 && j == 0) {
        const int groups = k / 64;
        uint32_t *sb = (uint32_t *)(dst + 1024 * S + 16 * GS * c);
#pragma unroll
        for (int g = 0; g < GS; ++g)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int col = 64 * b + 16 * t + c;
                const int gk = GS * u + g;
                uint32_t d = 0u;
                if (col < n && gk < groups)
                    d = (uint32_t)scales[(size_t)col * groups + gk] |
                        ((uint32_t)biases[(size_t)col * groups + gk] << 16);
                sb[4 * g + t] = d;
            }
    }
}

}  // namespace

hipError_t launch_pack(int32_t n, int32_t k, int bits, const void *codes, const uint16_t *scales,
                       const uint16_t *biases, void *tiles, hipStream_t s) {
    const int nst = (k + tile_k(bits) - 1) / tile_k(bits);
    const int64_t units = ((int64_t)n + 63) / 64 * nst;
    if (units > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid((unsigned)units), block(64);
    const unsigned char *cb = (const unsigned char *)codes;
    unsigned char *tb = (unsigned char *)tiles;
    switch (bits) {
        case 2: hipLaunchKernelGGL(pack_kernel<2>, grid, block, 0, s, n, k, cb, scales, biases, tb, nst); break;
        case 3: hipLaunchKernelGGL(pack_kernel<3>, grid, block, 0, s, n, k, cb, scales, biases, tb, nst); break;
        case 4: hipLaunchKernelGGL(pack_kernel<4>, grid, block, 0, s, n, k, cb, scales, biases, tb, nst); break;
        case 8: hipLaunchKernelGGL(pack_kernel<8>, grid, block, 0, s, n, k, cb, scales, biases, tb, nst); break;
        case 16: hipLaunchKernelGGL(pack_kernel<16>, grid, block, 0, s, n, k, cb, scales, biases, tb, nst); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace dspk

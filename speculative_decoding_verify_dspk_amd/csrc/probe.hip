// Streaming-read probe (measurement only, not part of the verify pass): how
// fast this device streams a large buffer from HBM with the access pattern the
// projection kernels use -- each wave reads consecutive 1 KiB pieces (16 bytes
// per lane, non-temporal), several in flight, each workgroup one contiguous
// range of the buffer.  The benchmark reports it next to the published HBM
// peak as the "achievable" bandwidth.  Built into its own library
// (libdspk_probe.so) by the package's build script.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kInFlight = 8;     // 1 KiB pieces in flight per wave

// Workgroup b reads pieces [b * n / grid, (b + 1) * n / grid) of the n
// pieces; wave w of the workgroup takes every fourth group of kInFlight
// consecutive pieces.  The XOR of everything read goes to sink[b], so no load
// is dead.
__global__ __launch_bounds__(256) void stream_read_kernel(const unsigned char *__restrict__ buf, int64_t pieces,
                                                          uint32_t *__restrict__ sink) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t b = blockIdx.x, g = gridDim.x;
    const int64_t p0 = b * pieces / g, p1 = (b + 1) * pieces / g;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int64_t p = p0 + (int64_t)w * kInFlight; p < p1; p += 4 * kInFlight) {
        u32x4 v[kInFlight];
#pragma unroll
        for (int i = 0; i < kInFlight; ++i) {
            const int64_t q = p + i < p1 ? p + i : p1 - 1;     // stay inside the range
            v[i] = __builtin_nontemporal_load((const u32x4 *)(buf + q * 1024 + 16 * lane));
        }
#pragma unroll
        for (int i = 0; i < kInFlight; ++i) acc ^= v[i];
    }
    uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    for (int off = 32; off > 0; off >>= 1) x ^= __shfl_xor(x, off);
    __shared__ uint32_t s[4];
    if (lane == 0) s[w] = x;
    __syncthreads();
    if (threadIdx.x == 0) sink[b] = s[0] ^ s[1] ^ s[2] ^ s[3];
}

}  // namespace

extern "C" {

// Enqueue one streaming read of `bytes` (a multiple of 1024) from device
// buffer `buf` on `stream`, with `grid` workgroups of 256 threads; sink is
// device memory of grid 32-bit words.  Returns 0, or -1 on bad arguments or a
// launch error.
int dspk_probe_stream_read(const void *buf, int64_t bytes, int32_t grid, void *sink, void *stream) {
    if (buf == nullptr || sink == nullptr || bytes < 1024 || bytes % 1024 || grid < 1) return -1;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream,
                       (const unsigned char *)buf, bytes / 1024, (uint32_t *)sink);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // extern "C"

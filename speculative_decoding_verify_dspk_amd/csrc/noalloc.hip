// Workspace of the allocation-free projection entry point
// (dspk_qgemm_verify_grouped_noalloc): one file-scope device array per GPU,
// used in place of a caller-provided workspace, for callers that cannot
// allocate (code under HIP graph capture, tight serving loops).
//
// The array holds the same regions as a projection workspace (head words,
// partial sums of split blocks, arrival counters; see dspk_internal.h), sized
// for a device of up to kScratchCus CUs and launches of up to
// kScratchMaxBlocks 64-column blocks.  Its host-side name is only a handle:
// host code uses the device address that hipGetSymbolAddress returns for the
// current device, fetched once per device and kept.
#include <hip/hip_runtime.h>

#include <mutex>

#include "dspk_internal.h"

namespace dspk {
namespace {

constexpr size_t kScratchBytes =
    kWsHead + partial_region_bytes(kScratchCus) + ((kScratchMaxBlocks * kWavesPerWG * 4 + 255) / 256) * 256;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Zero the words that must start at zero (head words and counters); the
// partial sums are always written before they are read.  A kernel rather than
// a memset, so that it may also be recorded into a captured graph.
__global__ void clear_words(uint32_t *head, size_t head_words, uint32_t *ctr, size_t ctr_words) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < head_words) head[i] = 0u;
    if (i < ctr_words) ctr[i] = 0u;
}

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_ptr[kMaxDevices] = {};

}  // namespace

size_t static_scratch_bytes() { return kScratchBytes; }

hipError_t static_scratch(void **ptr, hipStream_t s) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_ptr[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        // once per device: clear the head words and the counter region
        const size_t head_words = kWsHead / 4;
        const size_t ctr_off = kWsHead + partial_region_bytes(device_cus());   // the plans' counter offset
        if (ctr_off >= kScratchBytes) return hipErrorInvalidValue;
        const size_t ctr_words = (kScratchBytes - ctr_off) / 4;
        const size_t n = head_words > ctr_words ? head_words : ctr_words;
        hipLaunchKernelGGL(clear_words, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, (uint32_t *)p,
                           head_words, (uint32_t *)((char *)p + ctr_off), ctr_words);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        g_ptr[dev] = p;
    }
    *ptr = g_ptr[dev];
    return hipSuccess;
}

}  // namespace dspk

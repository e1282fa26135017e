// Workspace layout of the sampling kernels (host and device): byte offsets of
// each region for m_rows rows over a vocabulary of v entries.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "dspk_internal.h"

namespace dspk {

constexpr int kSampleSlice = 8192;   // entries per workgroup of the binning pass (<= 2^13)
constexpr int kSampleBins = 2048;    // histogram bins per level
constexpr int kSampleSeg = 256;      // columns per segment of the drawing row's masses

struct SampleWsLayout {
    size_t stats, flags, qmax, mass, trunc, pcnt, pmass, bin1, total;
    int nslices, vpad;
};

constexpr size_t sample_align256(size_t x) { return (x + 255) / 256 * 256; }

// [0, 256) arrival counter; then per (row, chunk) {max, sum exp} (8 B), the
// fault flag (4 B) and the max of q (4 B); per 256-column segment the
// {residual, p} masses of the drawing row (8 B); per (row, distribution) the truncation record
// (16 B); and, used only when truncating, per (row, distribution, slice) the
// first-level histograms (NB x u32 counts, NB x u64 masses) and per (row,
// distribution) the first-level bin of every entry (u16).
constexpr SampleWsLayout sample_ws_layout(int rows, int v) {
    const size_t nchunks = (size_t)(v + kSampleChunk - 1) / kSampleChunk;
    SampleWsLayout L{};
    L.nslices = (v + kSampleSlice - 1) / kSampleSlice;
    L.vpad = (v + 127) / 128 * 128;
    const size_t nh = (size_t)rows * 2 * L.nslices * kSampleBins;
    size_t o = 256;
    L.stats = o;
    o += sample_align256(rows * nchunks * 8);
    L.flags = o;
    o += sample_align256(rows * nchunks * 4);
    L.qmax = o;
    o += sample_align256(rows * nchunks * 4);
    L.mass = o;
    o += sample_align256(nchunks * (kSampleChunk / kSampleSeg) * 8);
    L.trunc = o;
    o += sample_align256((size_t)rows * 2 * 16);
    L.pcnt = o;
    o += sample_align256(nh * 4);
    L.pmass = o;
    o += sample_align256(nh * 8);
    L.bin1 = o;
    o += sample_align256((size_t)rows * 2 * L.vpad * 2);
    L.total = o;
    return L;
}

}  // namespace dspk

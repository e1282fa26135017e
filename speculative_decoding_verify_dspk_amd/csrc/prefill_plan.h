// Host-side choice of the prefill kernel's row block (declared apart from
// the verify kernels' shared header so that neither depends on it).
#pragma once

#include <stdint.h>

namespace dspk {

// Rows per prefill workgroup, 64 or 128, for m rows, nblocks 64-column
// blocks and a weight format of `bits` on a device of `cus` CUs (planning
// only; both blocks give identical results).
int prefill_block_rows(int32_t m, int32_t nblocks, int bits, int cus);
// The block for a launch: the override below, else prefill_block_rows on the
// current device.
int prefill_rows_for(int32_t m, int32_t nblocks, int bits);
// Process-wide override: 0 automatic, 64 or 128 forced.  Returns the previous
// setting, or -1 for another value.
int set_prefill_block_rows(int rows);

// K splits of a launch of `wgs` workgroups over nst units of K, on a device
// of `cus` CUs holding `occ` workgroups each (planning only).
int prefill_splits(int64_t wgs, int32_t nst, int occ, int cus);

// The whole plan of one prefill call: rows per workgroup, K splits (1 unless
// a workspace may be used) and the workspace it needs (0 for one split):
// arrival counters at offset 0, partial tiles at off_part.
struct PrefillPlan {
    int rows, ks;
    size_t off_part, ws_bytes;
};
PrefillPlan prefill_plan(int32_t m, int32_t nblocks, int32_t nst, int bits, bool may_split);

}  // namespace dspk

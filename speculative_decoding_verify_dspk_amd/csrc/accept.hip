// Acceptance of a verify block on gfx950: greedy longest-prefix match and
// Leviathan/Chen speculative sampling ("mlx-dspark" wiki summary,
// "Architecture"; "mlx-dspark 0.7.0", "How it works").
#include <math.h>

#include <hip/hip_runtime.h>

#include "dspk_internal.h"
#include "sample_layout.h"

namespace dspk {
namespace {

// ---------------------------------------------------------------- greedy
// One thread per request: drafts are accepted while they equal the target's
// token of the same row; the target's token of the first mismatching row (or
// of the last row) is always committed, so 1 .. M tokens are committed.
__global__ void accept_greedy_kernel(const int32_t *__restrict__ t, const int32_t *__restrict__ d,
                                     int32_t b, int32_t M, int32_t *__restrict__ accept_len,
                                     int32_t *__restrict__ committed) {
    const int r = blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= b) return;
    const int32_t *tr = t + (int64_t)r * M;
    const int32_t *dr = d + (int64_t)r * (M - 1);
    int32_t *cr = committed + (int64_t)r * M;
    int a = 0;
    while (a < M - 1 && dr[a] == tr[a]) {
        cr[a] = dr[a];
        ++a;
    }
    cr[a] = tr[a];
    for (int i = a + 1; i < M; ++i) cr[i] = -1;
    accept_len[r] = a + 1;
}

// -------------------------------------------------------------- sampling
// Workspace: see sample_layout.h.
constexpr int CH = kSampleChunk;
constexpr int TPB = 256;
constexpr int EPT = CH / TPB;    // logits per thread per chunk
constexpr int FT = 1024;         // threads of a truncation workgroup
constexpr int NB = kSampleBins;  // histogram bins per level
constexpr int SLICE = kSampleSlice;
constexpr int BT = 512;          // threads of a binning workgroup
static_assert(SLICE <= 8192, "the binning histogram's 32-bit mass halves hold 2^13 entries");

struct Trunc {
    unsigned long long key;      // kept iff order key >= key
    float mass;                  // kept mass (of p, or of q as supplied)
    int32_t pad;
};
static_assert(sizeof(Trunc) == 16, "truncation record size is fixed by the workspace layout");

struct SampleWs {
    uint32_t *counter;
    float2 *stats;   // [rows][nchunks]
    int32_t *flags;  // [rows][nchunks]
    float *qmax;     // [rows][nchunks] (draft rows)
    float2 *mass;    // [nchunks][chunk / kSampleSeg]: per segment of the drawing row
    Trunc *trunc;    // [rows][2]: target p, draft q
    uint32_t *pcnt;            // [rows][2][nslices][NB]
    unsigned long long *pmass; // [rows][2][nslices][NB]
    uint16_t *bin1;            // [rows][2][vpad]
    int nslices, vpad;
};

__device__ inline SampleWs carve(void *ws, int rows, int v) {
    const SampleWsLayout L = sample_ws_layout(rows, v);
    char *p = (char *)ws;
    SampleWs s;
    s.counter = (uint32_t *)p;
    s.stats = (float2 *)(p + L.stats);
    s.flags = (int32_t *)(p + L.flags);
    s.qmax = (float *)(p + L.qmax);
    s.mass = (float2 *)(p + L.mass);
    s.trunc = (Trunc *)(p + L.trunc);
    s.pcnt = (uint32_t *)(p + L.pcnt);
    s.pmass = (unsigned long long *)(p + L.pmass);
    s.bin1 = (uint16_t *)(p + L.bin1);
    s.nslices = L.nslices;
    s.vpad = L.vpad;
    return s;
}

// Everything the sampling kernels read (kernel argument, by value).
struct SampleArgs {
    const float *z;
    int64_t ldz;
    const float *q;
    int64_t ldq;
    const int32_t *d;
    const float *u;
    int32_t rows, v;
    float inv_t;                 // 1 / temperature
    int32_t top_k;               // 0: off
    float top_p;                 // 1: off
    float presence, frequency;   // penalties
    const int32_t *counts;       // history token counts [v], or NULL
    int32_t pen;                 // any penalty applies
    int32_t trunc;               // top-k or top-p applies
    bool vec_z, vec_q;           // rows of z / q start on 16-byte boundaries
    int32_t *accept_len, *committed;
    void *ws;
};

// Penalised, temperature-scaled logit of column col in row j ("mlx-dspark
// releases", v0.2.0 notes: OpenAI presence/frequency penalties on the target
// logits; the committed tokens are those one-token decoding of the penalised
// target would give).  Row j is reached only when drafts 0..j-1 were accepted,
// so its counts include them; drafts are in LDS (s_d).  bloom (or NULL): a 1024-bit
// filter of the columns of drafts 0..j-1 -- a clear bit means none of them
// is col, and the scan over the drafts is skipped.
// hist: counts[col] (0 without counts), loaded by the caller.
__device__ inline float scaled_logit_h(const SampleArgs &A, const int32_t *s_d, const uint32_t *bloom, int j,
                                       int col, float zz, int hist) {
    if (A.pen) {
        int c = hist;
        const uint32_t h = (uint32_t)col & 1023u;
        if (bloom == nullptr || ((bloom[h >> 5] >> (h & 31u)) & 1u))
            for (int i = 0; i < j; ++i) c += s_d[i] == col;
        zz = zz - A.presence * (c > 0 ? 1.f : 0.f) - A.frequency * (float)c;
    }
    return zz * A.inv_t;
}

__device__ inline float scaled_logit(const SampleArgs &A, const int32_t *s_d, const uint32_t *bloom, int j, int col,
                                     float zz) {
    return scaled_logit_h(A, s_d, bloom, j, col, zz, A.pen && A.counts != nullptr ? A.counts[col] : 0);
}

// Fill the filter of drafts 0..j-1 (bloom: 32 words of LDS; s_d already
// loaded); ends with a barrier.
__device__ inline void build_bloom(uint32_t *bloom, const int32_t *s_d, int j) {
    if (threadIdx.x < 32) bloom[threadIdx.x] = 0u;
    __syncthreads();
    if ((int)threadIdx.x < j) {
        const uint32_t h = (uint32_t)s_d[threadIdx.x] & 1023u;
        atomicOr(&bloom[h >> 5], 1u << (h & 31u));
    }
    __syncthreads();
}

// Order key of an entry: larger value first, then the smaller column; unique.
// -0 and +0 are one value.
__device__ inline unsigned long long order_key(float x, int col) {
    uint32_t b = __float_as_uint(x + 0.0f);
    b = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    return ((unsigned long long)b << 32) | (unsigned long long)(0xffffffffu - (uint32_t)col);
}

// Values one workgroup hands to another inside a kernel move through
// device-scope atomic accesses: they are performed where all XCDs see them,
// so no cache writeback or invalidation (a device-scope fence) is needed;
// the writer waits for its stores to complete before it signals arrival.
__device__ inline void store_f2(float2 *p, float2 v) {
    __hip_atomic_store((unsigned long long *)p, __builtin_bit_cast(unsigned long long, v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline float2 load_f2(const float2 *p) {
    return __builtin_bit_cast(float2, __hip_atomic_load((unsigned long long *)p, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT));
}

// Row maximum and normaliser of z'/T from the chunk statistics, eight threads
// per row (k = tid % 8 takes chunks k, k + 8, ...), then a fixed butterfly.
__device__ inline float2 row_stats8(const float2 *st, int nchunks, int k) {
    constexpr int R = 8;     // chunks per thread fetched together (all of them up to 64 chunks)
    float2 a[R];
#pragma unroll
    for (int r = 0; r < R; ++r) a[r] = k + 8 * r < nchunks ? st[k + 8 * r] : make_float2(-INFINITY, 0.f);
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < R; ++r) mx = fmaxf(mx, a[r].x);
    for (int cc = k + 8 * R; cc < nchunks; cc += 8) mx = fmaxf(mx, st[cc].x);
    for (int off = 1; off < 8; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    float sm = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r)
        if (k + 8 * r < nchunks) sm += a[r].y * expf(a[r].x - mx);
    for (int cc = k + 8 * R; cc < nchunks; cc += 8) sm += st[cc].y * expf(st[cc].x - mx);
    for (int off = 1; off < 8; off <<= 1) sm += __shfl_xor(sm, off);
    return make_float2(mx, sm);
}

// Four consecutive entries of a row from col on, entries at or past v1
// reading as `fill`: one 16-byte load when `full` (in range and 16-byte
// aligned), else four loads clamped into the row (never a branch per entry,
// so every load of a batch is in flight at once).
__device__ inline float4 load4(const float *row, int col, int v1, bool full, float fill) {
    if (full) return *(const float4 *)(row + col);
    const int last = v1 - 1;
    const float a = row[min(col, last)], b = row[min(col + 1, last)];
    const float c = row[min(col + 2, last)], d = row[min(col + 3, last)];
    return make_float4(col < v1 ? a : fill, col + 1 < v1 ? b : fill, col + 2 < v1 ? c : fill, col + 3 < v1 ? d : fill);
}
__device__ inline float f4(const float4 &a, int e) { return e == 0 ? a.x : e == 1 ? a.y : e == 2 ? a.z : a.w; }

__device__ inline float wave_max(float v) {
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    return v;
}
__device__ inline float wave_sum(float v) {
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

// A chunk is read as G4 steps of TPB float4 groups: thread tid's group i holds
// columns v0 + 4 (tid + TPB i) .. + 3, so wave w's step i covers the SEG
// columns of segment NW i + w of the chunk.
constexpr int G4 = EPT / 4;
constexpr int NW = TPB / 64;
constexpr int SEG = kSampleSeg;
constexpr int NSEG = CH / SEG;
static_assert(EPT % 4 == 0 && SEG == 4 * 64 && NSEG == NW * G4, "chunk, segment and thread layout disagree");
static_assert(kMaxRows <= 64, "the accept tests and the final writes take one lane of wave 0 per row");

// This thread's NG groups of four of a chunk [v0, v1) of a row, for NT
// threads (group i of thread t: columns v0 + 4 (t + NT i) .. + 3; entries past
// v1 read as 0).  One branch for the whole chunk -- 16-byte loads when the
// chunk is full and the row 16-byte aligned, else clamped loads -- so that
// all of them are in flight together.
template <int NT, int NG>
__device__ inline void load_chunk(float4 (&out)[NG], const float *row, int v0, int v1, bool vec) {
    const int t = threadIdx.x;
    if (vec && v0 + CH <= v1) {
#pragma unroll
        for (int i = 0; i < NG; ++i) out[i] = *(const float4 *)(row + v0 + 4 * (t + NT * i));
    } else {
#pragma unroll
        for (int i = 0; i < NG; ++i) out[i] = load4(row, v0 + 4 * (t + NT * i), v1, false, 0.f);
    }
}

// The decide kernel runs 1024 threads per chunk: one group of four per
// thread, so wave w covers exactly segment w of the chunk.
constexpr int DT = 1024;
constexpr int DW = DT / 64;
constexpr int DG = CH / (4 * DT);
static_assert(DG == 1 && DW == NSEG, "decide layout: one wave per segment");

// Pass 1: per (row, chunk) max and sum of exp of z'/T, and the fault flag
// (non-finite logit; non-finite or negative q on draft rows; negative count).
// Every load of the chunk is issued before any of them is used.
__global__ __launch_bounds__(TPB) void sample_stats_kernel(const SampleArgs A) {
    __shared__ float s_mx[NW], s_qm[NW], s_sm[NW];
    __shared__ int s_bad[NW];
    __shared__ int32_t s_d[kMaxRows];
    __shared__ uint32_t s_bloom[32];
    const int nchunks = (A.v + CH - 1) / CH;
    const SampleWs W = carve(A.ws, A.rows, A.v);
    const int c = blockIdx.x, j = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);     // wave-uniform (scalar branches)
    const int v0 = c * CH, v1 = min(A.v, v0 + CH);
    const bool draft = j < A.rows - 1;
    const float *zr = A.z + (int64_t)j * A.ldz;
    const float *qr = A.q + (int64_t)j * A.ldq;
    float4 zv[G4], qv[G4];
    load_chunk<TPB, G4>(zv, zr, v0, v1, A.vec_z);
    if (draft) load_chunk<TPB, G4>(qv, qr, v0, v1, A.vec_q);
    if (A.pen) {
        if (tid < A.rows - 1) s_d[tid] = A.d[tid];
        __syncthreads();
        build_bloom(s_bloom, s_d, j);
    }
    float a[G4][4];
    float mx = -INFINITY, qm = 0.f;
    int bad = 0;
#pragma unroll
    for (int i = 0; i < G4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int col = v0 + 4 * (tid + TPB * i) + e;
            a[i][e] = -INFINITY;
            if (col < v1) {
                const float zz = f4(zv[i], e);
                bad |= !isfinite(zz);
                if (A.counts != nullptr) bad |= A.counts[col] < 0;
                a[i][e] = scaled_logit(A, s_d, s_bloom, j, col, zz);
                mx = fmaxf(mx, a[i][e]);
                if (draft) {
                    const float qq = f4(qv[i], e);
                    bad |= !(isfinite(qq) && qq >= 0.f);
                    qm = fmaxf(qm, qq);
                }
            }
        }
    mx = wave_max(mx);
    qm = wave_max(qm);
    const int wbad = __any(bad);
    if (lane == 0) {
        s_mx[w] = mx;
        s_qm[w] = qm;
        s_bad[w] = wbad;
    }
    __syncthreads();
    float cmax = s_mx[0];
    for (int k = 1; k < NW; ++k) cmax = fmaxf(cmax, s_mx[k]);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < G4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (v0 + 4 * (tid + TPB * i) + e < v1) s += expf(a[i][e] - cmax);
    s = wave_sum(s);
    if (lane == 0) s_sm[w] = s;
    __syncthreads();
    if (tid == 0) {
        float csum = s_sm[0], cq = s_qm[0];
        int cb = s_bad[0];
        for (int k = 1; k < NW; ++k) {
            csum += s_sm[k];
            cq = fmaxf(cq, s_qm[k]);
            cb |= s_bad[k];
        }
        W.stats[j * nchunks + c] = make_float2(cmax, csum);
        W.flags[j * nchunks + c] = cb;
        if (A.trunc) W.qmax[j * nchunks + c] = cq;
    }
}

// Truncation of one distribution ("mlx-dspark releases", v0.1.0 notes: the
// same top-k / top-p filter cuts down the target and the draft).  Entries are
// ordered by value (larger first, then the smaller column): their order keys
// are unique 64-bit values, so each bound is one key.  Top-k keeps the first
// k; top-p then keeps an entry iff the kept mass before it is below top_p
// times the top-k mass.  Masses are counted in fixed point -- unit = the
// row's largest weight / 2^37 (fewer bits for v > 2^25, so that v weights fit
// 64 bits) -- as integers, so sums do not depend on thread timing; every
// weight is off by less than one unit (rounded down, but a positive weight
// counts at least one) and the kept mass is at least the largest weight, so a
// bound is off by at most v * 2^-37 of the kept mass.  A top-k bound that
// falls among entries of weight exactly zero keeps all of them instead: they
// carry no mass, so the truncated distribution is the same.
//
// Every entry has a fine index fi (22 bits) that never decreases along the
// key order, from float bits, so that any spread of values splits evenly in
// log scale: for p, the bits of t = max(z'/T) - z'/T, clamped to
// [2^-24, 2^40), in steps of 128 ulps (32 first-level bins per octave); for
// q, bits of max(q) - bits of q in steps of 512 ulps (8 per octave, the whole
// float range down to 0).
//
// Two kernels.  sample_bins_kernel (one workgroup per slice of SLICE entries
// of a (row, distribution), the whole GPU) evaluates every entry once, stores
// its first-level bin fi >> 11 and the slice's histogram (count and mass per
// bin).  sample_trunc_kernel (one workgroup per (row, distribution)) adds the
// slice histograms, finds the bin holding a bound with a wave-parallel scan,
// and, when it holds at most CAP entries, gathers them (found through the
// stored bins) into LDS, sorts them by key (bitonic) and takes the first at
// which the running count (top-k) or mass (top-p) reaches its target.  A bin
// of more entries is split by a second histogram over fi & 2047, and a
// second-level bin still too full (equal values) falls back to a 64-bit radix
// selection over the keys (11-bit digits).
constexpr int CAP = 4096;                      // entries sorted in LDS
constexpr uint32_t FI_MAX = (1u << 22) - 1;
constexpr uint32_t kTLo = 103u << 23;          // float bits of 2^-24
constexpr uint32_t kTHi = (167u << 23) - 1u;   // just below 2^40

// What an entry's evaluation needs of its row.
struct RowCtx {
    float rmax;                  // p: max of z'/T
    float wmax, inv_wmax;        // the row's largest weight (p: 1 / sum exp(z'/T - rmax))
    uint32_t wbits;              // its bits
    int fx;                      // fixed point: weight / wmax in units of 2^-fx (fx <= 37)
};

// Row context of (row j, distribution dist); all threads call it (barriers).
__device__ inline RowCtx row_ctx(const SampleArgs &A, const SampleWs &W, int j, int dist, float2 *s_rs) {
    const int nchunks = (A.v + CH - 1) / CH;
    const int tid = threadIdx.x;
    if (dist == 0) {
        if (tid < 8) {
            const float2 rs = row_stats8(W.stats + (int64_t)j * nchunks, nchunks, tid);
            if (tid == 0) *s_rs = rs;
        }
    } else if (tid < 64) {
        float mx = 0.f;
        for (int cc = tid; cc < nchunks; cc += 64) mx = fmaxf(mx, W.qmax[j * nchunks + cc]);
        for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
        if (tid == 0) *s_rs = make_float2(mx, 0.f);
    }
    __syncthreads();
    RowCtx r;
    const float2 rs = *s_rs;
    r.rmax = rs.x;
    // largest weight: 1 / sum for p (its largest entry has x = rmax)
    r.wmax = dist == 0 ? 1.f / rs.y : rs.x;
    r.inv_wmax = r.wmax > 0.f ? 1.f / r.wmax : 0.f;
    r.wbits = __float_as_uint(r.wmax) & 0x7fffffffu;
    int lg = 0;
    while ((1 << lg) < A.v) ++lg;
    r.fx = min(37, 62 - lg);
    return r;
}

// Key, fine index and fixed-point weight of column col.
// raw: z[j][col] (p) or q[j][col]; hist: counts[col] (p with penalties and
// counts; else unused).
__device__ inline void trunc_entry_raw(const SampleArgs &A, const RowCtx &R, int dist, int j, int col, float raw,
                                       int hist, const int32_t *s_d, const uint32_t *bloom,
                                       unsigned long long &key, uint32_t &fi, unsigned long long &mfx) {
    float x, y;     // y: weight / wmax, in [0, 1]
    if (dist == 0) {
        x = scaled_logit_h(A, s_d, bloom, j, col, raw, hist);
        y = expf(x - R.rmax);
        const uint32_t tb = __float_as_uint(R.rmax - x);
        fi = tb >= 0x80000000u ? 0u : (min(max(tb, kTLo), kTHi) - kTLo) >> 7;
    } else {
        x = raw;
        y = fminf(x * R.inv_wmax, 1.f);
        const uint32_t b = __float_as_uint(x) & 0x7fffffffu;
        fi = b >= R.wbits ? 0u : (R.wbits - b) >> 9;
    }
    fi = min(fi, FI_MAX);
    key = order_key(x, col);
    // floor(y * 2^fx) from the float's fields (exact: y * 2^fx <= 2^37); a
    // positive weight counts at least one unit, so a bin's mass is zero only
    // when all its weights are
    const uint32_t yb = __float_as_uint(y);
    const int e = (int)((yb >> 23) & 0xffu) - 127 + R.fx;      // exponent of y * 2^fx
    const unsigned long long mant = (unsigned long long)((yb & 0x7fffffu) | 0x800000u);
    const unsigned long long u = e < 0 ? 0ull : (e >= 23 ? mant << (e - 23) : mant >> (23 - e));
    mfx = (y > 0.f && u == 0ull) ? 1ull : (y > 0.f ? u : 0ull);
}

// Add (1, mfx) to bin b of (cnt, mass) for the lanes with take set.  When
// every taking lane of the wave has the same bin (crowded bins: equal or
// nearly equal values, runs of columns), one lane adds the wave's sums: LDS
// atomics to one address from many lanes would be serialised.  The whole
// wave calls it.
__device__ inline void hist_add(uint32_t *cnt, unsigned long long *mass, bool take, int b, unsigned long long mfx) {
    const unsigned long long act = __ballot(take);
    if (act == 0ull) return;
    const int lane = threadIdx.x & 63;
    const int lead = __ffsll((long long)act) - 1;
    const int b0 = __builtin_amdgcn_readlane(b, lead);
    const unsigned long long same = __ballot(take && b == b0);
    if (same == act) {
        unsigned long long ms = take ? mfx : 0ull;
        for (int off = 32; off > 0; off >>= 1) ms += __shfl_xor(ms, off);
        if (lane == lead) {
            atomicAdd(&cnt[b0], (uint32_t)__popcll(act));
            atomicAdd(&mass[b0], ms);
        }
    } else if (take) {
        atomicAdd(&cnt[b], 1u);
        atomicAdd(&mass[b], mfx);
    }
}

// hist_add with the mass in two halves (low 19 bits, the rest) on 32-bit
// counters (64-bit LDS atomics are much slower): with mfx <= 2^37 and at most
// SLICE = 2^13 entries per histogram, neither half's sum reaches 2^32.
__device__ inline void hist_add_split(uint32_t *cnt, uint32_t *lo, uint32_t *hi, bool take, int b,
                                      unsigned long long mfx) {
    const unsigned long long act = __ballot(take);
    if (act == 0ull) return;
    const int lane = threadIdx.x & 63;
    const int lead = __ffsll((long long)act) - 1;
    const int b0 = __builtin_amdgcn_readlane(b, lead);
    const unsigned long long same = __ballot(take && b == b0);
    uint32_t l = take ? (uint32_t)(mfx & 0x7ffffu) : 0u, h = take ? (uint32_t)(mfx >> 19) : 0u;
    if (same == act) {
        for (int off = 32; off > 0; off >>= 1) {
            l += __shfl_xor(l, off);
            h += __shfl_xor(h, off);
        }
        if (lane == lead) {
            atomicAdd(&cnt[b0], (uint32_t)__popcll(act));
            atomicAdd(&lo[b0], l);
            atomicAdd(&hi[b0], h);
        }
    } else if (take) {
        atomicAdd(&cnt[b], 1u);
        if (l != 0u) atomicAdd(&lo[b], l);
        if (h != 0u) atomicAdd(&hi[b], h);
    }
}

__device__ inline unsigned long long wave_incl_scan(unsigned long long x, int lane) {
    for (int off = 1; off < 64; off <<= 1) {
        const unsigned long long y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    return x;
}

// Binning pass: grid (nslices, rows, 2).
__global__ __launch_bounds__(BT) void sample_bins_kernel(const SampleArgs A) {
    __shared__ uint32_t h_cnt[NB];
    __shared__ uint32_t h_lo[NB], h_hi[NB];   // mass = hi * 2^19 + lo
    __shared__ int32_t s_d[kMaxRows];
    __shared__ uint32_t s_bloom[32];
    __shared__ float2 s_rs;
    const int sl = blockIdx.x, j = blockIdx.y, dist = blockIdx.z, tid = threadIdx.x;
    if (dist == 1 && j >= A.rows - 1) return;
    const SampleWs W = carve(A.ws, A.rows, A.v);
    if (tid < A.rows - 1) s_d[tid] = A.d[tid];
    for (int b = tid; b < NB; b += BT) {
        h_cnt[b] = 0u;
        h_lo[b] = 0u;
        h_hi[b] = 0u;
    }
    __syncthreads();
    build_bloom(s_bloom, s_d, dist == 0 ? j : 0);
    const RowCtx R = row_ctx(A, W, j, dist, &s_rs);
    uint16_t *bins = W.bin1 + (size_t)(j * 2 + dist) * W.vpad;
    const int c_beg = sl * SLICE, c_end = min(A.v, c_beg + SLICE);
    // the slice's values (and counts) first, all loads in flight
    constexpr int PER = SLICE / BT;
    const float *src = dist == 0 ? A.z + (int64_t)j * A.ldz : A.q + (int64_t)j * A.ldq;
    const bool with_hist = dist == 0 && A.pen && A.counts != nullptr;
    float raw[PER];
    int hist[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int col = c_beg + BT * i + tid;
        raw[i] = col < c_end ? src[col] : 0.f;
        hist[i] = with_hist && col < c_end ? A.counts[col] : 0;
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int col = c_beg + BT * i + tid;
        unsigned long long key = 0, mfx = 0;
        uint32_t fi = 0;
        const bool take = col < c_end;
        if (take) {
            trunc_entry_raw(A, R, dist, j, col, raw[i], hist[i], s_d, s_bloom, key, fi, mfx);
            bins[col] = (uint16_t)(fi >> 11);
        }
        hist_add_split(h_cnt, h_lo, h_hi, take, (int)(fi >> 11), mfx);
    }
    __syncthreads();
    const size_t slot = ((size_t)(j * 2 + dist) * W.nslices + sl) * NB;
    for (int b = tid; b < NB; b += BT) {
        W.pcnt[slot + b] = h_cnt[b];
        W.pmass[slot + b] = ((unsigned long long)h_hi[b] << 19) + h_lo[b];
    }
}

// Running sums at a bound: the count and fixed-point mass of the entries
// whose keys are >= the bound's key (among those with key >= lo).
struct Found {
    unsigned long long key, cnt, mass;
    int ok;
};

// Selection: grid (rows, 2).
__global__ __launch_bounds__(FT) void sample_trunc_kernel(const SampleArgs A) {
    __shared__ uint32_t h_cnt[NB];
    __shared__ unsigned long long h_mass[NB];
    __shared__ unsigned long long c_key[CAP];
    __shared__ unsigned long long c_mass[CAP];
    __shared__ unsigned long long s_wsum[FT / 64][2];
    __shared__ int32_t s_d[kMaxRows];
    __shared__ uint32_t s_bloom[32];
    __shared__ float2 s_rs;
    __shared__ int s_bin, s_n;
    __shared__ unsigned long long s_acnt, s_amass;
    __shared__ Found s_found;
    const int j = blockIdx.x, dist = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    if (dist == 1 && j >= A.rows - 1) return;
    const SampleWs W = carve(A.ws, A.rows, A.v);
    if (tid < A.rows - 1) s_d[tid] = A.d[tid];
    __syncthreads();
    build_bloom(s_bloom, s_d, dist == 0 ? j : 0);
    const RowCtx R = row_ctx(A, W, j, dist, &s_rs);
    const uint16_t *bins = W.bin1 + (size_t)(j * 2 + dist) * W.vpad;
    const size_t slot0 = (size_t)(j * 2 + dist) * W.nslices * NB;

    // An entry's key, fine index and weight from its value (and count).
    auto entry = [&](int col, float raw, int hist, unsigned long long &key, uint32_t &fi, unsigned long long &mfx)
        __attribute__((always_inline)) { trunc_entry_raw(A, R, dist, j, col, raw, hist, s_d, s_bloom, key, fi, mfx); };
    const float *vrow = dist == 0 ? A.z + (int64_t)j * A.ldz : A.q + (int64_t)j * A.ldq;
    const bool with_hist = dist == 0 && A.pen && A.counts != nullptr;

    // Calls visit(match, col, raw, hist) until every entry of first-level bin
    // b1 has been visited once with match set (col < v; raw its value, hist
    // its count); the calls are wave-uniform, so visit may use wave-wide
    // operations.  The stored bins are read 16 bytes (8 entries) at a time,
    // 4 loads in flight per thread; each thread then takes the matches of its
    // 32 entries VB at a time, lowest first, with the values of all VB
    // loaded together (a crowded bin gives a thread many matches, and one
    // dependent load per visit made them a chain of round trips).
    auto scan_bin = [&](int b1, auto &&visit) __attribute__((always_inline)) {
        const uint4 *bv = reinterpret_cast<const uint4 *>(bins);
        const int ng = (A.v + 7) >> 3;
        constexpr int K = 4;
        for (int g0 = 0; g0 < ng; g0 += FT * K) {
            uint4 vv[K];
#pragma unroll
            for (int i = 0; i < K; ++i) {
                const int gi = g0 + FT * i + tid;
                vv[i] = gi < ng ? bv[gi] : make_uint4(~0u, ~0u, ~0u, ~0u);
            }
            uint32_t mask = 0;
#pragma unroll
            for (int i = 0; i < K; ++i) {
                const uint32_t w4[4] = {vv[i].x, vv[i].y, vv[i].z, vv[i].w};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int col = (g0 + FT * i + tid) * 8 + e;
                    const uint32_t bb = (w4[e >> 1] >> ((e & 1) * 16)) & 0xffffu;
                    if (col < A.v && bb == (uint32_t)b1) mask |= 1u << (i * 8 + e);
                }
            }
            constexpr int VB = 8;
            for (;;) {
                if (__ballot(mask != 0u) == 0ull) break;
                bool has[VB];
                int cols[VB];
#pragma unroll
                for (int t = 0; t < VB; ++t) {
                    has[t] = mask != 0u;
                    const int e = has[t] ? __ffs(mask) - 1 : 0;
                    mask &= mask - 1u;
                    cols[t] = has[t] ? (g0 + FT * (e >> 3) + tid) * 8 + (e & 7) : 0;   // column 0: a valid address
                }
                float raw[VB];
                int hist[VB];
#pragma unroll
                for (int t = 0; t < VB; ++t) {
                    raw[t] = vrow[cols[t]];
                    hist[t] = with_hist ? A.counts[cols[t]] : 0;
                }
#pragma unroll
                for (int t = 0; t < VB; ++t) visit(has[t], cols[t], raw[t], hist[t]);
            }
        }
    };

    // (the barrier first: every thread has read what it needs of the bins)
    auto clear_hist = [&]() __attribute__((always_inline)) {
        __syncthreads();
        for (int b = tid; b < NB; b += FT) {
            h_cnt[b] = 0u;
            h_mass[b] = 0ull;
        }
        __syncthreads();
    };

    // first-level histogram of the whole row: the sum of the slices'
    auto load_level1 = [&]() __attribute__((always_inline)) {
        __syncthreads();
        for (int b = tid; b < NB; b += FT) {
            unsigned long long c = 0, m = 0;
            for (int sl0 = 0; sl0 < W.nslices; sl0 += 8) {   // 8 slices' loads in flight
                uint32_t cc[8];
                unsigned long long mm[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const size_t at = slot0 + (size_t)(sl0 + i) * NB + b;
                    cc[i] = sl0 + i < W.nslices ? W.pcnt[at] : 0u;
                    mm[i] = sl0 + i < W.nslices ? W.pmass[at] : 0ull;
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    c += cc[i];
                    m += mm[i];
                }
            }
            h_cnt[b] = (uint32_t)c;
            h_mass[b] = m;
        }
        __syncthreads();
    };

    // Wave 0: the first bin, in the order 'ascending' (bin 0 first) or
    // descending, at which base + running weight (count or mass) reaches
    // target; s_bin = -1 if none.  s_acnt / s_amass: count and mass before
    // it.  All threads call it (barriers on both sides).
    auto find_bin = [&](bool ascending, bool by_mass, unsigned long long target, unsigned long long base_cnt,
                        unsigned long long base_mass) __attribute__((always_inline)) {
        __syncthreads();
        if (wv == 0) {
            constexpr int PER = NB / 64;
            unsigned long long lc = 0, lm = 0;
#pragma unroll 4
            for (int i = 0; i < PER; ++i) {
                const int pos = lane * PER + i;
                const int b = ascending ? pos : NB - 1 - pos;
                lc += h_cnt[b];
                lm += h_mass[b];
            }
            const unsigned long long ic = wave_incl_scan(lc, lane), im = wave_incl_scan(lm, lane);
            const unsigned long long reach = by_mass ? base_mass + im : base_cnt + ic;
            const unsigned long long mask = __ballot(reach >= target);
            if (lane == 0) s_bin = -1;
            if (mask != 0ull && lane == __ffsll((long long)mask) - 1) {
                unsigned long long c = base_cnt + ic - lc, mm = base_mass + im - lm;
                int bin = -1;
#pragma unroll 1
                for (int i = 0; i < PER; ++i) {
                    const int pos = lane * PER + i;
                    const int b = ascending ? pos : NB - 1 - pos;
                    const unsigned long long nc = c + h_cnt[b], nm = mm + h_mass[b];
                    if ((by_mass ? nm : nc) >= target) {
                        bin = b;
                        break;
                    }
                    c = nc;
                    mm = nm;
                }
                s_bin = bin;
                s_acnt = c;
                s_amass = mm;
            }
        }
        __syncthreads();
    };

    // Gather the entries of first-level bin b1 with key >= lo and fi in
    // [f0, f1] into LDS (at most CAP of them) and find the first, in
    // descending key order, at which base + running weight reaches target;
    // result in s_found.  base is below target (the sums before the bin that
    // find_bin chose), so the selection below never settles on an empty
    // digit.
    auto gather_select_find = [&](int b1, unsigned long long lo, uint32_t f0, uint32_t f1, bool by_mass,
                                unsigned long long target, unsigned long long base_cnt,
                                unsigned long long base_mass) __attribute__((always_inline)) {
        if (tid == 0) s_n = 0;
        __syncthreads();
        scan_bin(b1, [&](bool match, int col, float raw, int hist) __attribute__((always_inline)) {
            bool take = false;
            unsigned long long key = 0, mfx = 0;
            if (match) {
                uint32_t fi;
                entry(col, raw, hist, key, fi, mfx);
                take = key >= lo && fi >= f0 && fi <= f1;
            }
            const unsigned long long bal = __ballot(take);
            if (bal != 0ull) {
                const int lead = __ffsll((long long)bal) - 1;
                int basei = 0;
                if (lane == lead) basei = atomicAdd(&s_n, (int)__popcll(bal));
                basei = __shfl(basei, lead);
                const int slot = basei + (int)__popcll(bal & ((1ull << lane) - 1ull));
                if (take && slot < CAP) {
                    c_key[slot] = key;
                    c_mass[slot] = mfx;
                }
            }
        });
        __syncthreads();
        const int n = min(s_n, CAP);
        // The bound among the gathered entries, without sorting them: a
        // radix selection over the 64-bit keys, one 8-bit digit per pass from
        // the top.  Each pass histograms (count, mass) by digit the entries
        // that share the digits chosen so far and takes the largest digit at
        // which base + the weight of every larger key reaches target; the
        // digits above it join the base.  After eight passes the digits are
        // the bound's key (keys are unique) and the base counts every larger
        // key.  (A bitonic sort of up to 4096 entries by one workgroup was
        // most of the selection's time.)
        static_assert(CAP == 4 * FT, "four gathered entries per thread");
        if (n <= 64) {
            // few entries (the usual case): wave 0 sorts them across its
            // lanes with shuffles (bitonic, descending, no barriers) and
            // scans the running weight
            if (wv == 0) {
                unsigned long long k1 = lane < n ? c_key[lane] : 0ull, m1 = lane < n ? c_mass[lane] : 0ull;
                for (int k = 2; k <= 64; k <<= 1)
                    for (int jj = k >> 1; jj > 0; jj >>= 1) {
                        const unsigned long long pk = __shfl_xor(k1, jj), pm = __shfl_xor(m1, jj);
                        const bool keep_max = ((lane & k) == 0) == ((lane & jj) == 0);
                        if (keep_max ? pk > k1 : pk < k1) {
                            k1 = pk;
                            m1 = pm;
                        }
                    }
                const unsigned long long ic = wave_incl_scan(lane < n ? 1ull : 0ull, lane) + base_cnt;
                const unsigned long long im = wave_incl_scan(lane < n ? m1 : 0ull, lane) + base_mass;
                const unsigned long long hit = __ballot(lane < n && (by_mass ? im : ic) >= target);
                if (hit != 0ull && lane == __ffsll((long long)hit) - 1) {
                    s_found.key = k1;
                    s_found.cnt = ic;
                    s_found.mass = im;
                    s_found.ok = 1;
                }
            }
            __syncthreads();
            return;
        }
        unsigned long long kv[4], mv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int e = 4 * tid + r;
            kv[r] = e < n ? c_key[e] : 0ull;
            mv[r] = e < n ? c_mass[e] : 0ull;
        }
        unsigned long long prefix = 0, acnt = base_cnt, amass = base_mass;
        bool found = true;
        for (int shift = 56; shift >= 0; shift -= 8) {
            __syncthreads();            // the previous pass's histogram has been read
            for (int b = tid; b < 256; b += FT) {
                h_cnt[b] = 0u;
                h_mass[b] = 0ull;
            }
            __syncthreads();
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int e = 4 * tid + r;
                const bool take = e < n && (shift == 56 || (kv[r] >> (shift + 8)) == (prefix >> (shift + 8)));
                hist_add(h_cnt, h_mass, take, (int)((kv[r] >> shift) & 255u), mv[r]);
            }
            __syncthreads();
            if (wv == 0) {
                // digits in descending order, four per lane
                unsigned long long lc = 0, lm = 0;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int b = 255 - (4 * lane + i);
                    lc += h_cnt[b];
                    lm += h_mass[b];
                }
                const unsigned long long ic = wave_incl_scan(lc, lane), im = wave_incl_scan(lm, lane);
                const unsigned long long reach = by_mass ? amass + im : acnt + ic;
                const unsigned long long mask = __ballot(reach >= target);
                if (lane == 0) s_bin = -1;
                if (mask != 0ull && lane == __ffsll((long long)mask) - 1) {
                    unsigned long long c = acnt + ic - lc, m = amass + im - lm;
                    int bin = -1;
                    for (int i = 0; i < 4; ++i) {
                        const int b = 255 - (4 * lane + i);
                        const unsigned long long nc = c + h_cnt[b], nm = m + h_mass[b];
                        if ((by_mass ? nm : nc) >= target) {
                            bin = b;
                            break;
                        }
                        c = nc;
                        m = nm;
                    }
                    s_bin = bin;
                    s_acnt = c;
                    s_amass = m;
                }
            }
            __syncthreads();
            if (s_bin < 0) {            // not reached (only possible in the first pass)
                found = false;
                break;
            }
            prefix |= (unsigned long long)s_bin << shift;
            acnt = s_acnt;
            amass = s_amass;
        }
        if (found) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (4 * tid + r < n && kv[r] == prefix) {
                    s_found.key = prefix;
                    s_found.cnt = acnt + 1;
                    s_found.mass = amass + mv[r];
                    s_found.ok = 1;
                }
            }
        }
        __syncthreads();
    };

    // Exact radix selection over keys (rare path: more than CAP entries with
    // one fine index f in bin b1): the largest key K with key >= lo, fi == f
    // and base + weight(keys >= K) >= target; then its running sums.
    auto radix_find = [&](int b1, unsigned long long lo, uint32_t f, bool by_mass, unsigned long long target,
                          unsigned long long base_cnt, unsigned long long base_mass) __attribute__((always_inline)) {
        unsigned long long prefix = 0, acnt = base_cnt, amass = base_mass;
        for (int pass = 0; pass < 6; ++pass) {
            const int shift = pass < 5 ? 53 - 11 * pass : 0;
            const int width = pass < 5 ? 11 : 9;
            const int top = shift + width;
            clear_hist();
            scan_bin(b1, [&](bool match, int col, float raw, int hist) __attribute__((always_inline)) {
                unsigned long long key = 0, mfx = 0;
                bool take = false;
                if (match) {
                    uint32_t fi;
                    entry(col, raw, hist, key, fi, mfx);
                    take = key >= lo && fi == f && (top >= 64 || (key >> top) == (prefix >> top));
                }
                hist_add(h_cnt, h_mass, take, (int)((key >> shift) & ((1u << width) - 1u)), mfx);
            });
            find_bin(false, by_mass, target, acnt, amass);
            if (s_bin < 0) return;      // s_found.ok stays 0
            prefix |= (unsigned long long)s_bin << shift;
            acnt = s_acnt;
            amass = s_amass;
        }
        // acnt / amass count the keys above 'prefix'; add the entry itself
        // (one entry has this key)
        scan_bin(b1, [&](bool match, int col, float raw, int hist) __attribute__((always_inline)) {
            if (match) {
                unsigned long long key, mfx;
                uint32_t fi;
                entry(col, raw, hist, key, fi, mfx);
                if (key == prefix) {
                    s_found.key = prefix;
                    s_found.cnt = acnt + 1;
                    s_found.mass = amass + mfx;
                    s_found.ok = 1;
                }
            }
        });
        __syncthreads();
    };

    // The first entry (key >= lo) at which the running count (by_mass =
    // false) or mass reaches target, given the first-level histogram of the
    // entries with key >= lo in h_cnt / h_mass.  Result in s_found (ok = 0:
    // not reached, 2: see below); the first-level bin and the sums before it in
    // l1_bin / l1_acnt / l1_amass.
    int l1_bin = -1;
    unsigned long long l1_acnt = 0, l1_amass = 0;
    auto find_bound = [&](unsigned long long lo, bool by_mass, unsigned long long target)
        __attribute__((always_inline)) {
        if (tid == 0) s_found.ok = 0;
        find_bin(true, by_mass, target, 0ull, 0ull);
        const int b1 = s_bin;
        l1_bin = b1;
        if (b1 < 0) return;
        unsigned long long acnt = s_acnt, amass = s_amass;
        l1_acnt = acnt;
        l1_amass = amass;
        if (!by_mass && h_mass[b1] == 0ull) {
            // weight-zero bin: every later entry weighs zero too (weights do
            // not increase along the key order), so the first k hold every
            // positive weight: ok = 2
            __syncthreads();
            if (tid == 0) s_found.ok = 2;
            __syncthreads();
            return;
        }
        if (h_cnt[b1] <= (uint32_t)CAP) {
            gather_select_find(b1, lo, (uint32_t)b1 << 11, ((uint32_t)b1 << 11) | 2047u, by_mass, target, acnt, amass);
            return;
        }
        clear_hist();
        scan_bin(b1, [&](bool match, int col, float raw, int hist) __attribute__((always_inline)) {
            unsigned long long key = 0, mfx = 0;
            uint32_t fi = 0;
            bool take = false;
            if (match) {
                entry(col, raw, hist, key, fi, mfx);
                take = key >= lo;
            }
            hist_add(h_cnt, h_mass, take, (int)(fi & 2047u), mfx);
        });
        find_bin(true, by_mass, target, acnt, amass);
        const int b2 = s_bin;
        if (b2 < 0) return;
        acnt = s_acnt;
        amass = s_amass;
        const uint32_t f = ((uint32_t)b1 << 11) | (uint32_t)b2;
        if (!by_mass && h_mass[b2] == 0ull) {
            __syncthreads();
            if (tid == 0) s_found.ok = 2;
            __syncthreads();
            return;
        }
        if (h_cnt[b2] <= (uint32_t)CAP) {
            gather_select_find(b1, lo, f, f, by_mass, target, acnt, amass);
            return;
        }
        radix_find(b1, lo, f, by_mass, target, acnt, amass);
    };

    load_level1();
    unsigned long long lo = 0, kmass = 0;
    const bool topk = A.top_k > 0 && A.top_k < A.v;
    bool have_k = false;
    int bk = -1;
    unsigned long long bk_acnt = 0, bk_amass = 0;
    if (topk) {
        // ok = 2: the first k entries hold every positive weight, which is
        // the same truncation as none
        find_bound(0ull, false, (unsigned long long)A.top_k);
        if (s_found.ok == 1) {
            lo = s_found.key;
            kmass = s_found.mass;
            have_k = true;
            bk = l1_bin;
            bk_acnt = l1_acnt;
            bk_amass = l1_amass;
        }
    }
    if (!have_k) {
        // total mass: the first-level bins' sums, in bin order (reloaded:
        // the top-k search may have left a finer histogram)
        if (topk) load_level1();
        __syncthreads();
        if (wv == 0) {
            unsigned long long m = 0;
            for (int b = lane; b < NB; b += 64) m += h_mass[b];
            m = wave_incl_scan(m, lane);
            if (lane == 63) s_wsum[0][1] = m;
        }
        __syncthreads();
        kmass = s_wsum[0][1];
    }
    unsigned long long bound = lo, kept = kmass;
    if (A.top_p < 1.f) {
        const unsigned long long target = (unsigned long long)ceil((double)A.top_p * (double)kmass);
        if (target == 0) {
            bound = ~0ull;            // a row without weight keeps nothing
            kept = 0;
        } else {
            if (have_k) {
                // first-level histogram of the top-k entries: the bins before
                // bk whole, bk's part above the bound, nothing after
                load_level1();
                for (int b = tid; b < NB; b += FT) {
                    if (b > bk) {
                        h_cnt[b] = 0u;
                        h_mass[b] = 0ull;
                    } else if (b == bk) {
                        h_cnt[b] = (uint32_t)((unsigned long long)A.top_k - bk_acnt);
                        h_mass[b] = kmass - bk_amass;
                    }
                }
                __syncthreads();
            }
            find_bound(lo, true, target);
            if (s_found.ok == 1) {
                bound = s_found.key;
                kept = s_found.mass;
            }
        }
    }
    if (tid == 0) {
        Trunc t;
        t.key = bound;
        t.mass = (float)ldexp((double)kept * (double)R.wmax, -R.fx);
        t.pad = 0;
        W.trunc[j * 2 + dist] = t;
    }
}

// Probability of column col in the (truncated) target row j and draft row j.
struct RowView {
    float rmax, rsum;
    unsigned long long kp, kq;   // truncation bounds (0: keep all)
    float mp, mq;                // kept masses (p: 1 untruncated; q: 1 means "as supplied")
};

__device__ inline float p_of(const SampleArgs &A, const int32_t *s_d, const uint32_t *bloom, const RowView &r, int j,
                            int col, float zz) {
    const float x = scaled_logit(A, s_d, bloom, j, col, zz);
    const float p = expf(x - r.rmax) / r.rsum;
    if (!A.trunc) return p;
    return (order_key(x, col) >= r.kp && r.mp > 0.f) ? p / r.mp : 0.f;
}

__device__ inline float q_of(const SampleArgs &A, const RowView &r, int col, float qq) {
    if (!A.trunc) return qq;
    return (order_key(qq, col) >= r.kq && r.mq > 0.f) ? qq / r.mq : 0.f;
}

__device__ inline RowView row_view(const SampleArgs &A, const SampleWs &W, float2 rs, int j) {
    RowView r;
    r.rmax = rs.x;
    r.rsum = rs.y;
    r.kp = 0;
    r.kq = 0;
    r.mp = 1.f;
    r.mq = 1.f;
    if (A.trunc) {
        const Trunc tp = W.trunc[j * 2];
        r.kp = tp.key;
        r.mp = tp.mass;
        if (j < A.rows - 1) {
            const Trunc tq = W.trunc[j * 2 + 1];
            r.kq = tq.key;
            r.mq = tq.mass;
        }
    }
    return r;
}

// Pass 2, one workgroup per chunk.  Every workgroup repeats the (cheap,
// deterministic) accept decisions from the row statistics of pass 1 -- so all
// agree on the row jr that supplies the final draw -- and adds up, over its
// chunk of row jr only, the mass of the residual max(0, p - q) and of p per
// 256-column segment; the last workgroup to finish finds the segment holding
// the draw (prefix sums in column order) and draws the token inside it.
__global__ __launch_bounds__(DT) void sample_decide_kernel(const SampleArgs A) {
    __shared__ float2 s_rows[kMaxRows];
    __shared__ int32_t s_d[kMaxRows];
    __shared__ uint32_t s_bloom[32];
    __shared__ float s_tot[2][DW], s_scan[DW];
    __shared__ int s_flag, s_jr, s_lastseg;
    __shared__ unsigned long long s_cut;
    const int rows = A.rows, v = A.v;
    const int nchunks = (v + CH - 1) / CH, nseg = nchunks * NSEG;
    const SampleWs W = carve(A.ws, rows, v);
    const int c = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

    // draft ids and uniforms in range (they index memory below); thread j
    // fetches the two entries its accept test reads as soon as d_j is known
    int bad = 0, dj = 0;
    float uj = 0.f, zd = 0.f, qd = 0.f;
    const float ulast = A.u[rows - 1];      // the final draw's uniform (checked below by thread rows - 1)
    if (tid < rows) {
        uj = A.u[tid];
        bad |= !(uj >= 0.f && uj < 1.f);
    }
    if (tid < rows - 1) {
        dj = A.d[tid];
        s_d[tid] = dj;
        if (dj >= 0 && dj < v) {
            zd = A.z[(int64_t)tid * A.ldz + dj];
            qd = A.q[(int64_t)tid * A.ldq + dj];
        } else {
            bad = 1;
        }
    }
    if (tid < 8 * kMaxRows) {      // whole waves: eight lanes per row
        const int jj = tid >> 3, k = tid & 7;
        const float2 rs = row_stats8(W.stats + (int64_t)min(jj, rows - 1) * nchunks, nchunks, k);
        if (k == 0 && jj < rows) s_rows[jj] = rs;
    }
    bad = __syncthreads_or(bad);
    // Accept tests of all drafts at once (thread j of wave 0 tests draft j):
    // the first reject ends the accepted prefix and supplies the final draw,
    // else the last row does.
    if (w == 0) {
        bool reject = false;
        if (!bad && tid < rows - 1) {
            const RowView r = row_view(A, W, s_rows[tid], tid);
            const float pd = p_of(A, s_d, nullptr, r, tid, dj, zd);
            reject = !(uj * q_of(A, r, dj, qd) < pd);
        }
        const unsigned long long b = __ballot(reject);
        if (lane == 0) s_jr = b != 0ull ? __ffsll((long long)b) - 1 : rows - 1;
    }
    __syncthreads();
    const int jr = __builtin_amdgcn_readfirstlane(s_jr);     // the same on every thread
    if (A.pen) build_bloom(s_bloom, s_d, jr);
    const bool draft_row = jr < rows - 1;
    const RowView rv = row_view(A, W, s_rows[jr], jr);
    const float *zj = A.z + (int64_t)jr * A.ldz;
    const float *qj = A.q + (int64_t)jr * A.ldq;
    {
        const int v0 = c * CH, v1 = min(v, v0 + CH);
        float4 zv[DG], qv[DG];
        load_chunk<DT, DG>(zv, zj, v0, v1, A.vec_z);
        if (draft_row) load_chunk<DT, DG>(qv, qj, v0, v1, A.vec_q);
#pragma unroll
        for (int i = 0; i < DG; ++i) {
            float res = 0.f, pm = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int col = v0 + 4 * (tid + DT * i) + e;
                if (col < v1) {
                    const float p = p_of(A, s_d, s_bloom, rv, jr, col, f4(zv[i], e));
                    pm += p;
                    if (draft_row) res += fmaxf(0.f, p - q_of(A, rv, col, f4(qv[i], e)));
                }
            }
            res = wave_sum(res);
            pm = wave_sum(pm);
            if (lane == 0) store_f2(&W.mass[(int64_t)c * NSEG + DW * i + w], make_float2(res, pm));
        }
        // arrival: each wave's stores complete before the workgroup signals
        __builtin_amdgcn_s_waitcnt(0x0f70);     // vmcnt(0)
    }
    __syncthreads();
    if (tid == 0) s_flag = atomicAdd(W.counter, 1u) == (uint32_t)(nchunks - 1);
    __syncthreads();
    if (!s_flag) return;

    // The last workgroup.  Faults (any flagged chunk; ids and uniforms were
    // checked above) and this thread's run of consecutive segments, read
    // together; the first kRun masses stay in registers.
    constexpr int kRun = 2;
    const int per = (nseg + DT - 1) / DT;
    const int s0 = min(nseg, tid * per), s1 = min(nseg, s0 + per);
    {
        constexpr int F = 2;     // flag words per thread fetched together
        const int nf = rows * nchunks;
        int32_t fl[F];
#pragma unroll
        for (int f = 0; f < F; ++f) fl[f] = W.flags[min(tid + DT * f, nf - 1)];     // no branch: one wait
        for (int i = tid + DT * F; i < nf; i += DT) bad |= W.flags[i] != 0;
#pragma unroll
        for (int f = 0; f < F; ++f) bad |= fl[f] != 0;
    }
    float2 mr[kRun];
    float tr = 0.f, tp = 0.f;
#pragma unroll
    for (int k = 0; k < kRun; ++k) {
        mr[k] = s0 + k < s1 ? load_f2(&W.mass[s0 + k]) : make_float2(0.f, 0.f);
        tr += mr[k].x;
        tp += mr[k].y;
    }
    for (int s = s0 + kRun; s < s1; ++s) {
        const float2 mm = load_f2(&W.mass[s]);
        tr += mm.x;
        tp += mm.y;
    }
    bad = __syncthreads_or(bad);
    if (bad) {
        if (tid < rows) A.committed[tid] = -1;
        if (tid == 0) {
            A.accept_len[0] = -1;
            atomicExch(W.counter, 0u);
        }
        return;
    }
    // totals over the segments in a fixed order (runs in thread order)
    {
        const float a = wave_sum(tr), b = wave_sum(tp);
        if (lane == 0) {
            s_tot[0][w] = a;
            s_tot[1][w] = b;
        }
    }
    if (tid == 0) {
        s_cut = ~0ull;
        s_lastseg = -1;
    }
    __syncthreads();
    float total_res = s_tot[0][0], total_p = s_tot[1][0];
    for (int k = 1; k < DW; ++k) {
        total_res += s_tot[0][k];
        total_p += s_tot[1][k];
    }
    // mass to sample from: the residual on a reject (p if it has none), p for
    // the bonus
    const bool use_res = __builtin_amdgcn_readfirstlane(draft_row && total_res > 0.f);
    const float thr = ulast * (use_res ? total_res : total_p);
    // exclusive prefix of the run totals in thread order (wave scan, then the
    // waves before), then the first segment whose inclusive prefix exceeds thr
    const float mine = use_res ? tr : tp;
    float incl = mine;
    for (int off = 1; off < 64; off <<= 1) {
        const float t = __shfl_up(incl, off);
        if (lane >= off) incl += t;
    }
    float run = __shfl_up(incl, 1);
    if (lane == 0) run = 0.f;
    if (lane == 63) s_scan[w] = incl;
    __syncthreads();
    for (int k = 0; k < w; ++k) run += s_scan[k];
    // this thread's first crossing (segment and exclusive prefix) and its last
    // segment with mass
    bool found = false;
    int lastseg = -1;
    unsigned long long key = ~0ull;
#pragma unroll
    for (int k = 0; k < kRun; ++k) {
        const float m = use_res ? mr[k].x : mr[k].y;
        if (s0 + k < s1 && !found) {
            if (run + m > thr) {
                key = ((unsigned long long)(s0 + k) << 32) | __float_as_uint(run);
                found = true;
            }
            run += m;
        }
        if (s0 + k < s1 && m > 0.f) lastseg = s0 + k;
    }
    for (int s = s0 + kRun; s < s1; ++s) {
        const float2 mm = load_f2(&W.mass[s]);
        const float m = use_res ? mm.x : mm.y;
        if (!found) {
            if (run + m > thr) {
                key = ((unsigned long long)s << 32) | __float_as_uint(run);
                found = true;
            }
            run += m;
        }
        if (m > 0.f) lastseg = s;
    }
    // segments grow with the lane, so the wave's first crossing is its lowest
    // finding lane and its last segment with mass its highest lane that has
    // one: one LDS atomic per wave each
    {
        const unsigned long long bf = __ballot(found), bl = __ballot(lastseg >= 0);
        if (bf != 0ull && lane == __ffsll((long long)bf) - 1) atomicMin(&s_cut, key);
        if (bl != 0ull && lane == 63 - __clzll((long long)bl)) atomicMax(&s_lastseg, lastseg);
    }
    __syncthreads();
    if (w != 0) return;
    const unsigned long long cut = s_cut;
    int sstar;
    bool last_pos;
    float thr_local;
    if (cut != ~0ull) {
        sstar = (int)(cut >> 32);
        last_pos = false;
        thr_local = thr - __uint_as_float((uint32_t)cut);
    } else {
        // no segment crosses the threshold (rounding): the last one with mass
        sstar = s_lastseg >= 0 ? s_lastseg : nseg - 1;
        last_pos = true;
        thr_local = 0.f;
    }
    sstar = __builtin_amdgcn_readfirstlane(sstar);
    // inverse CDF inside segment sstar: one wave, four consecutive columns per
    // lane, prefix sums in column order
    const int col0 = sstar * SEG + 4 * lane;
    const bool in = sstar * SEG + SEG <= v;
    const float4 z4 = load4(zj, col0, v, in && A.vec_z, 0.f);
    float4 q4 = make_float4(0.f, 0.f, 0.f, 0.f);
    if (use_res) q4 = load4(qj, col0, v, in && A.vec_q, 0.f);
    float wv[4];
    float tot = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int col = col0 + e;
        float wgt = 0.f;
        if (col < v) {
            const float p = p_of(A, s_d, s_bloom, rv, jr, col, f4(z4, e));
            wgt = use_res ? fmaxf(0.f, p - q_of(A, rv, col, f4(q4, e))) : p;
        }
        wv[e] = wgt;
        tot += wgt;
    }
    float incl2 = tot;
    for (int off = 1; off < 64; off <<= 1) {
        const float t = __shfl_up(incl2, off);
        if (lane >= off) incl2 += t;
    }
    float run2 = __shfl_up(incl2, 1);
    if (lane == 0) run2 = 0.f;
    int pick = 0x7fffffff, lastp = -1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        run2 += wv[e];
        if (!last_pos && pick == 0x7fffffff && run2 > thr_local) pick = col0 + e;
        if (wv[e] > 0.f) lastp = col0 + e;
    }
    // the smallest pick over the wave; the largest positive column as the
    // rounding fallback
    for (int off = 32; off > 0; off >>= 1) {
        pick = min(pick, __shfl_xor(pick, off));
        lastp = max(lastp, __shfl_xor(lastp, off));
    }
    // the accepted drafts, the drawn token, -1 after it (rows <= 64 = one wave)
    const int tok = pick != 0x7fffffff ? pick : lastp >= 0 ? lastp : min(v - 1, sstar * SEG + SEG - 1);
    if (lane < rows) A.committed[lane] = lane < jr ? s_d[lane] : lane == jr ? tok : -1;
    if (lane == 0) {
        A.accept_len[0] = jr + 1;
        atomicExch(W.counter, 0u);
    }
}

}  // namespace


hipError_t launch_accept_greedy(const int32_t *t, const int32_t *d, int32_t b, int32_t m_rows,
                                int32_t *accept_len, int32_t *committed, hipStream_t s) {
    const int blocks = (b + 63) / 64;
    hipLaunchKernelGGL(accept_greedy_kernel, dim3(blocks), dim3(64), 0, s, t, d, b, m_rows, accept_len,
                       committed);
    return hipGetLastError();
}

hipError_t launch_accept_sample(const SampleParams &P, hipStream_t s) {
    SampleArgs A;
    A.z = P.z;
    A.ldz = P.ldz;
    A.q = P.q;
    A.ldq = P.ldq;
    A.d = P.d;
    A.u = P.u;
    A.rows = P.m_rows;
    A.v = P.v;
    A.inv_t = 1.f / P.temperature;
    A.top_k = P.top_k;
    A.top_p = P.top_p;
    A.presence = P.presence;
    A.frequency = P.frequency;
    A.counts = P.counts;
    A.pen = P.presence != 0.f || P.frequency != 0.f;
    A.trunc = (P.top_k > 0 && P.top_k < P.v) || P.top_p < 1.f;
    A.vec_z = ((uintptr_t)P.z % 16) == 0 && P.ldz % 4 == 0;
    A.vec_q = ((uintptr_t)P.q % 16) == 0 && P.ldq % 4 == 0;
    A.accept_len = P.accept_len;
    A.committed = P.committed;
    A.ws = P.ws;
    const int nchunks = (P.v + CH - 1) / CH;
    hipLaunchKernelGGL(sample_stats_kernel, dim3(nchunks, P.m_rows), dim3(TPB), 0, s, A);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (A.trunc) {
        hipLaunchKernelGGL(sample_bins_kernel, dim3((P.v + SLICE - 1) / SLICE, P.m_rows, 2), dim3(BT), 0, s, A);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(sample_trunc_kernel, dim3(P.m_rows, 2), dim3(FT), 0, s, A);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(sample_decide_kernel, dim3(nchunks), dim3(DT), 0, s, A);
    return hipGetLastError();
}

}  // namespace dspk

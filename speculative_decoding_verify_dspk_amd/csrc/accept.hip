// Acceptance of a verify block on gfx950: greedy longest-prefix match and
// Leviathan/Chen speculative sampling ("mlx-dspark" wiki summary,
// "Architecture"; "mlx-dspark 0.7.0", "How it works").
#include <math.h>

#include "dspk_internal.h"

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
// Workspace layout (bytes): [0, 256) arrival counter; then per (row, chunk):
// stats {max of z/T, sum exp(z/T - max)} and the fault flag; then per chunk
// the masses {residual, p} of the row that supplies the final draw.
constexpr int CH = kSampleChunk;
constexpr int TPB = 256;
constexpr int EPT = CH / TPB;    // logits per thread per chunk
constexpr int kMaxRowsSample = kMaxRows;

struct SampleWs {
    uint32_t *counter;
    float2 *stats;   // [rows][nchunks]
    int32_t *flags;  // [rows][nchunks]
    float2 *mass;    // [nchunks]
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) / 256 * 256; }

__host__ __device__ inline SampleWs carve(void *ws, int rows, int nchunks) {
    char *p = (char *)ws;
    SampleWs s;
    s.counter = (uint32_t *)p;
    p += 256;
    s.stats = (float2 *)p;
    p += align256((size_t)rows * nchunks * sizeof(float2));
    s.flags = (int32_t *)p;
    p += align256((size_t)rows * nchunks * sizeof(int32_t));
    s.mass = (float2 *)p;
    return s;
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

// block-wide reductions in a fixed order (wave butterfly, then waves in order)
__device__ inline float block_sum(float v, float *scratch) {
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) scratch[w] = v;
    __syncthreads();
    float r = scratch[0];
    for (int i = 1; i < TPB / 64; ++i) r += scratch[i];
    return r;
}

__device__ inline float block_max(float v, float *scratch) {
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) scratch[w] = v;
    __syncthreads();
    float r = scratch[0];
    for (int i = 1; i < TPB / 64; ++i) r = fmaxf(r, scratch[i]);
    return r;
}

// Pass 1: per (row, chunk) max and sum of exp of z/T, and the fault flag
// (non-finite logit; non-finite or negative q on draft rows).
__global__ __launch_bounds__(TPB) void sample_stats_kernel(const float *__restrict__ z, int64_t ldz,
                                                           const float *__restrict__ q, int64_t ldq,
                                                           int32_t rows, int32_t v, float temperature,
                                                           void *ws) {
    __shared__ float scratch[TPB / 64];
    const int nchunks = (v + CH - 1) / CH;
    const SampleWs W = carve(ws, rows, nchunks);
    const int c = blockIdx.x, j = blockIdx.y, tid = threadIdx.x;
    const int v0 = c * CH, v1 = min(v, v0 + CH);
    const float *zr = z + (int64_t)j * ldz;
    float a[EPT];
    float mx = -INFINITY;
    int bad = 0;
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        const int col = v0 + tid + TPB * i;
        a[i] = -INFINITY;
        if (col < v1) {
            const float zz = zr[col];
            bad |= !isfinite(zz);
            a[i] = zz / temperature;
            mx = fmaxf(mx, a[i]);
        }
    }
    if (j < rows - 1) {
        const float *qr = q + (int64_t)j * ldq;
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            const int col = v0 + tid + TPB * i;
            if (col < v1) {
                const float qq = qr[col];
                bad |= !(isfinite(qq) && qq >= 0.f);
            }
        }
    }
    bad = __syncthreads_or(bad);
    const float cmax = block_max(mx, scratch);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < EPT; ++i)
        if (v0 + tid + TPB * i < v1) s += expf(a[i] - cmax);
    const float csum = block_sum(s, scratch);
    if (tid == 0) {
        W.stats[j * nchunks + c] = make_float2(cmax, csum);
        W.flags[j * nchunks + c] = bad;
    }
}

// Pass 2, one workgroup per chunk.  Every workgroup repeats the (cheap,
// deterministic) accept decisions from the row statistics of pass 1 -- so all
// agree on the row jr that supplies the final draw -- and adds up, over its
// chunk of row jr only, the mass of the residual max(0, p - q) and of p; the
// last workgroup to finish draws the token.
__global__ __launch_bounds__(TPB) void sample_decide_kernel(
    const float *__restrict__ z, int64_t ldz, const float *__restrict__ q, int64_t ldq,
    const int32_t *__restrict__ d, const float *__restrict__ u, int32_t rows, int32_t v,
    float temperature, int32_t *__restrict__ accept_len, int32_t *__restrict__ committed, void *ws) {
    __shared__ float scratch[TPB / 64];
    __shared__ float2 s_rows[kMaxRowsSample];
    __shared__ float s_pref[TPB];
    __shared__ int s_flag[2];
    __shared__ int s_jr, s_lastc;
    __shared__ unsigned long long s_cut;
    const int nchunks = (v + CH - 1) / CH;
    const SampleWs W = carve(ws, rows, nchunks);
    const int c = blockIdx.x, tid = threadIdx.x;

    // row maxima and normalisers from the chunk statistics: eight threads per
    // row, chunks k, k + 8, ... each, then a fixed butterfly over the eight
    {
        const int j = tid >> 3, k = tid & 7;
        const float2 *st = W.stats + (int64_t)min(j, rows - 1) * nchunks;
        float mx = -INFINITY;
        for (int cc = k; cc < nchunks; cc += 8) mx = fmaxf(mx, st[cc].x);
        for (int off = 1; off < 8; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
        float sm = 0.f;
        for (int cc = k; cc < nchunks; cc += 8) sm += st[cc].y * expf(st[cc].x - mx);
        for (int off = 1; off < 8; off <<= 1) sm += __shfl_xor(sm, off);
        if (k == 0 && j < rows) s_rows[j] = make_float2(mx, sm);
    }
    // draft ids and uniforms in range (they index memory below)
    int bad = 0;
    if (tid < rows) {
        const float uu = u[tid];
        bad |= !(uu >= 0.f && uu < 1.f);
    }
    if (tid < rows - 1) bad |= (d[tid] < 0 || d[tid] >= v);
    if (tid == 0) s_jr = rows - 1;
    bad = __syncthreads_or(bad);
    // Accept tests of all drafts at once (thread j tests draft j): the first
    // reject ends the accepted prefix and supplies the final draw, else the
    // last row does.
    if (!bad && tid < rows - 1) {
        const float2 rs = s_rows[tid];
        const int dj = d[tid];
        const float pd = expf(z[(int64_t)tid * ldz + dj] / temperature - rs.x) / rs.y;
        const float qd = q[(int64_t)tid * ldq + dj];
        if (!(u[tid] * qd < pd)) atomicMin(&s_jr, tid);
    }
    __syncthreads();
    const int jr = s_jr;
    const bool draft_row = jr < rows - 1;
    {
        const float2 rs = s_rows[jr];
        const int v0 = c * CH, v1 = min(v, v0 + CH);
        const float *zr = z + (int64_t)jr * ldz;
        const float *qr = q + (int64_t)jr * ldq;
        float res = 0.f, pm = 0.f;
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            const int col = v0 + tid + TPB * i;
            if (col < v1) {
                const float p = expf(zr[col] / temperature - rs.x) / rs.y;
                pm += p;
                if (draft_row) res += fmaxf(0.f, p - qr[col]);
            }
        }
        const float rmass = block_sum(res, scratch);
        const float pmass = block_sum(pm, scratch);
        // arrival: thread 0 wrote this workgroup's masses and waits for them
        // to complete before it signals
        if (tid == 0) {
            store_f2(&W.mass[c], make_float2(rmass, pmass));
            __builtin_amdgcn_s_waitcnt(0x0f70);     // vmcnt(0)
            s_flag[0] = atomicAdd(W.counter, 1u) == (uint32_t)(nchunks - 1);
        }
    }
    __syncthreads();
    if (!s_flag[0]) return;

    // faults: any flagged chunk (non-finite logit, bad q), a uniform or draft id out of range
    for (int i = tid; i < rows * nchunks; i += TPB) bad |= W.flags[i] != 0;
    bad = __syncthreads_or(bad);
    if (bad) {
        if (tid < rows) committed[tid] = -1;
        if (tid == 0) {
            accept_len[0] = -1;
            atomicExch(W.counter, 0u);
        }
        return;
    }
    if (tid < jr) committed[tid] = d[tid];
    if (tid == 0) {
        s_lastc = -1;
        s_cut = ~0ull;
    }
    // mass to sample from: the residual on a reject (p if it has none), p for
    // the bonus; totals over the chunks in a fixed order
    float tr = 0.f, tp = 0.f;
    for (int cc = tid; cc < nchunks; cc += TPB) {
        const float2 mm = load_f2(&W.mass[cc]);
        tr += mm.x;
        tp += mm.y;
    }
    const float total_res = block_sum(tr, scratch);
    const float total_p = block_sum(tp, scratch);
    const int use_res = draft_row && total_res > 0.f;
    const float thr = u[rows - 1] * (use_res ? total_res : total_p);
    // chunk holding the draw: the first whose inclusive prefix of masses
    // exceeds thr (prefix sums in chunk order, TPB chunks per round); its
    // exclusive prefix travels with it in one 64-bit key
    float carry = 0.f;
    for (int b0 = 0; b0 < nchunks; b0 += TPB) {
        const int cc = b0 + tid;
        float mc = 0.f;
        if (cc < nchunks) {
            const float2 mm = load_f2(&W.mass[cc]);
            mc = use_res ? mm.x : mm.y;
        }
        s_pref[tid] = mc;
        __syncthreads();
        for (int off = 1; off < TPB; off <<= 1) {
            const float add = tid >= off ? s_pref[tid - off] : 0.f;
            __syncthreads();
            s_pref[tid] += add;
            __syncthreads();
        }
        const float incl = carry + s_pref[tid];
        if (cc < nchunks && incl > thr)
            atomicMin(&s_cut, ((unsigned long long)cc << 32) | __float_as_uint(incl - mc));
        if (cc < nchunks && mc > 0.f) atomicMax(&s_lastc, cc);
        carry += s_pref[TPB - 1];
        __syncthreads();
    }
    const unsigned long long cut = s_cut;
    int cstar, last_pos;
    float thr_local;
    if (cut != ~0ull) {
        cstar = (int)(cut >> 32);
        last_pos = 0;
        thr_local = thr - __uint_as_float((uint32_t)cut);
    } else {
        // no chunk crosses the threshold (rounding): the last chunk with mass
        cstar = s_lastc >= 0 ? s_lastc : nchunks - 1;
        last_pos = 1;
        thr_local = 0.f;
    }
    const float2 rs = s_rows[jr];
    __syncthreads();

    // inverse CDF inside chunk cstar: thread t owns EPT consecutive logits
    const int base = cstar * CH + tid * EPT;
    const float *zj = z + (int64_t)jr * ldz;
    const float *qj = q + (int64_t)jr * ldq;
    float wv[EPT];
    float tot = 0.f;
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        const int col = base + i;
        float wgt = 0.f;
        if (col < v) {
            const float p = expf(zj[col] / temperature - rs.x) / rs.y;
            wgt = use_res ? fmaxf(0.f, p - qj[col]) : p;
        }
        wv[i] = wgt;
        tot += wgt;
    }
    // exclusive prefix of the per-thread totals, in thread order
    s_pref[tid] = tot;
    __syncthreads();
    for (int off = 1; off < TPB; off <<= 1) {
        const float add = tid >= off ? s_pref[tid - off] : 0.f;
        __syncthreads();
        s_pref[tid] += add;
        __syncthreads();
    }
    float run = s_pref[tid] - tot;   // exclusive prefix
    int pick = 0x7fffffff, lastp = -1;
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        run += wv[i];
        if (!last_pos && pick == 0x7fffffff && run > thr_local) pick = base + i;
        if (wv[i] > 0.f) lastp = base + i;
    }
    // smallest pick over threads; largest positive index as the rounding fallback
    __shared__ int s_pick, s_last;
    if (tid == 0) {
        s_pick = 0x7fffffff;
        s_last = -1;
    }
    __syncthreads();
    atomicMin(&s_pick, pick);
    atomicMax(&s_last, lastp);
    __syncthreads();
    if (tid == 0) {
        int tok = s_pick;
        if (tok == 0x7fffffff) tok = s_last >= 0 ? s_last : min(v - 1, cstar * CH + CH - 1);
        committed[jr] = tok;
        for (int i = jr + 1; i < rows; ++i) committed[i] = -1;
        accept_len[0] = jr + 1;
        atomicExch(W.counter, 0u);
    }
}

}  // namespace

size_t sample_workspace_bytes(int32_t v, int32_t m_rows) {
    const size_t nchunks = (size_t)(v + CH - 1) / CH;
    return 256 + align256(m_rows * nchunks * sizeof(float2)) + align256(m_rows * nchunks * sizeof(int32_t)) +
           align256(nchunks * sizeof(float2));
}

hipError_t launch_accept_greedy(const int32_t *t, const int32_t *d, int32_t b, int32_t m_rows,
                                int32_t *accept_len, int32_t *committed, hipStream_t s) {
    const int blocks = (b + 63) / 64;
    hipLaunchKernelGGL(accept_greedy_kernel, dim3(blocks), dim3(64), 0, s, t, d, b, m_rows, accept_len,
                       committed);
    return hipGetLastError();
}

hipError_t launch_accept_sample(const float *z, int64_t ldz, const float *q, int64_t ldq,
                                const int32_t *d, const float *u, int32_t m_rows, int32_t v,
                                float temperature, int32_t *accept_len, int32_t *committed, void *ws,
                                hipStream_t s) {
    const int nchunks = (v + CH - 1) / CH;
    hipLaunchKernelGGL(sample_stats_kernel, dim3(nchunks, m_rows), dim3(TPB), 0, s, z, ldz, q, ldq, m_rows, v,
                       temperature, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(sample_decide_kernel, dim3(nchunks), dim3(TPB), 0, s, z, ldz, q, ldq, d, u, m_rows, v,
                       temperature, accept_len, committed, ws);
    return hipGetLastError();
}

}  // namespace dspk

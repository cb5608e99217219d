// Radius -> key-block index lists.
//
// Token Radius Attention for Efficient Video Generation, "The TRA Pipeline:
// Fused CUDA Kernels": distance computation, radius comparison and block
// pruning turn per-query radii into a regular block-sparse mask.  Here the
// distance is Chebyshev on block coordinates (frame, tile row, tile column)
// against the query block's own radius, and each list is compacted with a
// wavefront ballot plus a lane prefix count (mbcnt), in ascending block order.
#include "tra_internal.h"

namespace tra {
namespace {

// One wave64 per (head, query block); four waves per workgroup.
__global__ __launch_bounds__(256) void mask_kernel(const int32_t *__restrict__ radius, Grid g,
                                                   int64_t rows, int r_max, int64_t maxcnt,
                                                   int32_t *__restrict__ idx,
                                                   int32_t *__restrict__ cnt) {
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;
    const int qb = (int)(row % g.nb);
    const int64_t plane = (int64_t)g.nby * g.nbx;
    const int t0 = (int)(qb / plane);
    const int by0 = (int)((qb / g.nbx) % g.nby);
    const int bx0 = qb % g.nbx;

    int64_t r = radius[row];
    r = r < 0 ? 0 : (r > r_max ? r_max : r);
    const int64_t tlo = t0 - r < 0 ? 0 : t0 - r;
    const int64_t thi = t0 + r > g.T - 1 ? g.T - 1 : t0 + r;
    const int64_t first = tlo * plane, end = (thi + 1) * plane;

    int32_t *out = idx + row * maxcnt;
    int64_t count = 0;
    for (int64_t c0 = first; c0 < end; c0 += 64) {
        const int64_t kb = c0 + lane;
        bool keep = false;
        if (kb < end) {
            const int64_t dy = (kb / g.nbx) % g.nby - by0;
            const int64_t dx = kb % g.nbx - bx0;
            keep = (dy < 0 ? -dy : dy) <= r && (dx < 0 ? -dx : dx) <= r;
        }
        const uint64_t bal = __ballot(keep);
        const uint32_t before = __builtin_amdgcn_mbcnt_hi(
            (uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
        const int64_t pos = count + before;
        if (keep && pos < maxcnt) out[pos] = (int32_t)kb;
        count += __popcll(bal);
    }
    if (lane == 0) cnt[row] = (int32_t)(count < maxcnt ? count : maxcnt);
}

}  // namespace

hipError_t launch_mask(const int32_t *radius, const Grid &g, int heads, int r_max, int64_t maxcnt,
                       int32_t *idx, int32_t *cnt, hipStream_t s) {
    const int64_t rows = (int64_t)heads * g.nb;
    hipLaunchKernelGGL(mask_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, radius, g,
                       rows, r_max, maxcnt, idx, cnt);
    return hipGetLastError();
}

}  // namespace tra

namespace tra {
namespace {

// Union of the two key lists of a work item (a pair of vertically adjacent
// query blocks), the walk the attention kernel takes: entries
// (block << 2) | sides, bit 0 set when the upper block keeps the block, bit 1
// when the lower one does.  One wave64 per item.  For strictly ascending lists
// inside [0, nb) (as the radius mask writes them) the union is ascending and
// every block appears once: entry x = A[i] lands at
//   i + |{b in B : b < x}| - |{a in A[0 .. i) : a in B}|
// and an entry y = B[j] that A lacks at j + |{a in A : a < y}| - |{b in B[0 .. j) : b in A}|
// (merge path by binary search).  Other lists are concatenated (the valid
// entries of A, then those of B, each with its own side bit), which keeps the
// attention exact: every query block still sees exactly its own entries.
constexpr int kUnionWaves = 4;

__device__ __forceinline__ int lanes_before(uint64_t bal) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
}

__device__ int lower_bound_list(const int32_t *l, int n, int x) {
    int lo = 0, hi = n;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (l[mid] < x) lo = mid + 1;
        else hi = mid;
    }
    return lo;
}

// True when l[0 .. n) is strictly ascending with every entry in [0, nb).
__device__ bool list_ascending(const int32_t *l, int n, int nb, int lane) {
    int last = -1;
    for (int i0 = 0; i0 < n; i0 += 64) {
        const int i = i0 + lane;
        const int x = i < n ? l[i] : INT32_MAX;
        int prev = __shfl_up(x, 1);
        if (lane == 0) prev = last;
        const bool good = i >= n || ((unsigned)x < (unsigned)nb && x > prev);
        if (__any(!good)) return false;
        last = __shfl(x, min(63, n - 1 - i0));
    }
    return true;
}

// With per-entry log-weights lw (natural log, laid out like idx), every walk
// entry also gets its two blocks' weights in log2 units (ubias; 0 for a side
// that does not keep the block).
__global__ __launch_bounds__(64 * kUnionWaves) void union_kernel(
    const int32_t *__restrict__ idx, const int32_t *__restrict__ cnt,
    const float *__restrict__ lw, int64_t maxcnt, Grid g, int64_t items, int pairs_per_head,
    int64_t ustride, int32_t *__restrict__ ulist, int32_t *__restrict__ ulen,
    float2 *__restrict__ ubias) {
    constexpr float kLog2e = 1.4426950408889634f;
    const int64_t item = (int64_t)blockIdx.x * kUnionWaves + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (item >= items) return;
    const int64_t h = item / pairs_per_head;
    int qa, qb;
    pair_blocks((int)(item % pairs_per_head), g, qa, qb);
    auto len = [&](int b) -> int {
        if (b < 0) return 0;
        const int64_t m = cnt[h * g.nb + b];
        return (int)(m < 0 ? 0 : (m > maxcnt ? maxcnt : m));
    };
    const int32_t *A = idx + (h * g.nb + qa) * maxcnt;
    const int32_t *B = qb >= 0 ? idx + (h * g.nb + qb) * maxcnt : A;
    const float *wA = lw ? lw + (h * g.nb + qa) * maxcnt : nullptr;
    const float *wB = lw ? lw + (h * g.nb + (qb >= 0 ? qb : qa)) * maxcnt : nullptr;
    const int a = len(qa), b = len(qb);
    int32_t *out = ulist + item * ustride;
    float2 *bout = ubias ? ubias + item * ustride : nullptr;
    int n = 0;
    if (list_ascending(A, a, g.nb, lane) && list_ascending(B, b, g.nb, lane)) {
        int common = 0;
        for (int i0 = 0; i0 < a; i0 += 64) {
            const int i = i0 + lane;
            int x = 0, pos = 0;
            bool in_b = false;
            if (i < a) {
                x = A[i];
                pos = lower_bound_list(B, b, x);
                in_b = pos < b && B[pos] == x;
            }
            const uint64_t bal = __ballot(in_b);
            if (i < a) {
                const int64_t o = i + pos - common - lanes_before(bal);
                out[o] = (x << 2) | 1 | (in_b ? 2 : 0);
                if (bout) bout[o] = make_float2(wA[i] * kLog2e, in_b ? wB[pos] * kLog2e : 0.f);
            }
            common += __popcll(bal);
        }
        int common_b = 0;
        for (int j0 = 0; j0 < b; j0 += 64) {
            const int j = j0 + lane;
            int y = 0, pos = 0;
            bool in_a = false;
            if (j < b) {
                y = B[j];
                pos = lower_bound_list(A, a, y);
                in_a = pos < a && A[pos] == y;
            }
            const uint64_t bal = __ballot(in_a);
            if (j < b && !in_a) {
                const int64_t o = j + pos - common_b - lanes_before(bal);
                out[o] = (y << 2) | 2;
                if (bout) bout[o] = make_float2(0.f, wB[j] * kLog2e);
            }
            common_b += __popcll(bal);
        }
        n = a + b - common;
    } else {
#pragma unroll
        for (int side = 0; side < 2; ++side) {
            const int32_t *l = side ? B : A;
            const float *wl = side ? wB : wA;
            const int m = side ? b : a;
            for (int i0 = 0; i0 < m; i0 += 64) {
                const int i = i0 + lane;
                const int x = i < m ? l[i] : -1;
                const bool keep = i < m && (unsigned)x < (unsigned)g.nb;
                const uint64_t bal = __ballot(keep);
                if (keep) {
                    const int64_t o = n + lanes_before(bal);
                    out[o] = (x << 2) | (1 << side);
                    if (bout) {
                        const float w = wl[i] * kLog2e;
                        bout[o] = side ? make_float2(0.f, w) : make_float2(w, 0.f);
                    }
                }
                n += __popcll(bal);
            }
        }
    }
    if (lane == 0) ulen[item] = n;
}

// Work order for the attention kernel.  Workgroup ids are dealt to the eight
// XCDs round robin (id % 8), each XCD with its own L2, so XCD x is given a
// contiguous raster range of the items (neighbouring query blocks of the same
// head share most key tiles).  The ranges are cut at equal shares of the total
// work (walk length plus a fixed per-item cost), not at equal item counts: the
// whole launch waits for its busiest XCD.  A range holds at most `cap` items
// (the cut moves when a range would exceed it).  Each range is taken longest
// first, so that long items do not start last and leave a tail: the k-th
// longest item of range x goes to grid slot 8 k + x, and slots past a range's
// end hold -1.  One workgroup per XCD, each finding all eight cuts the same
// way: per-thread chunk sums, a block scan, a count of the items starting
// below each share; then a histogram of its range's lengths in LDS, a
// descending prefix scan and a scatter (the order among equal lengths is
// arbitrary; results do not depend on it).
constexpr int kOrderThreads = 1024;
constexpr int kOrderMaxBin = 8191;
constexpr int kXcds = 8;
constexpr int kItemCost = 4;  // prologue and epilogue of an item, in walk steps

// Exclusive prefix sum of one value per thread over the block (1024 threads):
// shuffles within each wave, then the 16 wave totals.  Every thread gets its
// exclusive prefix; *total receives the block total.
__device__ int64_t block_exclusive_scan(int64_t v, int64_t *wave_sums, int64_t *total) {
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    int64_t x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int64_t y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    if (lane == 63) wave_sums[wid] = x;
    __syncthreads();
    if (tid == 0) {
        int64_t run = 0;
        for (int w = 0; w < kOrderThreads / 64; ++w) {
            const int64_t t = wave_sums[w];
            wave_sums[w] = run;
            run += t;
        }
        *total = run;
    }
    __syncthreads();
    const int64_t r = wave_sums[wid] + x - v;
    __syncthreads();  // wave_sums may be reused by the next scan
    return r;
}

__global__ __launch_bounds__(kOrderThreads) void order_kernel(const int32_t *__restrict__ ulen,
                                                              int64_t items, int64_t cap,
                                                              int maxlen,
                                                              int32_t *__restrict__ order) {
    extern __shared__ int32_t bins[];  // maxlen + 1 bins
    __shared__ int64_t wave_sums[kOrderThreads / 64];
    __shared__ int64_t below[kXcds];  // items starting below share x / 8 of the work
    __shared__ int64_t total_work, total_bins;
    const int tid = threadIdx.x, x = blockIdx.x;
    auto length_of = [&](int64_t it) -> int {
        const int len = ulen[it];
        return len < 0 ? 0 : (len > maxlen ? maxlen : len);
    };
    // chunk sums and their exclusive block scan
    const int64_t chunk = (items + kOrderThreads - 1) / kOrderThreads;
    const int64_t c0 = min(items, tid * chunk), c1 = min(items, c0 + chunk);
    int64_t mine = 0;
    for (int64_t it = c0; it < c1; ++it) mine += length_of(it) + kItemCost;
    if (tid < kXcds) below[tid] = 0;
    int64_t start = block_exclusive_scan(mine, wave_sums, &total_work);
    const int64_t total = total_work;
    // count, for every share, the items of this chunk starting below it
    {
        int64_t cnt[kXcds] = {};
        for (int64_t it = c0; it < c1; ++it) {
#pragma unroll
            for (int s = 1; s < kXcds; ++s) cnt[s] += start * kXcds < s * total ? 1 : 0;
            start += length_of(it) + kItemCost;
        }
#pragma unroll
        for (int s = 1; s < kXcds; ++s)
            if (cnt[s]) atomicAdd((unsigned long long *)&below[s], (unsigned long long)cnt[s]);
    }
    for (int i = tid; i <= maxlen; i += kOrderThreads) bins[i] = 0;
    __syncthreads();
    // this XCD's range, cut at the shares within the cap
    int64_t lo = 0, hi = 0;
    for (int r = 0; r <= x; ++r) {
        lo = hi;
        hi = r == kXcds - 1 ? items : below[r + 1];
        hi = max(hi, items - cap * (kXcds - 1 - r));  // the rest must fit the later ranges
        hi = min(max(hi, lo), min(items, lo + cap));
    }
    for (int64_t it = lo + tid; it < hi; it += kOrderThreads) atomicAdd(&bins[length_of(it)], 1);
    __syncthreads();
    // descending exclusive scan of the bins (longest lengths first): thread t
    // owns a run of consecutive bins counted from the top
    {
        const int nbins = maxlen + 1;
        const int per = (nbins + kOrderThreads - 1) / kOrderThreads;
        const int b0 = tid * per, b1 = min(nbins, b0 + per);  // positions from the top
        int64_t sum = 0;
        for (int b = b0; b < b1; ++b) sum += bins[maxlen - b];
        int64_t run = block_exclusive_scan(sum, wave_sums, &total_bins);
        for (int b = b0; b < b1; ++b) {
            const int c = bins[maxlen - b];
            bins[maxlen - b] = (int)run;
            run += c;
        }
    }
    __syncthreads();
    for (int64_t it = lo + tid; it < hi; it += kOrderThreads) {
        const int64_t k = atomicAdd(&bins[length_of(it)], 1);
        order[kXcds * k + x] = (int32_t)it;
    }
    for (int64_t k = (hi - lo) + tid; k < cap; k += kOrderThreads) order[kXcds * k + x] = -1;
}

// Sampling with inclusion-probability weights (AB-Attention speeds up video
// diffusion transformers up to 2.23x, second paragraph): per (head, query
// block Q), importance p_K = softmax of the pooled logits over every key
// block, inclusion pi_K = min(1, m p_K) (pi_Q = 1: the own block is always
// kept), key block K kept when the caller's uniform u_QK < pi_K, with
// log-weight -ln pi_K.  One wave64 per row: a max and a sum over the row,
// then ballot compaction in ascending block order.
__global__ __launch_bounds__(256) void sip_kernel(const float *__restrict__ logits,
                                                  const float *__restrict__ u, int64_t rows,
                                                  int nb, float m, int64_t maxcnt,
                                                  int32_t *__restrict__ idx,
                                                  int32_t *__restrict__ cnt,
                                                  float *__restrict__ lw) {
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;
    const int qb = (int)(row % nb);
    const float *lr = logits + row * nb;
    const float *ur = u + row * nb;
    constexpr float kLog2e = 1.4426950408889634f;
    float mx = -INFINITY;
    for (int c = lane; c < nb; c += 64) mx = fmaxf(mx, lr[c]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    float z = 0.f;
    for (int c = lane; c < nb; c += 64) z += __builtin_amdgcn_exp2f((lr[c] - mx) * kLog2e);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) z += __shfl_xor(z, off);
    const float mz = m / z;
    int32_t *out = idx + row * maxcnt;
    float *wout = lw + row * maxcnt;
    int64_t count = 0;
    for (int c0 = 0; c0 < nb; c0 += 64) {
        const int c = c0 + lane;
        bool keep = false;
        float pi = 1.f;
        if (c < nb) {
            pi = c == qb ? 1.f : fminf(1.f, mz * __builtin_amdgcn_exp2f((lr[c] - mx) * kLog2e));
            keep = ur[c] < pi;
        }
        const uint64_t bal = __ballot(keep);
        const int64_t pos = count + lanes_before(bal);
        if (keep && pos < maxcnt) {
            out[pos] = c;
            wout[pos] = -0.69314718055994531f * __builtin_amdgcn_logf(pi);
        }
        count += __popcll(bal);
    }
    if (lane == 0) cnt[row] = (int32_t)(count < maxcnt ? count : maxcnt);
}

}  // namespace

int64_t union_stride(int64_t maxcnt) { return (2 * maxcnt + 63) / 64 * 64; }

hipError_t launch_union(const int32_t *idx, const int32_t *cnt, const float *lw, int64_t maxcnt,
                        const Grid &g, int heads, int32_t *ulist, int32_t *ulen, float2 *ubias,
                        hipStream_t s) {
    const int pph = pairs_per_head(g);
    const int64_t items = (int64_t)heads * pph;
    hipLaunchKernelGGL(union_kernel, dim3((unsigned)((items + kUnionWaves - 1) / kUnionWaves)),
                       dim3(64 * kUnionWaves), 0, s, idx, cnt, lw, maxcnt, g, items, pph,
                       union_stride(maxcnt), ulist, ulen, ubias);
    return hipGetLastError();
}

hipError_t launch_order(const int32_t *ulen, const Grid &g, int heads, int64_t maxcnt,
                        int32_t *order, hipStream_t s) {
    const int64_t items = (int64_t)heads * pairs_per_head(g);
    // lengths above kOrderMaxBin share the top bin (they still start first)
    const int maxlen = (int)(2 * maxcnt < kOrderMaxBin ? 2 * maxcnt : kOrderMaxBin);
    const size_t lds = (size_t)(maxlen + 1) * sizeof(int32_t);
    hipLaunchKernelGGL(order_kernel, dim3(kXcds), dim3(kOrderThreads), lds, s, ulen, items,
                       order_range_cap(g, heads), maxlen, order);
    return hipGetLastError();
}

}  // namespace tra

namespace tra {

hipError_t launch_sip(const float *logits, const float *u, const Grid &g, int heads, float m,
                      int32_t *idx, int32_t *cnt, float *lw, hipStream_t s) {
    const int64_t rows = (int64_t)heads * g.nb;
    hipLaunchKernelGGL(sip_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, logits, u,
                       rows, g.nb, m, (int64_t)g.nb, idx, cnt, lw);
    return hipGetLastError();
}

}  // namespace tra

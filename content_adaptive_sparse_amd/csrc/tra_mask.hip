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

// Work order for the attention kernel: the (head, query-block pair) items
// sorted by descending list length of the longer list of the pair, so that
// the longest items start first and the grid does not end on a long tail.
// One workgroup: histogram of lengths in LDS, a descending prefix scan, then a
// scatter (the order among equal lengths is arbitrary; results do not depend
// on it).
constexpr int kOrderThreads = 1024;
constexpr int kOrderMaxBin = 8191;

__global__ __launch_bounds__(kOrderThreads) void order_kernel(const int32_t *__restrict__ cnt,
                                                              Grid g, int64_t items,
                                                              int pairs_per_head, int maxlen,
                                                              int32_t *__restrict__ order) {
    extern __shared__ int32_t bins[];  // maxlen + 1 bins
    const int tid = threadIdx.x;
    for (int i = tid; i <= maxlen; i += kOrderThreads) bins[i] = 0;
    __syncthreads();
    auto length_of = [&](int64_t it) -> int {
        const int64_t h = it / pairs_per_head;
        int qa, qb;
        pair_blocks((int)(it % pairs_per_head), g, qa, qb);
        const int32_t *row = cnt + h * g.nb;
        int len = row[qa];
        if (qb >= 0) len = max(len, (int)row[qb]);
        return len < 0 ? 0 : (len > maxlen ? maxlen : len);
    };
    for (int64_t it = tid; it < items; it += kOrderThreads) atomicAdd(&bins[length_of(it)], 1);
    __syncthreads();
    if (tid == 0) {  // descending exclusive scan: longest lengths first
        int run = 0;
        for (int len = maxlen; len >= 0; --len) {
            const int c = bins[len];
            bins[len] = run;
            run += c;
        }
    }
    __syncthreads();
    for (int64_t it = tid; it < items; it += kOrderThreads) {
        const int slot = atomicAdd(&bins[length_of(it)], 1);
        order[slot] = (int32_t)it;
    }
}

}  // namespace

hipError_t launch_order(const int32_t *cnt, const Grid &g, int heads, int64_t maxcnt,
                        int32_t *order, hipStream_t s) {
    const int pph = pairs_per_head(g);
    const int64_t items = (int64_t)heads * pph;
    // lengths above kOrderMaxBin share the top bin (they still start first)
    const int maxlen = (int)(maxcnt < kOrderMaxBin ? maxcnt : kOrderMaxBin);
    const size_t lds = (size_t)(maxlen + 1) * sizeof(int32_t);
    hipLaunchKernelGGL(order_kernel, dim3(1), dim3(kOrderThreads), lds, s, cnt, g, items, pph,
                       maxlen, order);
    return hipGetLastError();
}

}  // namespace tra

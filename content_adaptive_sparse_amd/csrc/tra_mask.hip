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

// Work items: which two query blocks of a head share one attention workgroup
// (and its copied key/value tiles).  Neighbouring blocks -- vertically adjacent
// ones (tile rows 2 p and 2 p + 1 of one frame and column: short-axis
// neighbours, whose lists mostly coincide), or, in a head whose temporal pairs
// (one tile in frames 2 p and 2 p + 1) make walks at least 5% shorter in
// total, temporally adjacent ones (token-voted lists coincide more in time) --
// stay together when their list lengths are within a factor of two.  The
// blocks of every other neighbour pair are re-paired by length class: sorted
// by a key of four classes per octave of the length, longest first and in
// raster order inside a class, and paired in that order, so that a block that
// keeps every key block (binary routing) shares its walk with another such
// block instead of idling half the workgroup beside a short list.  (A plan
// built from radii pairs by radius instead; see pair_kernel.)  One workgroup
// of 1024 threads per head writes the head's plan_slots_per_head item slots:
// the kept neighbour pairs in raster order, then the re-paired ones, then
// unused slots (-1, -1).  The counting sort is stable: a chunk's ranks inside
// each class come from a 1024-bit membership mask.
constexpr int kScanThreads = 1024;

// Exclusive prefix sum of one value per thread over the block (1024 threads):
// shuffles within each wave, then the same over the 16 wave totals in the
// first wave.  Every thread gets its exclusive prefix; *total receives the
// block total.
__device__ int64_t block_exclusive_scan(int64_t v, int64_t *wave_sums, int64_t *total) {
    constexpr int kWaves = kScanThreads / 64;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    int64_t x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int64_t y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    if (lane == 63) wave_sums[wid] = x;
    __syncthreads();
    if (wid == 0) {
        int64_t w = lane < kWaves ? wave_sums[lane] : 0;
#pragma unroll
        for (int off = 1; off < kWaves; off <<= 1) {
            const int64_t y = __shfl_up(w, off);
            if (lane >= off) w += y;
        }
        if (lane < kWaves) wave_sums[lane] = w;  // inclusive
        if (lane == kWaves - 1) *total = w;
    }
    __syncthreads();
    const int64_t r = (wid ? wave_sums[wid - 1] : 0) + x - v;
    __syncthreads();  // wave_sums may be reused by the next scan
    return r;
}

// Lanes below this one whose ballot bit is set.
__device__ __forceinline__ int lanes_before(uint64_t bal) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
}

constexpr int kPairThreads = kScanThreads;
constexpr int kPairClasses = 128;
// The neighbour direction of a list plan is judged on every kCandidateStride-th
// candidate pair of a head (pair index 0, 4, 8, ...).
constexpr int kCandidateStride = 4;
__host__ __device__ inline int candidates(int pairs) {
    return (pairs + kCandidateStride - 1) / kCandidateStride;
}

__device__ __forceinline__ int length_class(int c) {
    const uint32_t x = (uint32_t)(c < 0 ? 0 : c) + 1u;
    const int e = 31 - __builtin_clz(x);  // floor(log2 x) <= 30
    const uint32_t f = e >= 2 ? (x >> (e - 2)) & 3u : (x << (2 - e)) & 3u;
    return 4 * e + (int)f;  // < 124
}

__device__ __forceinline__ bool lengths_pair_well(int a, int b) {
    return 2 * (int64_t)min(a, b) >= (int64_t)max(a, b);
}

// The key blocks of query block b within Chebyshev radius r (clamped to
// [0, r_max] as the radius mask clamps it) in block coordinates: a box of the
// (frame, tile row, tile column) grid.
struct KeyBox {
    int t0, t1, y0, y1, x0, x1;  // inclusive bounds; t0 > t1 when empty
    __device__ bool contains(int t, int y, int x) const {
        return t >= t0 && t <= t1 && y >= y0 && y <= y1 && x >= x0 && x <= x1;
    }
};

__device__ KeyBox key_box(int b, int32_t radius, int r_max, const Grid &g) {
    const int64_t r = radius < 0 ? 0 : (radius > r_max ? r_max : radius);
    const int plane = g.nby * g.nbx;
    const int t = b / plane, y = (b / g.nbx) % g.nby, x = b % g.nbx;
    KeyBox k;
    k.t0 = (int)max((int64_t)0, t - r);
    k.t1 = (int)min((int64_t)g.T - 1, t + r);
    k.y0 = (int)max((int64_t)0, y - r);
    k.y1 = (int)min((int64_t)g.nby - 1, y + r);
    k.x0 = (int)max((int64_t)0, x - r);
    k.x1 = (int)min((int64_t)g.nbx - 1, x + r);
    return k;
}

// cnt: list lengths; or, with radius non-null, the radius mask's lists known
// by their radii.  Then vertical neighbours stay together when their radii are
// equal (their key boxes then differ by at most one tile row), and the other
// blocks are classed by radius, largest first, and paired in (frame, tile
// column, tile row) order inside a class, so that a pair's two boxes are the
// same box shifted by a tile or two: at the Wan 81-frame layer's probe radii
// the walks' slot efficiency is 0.92 instead of 0.87 with the length rule, and
// the walks take 6% fewer steps.  (Pairing does not change any result: each
// block meets its own entries in ascending order whatever its partner.)
// wlen (list mode): the walk lengths of a sample of every head's vertical,
// then temporal candidate pairs (candidate_walk_kernel), which choose the
// neighbours: temporal ones when their sampled walks take at least 5% fewer
// steps per list entry.
__global__ __launch_bounds__(kPairThreads) void pair_kernel(const int32_t *__restrict__ cnt,
                                                           const int32_t *__restrict__ radius,
                                                           const int32_t *__restrict__ wlen,
                                                           int r_max, int64_t maxcnt, Grid g,
                                                           int slots, int2 *__restrict__ pairs) {
    __shared__ int64_t wave_sums[kPairThreads / 64];
    __shared__ int64_t total_sh;
    __shared__ int start[kPairClasses], run[kPairClasses];
    __shared__ uint32_t member[kPairClasses][kPairThreads / 32];
    const int h = blockIdx.x, tid = threadIdx.x;
    const int32_t *ch = radius ? radius + (int64_t)h * g.nb : cnt + (int64_t)h * g.nb;
    int2 *out = pairs + (int64_t)h * slots;
    const int plane = g.nby * g.nbx;
    auto len = [&](int b) -> int {  // list mode
        const int64_t m = ch[b];
        return (int)(m < 0 ? 0 : (m > maxcnt ? maxcnt : m));
    };
    // temporal neighbours when the sampled temporal candidates' walks hold at
    // least 5% fewer steps per list entry than the vertical ones'
    bool temporal = false;
    if (wlen) {
        const int vs = candidates(pairs_per_head(g)), ts = candidates(temporal_pairs_per_head(g));
        const int32_t *wv = wlen + (int64_t)h * vs;
        const int32_t *wt = wlen + (int64_t)gridDim.x * vs + (int64_t)h * ts;
        int64_t uv = 0, lv = 0, ut = 0, lt = 0;  // walk steps and list entries
        for (int i = tid; i < vs; i += kPairThreads) {
            int qa, qb;
            pair_blocks(i * kCandidateStride, g, qa, qb);
            uv += wv[i];
            lv += len(qa) + (qb >= 0 ? len(qb) : 0);
        }
        for (int i = tid; i < ts; i += kPairThreads) {
            int qa, qb;
            temporal_pair_blocks(i * kCandidateStride, g, qa, qb);
            ut += wt[i];
            lt += len(qa) + (qb >= 0 ? len(qb) : 0);
        }
        int64_t tot[4];
        const int64_t part[4] = {uv, lv, ut, lt};
        for (int j = 0; j < 4; ++j) {
            block_exclusive_scan(part[j], wave_sums, &total_sh);
            tot[j] = total_sh;
        }
        // ut / lt < 0.95 uv / lv (in double: the products may pass 2^63)
        temporal = 20.0 * (double)tot[2] * (double)tot[1] < 19.0 * (double)tot[0] * (double)tot[3];
    }
    // the neighbour of block b (-1 when its tile row, or frame, has none)
    auto partner = [&](int b) -> int {
        if (temporal) {
            const int t = b / plane;
            const int o = (t & 1) ? b - plane : b + plane;
            return ((t & 1) || t + 1 < g.T) ? o : -1;
        }
        const int by = (b / g.nbx) % g.nby;
        const int o = (by & 1) ? b - g.nbx : b + g.nbx;
        return ((by & 1) || by + 1 < g.nby) ? o : -1;
    };
    auto rad = [&](int b) -> int {
        const int32_t r = ch[b];
        return r < 0 ? 0 : (r > r_max ? r_max : r);
    };
    auto well = [&](int a, int b) -> bool {
        return radius ? rad(a) == rad(b) : lengths_pair_well(len(a), len(b));
    };
    auto klass = [&](int b) -> int {
        return radius ? min(rad(b), kPairClasses - 1) : length_class(len(b));
    };
    auto orphan = [&](int b) -> bool {
        const int o = partner(b);
        return o >= 0 && !well(b, o);
    };
    // the i-th block of the orphan order: raster, or (frame, column, row) for radii
    auto block_at = [&](int i) -> int {
        if (!radius) return i;
        const int t = i / plane, rem = i - t * plane;
        const int x = rem / g.nby, y = rem - x * g.nby;
        return (t * g.nby + y) * g.nbx + x;
    };
    // kept neighbour pairs, compacted in raster order
    const int npairs = temporal ? temporal_pairs_per_head(g) : pairs_per_head(g);
    int64_t kept = 0;
    for (int p0 = 0; p0 < npairs; p0 += kPairThreads) {
        const int p = p0 + tid;
        int qa = -1, qb = -1;
        bool keep = false;
        if (p < npairs) {
            if (temporal)
                temporal_pair_blocks(p, g, qa, qb);
            else
                pair_blocks(p, g, qa, qb);
            keep = qb < 0 || well(qa, qb);
        }
        int64_t tot;
        const int64_t at = block_exclusive_scan(keep ? 1 : 0, wave_sums, &total_sh);
        tot = total_sh;
        if (keep) out[kept + at] = make_int2(qa, qb);
        kept += tot;
        __syncthreads();
    }
    // orphans per length class, longest class first
    for (int k = tid; k < kPairClasses; k += kPairThreads) start[k] = run[k] = 0;
    __syncthreads();
    for (int b = tid; b < g.nb; b += kPairThreads)
        if (orphan(b)) atomicAdd(&start[klass(b)], 1);
    __syncthreads();
    int64_t norph = 0;
    if (tid == 0) {
        int acc = 0;
        for (int k = kPairClasses - 1; k >= 0; --k) {
            const int c = start[k];
            start[k] = acc;
            acc += c;
        }
        total_sh = acc;
    }
    __syncthreads();
    norph = total_sh;
    // stable scatter: position = class start + earlier orphans of the class
    for (int b0 = 0; b0 < g.nb; b0 += kPairThreads) {
        for (int i = tid; i < kPairClasses * (kPairThreads / 32); i += kPairThreads)
            (&member[0][0])[i] = 0u;
        __syncthreads();
        const int b = b0 + tid < g.nb ? block_at(b0 + tid) : g.nb;
        const bool orph = b < g.nb && orphan(b);
        const int k = orph ? klass(b) : 0;
        if (orph) atomicOr(&member[k][tid >> 5], 1u << (tid & 31));
        __syncthreads();
        if (orph) {
            int rank = __popc(member[k][tid >> 5] & ((1u << (tid & 31)) - 1u));
            for (int w = 0; w < (tid >> 5); ++w) rank += __popc(member[k][w]);
            const int64_t pos = start[k] + run[k] + rank;
            int *slot = reinterpret_cast<int *>(out + kept + pos / 2) + (pos & 1);
            *slot = b;
        }
        __syncthreads();
        for (int kk = tid; kk < kPairClasses; kk += kPairThreads) {
            int c = 0;
            for (int w = 0; w < kPairThreads / 32; ++w) c += __popc(member[kk][w]);
            run[kk] += c;
        }
        __syncthreads();
    }
    // an odd orphan count leaves the last item single; unused slots after it
    const int64_t used = kept + (norph + 1) / 2;
    if (tid == 0 && (norph & 1)) reinterpret_cast<int *>(out + kept + norph / 2)[1] = -1;
    for (int64_t i = used + tid; i < slots; i += kPairThreads) out[i] = make_int2(-1, -1);
}

// The pair table of the radius mask's lists, from the radii, frame by frame
// (the limits: at most kPairMaxPlane tiles per frame, kPairMaxFrames frames
// and kPairMaxOrphans blocks; pair_kernel's radius mode otherwise).  Vertical
// neighbours (tile rows 2 p, 2 p + 1) stay together when their radii are equal
// (their key boxes then differ by at most one tile row); the other blocks of a
// frame are ordered by radius, largest first, then tile column, then tile row,
// the frames one after another, and paired in that order, so that a pair's two
// boxes are one box shifted by a tile or two.  The items are listed frame by
// frame -- each frame's kept pairs in raster order, then the re-paired items
// whose first block lies in that frame -- so that the work order's contiguous
// XCD ranges hold neighbouring frames and their key tiles share each XCD's L2.
// One workgroup of 1024 threads per head; one wave per frame at a time.
constexpr int kPairMaxPlane = 256;
constexpr int kPairMaxFrames = 1024;
constexpr int kPairMaxOrphans = 8192;
constexpr int kNoKey = 0x7fffffff;

__global__ __launch_bounds__(kPairThreads) void pair_radius_kernel(const int32_t *__restrict__ radius,
                                                                  int r_max, Grid g, int slots,
                                                                  int2 *__restrict__ pairs) {
    constexpr int kWaves = kPairThreads / 64;
    __shared__ int kcnt[kPairMaxFrames + 1];  // kept items per frame, then their prefix
    __shared__ int ocnt[kPairMaxFrames + 1];  // re-paired blocks per frame, then their prefix
    __shared__ int okey[kWaves][kPairMaxPlane];
    __shared__ int oseq[kPairMaxOrphans];  // the re-paired blocks in pairing order
    __shared__ int64_t wave_sums[kWaves];
    __shared__ int64_t total_sh;
    const int h = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int plane = g.nby * g.nbx, npy = (g.nby + 1) / 2, fslots = npy * g.nbx;
    const int32_t *rh = radius + (int64_t)h * g.nb;
    int2 *out = pairs + (int64_t)h * slots;
    auto rad = [&](int b) -> int {
        const int32_t r = rh[b];
        return r < 0 ? 0 : (r > r_max ? r_max : r);
    };
    // block j = y nbx + x of frame f: its re-pairing key, or kNoKey when it
    // stays with its vertical neighbour (equal radii) or has none
    auto okey_of = [&](int f, int j) -> int {
        const int y = j / g.nbx, x = j - y * g.nbx;
        if ((y ^ 1) >= g.nby) return kNoKey;
        const int r = rad(f * plane + j);
        if (r == rad(f * plane + (y ^ 1) * g.nbx + x)) return kNoKey;
        return (kPairClasses - 1 - min(r, kPairClasses - 1)) * plane + x * g.nby + y;
    };
    // pair slot p of frame f (tile-row pair p / nbx, column p % nbx)
    auto slot_blocks = [&](int f, int p, int &qa, int &qb) {
        const int pr = p / g.nbx, x = p - pr * g.nbx;
        qa = (f * g.nby + 2 * pr) * g.nbx + x;
        qb = 2 * pr + 1 < g.nby ? qa + g.nbx : -1;
    };
    auto kept_slot = [&](int f, int p) -> bool {
        int qa, qb;
        slot_blocks(f, p, qa, qb);
        return qb < 0 || rad(qa) == rad(qb);
    };
    // 1. per frame: kept items and re-paired blocks
    for (int f0 = 0; f0 < g.T; f0 += kWaves) {
        const int f = f0 + wave;
        if (f < g.T) {
            int kc = 0, oc = 0;
            for (int p0 = 0; p0 < fslots; p0 += 64)
                kc += __popcll(__ballot(p0 + lane < fslots && kept_slot(f, p0 + lane)));
            for (int j0 = 0; j0 < plane; j0 += 64)
                oc += __popcll(__ballot(j0 + lane < plane && okey_of(f, j0 + lane) != kNoKey));
            if (lane == 0) {
                kcnt[f] = kc;
                ocnt[f] = oc;
            }
        }
    }
    __syncthreads();
    // 2. exclusive prefixes over the frames (one frame per thread)
    {
        const int64_t kv = tid < g.T ? kcnt[tid] : 0, ov = tid < g.T ? ocnt[tid] : 0;
        const int64_t kx = block_exclusive_scan(kv, wave_sums, &total_sh);
        const int ktot = (int)total_sh;
        const int64_t ox = block_exclusive_scan(ov, wave_sums, &total_sh);
        const int otot = (int)total_sh;
        if (tid < g.T) {
            kcnt[tid] = (int)kx;
            ocnt[tid] = (int)ox;
        }
        if (tid == 0) {
            kcnt[g.T] = ktot;
            ocnt[g.T] = otot;
        }
    }
    __syncthreads();
    // 3. the re-paired blocks in order: frame, then key (rank among the frame's keys)
    for (int f0 = 0; f0 < g.T; f0 += kWaves) {
        const int f = f0 + wave;
        if (f < g.T)
            for (int j = lane; j < plane; j += 64) okey[wave][j] = okey_of(f, j);
        __syncthreads();
        if (f < g.T) {
            for (int j = lane; j < plane; j += 64) {
                const int my = okey[wave][j];
                if (my == kNoKey) continue;
                int rank = 0;
                for (int k = 0; k < plane; ++k) rank += okey[wave][k] < my ? 1 : 0;
                oseq[ocnt[f] + rank] = f * plane + j;
            }
        }
        __syncthreads();
    }
    // 4. the items, frame by frame: a frame's kept pairs, then the re-paired
    //    items whose first block lies in it
    const int norph = ocnt[g.T];
    const int nitems_orph = (norph + 1) / 2;
    const int used = kcnt[g.T] + nitems_orph;
    for (int f0 = 0; f0 < g.T; f0 += kWaves) {
        const int f = f0 + wave;
        if (f >= g.T) continue;
        int base = kcnt[f] + (ocnt[f] + 1) / 2;
        for (int p0 = 0; p0 < fslots; p0 += 64) {
            const int p = p0 + lane;
            const bool keep = p < fslots && kept_slot(f, p);
            const uint64_t bal = __ballot(keep);
            if (keep) {
                int qa, qb;
                slot_blocks(f, p, qa, qb);
                out[base + lanes_before(bal)] = make_int2(qa, qb);
            }
            base += __popcll(bal);
        }
    }
    for (int j = tid; j < nitems_orph; j += kPairThreads) {
        const int first = oseq[2 * j];
        const int second = 2 * j + 1 < norph ? oseq[2 * j + 1] : -1;
        const int f = first / plane;
        out[kcnt[f + 1] + j] = make_int2(first, second);
    }
    for (int64_t i = used + tid; i < slots; i += kPairThreads) out[i] = make_int2(-1, -1);
}

// Union of the two key lists of a work item (a pair of query blocks from the
// pair table), the walk the attention kernel takes: entries
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
    const float *__restrict__ lw, int64_t maxcnt, Grid g, int64_t items, int slots,
    const int2 *__restrict__ pairs, int64_t ustride, int32_t *__restrict__ ulist,
    int32_t *__restrict__ ulen, float2 *__restrict__ ubias) {
    constexpr float kLog2e = 1.4426950408889634f;
    const int64_t item = (int64_t)blockIdx.x * kUnionWaves + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (item >= items) return;
    const int64_t h = item / slots;
    const int2 pr = pairs[item];
    const int qa = pr.x, qb = pr.y;
    if (qa < 0) {  // an unused item slot: an empty walk
        if (lane == 0) ulen[item] = 0;
        return;
    }
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

// Walk length of a sample of the candidate pairs of a list set -- every
// kCandidateStride-th vertical pair of each head, then (after all heads) every
// kCandidateStride-th temporal pair -- as union_kernel makes it: |A| + |B| -
// |A n B| for strictly ascending lists inside [0, nb), else |A| + |B|.  One
// wave64 per candidate; pair_kernel sums them per head to choose the
// neighbours it keeps together.
__global__ __launch_bounds__(64 * kUnionWaves) void candidate_walk_kernel(
    const int32_t *__restrict__ idx, const int32_t *__restrict__ cnt, int64_t maxcnt, Grid g,
    int heads, int32_t *__restrict__ wlen) {
    const int vs = candidates(pairs_per_head(g)), ts = candidates(temporal_pairs_per_head(g));
    const int64_t nv = (int64_t)heads * vs, items = nv + (int64_t)heads * ts;
    const int64_t c = (int64_t)blockIdx.x * kUnionWaves + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (c >= items) return;
    int64_t h;
    int qa, qb;
    if (c < nv) {
        h = c / vs;
        pair_blocks((int)(c - h * vs) * kCandidateStride, g, qa, qb);
    } else {
        h = (c - nv) / ts;
        temporal_pair_blocks((int)(c - nv - h * ts) * kCandidateStride, g, qa, qb);
    }
    auto len = [&](int b) -> int {
        if (b < 0) return 0;
        const int64_t m = cnt[h * g.nb + b];
        return (int)(m < 0 ? 0 : (m > maxcnt ? maxcnt : m));
    };
    const int a = len(qa), b = len(qb);
    const int32_t *A = idx + (h * g.nb + qa) * maxcnt;
    const int32_t *B = qb >= 0 ? idx + (h * g.nb + qb) * maxcnt : A;
    int n = a + b;
    if (b > 0 && list_ascending(A, a, g.nb, lane) && list_ascending(B, b, g.nb, lane)) {
        for (int i0 = 0; i0 < a; i0 += 64) {
            const int i = i0 + lane;
            bool in_b = false;
            if (i < a) {
                const int x = A[i];
                const int pos = lower_bound_list(B, b, x);
                in_b = pos < b && B[pos] == x;
            }
            n -= __popcll(__ballot(in_b));
        }
    }
    if (lane == 0) wlen[c] = n;
}

// The walk of a work item straight from the two blocks' radii: the union of
// their key boxes in ascending block order, each entry (block << 2) | sides --
// exactly what union_kernel makes of the radius mask's lists for the same two
// blocks, without the lists.  One wave64 per item scans the frames either box
// touches, 64 candidate blocks at a time, and compacts with a ballot.
__global__ __launch_bounds__(64 * kUnionWaves) void radius_walk_kernel(
    const int32_t *__restrict__ radius, int r_max, Grid g, int64_t items, int slots,
    const int2 *__restrict__ pairs, int64_t ustride, int32_t *__restrict__ ulist,
    int32_t *__restrict__ ulen) {
    const int64_t item = (int64_t)blockIdx.x * kUnionWaves + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (item >= items) return;
    const int64_t h = item / slots;
    const int2 pr = pairs[item];
    if (pr.x < 0) {  // an unused item slot: an empty walk
        if (lane == 0) ulen[item] = 0;
        return;
    }
    const int32_t *rh = radius + h * g.nb;
    const KeyBox A = key_box(pr.x, rh[pr.x], r_max, g);
    KeyBox B = A;
    if (pr.y >= 0) B = key_box(pr.y, rh[pr.y], r_max, g);
    const int plane = g.nby * g.nbx;
    const int first = min(A.t0, B.t0) * plane, end = (max(A.t1, B.t1) + 1) * plane;
    const bool single = pr.y < 0;
    int32_t *out = ulist + item * ustride;
    int64_t n = 0;
    for (int c0 = first; c0 < end; c0 += 64) {
        const int kb = c0 + lane;
        int sides = 0;
        if (kb < end) {
            const int t = kb / plane, rem = kb - t * plane;
            const int y = rem / g.nbx, x = rem - y * g.nbx;
            sides = (A.contains(t, y, x) ? 1 : 0) | (!single && B.contains(t, y, x) ? 2 : 0);
        }
        const uint64_t bal = __ballot(sides != 0);
        const int64_t o = n + lanes_before(bal);
        if (sides && o < ustride) out[o] = (kb << 2) | sides;
        n += __popcll(bal);
    }
    if (lane == 0) ulen[item] = (int32_t)(n < ustride ? n : ustride);
}

// Work order for the attention kernel.  Workgroup ids are dealt to the eight
// XCDs round robin (id % 8), each XCD with its own L2, so XCD x is given a
// contiguous range of the items (plans list them frame by frame, so a range
// holds neighbouring query blocks of one or two heads, which share most key
// tiles in that XCD's L2).  The ranges are cut at equal shares of the total
// work (walk length plus a fixed per-item cost), not at equal item counts:
// the whole launch waits for its busiest XCD.  A range holds at most `cap`
// items (the cut moves when a range would exceed it).  Each range is taken by
// length class, longest class first (two classes per octave of the walk
// length), in item order inside a class: long items do not start last and
// leave a tail, and the items that run together on an XCD still come from
// neighbouring frames (exact longest-first scattered them over the range and
// measured 4-5% slower on the larger layers).  The k-th item of range x in
// that order goes to grid slot 8 k + x, and slots past a range's end hold -1;
// the eight range lengths follow the slots.
// One workgroup per XCD, each finding all eight cuts the same way: per-thread
// chunk sums, a block scan, the item whose work spans each share; then the
// class counts of its range, a descending prefix and a stable scatter.
constexpr int kOrderThreads = kScanThreads;
constexpr int kOrderMaxBin = 8191;
constexpr int kXcds = 8;
constexpr int kItemCost = 4;  // prologue and epilogue of an item, in walk steps
constexpr int kOrderRegItems = 8;  // chunk lengths held in registers (items <= 8192)
constexpr int kOrderClasses = 32;  // two per octave of lengths up to 2^15

// Length class: the length itself below 4, else two classes per octave.
__device__ __forceinline__ int order_class(int len) {
    if (len <= 3) return len;
    const int e = 31 - __builtin_clz((uint32_t)len);
    return 2 * e + ((len >> (e - 1)) & 1);
}

__global__ __launch_bounds__(kOrderThreads) void order_kernel(const int32_t *__restrict__ ulen,
                                                              int64_t items, int64_t cap,
                                                              int maxlen,
                                                              int32_t *__restrict__ order) {
    __shared__ int64_t wave_sums[kOrderThreads / 64];
    __shared__ int64_t below[kXcds];  // items starting below share x / 8 of the work
    __shared__ int64_t total_work;
    __shared__ int cstart[kOrderClasses], crun[kOrderClasses];
    __shared__ uint32_t member[kOrderClasses][kOrderThreads / 32];
    const int tid = threadIdx.x, x = blockIdx.x;
    auto length_of = [&](int64_t it) -> int {
        const int len = ulen[it];
        return len < 0 ? 0 : (len > maxlen ? maxlen : len);
    };
    // chunk sums and their exclusive block scan (a chunk of up to
    // kOrderRegItems lengths is loaded once, all loads in flight together)
    const int64_t chunk = (items + kOrderThreads - 1) / kOrderThreads;
    const int64_t c0 = min(items, tid * chunk), c1 = min(items, c0 + chunk);
    const bool in_regs = chunk <= kOrderRegItems;
    int len_reg[kOrderRegItems];
    int64_t mine = 0;
    if (in_regs) {
#pragma unroll
        for (int i = 0; i < kOrderRegItems; ++i) len_reg[i] = c0 + i < c1 ? length_of(c0 + i) : 0;
#pragma unroll
        for (int i = 0; i < kOrderRegItems; ++i) mine += c0 + i < c1 ? len_reg[i] + kItemCost : 0;
    } else {
        for (int64_t it = c0; it < c1; ++it) mine += length_of(it) + kItemCost;
    }
    if (tid < kXcds) below[tid] = tid == 0 ? 0 : items;
    int64_t start = block_exclusive_scan(mine, wave_sums, &total_work);
    const int64_t total = total_work;
    // below[s] = the number of items whose work starts below share s of the
    // total (8 start < s total).  Starts increase strictly (every item costs
    // at least kItemCost), so that count is one past the item whose work
    // interval [8 start, 8 (start + w)) holds s total: its thread writes it.
    {
        auto mark = [&](int64_t it, int64_t w) {
#pragma unroll
            for (int s = 1; s < kXcds; ++s)
                if (start * kXcds < s * total && s * total <= (start + w) * kXcds) below[s] = it + 1;
            start += w;
        };
        if (in_regs) {
#pragma unroll
            for (int i = 0; i < kOrderRegItems; ++i)
                if (c0 + i < c1) mark(c0 + i, len_reg[i] + kItemCost);
        } else {
            for (int64_t it = c0; it < c1; ++it) mark(it, length_of(it) + kItemCost);
        }
    }
    for (int k = tid; k < kOrderClasses; k += kOrderThreads) cstart[k] = crun[k] = 0;
    __syncthreads();
    // this XCD's range, cut at the shares within the cap
    int64_t lo = 0, hi = 0;
    for (int r = 0; r <= x; ++r) {
        lo = hi;
        hi = r == kXcds - 1 ? items : below[r + 1];
        hi = max(hi, items - cap * (kXcds - 1 - r));  // the rest must fit the later ranges
        hi = min(max(hi, lo), min(items, lo + cap));
    }
    // class counts, then their descending exclusive prefix (longest class first)
    for (int64_t it = lo + tid; it < hi; it += kOrderThreads)
        atomicAdd(&cstart[order_class(length_of(it))], 1);
    __syncthreads();
    if (tid == 0) {
        int acc = 0;
        for (int k = kOrderClasses - 1; k >= 0; --k) {
            const int c = cstart[k];
            cstart[k] = acc;
            acc += c;
        }
    }
    __syncthreads();
    // stable scatter in chunks of the range: slot = class start + earlier items of the class
    for (int64_t c0 = lo; c0 < hi; c0 += kOrderThreads) {
        for (int i = tid; i < kOrderClasses * (kOrderThreads / 32); i += kOrderThreads)
            (&member[0][0])[i] = 0u;
        __syncthreads();
        const int64_t it = c0 + tid;
        const bool in = it < hi;
        const int k = in ? order_class(length_of(it)) : 0;
        if (in) atomicOr(&member[k][tid >> 5], 1u << (tid & 31));
        __syncthreads();
        if (in) {
            int rank = __popc(member[k][tid >> 5] & ((1u << (tid & 31)) - 1u));
            for (int w = 0; w < (tid >> 5); ++w) rank += __popc(member[k][w]);
            order[kXcds * (int64_t)(cstart[k] + crun[k] + rank) + x] = (int32_t)it;
        }
        __syncthreads();
        for (int kk = tid; kk < kOrderClasses; kk += kOrderThreads) {
            int cnt = 0;
            for (int w = 0; w < kOrderThreads / 32; ++w) cnt += __popc(member[kk][w]);
            crun[kk] += cnt;
        }
        __syncthreads();
    }
    for (int64_t k = (hi - lo) + tid; k < cap; k += kOrderThreads) order[kXcds * k + x] = -1;
    if (tid == 0) order[kXcds * cap + x] = (int32_t)(hi - lo);  // the range's length
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
                        const Grid &g, int heads, const int2 *pairs, int32_t *ulist, int32_t *ulen,
                        float2 *ubias, hipStream_t s) {
    const int slots = plan_slots_per_head(g);
    const int64_t items = (int64_t)heads * slots;
    hipLaunchKernelGGL(union_kernel, dim3((unsigned)((items + kUnionWaves - 1) / kUnionWaves)),
                       dim3(64 * kUnionWaves), 0, s, idx, cnt, lw, maxcnt, g, items, slots, pairs,
                       union_stride(maxcnt), ulist, ulen, ubias);
    return hipGetLastError();
}

hipError_t launch_pair(const int32_t *idx, const int32_t *cnt, int64_t maxcnt, const Grid &g,
                       int heads, int2 *pairs, int32_t *scratch, hipStream_t s) {
    const int64_t cands =
        (int64_t)heads * (candidates(pairs_per_head(g)) + candidates(temporal_pairs_per_head(g)));
    hipLaunchKernelGGL(candidate_walk_kernel,
                       dim3((unsigned)((cands + kUnionWaves - 1) / kUnionWaves)),
                       dim3(64 * kUnionWaves), 0, s, idx, cnt, maxcnt, g, heads, scratch);
    hipLaunchKernelGGL(pair_kernel, dim3((unsigned)heads), dim3(kPairThreads), 0, s, cnt, nullptr,
                       scratch, 0, maxcnt, g, plan_slots_per_head(g), pairs);
    return hipGetLastError();
}

hipError_t launch_pair_radius(const int32_t *radius, int r_max, int64_t maxcnt, const Grid &g,
                              int heads, int2 *pairs, hipStream_t s) {
    if (g.nby * g.nbx <= kPairMaxPlane && g.T <= kPairMaxFrames && g.nb <= kPairMaxOrphans)
        hipLaunchKernelGGL(pair_radius_kernel, dim3((unsigned)heads), dim3(kPairThreads), 0, s,
                           radius, r_max, g, plan_slots_per_head(g), pairs);
    else
        hipLaunchKernelGGL(pair_kernel, dim3((unsigned)heads), dim3(kPairThreads), 0, s, nullptr,
                           radius, nullptr, r_max, maxcnt, g, plan_slots_per_head(g), pairs);
    return hipGetLastError();
}

hipError_t launch_radius_walk(const int32_t *radius, int r_max, int64_t maxcnt, const Grid &g,
                              int heads, const int2 *pairs, int32_t *ulist, int32_t *ulen,
                              hipStream_t s) {
    const int slots = plan_slots_per_head(g);
    const int64_t items = (int64_t)heads * slots;
    hipLaunchKernelGGL(radius_walk_kernel, dim3((unsigned)((items + kUnionWaves - 1) / kUnionWaves)),
                       dim3(64 * kUnionWaves), 0, s, radius, r_max, g, items, slots, pairs,
                       union_stride(maxcnt), ulist, ulen);
    return hipGetLastError();
}

hipError_t launch_order(const int32_t *ulen, const Grid &g, int heads, int64_t maxcnt,
                        int32_t *order, hipStream_t s) {
    const int64_t items = (int64_t)heads * plan_slots_per_head(g);
    // lengths above kOrderMaxBin count as kOrderMaxBin (work and class)
    const int maxlen = (int)(2 * maxcnt < kOrderMaxBin ? 2 * maxcnt : kOrderMaxBin);
    hipLaunchKernelGGL(order_kernel, dim3(kXcds), dim3(kOrderThreads), 0, s, ulen, items,
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

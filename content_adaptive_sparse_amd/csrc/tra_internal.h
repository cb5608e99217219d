// Internal declarations of the HIP path (gfx950).  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tra {

// A block is an 8 x 8 spatial tile of tokens inside one frame.
constexpr int kTileSide = 8;
constexpr int kBlockTokens = 64;

// Tile grid of one head's (T, H, W) token grid.
struct Grid {
    int T, H, W;
    int nby, nbx;  // tiles per frame along y and x (ceil)
    int nb;        // T * nby * nbx
};

// Packed key/value tiles (tile-major, one 64-token tile after another), each
// tile a sequence of 1 KB matrix-core operand pieces in which lane l of a
// wave64 finds its 8 operand elements at element 8 l, so that every operand
// read is one contiguous, conflict-free 1 KB LDS access.  Key row w of a tile
// is (y % 8) * 8 + x % 8; missing cells are zero.
//   kt  bf16 [heads][nb][2 halves][D/16 k-steps][64 lanes][8]: piece (hf, ks),
//       lane l holds K[32 hf + l % 32][16 ks + 8 (l / 32) + e], e = 0..7.
//   vt  fp16 [heads][nb][2 halves][D/32 row tiles][2 k-steps][64 lanes][8]:
//       piece (hf, mt, ks2), lane l holds V[32 hf + swap23(8 (2 ks2 + l / 32) + e)]
//       [32 mt + l % 32], where swap23 exchanges bits 2 and 3 of a key position
//       (so that the keys of a lane match the probabilities that lane holds).
size_t packed_tile_elems(int D);

// V enters the P.V product on fp16 matrix cores as v 2^e_h, with one
// power-of-two exponent e_h per head that puts the head's largest |v| into
// [2^15, 2^16) (exact for every finite bfloat16 within 2^30 of it); the output
// is multiplied back by 2^-e_h.  vmax_kernel writes vmax_parts(g, D) partial
// maxima per head (vpart [heads][parts], bfloat16 bits of |v|); the packing
// kernel reduces them, scales V and writes e_h to vexp [heads].
constexpr int kVmaxParts = 256;  // at most the packing kernel's 256 threads
int vmax_parts(const Grid &g, int D);
// sched (or null): the next attention launch's work-claiming counters (kSchedBytes),
// zeroed here -- every launch along a work order follows the packing of its K and V.
hipError_t launch_vmax(int D, const uint16_t *v, const Grid &g, int heads, uint32_t *vpart,
                       int32_t *sched, hipStream_t s);

hipError_t launch_pack_pool(int D, bool pool, bool pack, const uint16_t *q, const uint16_t *k,
                            const uint16_t *v, const Grid &g, int heads, float *qp, float *kp,
                            uint16_t *kt, uint16_t *vt, const uint32_t *vpart, int32_t *vexp,
                            hipStream_t s);

// logits (optional): the pooled logit matrix [heads][nb][nb] (scaled by 1/sqrt(D)).
hipError_t launch_entropy(int D, const float *qp, const float *kp, const Grid &g, int heads,
                          int r_min, int r_max, int32_t *radius, float *h_norm, hipStream_t s,
                          float *logits = nullptr);

hipError_t launch_fill_dense(const Grid &g, int heads, int32_t *radius, float *h_norm,
                             hipStream_t s);

hipError_t launch_mask(const int32_t *radius, const Grid &g, int heads, int r_max,
                       int64_t maxcnt, int32_t *idx, int32_t *cnt, hipStream_t s);

// Packed K tiles only (the token-entropy warm-up reads no v).
hipError_t launch_pack_k(int D, const uint16_t *k, const Grid &g, int heads, uint16_t *kt,
                         hipStream_t s);

// Token-level policy (tra_token.hip): entropy and base radius of every token
// ([heads][T][H][W] fp32) from packed K; voting lists ([heads][nb][maxcnt]).
hipError_t launch_token_entropy(int D, const uint16_t *q, const uint16_t *kt, const Grid &g,
                                int heads, float tau, float gamma, float *ent, float *r0,
                                hipStream_t s);
hipError_t launch_token_mask(const float *r0, const Grid &g, int heads, float gamma,
                             int min_votes, int64_t maxcnt, int32_t *idx, int32_t *cnt,
                             hipStream_t s);

// Attention work items are pairs of vertically adjacent query blocks: item p
// of a head is frame t, tile-row pair pr, tile column bx, holding blocks
// (t, 2 pr, bx) and (t, 2 pr + 1, bx) (the second is absent when nby is odd and
// 2 pr + 1 == nby).  Tile rows are the shortest axis of a video latent, so
// radii clip there first and the two blocks' key lists mostly coincide.
__host__ __device__ inline int pairs_per_head(const Grid &g) {
    return g.T * ((g.nby + 1) / 2) * g.nbx;
}
__host__ __device__ inline void pair_blocks(int p, const Grid &g, int &qa, int &qb) {
    const int npy = (g.nby + 1) / 2;
    const int t = p / (npy * g.nbx);
    const int pr = (p / g.nbx) % npy;
    const int bx = p % g.nbx;
    qa = (t * g.nby + 2 * pr) * g.nbx + bx;
    qb = 2 * pr + 1 < g.nby ? qa + g.nbx : -1;
}
// Temporal pairs: pair p of a head is the tile p % plane of frames 2 (p / plane)
// and 2 (p / plane) + 1 (the second absent when T is odd and that frame is the
// last).  Lists voted by query tokens (the token policy) coincide more in time
// than across tile rows; a list plan takes them when they save steps.
__host__ __device__ inline int temporal_pairs_per_head(const Grid &g) {
    return (g.T + 1) / 2 * (g.nby * g.nbx);
}
__host__ __device__ inline void temporal_pair_blocks(int p, const Grid &g, int &qa, int &qb) {
    const int plane = g.nby * g.nbx;
    const int tp = p / plane;
    qa = 2 * tp * plane + (p - tp * plane);
    qb = 2 * tp + 1 < g.T ? qa + plane : -1;
}
// Item slots per head of a walk plan: room for either kind of pairs.
__host__ __device__ inline int plan_slots_per_head(const Grid &g) {
    const int v = pairs_per_head(g), t = temporal_pairs_per_head(g);
    return v > t ? v : t;
}

// Union walk of each work item (see tra_mask.hip): ulist holds, at row stride
// union_stride(maxcnt), entries (block << 2) | sides, ulen their counts; with
// per-entry log-weights lw (laid out like idx, or null) ubias holds each
// entry's (upper, lower) block weight in log2 units.
int64_t union_stride(int64_t maxcnt);
hipError_t launch_union(const int32_t *idx, const int32_t *cnt, const float *lw, int64_t maxcnt,
                        const Grid &g, int heads, const int2 *pairs, int32_t *ulist, int32_t *ulen,
                        float2 *ubias, hipStream_t s);

// Pair table of a list set (see tra_mask.hip): for every head,
// plan_slots_per_head item slots (qa, qb) -- neighbours whose list lengths are
// within a factor of two, the other blocks re-paired by length class -- then
// unused slots (-1, -1); qb = -1 marks a single block.  The neighbours are
// vertical, or temporal in a head whose temporal pairs' walks take at least 5%
// fewer steps per list entry (judged on every fourth pair of either kind).  scratch:
// heads (pairs_per_head + temporal_pairs_per_head) int32 of device memory for
// those walk lengths (any memory the caller overwrites afterwards: the plan's
// work order).
hipError_t launch_pair(const int32_t *idx, const int32_t *cnt, int64_t maxcnt, const Grid &g,
                       int heads, int2 *pairs, int32_t *scratch, hipStream_t s);

// The same two steps for the radius mask's lists taken straight from the radii
// (no lists): the pair table from the radii (vertical neighbours of equal
// radius, the others classed by radius), then each item's walk, the union of its
// two blocks' key boxes.  Every block meets the same entries in the same order
// as along launch_pair + launch_union of tra_mask's lists when maxcnt holds the
// largest box (tra_maxcnt), so that no list is cut short: the same results.
hipError_t launch_pair_radius(const int32_t *radius, int r_max, int64_t maxcnt, const Grid &g,
                              int heads, int2 *pairs, hipStream_t s);
hipError_t launch_radius_walk(const int32_t *radius, int r_max, int64_t maxcnt, const Grid &g,
                              int heads, const int2 *pairs, int32_t *ulist, int32_t *ulen,
                              hipStream_t s);

// Sampled lists with log-weights from the pooled logit matrix and uniforms
// u[heads][nb][nb] (row stride nb for idx and lw).
hipError_t launch_sip(const float *logits, const float *u, const Grid &g, int heads, float m,
                      int32_t *idx, int32_t *cnt, float *lw, hipStream_t s);

// Per-item arrays of a walk plan (lengths, walks) hold walk_items(g, heads) rows.
inline int64_t walk_items(const Grid &g, int heads) {
    return ((int64_t)heads * plan_slots_per_head(g) + 7) / 8 * 8;
}
// XCD-aware order of the attention work items: eight contiguous ranges of
// equal work, each of at most order_range_cap items (twice the average count)
// and taken by walk length class, longest class first.  order holds
// order_slots(g, heads) = 8 x cap grid slots (-1: no item), then the eight range
// lengths (order_ints ints in all); the attention launch has one workgroup per
// slot (an empty slot's workgroup exits at once; empty slots come last on their
// XCD).
inline int64_t order_range_cap(const Grid &g, int heads) {
    return 2 * (((int64_t)heads * plan_slots_per_head(g) + 7) / 8);
}
inline int64_t order_slots(const Grid &g, int heads) { return 8 * order_range_cap(g, heads); }
inline int64_t order_ints(const Grid &g, int heads) { return order_slots(g, heads) + 8; }
hipError_t launch_order(const int32_t *ulen, const Grid &g, int heads, int64_t maxcnt,
                        int32_t *order, hipStream_t s);

// Optional per-query entropy of the attention row (the token policy's warm-up
// fused into dense attention): H_i in nats and the base radius r0_i, both
// [heads][T][H][W] fp32, with the budget parameter tau and the temporal decay
// as 2 gamma log2(e).
struct EntropyOut {
    float *ent;
    float *r0;
    float tau;
    float two_gamma_log2e;
};

// Along a work order the last quarter of each XCD range is claimed at run
// time: one int32 counter per range, kSchedStride int32 apart, in kSchedBytes
// of device memory that must be zero when the launch starts (launch_vmax zeroes
// it; launches in a row need a zeroed set each) and is used by that launch alone.
constexpr int kXcdRanges = 8;
constexpr int kSchedStride = 64;
constexpr size_t kSchedBytes = (size_t)kXcdRanges * kSchedStride * sizeof(int32_t);
// Zeroes n int32 at p (a fill kernel: nothing that a captured graph could not replay).
hipError_t launch_zero(int32_t *p, int64_t n, hipStream_t s);

// ulist == nullptr: the dense mode (every block, both sides; order and pairs
// null, vertical pairs in XCD-contiguous raster order).  vexp: the per-head V
// exponents.  pairs: the plan's pair table.  sched: kSchedBytes of scratch for
// the work-claiming counters of a launch along a work order.
hipError_t launch_attn(int D, const uint16_t *q, const uint16_t *kt, const uint16_t *vt,
                       const int32_t *vexp, const int2 *pairs, const int32_t *ulist,
                       const int32_t *ulen, const float2 *ubias, int64_t ustride,
                       const int32_t *order, int32_t *sched, const Grid &g, int heads, float *out,
                       hipStream_t s, const EntropyOut *entropy = nullptr);

// Static device scratch of tra_probe_static (tra_static.hip): one array of
// kStaticScratchBytes per GPU, held until the process ends.  static_scratch
// returns the current device's copy (its address taken with
// hipGetSymbolAddress on the first call on that device).
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
hipError_t static_scratch(void **ptr);

}  // namespace tra

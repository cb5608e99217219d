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

hipError_t launch_pack_pool(int D, bool pool, bool pack, const uint16_t *q, const uint16_t *k,
                            const uint16_t *v, const Grid &g, int heads, float *qp, float *kp,
                            uint16_t *kt, uint16_t *vt, hipStream_t s);

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

// Union walk of each work item (see tra_mask.hip): ulist holds, at row stride
// union_stride(maxcnt), entries (block << 2) | sides, ulen their counts; with
// per-entry log-weights lw (laid out like idx, or null) ubias holds each
// entry's (upper, lower) block weight in log2 units.
int64_t union_stride(int64_t maxcnt);
hipError_t launch_union(const int32_t *idx, const int32_t *cnt, const float *lw, int64_t maxcnt,
                        const Grid &g, int heads, int32_t *ulist, int32_t *ulen, float2 *ubias,
                        hipStream_t s);

// Sampled lists with log-weights from the pooled logit matrix and uniforms
// u[heads][nb][nb] (row stride nb for idx and lw).
hipError_t launch_sip(const float *logits, const float *u, const Grid &g, int heads, float m,
                      int32_t *idx, int32_t *cnt, float *lw, hipStream_t s);

// Per-item arrays of a walk plan (lengths, walks) hold walk_items(g, heads) rows.
inline int64_t walk_items(const Grid &g, int heads) {
    return ((int64_t)heads * pairs_per_head(g) + 7) / 8 * 8;
}
// XCD-aware, longest-first order of the attention work items: eight contiguous
// ranges of equal work, each of at most order_range_cap items (twice the
// average count); order holds order_slots(g, heads) = 8 x cap grid slots (-1:
// no item), and the attention launch has one workgroup per slot (an empty
// slot's workgroup exits at once; empty slots come last on their XCD).
inline int64_t order_range_cap(const Grid &g, int heads) {
    return 2 * (((int64_t)heads * pairs_per_head(g) + 7) / 8);
}
inline int64_t order_slots(const Grid &g, int heads) { return 8 * order_range_cap(g, heads); }
hipError_t launch_order(const int32_t *ulen, const Grid &g, int heads, int64_t maxcnt,
                        int32_t *order, hipStream_t s);

// ulist == nullptr: the dense mode (every block, both sides; order null, items
// in XCD-contiguous raster order).
hipError_t launch_attn(int D, const uint16_t *q, const uint16_t *kt, const uint16_t *vt,
                       const int32_t *ulist, const int32_t *ulen, const float2 *ubias,
                       int64_t ustride, const int32_t *order, const Grid &g, int heads,
                       float *out, hipStream_t s);

}  // namespace tra

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

// Packed key/value tiles (tile-major, one 64-token tile after another):
//   kt  bf16 [heads][nb][64 keys][D], key row w = (y % 8) * 8 + x % 8, missing
//       cells zero; the 16-byte chunk c of row w is stored at chunk c ^ (w & KSW)
//       with KSW = min(D/8, 16) - 1 so that the matrix-core operand reads of 16
//       consecutive key rows hit distinct LDS banks.
//   vt  fp16 [heads][nb][2 halves][D][32 positions] (V transposed, keys
//       0..31 then 32..63), position p of a half holds key p with bits 2 and 3
//       swapped, so that the 8 keys one lane feeds to the P.V product are
//       contiguous; the 16-byte chunk c of row d is stored at c ^ ((d >> 2) & 3).
size_t packed_tile_elems(int D);

hipError_t launch_pack_pool(int D, bool pool, bool pack, const uint16_t *q, const uint16_t *k,
                            const uint16_t *v, const Grid &g, int heads, float *qp, float *kp,
                            uint16_t *kt, uint16_t *vt, hipStream_t s);

hipError_t launch_entropy(int D, const float *qp, const float *kp, const Grid &g, int heads,
                          int r_min, int r_max, int32_t *radius, float *h_norm, hipStream_t s);

hipError_t launch_fill_dense(const Grid &g, int heads, int32_t *radius, float *h_norm,
                             hipStream_t s);

hipError_t launch_mask(const int32_t *radius, const Grid &g, int heads, int r_max,
                       int64_t maxcnt, int32_t *idx, int32_t *cnt, hipStream_t s);

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

// Longest-first order of the attention work items (query-block pairs); see
// tra_mask.hip.  order has heads * pairs_per_head(g) entries.
hipError_t launch_order(const int32_t *cnt, const Grid &g, int heads, int64_t maxcnt,
                        int32_t *order, hipStream_t s);

// order may be null (items in XCD-contiguous raster order, the dense mode).
hipError_t launch_attn(int D, const uint16_t *q, const uint16_t *kt, const uint16_t *vt,
                       const int32_t *idx, const int32_t *cnt, int64_t maxcnt,
                       const int32_t *order, const Grid &g, int heads, float *out,
                       hipStream_t s);

}  // namespace tra

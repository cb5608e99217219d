// Block-sparse flash attention over 8 x 8-token tiles, gfx950 matrix cores.
//
// AB-Attention speeds up video diffusion transformers up to 2.23x (first
// paragraph): dynamic block-sparse attention computes exact attention only on
// the key/value blocks kept for a query block.  Token Radius Attention for
// Efficient Video Generation ("The TRA Pipeline: Fused CUDA Kernels"): the
// kept blocks come from the radius mask and run on a block-sparse backend,
// which this kernel is.
//
// One workgroup (two wave64) per (head, query block); wave w owns query rows
// 32 w .. 32 w + 31 of the tile.  For each kept key block, its packed K tile
// (bf16) and V^T tile (fp16) are copied into LDS, then every wave computes
//   S^T = K Q^T        v_mfma_f32_32x32x16_bf16, fp32 accumulation
//   online softmax     per query = per lane column, exp2 with the scale folded
//   O^T += V^T P^T     v_mfma_f32_32x32x16_f16 (P rounded to fp16)
// Working on the transposed products keeps every query's logits and output in
// one lane pair (lanes l and l + 32), so the softmax needs a single cross-lane
// exchange per tile and P feeds the second product without moving data.
#include <math.h>

#include "tra_internal.h"

namespace tra {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

template <typename T>
__device__ __forceinline__ T lds_load16(const uint16_t *p) {
    return *reinterpret_cast<const T *>(p);
}

constexpr int kAttnThreads = 128;
// The running max is only moved (and O, l rescaled) when a tile's max exceeds
// it by more than this many powers of two; in between, probabilities are
// taken against the stale max (at most 2^8, exact in fp16) and the final
// normalisation by l uses the same reference, so the result is unchanged.
constexpr float kRescaleLog2 = 8.0f;

template <int D>
__global__ __launch_bounds__(kAttnThreads, 2) void attn_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kt,
    const uint16_t *__restrict__ vt, const int32_t *__restrict__ idx,
    const int32_t *__restrict__ cnt, int64_t maxcnt, Grid g, int heads, int per_xcd,
    float *__restrict__ out, float scale_log2) {
    constexpr int KS = D / 16;                  // k-steps of Q.K^T
    constexpr int MT = D / 32;                  // 32-row tiles of O^T
    constexpr int CH = D / 8;                   // 16-byte chunks per K row
    constexpr int KSW = (CH < 16 ? CH : 16) - 1;
    constexpr int TILE = kBlockTokens * D;      // elements of one K or V^T tile
    constexpr int CPT = TILE / 8 / kAttnThreads;  // 16-byte chunks per thread per tile

    __shared__ __attribute__((aligned(16))) uint16_t k_lds[TILE];
    __shared__ __attribute__((aligned(16))) uint16_t v_lds[TILE];

    // Consecutive workgroup ids land on different XCDs; give every XCD a
    // contiguous range of (head, query block) so its L2 sees neighbouring
    // query blocks, whose key lists overlap.
    const int64_t total = (int64_t)heads * g.nb;
    const int64_t wg = (int64_t)(blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    if (wg >= total) return;
    const int h = (int)(wg / g.nb);
    const int qb = (int)(wg % g.nb);

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int hl = lane >> 5, l32 = lane & 31;

    int n;
    const int32_t *list = nullptr;
    if (idx) {
        const int64_t c = cnt[wg];
        n = (int)(c < 0 ? 0 : (c > maxcnt ? maxcnt : c));
        list = idx + wg * maxcnt;
    } else {
        n = g.nb;
    }

    // This lane's query token (clamped into the grid for the missing cells of
    // an edge tile; such rows are computed but never stored).
    const int plane = g.nby * g.nbx;
    const int t = qb / plane, by = (qb / g.nbx) % g.nby, bx = qb % g.nbx;
    const int qi = 32 * wave + l32;
    const int qy = kTileSide * by + (qi >> 3), qx = kTileSide * bx + (qi & 7);
    const bool qreal = qy < g.H && qx < g.W;
    const size_t qtok = (size_t)h * g.T * g.H * g.W +
                        ((size_t)t * g.H + min(qy, g.H - 1)) * g.W + min(qx, g.W - 1);

    auto block_at = [&](int j) -> int { return list ? list[j] : j; };
    auto next_valid = [&](int j) -> int {
        while (j < n && (unsigned)block_at(j) >= (unsigned)g.nb) ++j;
        return j;
    };

    // Register staging of one 16 KB tile: global -> VGPR -> LDS.  (Written as
    // macros over a fixed-size array so it stays in registers.)
    u32x4_t stage[CPT];
    const size_t head_tiles = (size_t)h * g.nb;
#define TRA_FETCH(base, blk)                                                                 \
    do {                                                                                     \
        const u32x4_t *src_ = reinterpret_cast<const u32x4_t *>((base) + (head_tiles + (blk)) * TILE); \
        _Pragma("unroll") for (int i_ = 0; i_ < CPT; ++i_) stage[i_] = src_[tid + kAttnThreads * i_]; \
    } while (0)
#define TRA_PUT(dst)                                                                         \
    do {                                                                                     \
        _Pragma("unroll") for (int i_ = 0; i_ < CPT; ++i_)                                   \
            reinterpret_cast<u32x4_t *>(dst)[tid + kAttnThreads * i_] = stage[i_];            \
    } while (0)

    int j = next_valid(0);
    int kb = j < n ? block_at(j) : -1;
    float *o = out + qtok * D;
    if (kb < 0) {  // nothing kept: zeros
        if (qreal)
            for (int c = 0; c < D / 2; c += 4)
                *reinterpret_cast<float4 *>(o + c + (D / 2) * hl) = make_float4(0.f, 0.f, 0.f, 0.f);
        return;
    }

    bf16x8_t qreg[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        qreg[ks] = *reinterpret_cast<const bf16x8_t *>(q + qtok * D + 16 * ks + 8 * hl);

    f32x16_t acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mt][r] = 0.f;
    float m_ref = -1e30f, l_run = 0.f;

    // prologue: tile 0 into LDS, K of tile 1 in flight
    TRA_FETCH(kt, kb);
    TRA_PUT(k_lds);
    TRA_FETCH(vt, kb);
    TRA_PUT(v_lds);
    int jn = next_valid(j + 1);
    int kbn = jn < n ? block_at(jn) : -1;
    TRA_FETCH(kt, kbn >= 0 ? kbn : kb);
    __syncthreads();

    while (true) {
        // ---- S^T = K Q^T (keys 0..31 and 32..63 of the tile) ----
        f32x16_t s[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[mt][r] = 0.f;
            const int key = 32 * mt + l32;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int cs = (2 * ks + hl) ^ (key & KSW);
                const bf16x8_t a = lds_load16<bf16x8_t>(k_lds + key * D + 8 * cs);
                s[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[ks], s[mt], 0, 0, 0);
            }
        }
        __syncthreads();  // every wave is done with k_lds; v_lds holds this tile's V
        // (past the end of the list this restages the current tile: harmless)
        TRA_PUT(k_lds);
        TRA_FETCH(vt, kbn >= 0 ? kbn : kb);

        // ---- missing key cells of an edge tile -> -inf ----
        const int kby = (kb / g.nbx) % g.nby, kbx = kb % g.nbx;
        const int kny = min(kTileSide, g.H - kTileSide * kby);
        const int knx = min(kTileSide, g.W - kTileSide * kbx);
        if (kny < kTileSide || knx < kTileSide) {
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int ky = 4 * mt + (r >> 2);
                    const int kx = 4 * hl + (r & 3);
                    if (ky >= kny || kx >= knx) s[mt][r] = -INFINITY;
                }
        }

        // ---- online softmax, base 2 with the scale folded into one FMA ----
        float mx = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mt][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32)) * scale_log2;
        const bool grow = mx > m_ref + kRescaleLog2;
        if (__any(grow)) {
            const float m_new = grow ? mx : m_ref;
            const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
            l_run *= alpha;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[mt][r] *= alpha;
            m_ref = m_new;
        }
        float psum = 0.f;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mt][r], scale_log2, -m_ref));
                s[mt][r] = p;
                psum += p;
            }
        l_run += psum;

        // P^T as the B operand: k-step ks2 covers keys 16 ks2 .. 16 ks2 + 15,
        // held in s[ks2 / 2] registers 8 (ks2 % 2) .. + 7.
        f16x8_t pk[4];
#pragma unroll
        for (int ks2 = 0; ks2 < 4; ++ks2)
#pragma unroll
            for (int e = 0; e < 8; ++e) pk[ks2][e] = (_Float16)s[ks2 >> 1][8 * (ks2 & 1) + e];

        // ---- O^T += V^T P^T ----
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int d = 32 * mt + l32;
#pragma unroll
            for (int ks2 = 0; ks2 < 4; ++ks2) {
                const int cs = (2 * ks2 + hl) ^ ((d >> 1) & 7);
                const f16x8_t a = lds_load16<f16x8_t>(v_lds + d * 64 + 8 * cs);
                acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pk[ks2], acc[mt], 0, 0, 0);
            }
        }
        if (kbn < 0) break;
        __syncthreads();  // every wave is done with v_lds; k_lds holds the next K
        TRA_PUT(v_lds);
        j = jn;
        kb = kbn;
        jn = next_valid(j + 1);
        kbn = jn < n ? block_at(jn) : -1;
        TRA_FETCH(kt, kbn >= 0 ? kbn : kb);
    }
#undef TRA_FETCH
#undef TRA_PUT

    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    if (qreal) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int d0 = 32 * mt + 8 * g4 + 4 * hl;
                *reinterpret_cast<float4 *>(o + d0) =
                    make_float4(acc[mt][4 * g4] * inv, acc[mt][4 * g4 + 1] * inv,
                                acc[mt][4 * g4 + 2] * inv, acc[mt][4 * g4 + 3] * inv);
            }
    }
}

}  // namespace

hipError_t launch_attn(int D, const uint16_t *q, const uint16_t *kt, const uint16_t *vt,
                       const int32_t *idx, const int32_t *cnt, int64_t maxcnt, const Grid &g,
                       int heads, float *out, hipStream_t s) {
    const int64_t total = (int64_t)heads * g.nb;
    const int per_xcd = (int)((total + 7) / 8);
    const dim3 grid((unsigned)(8 * (int64_t)per_xcd)), block(kAttnThreads);
    const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
    if (D == 128)
        hipLaunchKernelGGL(attn_kernel<128>, grid, block, 0, s, q, kt, vt, idx, cnt, maxcnt, g,
                           heads, per_xcd, out, scale_log2);
    else if (D == 64)
        hipLaunchKernelGGL(attn_kernel<64>, grid, block, 0, s, q, kt, vt, idx, cnt, maxcnt, g,
                           heads, per_xcd, out, scale_log2);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace tra

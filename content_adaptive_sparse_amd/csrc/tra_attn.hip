// Block-sparse flash attention over 8 x 8-token tiles, gfx950 matrix cores.
//
// AB-Attention speeds up video diffusion transformers up to 2.23x (first
// paragraph): dynamic block-sparse attention computes exact attention only on
// the key/value blocks kept for a query block.  Token Radius Attention for
// Efficient Video Generation ("The TRA Pipeline: Fused CUDA Kernels"): the
// kept blocks come from the radius mask and run on a block-sparse backend,
// which this kernel is.
//
// One workgroup of four wave64 computes two vertically adjacent query blocks
// of one head (two waves per block, 32 queries per wave) over the union of the
// two blocks' key lists.  Every kept key block's packed K rows (bf16) and V^T
// rows (fp16) are copied straight from global memory into a two-slot LDS ring
// (the next block lands while the current one is computed), and each wave
// whose block keeps it computes, per 32-key half:
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
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

template <typename T>
__device__ __forceinline__ T lds_load16(const uint16_t *p) {
    return *reinterpret_cast<const T *>(p);
}

// Exact n / d for 0 <= n < 2^24 and 1 <= d < 2^15 with m = ceil(2^39 / d):
// the product's error term is below n / 2^39 < 1 / d, so the floor is exact.
struct FastDiv {
    uint64_t m;
    uint32_t d;
};
__device__ __forceinline__ uint32_t fdiv(uint32_t n, FastDiv f) {
    return (uint32_t)(((uint64_t)n * f.m) >> 39);
}

// Lanes l and l + 32 hold the same query: combine a value with the other
// half's copy in registers (v_permlane32_swap: with the value in both
// operands, the results are the lower-half and the upper-half copies).
__device__ __forceinline__ float half_swap_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

constexpr int kAttnThreads = 256;
constexpr int kRingSlots = 2;
// s_waitcnt immediates for gfx9 (vmcnt bits [3:0] and [15:14], expcnt [6:4],
// lgkmcnt [11:8]); counters not waited on are left at their no-wait maxima.
constexpr int wait_vmcnt(int n) { return 0x0F70 | (n & 15) | (((n >> 4) & 3) << 14); }
constexpr int kWaitVmcnt0 = wait_vmcnt(0);
constexpr int kWaitLgkmcnt0 = 0xC07F;
// The running max is only moved (and O, l rescaled) when a tile's max exceeds
// it by more than this many powers of two; in between, probabilities are
// taken against the stale max (at most 2^8, exact in fp16) and the final
// normalisation by l uses the same reference, so the result is unchanged.
constexpr float kRescaleLog2 = 8.0f;

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void global_void_t;
// The key lists are never written while the kernel runs; reading them through
// the constant address space lets wave-uniform reads use scalar loads, which
// do not share the vector-memory counter with the in-flight LDS copies.
typedef __attribute__((address_space(4))) const int32_t const_i32_t;

template <int N>
struct SlotTag {
    static constexpr int value = N;
};

// A query block's key list read through scalar loads: entries outside
// [0, nb) are skipped; `cur` is the block at the cursor or INT32_MAX once the
// list is exhausted (so the smaller of two cursors is the next union entry).
struct ListCursor {
    const const_i32_t *list;  // nullptr: every block 0 .. nb-1 (dense)
    int n, j, cur;
};

__device__ __forceinline__ void list_seek(ListCursor &c, int nb) {
    while (c.j < c.n) {
        const int b = c.list ? c.list[c.j] : c.j;
        if ((unsigned)b < (unsigned)nb) {
            c.cur = b;
            return;
        }
        ++c.j;
    }
    c.cur = INT32_MAX;
}

template <int D>
__global__ __launch_bounds__(kAttnThreads, 2) void attn_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kt,
    const uint16_t *__restrict__ vt, const int32_t *__restrict__ idx,
    const int32_t *__restrict__ cnt, int64_t maxcnt, const int32_t *__restrict__ order, Grid g,
    int heads, int pairs_per_head, int per_xcd, FastDiv div_nbx, FastDiv div_nby,
    float *__restrict__ out, float scale_log2) {
    constexpr int KS = D / 16;                  // k-steps of Q.K^T
    constexpr int MT = D / 32;                  // 32-row tiles of O^T
    constexpr int CH = D / 8;                   // 16-byte chunks per K row
    constexpr int KSW = (CH < 16 ? CH : 16) - 1;
    constexpr int HALF = 32 * D;                // elements of a 32-key K or V^T half tile
    constexpr int PIECES = HALF * 2 / 1024;     // 1 KB copies per half tile and operand
    constexpr int WAVES = kAttnThreads / 64;
    constexpr int PPW = PIECES / WAVES;         // pieces per wave and operand
    static_assert(PPW * WAVES == PIECES, "every piece copied exactly once");
    static_assert(PIECES * 512 == HALF, "pieces tile the half exactly (no copy past a slot)");

    // Ring of whole packed tiles: [slot][0 = K rows, 1 = V^T rows]; the copy of
    // the next block runs while the current one is computed.
    __shared__ __attribute__((aligned(1024))) uint16_t ring[kRingSlots][2][2 * HALF];

    // Work item: a pair of vertically adjacent query blocks of one head.
    // With a work order (lists of unequal length), items are taken longest
    // first.  Without one (dense mode: equal work), consecutive workgroup ids,
    // which land on different XCDs, are remapped so every XCD gets a contiguous
    // range of items and its L2 sees neighbouring query blocks.
    const int64_t total = (int64_t)heads * pairs_per_head;
    int64_t item;
    if (order) {
        if ((int64_t)blockIdx.x >= total) return;
        item = ((const const_i32_t *)order)[blockIdx.x];
    } else {
        item = (int64_t)(blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    }
    if (item >= total) return;
    const int h = (int)(item / pairs_per_head);
    int blk[2];
    pair_blocks((int)(item % pairs_per_head), g, blk[0], blk[1]);

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int hl = lane >> 5, l32 = lane & 31;
    const int side = wave >> 1;          // which block of the pair this wave computes
    const int qb = blk[side];            // -1: absent (odd tile-row count)

    // Both cursors are tracked (redundantly) by every wave.
    ListCursor ca, cb;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        ListCursor &c = k ? cb : ca;
        const int b = blk[k];
        c.j = 0;
        c.list = nullptr;
        if (b < 0) {
            c.n = 0;
        } else if (idx) {
            const int64_t row = (int64_t)h * g.nb + b;
            const int64_t m = ((const const_i32_t *)cnt)[row];
            c.n = (int)(m < 0 ? 0 : (m > maxcnt ? maxcnt : m));
            c.list = (const const_i32_t *)idx + row * maxcnt;
        } else {
            c.n = g.nb;
        }
        list_seek(c, g.nb);
    }

    // This lane's query token (clamped into the grid for the missing cells of
    // an edge tile, and for an absent block; such rows are never stored).
    const int plane = g.nby * g.nbx;
    const int qbc = qb >= 0 ? qb : blk[0];
    const int t = qbc / plane, by = (qbc / g.nbx) % g.nby, bx = qbc % g.nbx;
    const int qi = 32 * (wave & 1) + l32;
    const int qy = kTileSide * by + (qi >> 3), qx = kTileSide * bx + (qi & 7);
    const bool qreal = qb >= 0 && qy < g.H && qx < g.W;
    const size_t qtok = (size_t)h * g.T * g.H * g.W +
                        ((size_t)t * g.H + min(qy, g.H - 1)) * g.W + min(qx, g.W - 1);
    float *o = out + qtok * D;

    int kb = min(ca.cur, cb.cur);
    if (kb == INT32_MAX) {  // neither block keeps anything: zeros
        if (qreal)
            for (int c = 0; c < D / 2; c += 4)
                *reinterpret_cast<float4 *>(o + c + (D / 2) * hl) = make_float4(0.f, 0.f, 0.f, 0.f);
        return;
    }

    // Direct global -> LDS copy of block `blk`'s packed tiles into ring slot
    // `slot`: each wave moves 2 PPW 1 KB pieces of K and of V^T; lane l lands 16
    // bytes at piece base + 16 l.
    const size_t head_tiles = (size_t)h * g.nb;
#define TRA_ISSUE(blk, slot)                                                                  \
    do {                                                                                      \
        const char *ks_ = reinterpret_cast<const char *>(kt + (head_tiles + (blk)) * 64 * D) + wave_piece_bytes; \
        const char *vs_ = reinterpret_cast<const char *>(vt + (head_tiles + (blk)) * 64 * D) + wave_piece_bytes; \
        _Pragma("unroll") for (int i_ = 0; i_ < 2 * PPW; ++i_) {                             \
            __builtin_amdgcn_global_load_lds((const global_void_t *)(ks_ + lane16 + i_ * 1024), \
                                             (lds_void_t *)&ring[slot][0][wave_piece_elems + i_ * 512], 16, 0, 0); \
            __builtin_amdgcn_global_load_lds((const global_void_t *)(vs_ + lane16 + i_ * 1024), \
                                             (lds_void_t *)&ring[slot][1][wave_piece_elems + i_ * 512], 16, 0, 0); \
        }                                                                                     \
    } while (0)
    // this wave's share of every copy, and this lane's 16 bytes of a piece
    const int wave_piece_bytes = wave * 2 * PPW * 1024;
    const int wave_piece_elems = wave * 2 * PPW * 512;
    const int lane16 = lane * 16;

    // Per-lane LDS element offsets of the matrix-core operands inside a slot:
    // K row l32, chunk (2 ks + hl) swizzled; V^T row d = 32 mt + l32, chunk
    // (2 ks2 + hl) swizzled.
    int kofs[KS], vofs[MT][2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kofs[ks] = l32 * D + 8 * ((2 * ks + hl) ^ (l32 & KSW));
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int ks2 = 0; ks2 < 2; ++ks2) {
            const int d = 32 * mt + l32;
            vofs[mt][ks2] = d * 32 + 8 * ((2 * ks2 + hl) ^ ((d >> 2) & 3));
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

    // Union walk over whole blocks: the copy cursor (pa, pb, pkb) runs one
    // block ahead of the compute cursor (ca, cb, kb).
    ListCursor pa = ca, pb = cb;
    int pkb = kb;
    auto advance = [&](ListCursor &xa, ListCursor &xb, int &xkb) {
        if (xa.cur == xkb) { ++xa.j; list_seek(xa, g.nb); }
        if (xb.cur == xkb) { ++xb.j; list_seek(xb, g.nb); }
        xkb = min(xa.cur, xb.cur);
    };
    TRA_ISSUE(pkb, 0);
    advance(pa, pb, pkb);
    const bool two = pkb != INT32_MAX;
    if (two) {
        TRA_ISSUE(pkb, 1);
        advance(pa, pb, pkb);
        __builtin_amdgcn_s_waitcnt(wait_vmcnt(4 * PPW));  // block 0 landed
    } else {
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    }
    __syncthreads();

    auto block_step = [&](auto slot_tag) -> bool {
        constexpr int slot = decltype(slot_tag)::value;
        const bool mine = (side ? cb.cur : ca.cur) == kb;
        if (mine) {
            const uint32_t row = fdiv((uint32_t)kb, div_nbx);
            const int kbx = (int)((uint32_t)kb - row * div_nbx.d);
            const int kby = (int)(row - fdiv(row, div_nby) * div_nby.d);
            const int kny = min(kTileSide, g.H - kTileSide * kby);
            const int knx = min(kTileSide, g.W - kTileSide * kbx);
            const uint16_t *Kt = ring[slot][0];
            const uint16_t *Vt = ring[slot][1];
            f32x16_t s[2];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                bf16x8_t ka[KS];
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) ka[ks] = lds_load16<bf16x8_t>(Kt + hf * 32 * D + kofs[ks]);
#pragma unroll
                for (int r = 0; r < 16; ++r) s[hf][r] = 0.f;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    s[hf] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks], qreg[ks], s[hf], 0, 0, 0);
            }
            if (kny < kTileSide || knx < kTileSide) {
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const bool bad = (4 * hf + (r >> 2) >= kny) || (4 * hl + (r & 3) >= knx);
                        s[hf][r] = bad ? -INFINITY : s[hf][r];
                    }
            }
            float mx = -INFINITY;
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[hf][r]);
            mx = half_swap_max(mx) * scale_log2;
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
            f16x8_t pk[2][2];
            float psum0 = 0.f, psum1 = 0.f;
            const f16x2_t one2 = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    s[hf][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[hf][r], scale_log2, -m_ref));
#pragma unroll
                for (int ks2 = 0; ks2 < 2; ++ks2) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) pk[hf][ks2][e] = (_Float16)s[hf][8 * ks2 + e];
#pragma unroll
                    for (int e = 0; e < 8; e += 4) {
                        const f16x2_t a = {pk[hf][ks2][e], pk[hf][ks2][e + 1]};
                        const f16x2_t b = {pk[hf][ks2][e + 2], pk[hf][ks2][e + 3]};
                        psum0 = __builtin_amdgcn_fdot2(a, one2, psum0, false);
                        psum1 = __builtin_amdgcn_fdot2(b, one2, psum1, false);
                    }
                }
            }
            l_run += psum0 + psum1;
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int ks2 = 0; ks2 < 2; ++ks2) {
                        const f16x8_t a = lds_load16<f16x8_t>(Vt + hf * HALF + vofs[mt][ks2]);
                        acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pk[hf][ks2], acc[mt], 0, 0, 0);
                    }
        }
        advance(ca, cb, kb);
        if (kb == INT32_MAX) return false;
        // the next block is the only copy in flight: wait for it, then refill this slot
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        __syncthreads();
        if (pkb != INT32_MAX) {
            TRA_ISSUE(pkb, slot);
            advance(pa, pb, pkb);
        }
        return true;
    };
    while (block_step(SlotTag<0>{}) && block_step(SlotTag<1>{})) {
    }
#undef TRA_ISSUE

    const float l_tot = half_swap_sum(l_run);
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
                       const int32_t *idx, const int32_t *cnt, int64_t maxcnt,
                       const int32_t *order, const Grid &g, int heads, float *out,
                       hipStream_t s) {
    const int pph = pairs_per_head(g);
    const int64_t total = (int64_t)heads * pph;
    const int per_xcd = (int)((total + 7) / 8);
    const dim3 grid((unsigned)(8 * (int64_t)per_xcd)), block(kAttnThreads);
    const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
    auto magic = [](int d) {
        FastDiv f;
        f.d = (uint32_t)d;
        f.m = (((uint64_t)1 << 39) + (uint64_t)d - 1) / (uint64_t)d;
        return f;
    };
    const FastDiv div_nbx = magic(g.nbx), div_nby = magic(g.nby);
    if (D == 128)
        hipLaunchKernelGGL(attn_kernel<128>, grid, block, 0, s, q, kt, vt, idx, cnt, maxcnt, order,
                           g, heads, pph, per_xcd, div_nbx, div_nby, out, scale_log2);
    else if (D == 64)
        hipLaunchKernelGGL(attn_kernel<64>, grid, block, 0, s, q, kt, vt, idx, cnt, maxcnt, order,
                           g, heads, pph, per_xcd, div_nbx, div_nby, out, scale_log2);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace tra

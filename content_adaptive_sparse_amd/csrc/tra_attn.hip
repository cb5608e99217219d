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

#include "tra_device.h"

namespace tra {
namespace {

constexpr int kAttnThreads = 256;
// The running max is only moved (and O, l rescaled) when a tile's max exceeds
// it by more than this many powers of two; in between, probabilities are
// taken against the stale max (at most 2^8, exact in fp16) and the final
// normalisation by l uses the same reference, so the result is unchanged.
constexpr float kRescaleLog2 = 8.0f;

// WEIGHTED: every walk entry carries, per side, a log2 weight added to the
// logits of its keys (inverse inclusion probabilities of sampled blocks).
template <int D, bool WEIGHTED>
__global__ __launch_bounds__(kAttnThreads, 2) void attn_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kt,
    const uint16_t *__restrict__ vt, const int32_t *__restrict__ ulist,
    const int32_t *__restrict__ ulen, const float2 *__restrict__ ubias, int64_t ustride,
    const int32_t *__restrict__ order, Grid g,
    int heads, int pairs_per_head, int per_xcd, FastDiv div_nbx, FastDiv div_nby,
    float *__restrict__ out, float scale_log2) {
    constexpr int KS = D / 16;                  // k-steps of Q.K^T
    constexpr int MT = D / 32;                  // 32-row tiles of O^T
    constexpr int TILE = 64 * D;                // elements of a packed K or V^T tile
    constexpr int PIECES = TILE * 2 / 1024;     // 1 KB copies per tile
    constexpr int WAVES = kAttnThreads / 64;
    constexpr int PPW = PIECES / WAVES;         // pieces per wave and tile
    static_assert(PPW * WAVES == PIECES, "every piece copied exactly once");
    static_assert(PIECES * 512 == TILE, "pieces tile a tile exactly (no copy past a slot)");

    // Two-slot rings of packed K tiles (bf16) and V^T tiles (fp16).  Step u
    // reads K of union entry u and V^T of entry u - 1, while K of entry u + 1
    // and V^T of entry u land in the other slots.
    __shared__ __attribute__((aligned(1024))) uint16_t kring[2][TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t vring[2][TILE];

    // Work item: a pair of vertically adjacent query blocks of one head.
    // Consecutive workgroup ids land on different XCDs; every XCD is given a
    // contiguous range of items so its L2 sees neighbouring query blocks.  With
    // a work order (lists of unequal length) the ranges hold equal shares of
    // the total work and each is taken longest first; without one (dense mode:
    // equal work) the ranges hold equal item counts in raster order.
    const int64_t total = (int64_t)heads * pairs_per_head;
    int64_t item;
    if (order) {
        item = ((const const_i32_t *)order)[blockIdx.x];  // one slot per workgroup
        if (item < 0) return;
    } else {
        item = (int64_t)(blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    }
    if (item >= total) return;
    const int h = (int)(item / pairs_per_head);
    int blk[2];
    pair_blocks((int)(item % pairs_per_head), g, blk[0], blk[1]);

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int hl = lane >> 5, l32 = lane & 31;
    const int side = wave >> 1;          // which block of the pair this wave computes
    const int qb = blk[side];            // -1: absent (odd tile-row count)

    // This lane's query token.  The real queries of a block are numbered
    // first (row-major over the tile's real rows and columns), so an edge tile
    // with at most 32 of them leaves its second wave without work.  Lanes past
    // the real queries (and an absent block) take a clamped token and never
    // store.
    const int plane = g.nby * g.nbx;
    const int qbc = qb >= 0 ? qb : blk[0];
    const int t = qbc / plane, by = (qbc / g.nbx) % g.nby, bx = qbc % g.nbx;
    const int qny = min(kTileSide, g.H - kTileSide * by), qnx = min(kTileSide, g.W - kTileSide * bx);
    const int nq = qb >= 0 ? qny * qnx : 0;
    const bool live = 32 * (wave & 1) < nq;  // this wave has real queries
    const int qi = min(32 * (wave & 1) + l32, qny * qnx - 1);
    const bool qreal = 32 * (wave & 1) + l32 < nq;
    const int qy = kTileSide * by + qi / qnx, qx = kTileSide * bx + qi % qnx;
    const size_t qtok = (size_t)h * g.T * g.H * g.W + ((size_t)t * g.H + qy) * g.W + qx;
    float *o = out + qtok * D;

    // The item's union walk: n entries (block << 2) | sides (bit 0: the upper
    // block keeps it, bit 1: the lower one), read through a 64-entry window
    // held one entry per lane (the next window is fetched 64 entries early).
    // The dense mode walks every block with both sides.
    const int32_t *ul = ulist ? ulist + item * ustride : nullptr;
    int n = g.nb;
    if (ul) {
        const int64_t m = ((const const_i32_t *)ulen)[item];
        n = (int)(m < 0 ? 0 : (m > ustride ? ustride : m));
    }
    if (n == 0) {  // neither block keeps anything: zeros
        if (qreal)
            for (int c = 0; c < D / 2; c += 4)
                *reinterpret_cast<float4 *>(o + c + (D / 2) * hl) = make_float4(0.f, 0.f, 0.f, 0.f);
        return;
    }
    int win = 0, win_next = 0, wbase = 0;
    // this wave's side's weight of every entry, windowed like the entries
    const float *ubw = WEIGHTED ? reinterpret_cast<const float *>(ubias + item * ustride) + side
                                : nullptr;
    float bwin = 0.f, bwin_next = 0.f;
    if (ul) {
        win = lane < n ? ul[lane] : 0;
        win_next = 64 + lane < n ? ul[64 + lane] : 0;
        if (WEIGHTED) {
            bwin = lane < n ? ubw[2 * lane] : 0.f;
            bwin_next = 64 + lane < n ? ubw[2 * (64 + lane)] : 0.f;
        }
    }
    // Entry i (-1 past the end); called with i = 0, 1, 2, ... in turn.
    auto entry = [&](int i) -> int {
        if (i >= n) return -1;
        if (!ul) return (i << 2) | 3;
        if (i >= wbase + 64) {
            win = win_next;
            wbase += 64;
            win_next = wbase + 64 + lane < n ? ul[wbase + 64 + lane] : 0;
            if (WEIGHTED) {
                bwin = bwin_next;
                bwin_next = wbase + 64 + lane < n ? ubw[2 * (wbase + 64 + lane)] : 0.f;
            }
        }
        return __builtin_amdgcn_readlane(win, i - wbase);
    };
    // weight of entry i for this wave's side (right after entry(i): same window)
    auto weight = [&](int i) -> float {
        if (!WEIGHTED || i >= n) return 0.f;
        return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bwin), i - wbase));
    };

    // Direct global -> LDS copy of one packed tile of block `blk` into `dst`:
    // each wave moves PPW 1 KB pieces; lane l lands 16 bytes at piece base +
    // 16 l.  One global address and one LDS base (M0, wave-uniform) serve the
    // wave's pieces: a piece's 1 KB step is the instruction's immediate
    // offset, which applies to both the global and the LDS address.
    static_assert(PPW == 2 || PPW == 4, "pieces per wave");
    const size_t head_tiles = (size_t)h * g.nb;
    const int wave_lds_bytes = __builtin_amdgcn_readfirstlane(wave * PPW * 1024);
    const uint32_t lane_bytes = (uint32_t)(wave * PPW * 1024 + lane * 16);
#define TRA_ISSUE(src, dst, blk)                                                              \
    do {                                                                                      \
        const global_void_t *g_ = (const global_void_t *)(                                    \
            reinterpret_cast<const char *>(src + (head_tiles + (blk)) * 64 * D) + lane_bytes); \
        lds_void_t *l_ = (lds_void_t *)(reinterpret_cast<char *>(dst) + wave_lds_bytes);      \
        __builtin_amdgcn_global_load_lds(g_, l_, 16, 0, 0);                                   \
        __builtin_amdgcn_global_load_lds(g_, l_, 16, 1024, 0);                                \
        if constexpr (PPW == 4) {                                                             \
            __builtin_amdgcn_global_load_lds(g_, l_, 16, 2048, 0);                            \
            __builtin_amdgcn_global_load_lds(g_, l_, 16, 3072, 0);                            \
        }                                                                                     \
    } while (0)

    // Every matrix-core operand of a packed tile is a 1 KB piece in which this
    // lane's 8 elements sit at element 8 * lane.
    const int lane8 = lane * 8;

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

    int e0 = entry(0);
    float w0 = weight(0);
    int e1 = entry(1);  // entries u and u + 1
    float w1 = weight(1);
    TRA_ISSUE(kt, kring[0], e0 >> 2);
    if (e1 >= 0) {
        TRA_ISSUE(kt, kring[1], e1 >> 2);
        TRA_ISSUE(vt, vring[0], e0 >> 2);
        __builtin_amdgcn_s_waitcnt(wait_vmcnt(2 * PPW));  // K of entry 0 landed
    } else {
        TRA_ISSUE(vt, vring[0], e0 >> 2);
        __builtin_amdgcn_s_waitcnt(wait_vmcnt(PPW));
    }
    __syncthreads();

    // Probabilities (fp16) of the previous entry, waiting for their P.V, and
    // the rescale of O their reference asks for.
    f16x8_t pk[2][2];
    bool rescale = false;
    float alpha_o = 1.f;
    bool prev_mine = false;  // this wave's block kept the previous entry

    // One step of the software pipeline for this wave: the logits of entry u
    // (DS) on the matrix cores; then O += V^T P^T for the previous entry (DP)
    // on the matrix cores while the VALU turns entry u's logits into
    // probabilities (max, reference, exp, fp16, row sums).  A move of the
    // reference rescales O before the next product, after the previous
    // entry's product has landed in it.
    auto work = [&](auto slot_tag, auto ds_tag, auto dp_tag) {
        constexpr int s = decltype(slot_tag)::value;
        constexpr bool DS = decltype(ds_tag)::value != 0;
        constexpr bool DP = decltype(dp_tag)::value != 0;
        f32x16_t sb[2];
        if constexpr (DS) {
            const uint16_t *Kt = kring[s];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
                for (int r = 0; r < 16; ++r) sb[hf][r] = 0.f;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const bf16x8_t ka = lds_load16<bf16x8_t>(Kt + (hf * KS + ks) * 512 + lane8);
                    sb[hf] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[ks], sb[hf], 0, 0, 0);
                }
            }
            const uint32_t kb = (uint32_t)(e0 >> 2);
            const uint32_t row = fdiv(kb, div_nbx);
            const int kbx = (int)(kb - row * div_nbx.d);
            const int kby = (int)(row - fdiv(row, div_nby) * div_nby.d);
            mask_edge_keys(sb, min(kTileSide, g.H - kTileSide * kby),
                           min(kTileSide, g.W - kTileSide * kbx), hl, -INFINITY);
        }
        if constexpr (DP) {
            if (rescale) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[mt][r] *= alpha_o;
            }
            const uint16_t *Vt = vring[s ^ 1];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int ks2 = 0; ks2 < 2; ++ks2) {
                        const f16x8_t a = lds_load16<f16x8_t>(Vt + ((hf * MT + mt) * 2 + ks2) * 512 + lane8);
                        acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pk[hf][ks2], acc[mt], 0, 0, 0);
                    }
        }
        if constexpr (DS) {
            float mx = -INFINITY;
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sb[hf][r]);
            mx = half_swap_max(mx) * scale_log2 + w0;
            const bool grow = mx > m_ref + kRescaleLog2;
            const float m_new = grow ? mx : m_ref;
            const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
            m_ref = m_new;
            const float bias = w0 - m_ref;
            float psum0 = 0.f, psum1 = 0.f;
            const f16x2_t one2 = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    sb[hf][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sb[hf][r], scale_log2, bias));
#pragma unroll
                for (int ks2 = 0; ks2 < 2; ++ks2) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) pk[hf][ks2][e] = (_Float16)sb[hf][8 * ks2 + e];
#pragma unroll
                    for (int e = 0; e < 8; e += 4) {
                        const f16x2_t a = {pk[hf][ks2][e], pk[hf][ks2][e + 1]};
                        const f16x2_t b = {pk[hf][ks2][e + 2], pk[hf][ks2][e + 3]};
                        psum0 = __builtin_amdgcn_fdot2(a, one2, psum0, false);
                        psum1 = __builtin_amdgcn_fdot2(b, one2, psum1, false);
                    }
                }
            }
            l_run = l_run * alpha + (psum0 + psum1);
            rescale = __any(grow);  // O follows before this entry's P.V
            alpha_o = alpha;
        }
    };
    using T0 = SlotTag<0>;
    using T1 = SlotTag<1>;

    // Step u: K of entry u is in kring[u & 1], V^T of entry u - 1 in
    // vring[(u - 1) & 1].  One extra step after the last entry drains the
    // pipeline (e0 == -1).
    int u = 0;
    auto step = [&](auto slot_tag) -> bool {
        const bool mine = live && e0 >= 0 && ((e0 >> side) & 1);
        if (mine) {
            if (prev_mine) work(slot_tag, T1{}, T1{});
            else work(slot_tag, T1{}, T0{});
        } else if (prev_mine) {
            work(slot_tag, T0{}, T1{});
        }
        prev_mine = mine;
        if (e0 < 0) return false;
        // K of entry u + 1 and V^T of entry u were the copies in flight
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        __syncthreads();
        constexpr int s = decltype(slot_tag)::value;
        const int e2 = entry(u + 2);
        const float w2 = weight(u + 2);
        if (e2 >= 0) TRA_ISSUE(kt, kring[s], e2 >> 2);      // entry u + 2
        if (e1 >= 0) TRA_ISSUE(vt, vring[s ^ 1], e1 >> 2);  // entry u + 1
        e0 = e1;
        e1 = e2;
        w0 = w1;
        w1 = w2;
        ++u;
        return true;
    };
    while (step(T0{}) && step(T1{})) {
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
                       const int32_t *ulist, const int32_t *ulen, const float2 *ubias,
                       int64_t ustride, const int32_t *order, const Grid &g, int heads,
                       float *out, hipStream_t s) {
    const int pph = pairs_per_head(g);
    const int64_t total = (int64_t)heads * pph;
    const int per_xcd = (int)((total + 7) / 8);
    // one workgroup per slot of the work order, or per item in XCD ranges
    const dim3 grid((unsigned)(order ? order_slots(g, heads) : 8 * (int64_t)per_xcd)),
        block(kAttnThreads);
    const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
    const FastDiv div_nbx = make_fastdiv(g.nbx), div_nby = make_fastdiv(g.nby);
#define TRA_LAUNCH(DD, WW)                                                                    \
    hipLaunchKernelGGL((attn_kernel<DD, WW>), grid, block, 0, s, q, kt, vt, ulist, ulen, ubias,  \
                       ustride, order, g, heads, pph, per_xcd, div_nbx, div_nby, out, scale_log2)
    const bool weighted = ubias != nullptr && ulist != nullptr;
    if (D == 128 && weighted)
        TRA_LAUNCH(128, true);
    else if (D == 128)
        TRA_LAUNCH(128, false);
    else if (D == 64 && weighted)
        TRA_LAUNCH(64, true);
    else if (D == 64)
        TRA_LAUNCH(64, false);
    else
        return hipErrorInvalidValue;
#undef TRA_LAUNCH
    return hipGetLastError();
}

}  // namespace tra

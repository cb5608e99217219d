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
//   online softmax     per query = per lane column, exp2 with the scale folded,
//                      against a running reference that only moves when a
//                      probability would overflow fp16 (no max per tile)
//   O^T += V^T P^T     v_mfma_f32_32x32x16_f16 (P rounded to fp16)
// Working on the transposed products keeps every query's logits and output in
// one lane pair (lanes l and l + 32), so the softmax needs a single cross-lane
// exchange per tile and P feeds the second product without moving data.
#include <math.h>

#include "tra_device.h"

namespace tra {
namespace {

constexpr int kAttnThreads = 256;
// Probabilities are taken against a running reference m: 2^(s log2(e)/sqrt(d)
// - m) in fp16, which holds up to 2^16.  m is not the running max: a tile only
// moves it when one of its probabilities overflows fp16 (the row sum becomes
// inf), and then to the tile's max if that exceeds m by more than this many
// powers of two (O and l rescaled).  The final normalisation by l uses the same
// reference, so the result does not depend on it; fp16 keeps 11 significant
// bits anywhere in its normal range.
constexpr float kRescaleLog2 = 8.0f;
// Slots past the end of an XCD range that look for other ranges' last items
// (later slots of that XCD exit at once).
constexpr int kThieves = 32;

// WEIGHTED: every walk entry carries, per side, a log2 weight added to the
// logits of its keys (inverse inclusion probabilities of sampled blocks).
// ENTROPY: each query also keeps, against the same lazy reference m, the fp32
// sums Z = sum 2^x and A = sum x 2^x over x = s log2(e) / sqrt(d) - m, and
// writes its row's entropy H = ln Z - ln 2 A / Z with the base radius it
// implies (the token policy's warm-up, fused into the attention pass).
template <int D, bool WEIGHTED, bool ENTROPY>
__global__ __launch_bounds__(kAttnThreads, 2) void attn_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kt,
    const uint16_t *__restrict__ vt, const int32_t *__restrict__ vexp,
    const int2 *__restrict__ pairs, const int32_t *__restrict__ ulist,
    const int32_t *__restrict__ ulen,
    const float2 *__restrict__ ubias, int64_t ustride, const int32_t *__restrict__ order,
    int32_t *__restrict__ sched, Grid g,
    int heads, int items_per_head, int per_xcd, FastDiv div_nbx, FastDiv div_nby,
    float *__restrict__ out, float scale_log2, EntropyOut eo) {
    static_assert(!(WEIGHTED && ENTROPY), "entropy of unweighted rows only");
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

    // Work item: two query blocks of one head -- the plan's pair table, or
    // vertically adjacent blocks in dense mode.  Consecutive workgroup ids land
    // on different XCDs; every XCD is given a contiguous range of items so its
    // L2 sees neighbouring query blocks.  With a work order (lists of unequal
    // length) the ranges hold equal shares of the total work and each is taken
    // by walk length class, longest class first; without one (dense mode: equal
    // work) the ranges hold equal item counts in raster order.  Along a work
    // order the first three quarters of each range are taken in place; the last
    // quarter (its shortest items) is claimed at run time, by the range's own
    // workgroups and, once their range is spent, by other XCDs': the XCDs do
    // not run at one speed (equal ranges of dense work finish up to 6% apart),
    // so the fast ones take over the slow ones' last items, and only those
    // items pay for the claim's atomic.
    const int64_t total = (int64_t)heads * items_per_head;
    int64_t item;
    if (!ENTROPY && order) {  // the entropy warm-up is dense: no work order
        const const_i32_t *ord = (const const_i32_t *)order;
        const int64_t cap = gridDim.x / kXcdRanges;  // slots per range
        const int x = (int)(blockIdx.x % kXcdRanges);
        const int64_t k = blockIdx.x / kXcdRanges;
        const int nx = ord[kXcdRanges * cap + x];  // the range's length
        const int mine = ord[blockIdx.x];          // loaded beside it
        if (k < nx - nx / 4) {
            item = mine;
        } else if (k >= nx + kThieves) {
            item = -1;  // enough slots past the range's end look for other ranges' items
        } else {
            // the own range's last quarter first (slots inside the range); once
            // that is spent, one look at every other range's counter (a lane
            // each), then a claim on the first range with items left, looked at
            // again if that claim comes late
            __shared__ int32_t claimed;
            if (threadIdx.x < 64) {
                const int lane = threadIdx.x;
                int it = -1;
                if (lane == 0 && k < nx) {
                    const int c = atomicAdd(sched + x * kSchedStride, 1);
                    if (c < nx / 4) it = ord[kXcdRanges * (int64_t)(nx - nx / 4 + c) + x];
                }
                it = __shfl(it, 0);
                for (int round = 0; round < kXcdRanges && it < 0; ++round) {
                    const int y = (x + 1 + lane) % kXcdRanges;
                    bool left = false;
                    int ny = 0;
                    if (lane < kXcdRanges - 1) {
                        ny = ord[kXcdRanges * cap + y];
                        left = atomicAdd(sched + y * kSchedStride, 0) < ny / 4;
                    }
                    const uint64_t cand = __ballot(left);
                    if (!cand) break;  // every range's last quarter is spent
                    const int j = __builtin_ctzll(cand);
                    if (lane == j) {
                        const int c = atomicAdd(sched + y * kSchedStride, 1);
                        if (c < ny / 4) it = ord[kXcdRanges * (int64_t)(ny - ny / 4 + c) + y];
                    }
                    it = __shfl(it, j);
                }
                if (lane == 0) claimed = it;
            }
            __syncthreads();
            item = claimed;
        }
    } else {
        item = (int64_t)(blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    }
    if (item < 0 || item >= total) return;
    const int h = (int)(item / items_per_head);
    int blk[2];
    if (pairs) {
        const int2 pr = reinterpret_cast<const int2 *>(pairs)[item];
        blk[0] = __builtin_amdgcn_readfirstlane(pr.x);
        blk[1] = __builtin_amdgcn_readfirstlane(pr.y);
        if (blk[0] < 0) return;  // an unused slot of the pair table
    } else {
        pair_blocks((int)(item % items_per_head), g, blk[0], blk[1]);
    }

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
    if (n == 0) {  // neither block keeps anything: zeros (and, for ENTROPY, an empty row's H = 0)
        if (qreal)
            for (int c = 0; c < D / 2; c += 4)
                *reinterpret_cast<float4 *>(o + c + (D / 2) * hl) = make_float4(0.f, 0.f, 0.f, 0.f);
        if (ENTROPY && qreal && hl == 0) {
            float r0;
            eo.ent[qtok] = entropy_and_radius(1.f, 0.f, t, g, eo.tau, eo.two_gamma_log2e, &r0);
            eo.r0[qtok] = r0;
        }
        return;
    }
    // V was packed as v 2^ve (fp16 range); the output is scaled back by 2^-ve
    const int ve = ((const const_i32_t *)vexp)[h];
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
    // The copies are written as inline assembly so that the compiler does not
    // track them: it cannot tell the ring slots apart and would otherwise wait
    // for every copy in flight before the next LDS operand read, although the
    // slot being filled is never read before the next barrier.  Every wave
    // waits for its own copies (vmcnt 0) before each barrier, and nothing
    // reads a slot between the copy into it and that barrier.  The copies
    // write LDS only (no register results), so no register is left in flight.
    static_assert(PPW == 2 || PPW == 4, "pieces per wave");
    const size_t head_tiles = (size_t)h * g.nb;
    const int wave_lds_bytes = __builtin_amdgcn_readfirstlane(wave * PPW * 1024);
    const uint32_t lane_bytes = (uint32_t)(wave * PPW * 1024 + lane * 16);
#define TRA_ISSUE(src, dst, blk)                                                                \
    do {                                                                                        \
        const char *g_ =                                                                        \
            reinterpret_cast<const char *>(src + (head_tiles + (blk)) * 64 * D) + lane_bytes;   \
        const uint32_t m_ = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t *)( \
            reinterpret_cast<char *>(dst) + wave_lds_bytes));                                   \
        if constexpr (PPW == 4)                                                                 \
            asm volatile("global_load_lds_dwordx4 %1, off\n\t"                                   \
                         "global_load_lds_dwordx4 %1, off offset:1024\n\t"                       \
                         "global_load_lds_dwordx4 %1, off offset:2048\n\t"                       \
                         "global_load_lds_dwordx4 %1, off offset:3072" ::"{m0}"(m_),              \
                         "v"(g_)                                                                \
                         : "memory");                                                           \
        else                                                                                    \
            asm volatile("global_load_lds_dwordx4 %1, off\n\t"                                   \
                         "global_load_lds_dwordx4 %1, off offset:1024" ::"{m0}"(m_), "v"(g_)      \
                         : "memory");                                                           \
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
    float ent_z = 0.f, ent_a = 0.f;  // ENTROPY: fp32 row sums Z and A of this lane's keys
    // Missing keys of edge tiles: -inf, or a finite -1e30 when x 2^x is summed
    // (so that 0 * x stays 0)
    constexpr float kMaskFill = ENTROPY ? -1e30f : -INFINITY;

    int e0 = entry(0);
    float w0 = weight(0);
    int e1 = entry(1);  // entries u and u + 1
    float w1 = weight(1);
    TRA_ISSUE(kt, kring[0], e0 >> 2);
    if (e1 >= 0) TRA_ISSUE(kt, kring[1], e1 >> 2);
    TRA_ISSUE(vt, vring[0], e0 >> 2);
    // every load so far (Q rows, walk windows, the first copies) has landed:
    // the compiler, which does not see the copies, then keeps no wait for the
    // Q rows inside the loop
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();

    // Row sums of fp16 probabilities (two independent chains).
    auto row_sum_f16 = [&](const f16x8_t &p, float s0, float &s1) -> float {
        const f16x2_t one2 = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
        for (int e = 0; e < 8; e += 4) {
            const f16x2_t a = {p[e], p[e + 1]};
            const f16x2_t b = {p[e + 2], p[e + 3]};
            s0 = __builtin_amdgcn_fdot2(a, one2, s0, false);
            s1 = __builtin_amdgcn_fdot2(b, one2, s1, false);
        }
        return s0;
    };
    // fp16 probabilities 2^(s log2(e) / sqrt(d) + bias) of one tile and their
    // row sum (this lane's keys).  Missing keys of an edge tile (rows >= kny,
    // columns >= knx; their logits are 0 from the zero K rows) are cleared in
    // the fp16 registers: a packed register holds key row 4 hf + 2 ks2 + j / 2
    // (register j of the 8-element group) and key columns 4 hl + 2 (j % 2) and
    // the next one.
    // ENTROPY: the logits of missing keys are already -1e30 (so their
    // probabilities are 0 here) and the fp32 sums z = sum 2^x, a = sum x 2^x of
    // this lane's keys are returned as well.
    auto softmax_fp16 = [&](const f32x16_t (&sv)[2], float bias, int kny_, int knx_,
                            f16x8_t (&pn)[2][2], float &z, float &a) -> float {
        float s0 = 0.f, s1 = 0.f;
        float z0 = 0.f, z1 = 0.f, a0 = 0.f, a1 = 0.f;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int ks2 = 0; ks2 < 2; ++ks2) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float x = __builtin_fmaf(sv[hf][8 * ks2 + e], scale_log2, bias);
                    const float p = __builtin_amdgcn_exp2f(x);
                    pn[hf][ks2][e] = (_Float16)p;
                    if constexpr (ENTROPY) {
                        if (e & 1) {
                            z1 += p;
                            a1 = __builtin_fmaf(p, x, a1);
                        } else {
                            z0 += p;
                            a0 = __builtin_fmaf(p, x, a0);
                        }
                    }
                }
            }
        z = z0 + z1;
        a = a0 + a1;
        if (kny_ < kTileSide || knx_ < kTileSide) {
            const int cm = knx_ - 4 * hl;  // real columns among this lane's four
            const uint32_t m01 = cm >= 2 ? 0xffffffffu : (cm == 1 ? 0x0000ffffu : 0u);
            const uint32_t m23 = cm >= 4 ? 0xffffffffu : (cm == 3 ? 0x0000ffffu : 0u);
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int ks2 = 0; ks2 < 2; ++ks2) {
                    u32x4_t w = __builtin_bit_cast(u32x4_t, pn[hf][ks2]);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const bool row_ok = 4 * hf + 2 * ks2 + j / 2 < kny_;
                        w[j] &= row_ok ? ((j & 1) ? m23 : m01) : 0u;
                    }
                    pn[hf][ks2] = __builtin_bit_cast(f16x8_t, w);
                }
        }
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int ks2 = 0; ks2 < 2; ++ks2) s0 = row_sum_f16(pn[hf][ks2], s0, s1);
        return s0 + s1;
    };

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
        int kny = kTileSide, knx = kTileSide;
        // a reference move of the previous entry rescales O before this step's
        // P.V (the multiply waits for the previous products); taken first so that
        // the products and the softmax below share one basic block
        if constexpr (DP) {
            if (rescale) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[mt][r] *= alpha_o;
            }
        }
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
            // the K operand reads run six ahead of the products that use them
            __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);  // 6 LDS reads
#pragma unroll
            for (int i = 0; i < 2 * KS - 6; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 product
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 LDS read
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);  // the last 6 products
            const uint32_t kb = (uint32_t)(e0 >> 2);
            const uint32_t row = fdiv(kb, div_nbx);
            const int kbx = (int)(kb - row * div_nbx.d);
            const int kby = (int)(row - fdiv(row, div_nby) * div_nby.d);
            kny = min(kTileSide, g.H - kTileSide * kby);
            knx = min(kTileSide, g.W - kTileSide * kbx);
            if constexpr (ENTROPY) mask_edge_keys(sb, kny, knx, hl, kMaskFill);
        }
        if constexpr (DP) {
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
            // Probabilities against the running reference without a max: a key
            // more than 2^16 above it overflows fp16 to inf, which the row sum
            // shows; only then is the step redone against a moved reference.
            f16x8_t pn[2][2];
            float z, a;
            float psum = softmax_fp16(sb, w0 - m_ref, ENTROPY ? kTileSide : kny,
                                      ENTROPY ? kTileSide : knx, pn, z, a);
            if (__builtin_expect(__any(!(psum < INFINITY)), 0)) {
                if constexpr (!ENTROPY) mask_edge_keys(sb, kny, knx, hl, -INFINITY);
                float mx = -INFINITY;
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sb[hf][r]);
                mx = half_swap_max(mx) * scale_log2 + w0;
                const bool grow = mx > m_ref + kRescaleLog2;
                const float m_new = grow ? mx : m_ref;
                alpha_o = __builtin_amdgcn_exp2f(m_ref - m_new);
                if constexpr (ENTROPY) {
                    // moving the reference by delta: Z' = 2^-delta Z, A' = 2^-delta (A - delta Z)
                    ent_a = alpha_o * __builtin_fmaf(m_ref - m_new, ent_z, ent_a);
                    ent_z *= alpha_o;
                }
                m_ref = m_new;
                l_run *= alpha_o;
                rescale = true;  // O follows before this entry's P.V
                psum = softmax_fp16(sb, w0 - m_ref, kTileSide, kTileSide, pn, z, a);
            } else {
                rescale = false;
            }
            l_run += psum;
            if constexpr (ENTROPY) {
                ent_z += z;
                ent_a += a;
            }
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int ks2 = 0; ks2 < 2; ++ks2) pk[hf][ks2] = pn[hf][ks2];
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
        // a wave computing a step issues ahead of one at the barrier or
        // issuing copies (two waves of different workgroups share a SIMD)
        __builtin_amdgcn_s_setprio(1);
        if (mine) {
            if (prev_mine) work(slot_tag, T1{}, T1{});
            else work(slot_tag, T1{}, T0{});
        } else if (prev_mine) {
            work(slot_tag, T0{}, T1{});
        }
        prev_mine = mine;
        __builtin_amdgcn_s_setprio(0);
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
                *reinterpret_cast<float4 *>(o + d0) = make_float4(
                    ldexpf(acc[mt][4 * g4] * inv, -ve), ldexpf(acc[mt][4 * g4 + 1] * inv, -ve),
                    ldexpf(acc[mt][4 * g4 + 2] * inv, -ve), ldexpf(acc[mt][4 * g4 + 3] * inv, -ve));
            }
    }
    if constexpr (ENTROPY) {
        const float zt = half_swap_sum(ent_z), at = half_swap_sum(ent_a);
        if (qreal && hl == 0) {
            float r0;
            eo.ent[qtok] = entropy_and_radius(zt, at, t, g, eo.tau, eo.two_gamma_log2e, &r0);
            eo.r0[qtok] = r0;
        }
    }
}

__global__ void zero_kernel(int32_t *p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0;
}

}  // namespace

hipError_t launch_zero(int32_t *p, int64_t n, hipStream_t s) {
    if (n > 0)
        hipLaunchKernelGGL(zero_kernel, dim3((unsigned)((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024)),
                           dim3(256), 0, s, p, n);
    return hipGetLastError();
}

hipError_t launch_attn(int D, const uint16_t *q, const uint16_t *kt, const uint16_t *vt,
                       const int32_t *vexp, const int2 *pairs, const int32_t *ulist,
                       const int32_t *ulen, const float2 *ubias, int64_t ustride,
                       const int32_t *order, int32_t *sched, const Grid &g, int heads, float *out,
                       hipStream_t s, const EntropyOut *entropy) {
    if (order && !sched) return hipErrorInvalidValue;
    // items per head: the plan's slots, or the vertical pairs of dense mode
    const int pph = pairs ? plan_slots_per_head(g) : pairs_per_head(g);
    const int64_t total = (int64_t)heads * pph;
    const int per_xcd = (int)((total + 7) / 8);
    // one workgroup per slot of the work order, or per item in XCD ranges
    const dim3 grid((unsigned)(order ? order_slots(g, heads) : 8 * (int64_t)per_xcd)),
        block(kAttnThreads);
    const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
    const FastDiv div_nbx = make_fastdiv(g.nbx), div_nby = make_fastdiv(g.nby);
    const EntropyOut eo = entropy ? *entropy : EntropyOut{nullptr, nullptr, 0.f, 0.f};
#define TRA_LAUNCH(DD, WW, EE)                                                                \
    hipLaunchKernelGGL((attn_kernel<DD, WW, EE>), grid, block, 0, s, q, kt, vt, vexp, pairs,     \
                       ulist, ulen, ubias, ustride, order, sched, g, heads, pph, per_xcd, div_nbx, \
                       div_nby, out, scale_log2, eo)
    const bool weighted = ubias != nullptr && ulist != nullptr;
    if (weighted && entropy) return hipErrorInvalidValue;
    if (entropy && order) return hipErrorInvalidValue;  // the entropy warm-up walks every block
    if (D == 128 && weighted)
        TRA_LAUNCH(128, true, false);
    else if (D == 128 && entropy)
        TRA_LAUNCH(128, false, true);
    else if (D == 128)
        TRA_LAUNCH(128, false, false);
    else if (D == 64 && weighted)
        TRA_LAUNCH(64, true, false);
    else if (D == 64 && entropy)
        TRA_LAUNCH(64, false, true);
    else if (D == 64)
        TRA_LAUNCH(64, false, false);
    else
        return hipErrorInvalidValue;
#undef TRA_LAUNCH
    return hipGetLastError();
}

}  // namespace tra

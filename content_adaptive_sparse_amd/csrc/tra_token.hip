// Token-level radius policy: entropy of every query's dense attention row (the
// warm-up), its token budget and base radius, and the block lists voted by the
// queries' spatiotemporal disks.
//
// Token Radius Attention for Efficient Video Generation:
//   "Insight I" / "The TRA Pipeline: Entropy-to-Budget" -- the entropy H_i of a
//   query's attention row decides its budget, about tau exp(H_i) keys (the
//   page's tau exp(H_i) / N as a fraction of the N keys);
//   "Insight II" / "Budget-to-Radius" -- the budget becomes a base radius r0_i,
//   and the radius in a frame delta frames away is r0_i exp(-gamma delta): a
//   disk per frame.  Here r0_i makes the disks' areas over the T frames add up
//   to the budget: r0_i = sqrt(b_i / (pi sum_t' exp(-2 gamma |t' - t_i|)));
//   "Fused CUDA Kernels" -- distance computation, radius comparison and token
//   voting turn the token disks into a block-sparse mask: key block K is kept
//   for query block Q when at least min_votes real query tokens of Q reach a
//   real key token of K.
#include <math.h>

#include "tra_device.h"

namespace tra {
namespace {

constexpr int kEntThreads = 256;
constexpr float kRefLog2 = 8.0f;     // lazy reference: move when a tile exceeds it by 2^8
constexpr float kMaskedLogit = -1e30f;  // finite, so that e * x stays 0 for masked keys

// One workgroup of four wave64 per pair of vertically adjacent query blocks of
// one head (two waves per block, 32 queries per wave), walking every key tile
// of the head.  Per tile: S^T = K Q^T on bf16 matrix cores (K pieces copied
// straight into a two-slot LDS ring), then per query, in base 2 with a lazy
// reference m: Z = sum 2^x, A = sum x 2^x over x = s log2(e) / sqrt(d) - m.
// The entropy of the row is H = ln Z - ln 2 A / Z.
template <int D>
__global__ __launch_bounds__(kEntThreads, 2) void token_entropy_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kt, Grid g, int heads,
    int pairs_per_head, int per_xcd, FastDiv div_nbx, FastDiv div_nby, float scale_log2,
    float tau, float two_gamma_log2e, float *__restrict__ ent, float *__restrict__ r0) {
    constexpr int KS = D / 16;
    constexpr int TILE = 64 * D;
    constexpr int PIECES = TILE * 2 / 1024;
    constexpr int WAVES = kEntThreads / 64;
    constexpr int PPW = PIECES / WAVES;
    static_assert(PPW * WAVES == PIECES, "every piece copied exactly once");

    __shared__ __attribute__((aligned(1024))) uint16_t kring[2][TILE];

    const int64_t total = (int64_t)heads * pairs_per_head;
    const int64_t item = (int64_t)(blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    if (item >= total) return;
    const int h = (int)(item / pairs_per_head);
    int blk[2];
    pair_blocks((int)(item % pairs_per_head), g, blk[0], blk[1]);

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int hl = lane >> 5, l32 = lane & 31;
    const int qb = blk[wave >> 1];
    const int plane = g.nby * g.nbx;
    const int qbc = qb >= 0 ? qb : blk[0];
    const int t = qbc / plane, by = (qbc / g.nbx) % g.nby, bx = qbc % g.nbx;
    // The block's real queries are numbered first (row-major over the tile's
    // real rows and columns): a tile with at most 32 leaves its second wave
    // without queries, and that wave only helps with the copies.
    const int qny = min(kTileSide, g.H - kTileSide * by), qnx = min(kTileSide, g.W - kTileSide * bx);
    const int nq = qb >= 0 ? qny * qnx : 0;
    const bool live = 32 * (wave & 1) < nq;
    const int qi = min(32 * (wave & 1) + l32, qny * qnx - 1);
    const bool qreal = 32 * (wave & 1) + l32 < nq;
    const int qy = kTileSide * by + qi / qnx, qx = kTileSide * bx + qi % qnx;
    const size_t qtok = ((size_t)t * g.H + qy) * g.W + qx;
    const size_t head_tok = (size_t)h * g.T * g.H * g.W;

    bf16x8_t qreg[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        qreg[ks] = *reinterpret_cast<const bf16x8_t *>(q + (head_tok + qtok) * D + 16 * ks + 8 * hl);

    // Copy of key tile kb into a slot: each wave moves PPW 1 KB pieces with one
    // global address and one wave-uniform LDS base, the pieces' 1 KB step in the
    // instruction's immediate offset (it moves the global and the LDS address).
    // Inline assembly, so that the compiler does not wait for the copy in flight
    // (into the other slot) before this tile's operand reads; each wave waits
    // for its own copies before the barrier that precedes the tile's use.
    static_assert(PPW == 2 || PPW == 4, "pieces per wave");
    const size_t head_tiles = (size_t)h * g.nb;
    const int wave_lds_bytes = __builtin_amdgcn_readfirstlane(wave * PPW * 1024);
    const uint32_t lane_bytes = (uint32_t)(wave * PPW * 1024 + lane * 16);
    const int lane8 = lane * 8;
    auto issue = [&](int kb, int slot) {
        const char *g_ = reinterpret_cast<const char *>(kt + (head_tiles + kb) * 64 * D) + lane_bytes;
        const uint32_t m_ = __builtin_amdgcn_readfirstlane(
            (uint32_t)(uintptr_t)(lds_void_t *)(reinterpret_cast<char *>(kring[slot]) + wave_lds_bytes));
        if constexpr (PPW == 4)
            asm volatile("global_load_lds_dwordx4 %1, off\n\t"
                         "global_load_lds_dwordx4 %1, off offset:1024\n\t"
                         "global_load_lds_dwordx4 %1, off offset:2048\n\t"
                         "global_load_lds_dwordx4 %1, off offset:3072" ::"{m0}"(m_), "v"(g_)
                         : "memory");
        else
            asm volatile("global_load_lds_dwordx4 %1, off\n\t"
                         "global_load_lds_dwordx4 %1, off offset:1024" ::"{m0}"(m_), "v"(g_)
                         : "memory");
    };

    issue(0, 0);
    if (g.nb > 1) issue(1, 1);
    // every load so far (Q rows, the first copies) has landed; the compiler, which
    // does not see the copies, then keeps no wait for the Q rows inside the loop
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();

    float m_ref = -1e30f, Z = 0.f, A = 0.f;
    for (int kb = 0; kb < g.nb; ++kb) {
        if (live) {  // a wave without real queries only copies
            const uint16_t *Kt = kring[kb & 1];
            f32x16_t sb[2];
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
            const uint32_t row = fdiv((uint32_t)kb, div_nbx);
            const int kbx = (int)((uint32_t)kb - row * div_nbx.d);
            const int kby = (int)(row - fdiv(row, div_nby) * div_nby.d);
            mask_edge_keys(sb, min(kTileSide, g.H - kTileSide * kby),
                           min(kTileSide, g.W - kTileSide * kbx), hl, kMaskedLogit);
            float mx = -INFINITY;
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sb[hf][r]);
            mx = half_swap_max(mx) * scale_log2;
            const bool grow = mx > m_ref + kRefLog2;
            if (__any(grow)) {
                // moving the reference from m to m': Z' = 2^(m - m') Z,
                // A' = 2^(m - m') (A + (m - m') Z)
                const float m_new = grow ? mx : m_ref;
                const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
                A = alpha * __builtin_fmaf(m_ref - m_new, Z, A);
                Z *= alpha;
                m_ref = m_new;
            }
            float z0 = 0.f, z1 = 0.f, a0 = 0.f, a1 = 0.f;
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    const float x0 = __builtin_fmaf(sb[hf][r], scale_log2, -m_ref);
                    const float x1 = __builtin_fmaf(sb[hf][r + 1], scale_log2, -m_ref);
                    const float e0 = __builtin_amdgcn_exp2f(x0), e1 = __builtin_amdgcn_exp2f(x1);
                    z0 += e0;
                    z1 += e1;
                    a0 = __builtin_fmaf(e0, x0, a0);
                    a1 = __builtin_fmaf(e1, x1, a1);
                }
            Z += z0 + z1;
            A += a0 + a1;
        }
        if (kb + 1 == g.nb) break;
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // the next tile has landed
        __syncthreads();                          // and every wave is done with this one
        if (kb + 2 < g.nb) issue(kb + 2, kb & 1);
    }

    const float Zt = half_swap_sum(Z), At = half_swap_sum(A);
    if (qreal && hl == 0) {
        // Z >= 1: the key that last set the reference contributes 2^0
        float rq;
        ent[head_tok + qtok] = entropy_and_radius(Zt, At, t, g, tau, two_gamma_log2e, &rq);
        r0[head_tok + qtok] = rq;
    }
}

// Voting lists: one wave64 per (head, query block), lane l = query token
// (y, x) = (8 by + l / 8, 8 bx + l % 8).  For every frame, the wave's largest
// radius bounds the candidate tiles; per candidate each lane tests its
// squared distance to the tile's real-token rectangle (an exact integer)
// against its squared radius, and the tile is kept when the ballot count
// reaches min_votes.  Lists come out ascending (frame, tile row, tile column).
__global__ __launch_bounds__(256) void token_mask_kernel(
    const float *__restrict__ r0, Grid g, int64_t rows, float gamma_log2e, int min_votes,
    int64_t maxcnt, int32_t *__restrict__ idx, int32_t *__restrict__ cnt) {
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;
    const int h = (int)(row / g.nb);
    const int qb = (int)(row % g.nb);
    const int plane = g.nby * g.nbx;
    const int t = qb / plane, by = (qb / g.nbx) % g.nby, bx = qb % g.nbx;
    const int y = kTileSide * by + (lane >> 3), x = kTileSide * bx + (lane & 7);
    const bool real = y < g.H && x < g.W;
    const float rq = real ? r0[(((size_t)h * g.T + t) * g.H + y) * g.W + x] : 0.f;
    const int ylo = kTileSide * by, yhi = min(g.H - 1, kTileSide * by + kTileSide - 1);
    const int xlo = kTileSide * bx, xhi = min(g.W - 1, kTileSide * bx + kTileSide - 1);

    int32_t *out = idx + row * maxcnt;
    int64_t count = 0;
    for (int tk = 0; tk < g.T; ++tk) {
        const float r = rq * __builtin_amdgcn_exp2f(-gamma_log2e * (float)abs(tk - t));
        const float r2 = r * r;
        float R = real ? r : 0.f;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) R = fmaxf(R, __shfl_xor(R, off));
        // tiles holding a token within R of the query block's token rectangle
        const int ky0 = max(0, (int)floorf(((float)ylo - R) / kTileSide));
        const int ky1 = min(g.nby - 1, (int)floorf(((float)yhi + R) / kTileSide));
        const int kx0 = max(0, (int)floorf(((float)xlo - R) / kTileSide));
        const int kx1 = min(g.nbx - 1, (int)floorf(((float)xhi + R) / kTileSide));
        for (int ky = ky0; ky <= ky1; ++ky) {
            const int ty0 = kTileSide * ky, ty1 = min(g.H - 1, ty0 + kTileSide - 1);
            const int dy = max(0, max(ty0 - y, y - ty1));
            for (int kx = kx0; kx <= kx1; ++kx) {
                const int tx0 = kTileSide * kx, tx1 = min(g.W - 1, tx0 + kTileSide - 1);
                const int dx = max(0, max(tx0 - x, x - tx1));
                const bool vote = real && (float)(dy * dy + dx * dx) <= r2;
                if (__popcll(__ballot(vote)) >= min_votes) {
                    if (count < maxcnt && lane == 0) out[count] = (tk * g.nby + ky) * g.nbx + kx;
                    ++count;
                }
            }
        }
    }
    if (lane == 0) cnt[row] = (int32_t)(count < maxcnt ? count : maxcnt);
}

}  // namespace

hipError_t launch_token_entropy(int D, const uint16_t *q, const uint16_t *kt, const Grid &g,
                                int heads, float tau, float gamma, float *ent, float *r0,
                                hipStream_t s) {
    const int pph = pairs_per_head(g);
    const int64_t total = (int64_t)heads * pph;
    const int per_xcd = (int)((total + 7) / 8);
    const dim3 grid((unsigned)(8 * (int64_t)per_xcd)), block(kEntThreads);
    const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
    const float tg = (float)(2.0 * gamma * 1.4426950408889634);
    const FastDiv div_nbx = make_fastdiv(g.nbx), div_nby = make_fastdiv(g.nby);
    if (D == 128)
        hipLaunchKernelGGL(token_entropy_kernel<128>, grid, block, 0, s, q, kt, g, heads, pph,
                           per_xcd, div_nbx, div_nby, scale_log2, tau, tg, ent, r0);
    else if (D == 64)
        hipLaunchKernelGGL(token_entropy_kernel<64>, grid, block, 0, s, q, kt, g, heads, pph,
                           per_xcd, div_nbx, div_nby, scale_log2, tau, tg, ent, r0);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_token_mask(const float *r0, const Grid &g, int heads, float gamma,
                             int min_votes, int64_t maxcnt, int32_t *idx, int32_t *cnt,
                             hipStream_t s) {
    const int64_t rows = (int64_t)heads * g.nb;
    const float gl = (float)(gamma * 1.4426950408889634);
    hipLaunchKernelGGL(token_mask_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, r0,
                       g, rows, gl, min_votes, maxcnt, idx, cnt);
    return hipGetLastError();
}

}  // namespace tra

// Probe kernels: block mean-pooling of q/k (fused with the tile-major packing
// of k and v for the attention kernel), and the pooled-logit softmax entropy
// that sets each query block's radius.
//
// Token Radius Attention for Efficient Video Generation:
//   "Insight I" / "The TRA Pipeline: Entropy-to-Budget" -- attention entropy
//   of a query decides how many keys it needs; here measured on block-pooled
//   queries and keys against every key block.
//   "Budget-to-Radius" -- entropy becomes a radius; here one linear quantiser
//   r = r_min + floor(h_norm * (r_max - r_min + 1)), clamped to [r_min, r_max].
//   "Tile-Major Layout" -- tokens regrouped so that an 8 x 8 spatial tile is
//   one contiguous block; the packing below writes k and v tile-major.
#include <float.h>
#include <math.h>

#include "tra_internal.h"

namespace tra {
namespace {

__device__ __forceinline__ float bf16_to_float(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Swap bits 2 and 3 of a key position inside its 16-key group (an involution).
__device__ __forceinline__ int swap_bits23(int p) {
    return (p & ~12) | ((p & 4) << 1) | ((p & 8) >> 1);
}

// One workgroup per (head, block).  256 threads; thread tid owns the 16-byte
// chunk c = tid % (D/8) of rows w = tid / (D/8) + i * (256 / (D/8)).  PACK
// writes the packed K tile, PACKV also the packed V^T tile.
template <int D, bool POOL, bool PACK, bool PACKV = PACK>
__global__ __launch_bounds__(256) void pack_pool_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, Grid g, float *__restrict__ qp, float *__restrict__ kp,
    uint16_t *__restrict__ kt, uint16_t *__restrict__ vt) {
    constexpr int CH = D / 8;
    constexpr int RG = 256 / CH;
    constexpr int RPT = 64 / RG;
    constexpr int KS = D / 16;     // 16-wide k-steps of Q.K^T
    constexpr int MT = D / 32;     // 32-row tiles of O^T
    constexpr int VPITCH = D + 8;  // fp16 elements per LDS row of the V tile

    __shared__ float red[POOL ? 2 : 1][POOL ? RG : 1][POOL ? D : 1];
    __shared__ __attribute__((aligned(16))) uint16_t vs[PACKV ? 64 : 1][PACKV ? VPITCH : 1];

    const int b = blockIdx.x;
    const int h = blockIdx.y;
    const int tid = threadIdx.x;
    const int c = tid % CH;
    const int rg = tid / CH;
    const int t = b / (g.nby * g.nbx);
    const int by = (b / g.nbx) % g.nby;
    const int bx = b % g.nbx;
    const int ny = min(kTileSide, g.H - kTileSide * by);
    const int nx = min(kTileSide, g.W - kTileSide * bx);
    const size_t head_tok = (size_t)h * g.T * g.H * g.W;
    const size_t tile = (size_t)h * g.nb + b;

    float sq[8], sk[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) sq[e] = sk[e] = 0.f;

#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int w = rg + RG * i;
        const int ty = w >> 3, tx = w & 7;
        const bool real = ty < ny && tx < nx;
        uint4 kk = make_uint4(0, 0, 0, 0), qq = kk, vv = kk;
        if (real) {
            const size_t tok = head_tok + ((size_t)t * g.H + kTileSide * by + ty) * g.W +
                               kTileSide * bx + tx;
            const size_t off = tok * D + 8 * c;
            kk = *reinterpret_cast<const uint4 *>(k + off);
            if (POOL) qq = *reinterpret_cast<const uint4 *>(q + off);
            if (PACKV) vv = *reinterpret_cast<const uint4 *>(v + off);
        }
        if (POOL) {
            const uint32_t qw[4] = {qq.x, qq.y, qq.z, qq.w};
            const uint32_t kw[4] = {kk.x, kk.y, kk.z, kk.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sq[2 * e] += bf16_to_float(qw[e] & 0xffffu);
                sq[2 * e + 1] += bf16_to_float(qw[e] >> 16);
                sk[2 * e] += bf16_to_float(kw[e] & 0xffffu);
                sk[2 * e + 1] += bf16_to_float(kw[e] >> 16);
            }
        }
        if (PACK) {
            // K fragment piece (w / 32, c / 2), lane 32 (c % 2) + w % 32
            const int piece = (w >> 5) * KS + (c >> 1);
            const int lane = 32 * (c & 1) + (w & 31);
            *reinterpret_cast<uint4 *>(kt + tile * 64 * D + (piece * 64 + lane) * 8) = kk;
        }
        if (PACKV) {
            const uint32_t vw[4] = {vv.x, vv.y, vv.z, vv.w};
            uint32_t hw[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                // bf16 -> fp16 is exact for |v| in the fp16 normal range
                const _Float16 lo = (_Float16)bf16_to_float(vw[e] & 0xffffu);
                const _Float16 hi = (_Float16)bf16_to_float(vw[e] >> 16);
                hw[e] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
            }
            *reinterpret_cast<uint4 *>(&vs[w][8 * c]) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        }
    }

    if (POOL) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            red[0][rg][8 * c + e] = sq[e];
            red[1][rg][8 * c + e] = sk[e];
        }
    }
    __syncthreads();
    if (POOL) {
        const float inv_n = 1.0f / (float)(ny * nx);
        for (int col = tid; col < 2 * D; col += 256) {
            const int which = col / D, dd = col % D;
            float s = 0.f;
            for (int r = 0; r < RG; ++r) s += red[which][r][dd];
            (which ? kp : qp)[tile * D + dd] = s * inv_n;
        }
    }
    if (PACKV) {
        // V^T fragment pieces (hf, mt, ks2): lane l holds row d = 32 mt + l % 32
        // at the eight keys 32 hf + swap_bits23(8 (2 ks2 + l / 32) + e).
        for (int o = tid; o < 2 * MT * 2 * 64; o += 256) {
            const int piece = o >> 6, lane = o & 63;
            const int hf = piece / (2 * MT), mt = (piece >> 1) % MT, ks2 = piece & 1;
            const int dd = 32 * mt + (lane & 31);
            const int cc = 2 * ks2 + (lane >> 5);
            uint32_t w32[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int k0 = 32 * hf + swap_bits23(8 * cc + 2 * e);
                const int k1 = 32 * hf + swap_bits23(8 * cc + 2 * e + 1);
                w32[e] = (uint32_t)vs[k0][dd] | ((uint32_t)vs[k1][dd] << 16);
            }
            *reinterpret_cast<uint4 *>(vt + tile * 64 * D + (size_t)o * 8) =
                make_uint4(w32[0], w32[1], w32[2], w32[3]);
        }
    }
}

// Pooled-logit entropy and radius.  One workgroup per (head, 32 query
// blocks); the key blocks stream through LDS in chunks of 64.  Thread
// (tq = tid / 16, tk = tid % 16) handles queries 2 tq, 2 tq + 1 and keys
// tk + 16 j of each chunk, keeping an online (max, sum, weighted-log) state
// per query that is merged over the 16 tk lanes at the end.
constexpr int kEntQ = 32;
constexpr int kEntK = 64;

struct EntState {
    float m, Z, A;  // running max, sum e^(s-m), sum e^(s-m) (s-m)
};

__device__ __forceinline__ EntState ent_merge(EntState a, EntState b) {
    const float mn = fmaxf(a.m, b.m);
    const float ea = expf(a.m - mn), eb = expf(b.m - mn);
    EntState r;
    r.m = mn;
    r.Z = ea * a.Z + eb * b.Z;
    r.A = ea * (a.A + (a.m - mn) * a.Z) + eb * (b.A + (b.m - mn) * b.Z);
    return r;
}

template <int D>
__global__ __launch_bounds__(256) void entropy_kernel(
    const float *__restrict__ qp, const float *__restrict__ kp, Grid g, int r_min,
    int64_t R, int r_max, float inv_ln_nb, float scale, int32_t *__restrict__ radius,
    float *__restrict__ h_norm, float *__restrict__ logits) {
    constexpr int P = D + 4;
    __shared__ __attribute__((aligned(16))) float Qs[kEntQ][P];
    __shared__ __attribute__((aligned(16))) float Ks[kEntK][P];

    const int h = blockIdx.y;
    const int q0 = blockIdx.x * kEntQ;
    const int tid = threadIdx.x;
    const int tq = tid >> 4, tk = tid & 15;
    const float *qh = qp + (size_t)h * g.nb * D;
    const float *kh = kp + (size_t)h * g.nb * D;

    for (int e = tid; e < kEntQ * D / 4; e += 256) {
        const int r = e / (D / 4), c4 = e % (D / 4);
        float4 val = make_float4(0.f, 0.f, 0.f, 0.f);
        if (q0 + r < g.nb) val = reinterpret_cast<const float4 *>(qh + (size_t)(q0 + r) * D)[c4];
        *reinterpret_cast<float4 *>(&Qs[r][4 * c4]) = val;
    }

    EntState st[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) st[i] = EntState{-1e30f, 0.f, 0.f};

    // Key chunks are double-buffered through registers: the next chunk's loads
    // are in flight while the current one is computed from LDS.
    constexpr int KCH = kEntK * D / 4 / 256;  // float4 per thread and chunk
    static_assert(KCH * 256 * 4 == kEntK * D, "chunk split");
    float4 stage[KCH];
    auto load_chunk = [&](int c0) {
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
            const int e = tid + 256 * i;
            const int r = e / (D / 4), c4 = e % (D / 4);
            stage[i] = c0 + r < g.nb ? reinterpret_cast<const float4 *>(kh + (size_t)(c0 + r) * D)[c4]
                                     : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };
    load_chunk(0);
    for (int c0 = 0; c0 < g.nb; c0 += kEntK) {
        __syncthreads();
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
            const int e = tid + 256 * i;
            *reinterpret_cast<float4 *>(&Ks[e / (D / 4)][4 * (e % (D / 4))]) = stage[i];
        }
        __syncthreads();
        if (c0 + kEntK < g.nb) load_chunk(c0 + kEntK);
        float s[2][4];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) s[i][j] = 0.f;
#pragma unroll 2
        for (int dd = 0; dd < D; dd += 4) {
            const float4 a0 = *reinterpret_cast<const float4 *>(&Qs[2 * tq][dd]);
            const float4 a1 = *reinterpret_cast<const float4 *>(&Qs[2 * tq + 1][dd]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float4 kk = *reinterpret_cast<const float4 *>(&Ks[tk + 16 * j][dd]);
                s[0][j] += a0.x * kk.x + a0.y * kk.y + a0.z * kk.z + a0.w * kk.w;
                s[1][j] += a1.x * kk.x + a1.y * kk.y + a1.z * kk.z + a1.w * kk.w;
            }
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            float mx = st[i].m;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                s[i][j] *= scale;
                if (c0 + tk + 16 * j < g.nb) mx = fmaxf(mx, s[i][j]);
                // the pooled logit matrix [heads][nb][nb], when asked for
                if (logits && c0 + tk + 16 * j < g.nb && q0 + 2 * tq + i < g.nb)
                    logits[((size_t)h * g.nb + q0 + 2 * tq + i) * g.nb + c0 + tk + 16 * j] = s[i][j];
            }
            if (mx > st[i].m) {
                const float a = expf(st[i].m - mx);
                st[i].A = a * (st[i].A + (st[i].m - mx) * st[i].Z);
                st[i].Z *= a;
                st[i].m = mx;
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (c0 + tk + 16 * j < g.nb) {
                    const float x = s[i][j] - st[i].m;
                    const float e = expf(x);
                    st[i].Z += e;
                    st[i].A += e * x;
                }
            }
        }
    }

#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) {
            EntState o;
            o.m = __shfl_xor(st[i].m, off);
            o.Z = __shfl_xor(st[i].Z, off);
            o.A = __shfl_xor(st[i].A, off);
            st[i] = ent_merge(st[i], o);
        }
        const int b = q0 + 2 * tq + i;
        if (tk == 0 && b < g.nb) {
            const float Hb = logf(st[i].Z) - st[i].A / st[i].Z;
            const float hn = Hb * inv_ln_nb;
            int64_t r = (int64_t)r_min + (int64_t)floor((double)hn * (double)R);
            r = r < r_min ? r_min : (r > r_max ? r_max : r);
            radius[(size_t)h * g.nb + b] = (int32_t)r;
            if (h_norm) h_norm[(size_t)h * g.nb + b] = hn;
        }
    }
}

__global__ __launch_bounds__(256) void fill_dense_kernel(int64_t n, int32_t *__restrict__ radius,
                                                         float *__restrict__ h_norm) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) {
        radius[i] = 2147483647;
        if (h_norm) h_norm[i] = 0.f;
    }
}

template <int D>
hipError_t pack_pool_dispatch(bool pool, bool pack, const uint16_t *q, const uint16_t *k,
                              const uint16_t *v, const Grid &g, int heads, float *qp, float *kp,
                              uint16_t *kt, uint16_t *vt, hipStream_t s) {
    const dim3 grid(g.nb, heads), block(256);
    if (pool && pack)
        hipLaunchKernelGGL((pack_pool_kernel<D, true, true>), grid, block, 0, s, q, k, v, g, qp, kp, kt, vt);
    else if (pool)
        hipLaunchKernelGGL((pack_pool_kernel<D, true, false>), grid, block, 0, s, q, k, v, g, qp, kp, kt, vt);
    else if (pack)
        hipLaunchKernelGGL((pack_pool_kernel<D, false, true>), grid, block, 0, s, q, k, v, g, qp, kp, kt, vt);
    return hipGetLastError();
}

}  // namespace

size_t packed_tile_elems(int D) { return (size_t)kBlockTokens * D; }

hipError_t launch_pack_k(int D, const uint16_t *k, const Grid &g, int heads, uint16_t *kt,
                         hipStream_t s) {
    const dim3 grid(g.nb, heads), block(256);
    if (D == 128)
        hipLaunchKernelGGL((pack_pool_kernel<128, false, true, false>), grid, block, 0, s, nullptr,
                           k, nullptr, g, nullptr, nullptr, kt, nullptr);
    else if (D == 64)
        hipLaunchKernelGGL((pack_pool_kernel<64, false, true, false>), grid, block, 0, s, nullptr,
                           k, nullptr, g, nullptr, nullptr, kt, nullptr);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_pack_pool(int D, bool pool, bool pack, const uint16_t *q, const uint16_t *k,
                            const uint16_t *v, const Grid &g, int heads, float *qp, float *kp,
                            uint16_t *kt, uint16_t *vt, hipStream_t s) {
    if (D == 128) return pack_pool_dispatch<128>(pool, pack, q, k, v, g, heads, qp, kp, kt, vt, s);
    if (D == 64) return pack_pool_dispatch<64>(pool, pack, q, k, v, g, heads, qp, kp, kt, vt, s);
    return hipErrorInvalidValue;
}

hipError_t launch_entropy(int D, const float *qp, const float *kp, const Grid &g, int heads,
                          int r_min, int r_max, int32_t *radius, float *h_norm, hipStream_t s,
                          float *logits) {
    const dim3 grid((g.nb + kEntQ - 1) / kEntQ, heads), block(256);
    const int64_t R = (int64_t)r_max - (int64_t)r_min + 1;
    const float inv_ln_nb = g.nb > 1 ? (float)(1.0 / log((double)g.nb)) : 0.f;
    const float scale = (float)(1.0 / sqrt((double)D));
    if (D == 128)
        hipLaunchKernelGGL(entropy_kernel<128>, grid, block, 0, s, qp, kp, g, r_min, R, r_max,
                           inv_ln_nb, scale, radius, h_norm, logits);
    else if (D == 64)
        hipLaunchKernelGGL(entropy_kernel<64>, grid, block, 0, s, qp, kp, g, r_min, R, r_max,
                           inv_ln_nb, scale, radius, h_norm, logits);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_fill_dense(const Grid &g, int heads, int32_t *radius, float *h_norm,
                             hipStream_t s) {
    const int64_t n = (int64_t)heads * g.nb;
    hipLaunchKernelGGL(fill_dense_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, n,
                       radius, h_norm);
    return hipGetLastError();
}

}  // namespace tra

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

// Largest |v| of a head, as the bit pattern of a non-negative bfloat16 (for
// finite non-negative values the bit patterns order like the values).  Grid
// (parts, heads): workgroup g scans the g-th of `parts` equal chunks of the
// head's T H W d elements, eight at a time, and writes its maximum.  The first
// workgroup also zeroes the attention launch's work-claiming counters.
__global__ __launch_bounds__(256) void vmax_kernel(const uint16_t *__restrict__ v, int64_t n,
                                                   int parts, uint32_t *__restrict__ vpart,
                                                   int32_t *__restrict__ sched) {
    if (sched && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x < kXcdRanges)
        sched[threadIdx.x * kSchedStride] = 0;
    __shared__ uint32_t red[4];
    const int h = blockIdx.y, gpart = blockIdx.x;
    const int64_t n8 = n / 8;  // n = T H W d is a multiple of 8 (d in {64, 128})
    const int64_t chunk = (n8 + parts - 1) / parts;
    const int64_t lo = min(n8, gpart * chunk), hi = min(n8, lo + chunk);
    const uint4 *src = reinterpret_cast<const uint4 *>(v + (size_t)h * n);
    uint32_t mx = 0;
    auto fold = [&](const uint4 &w) {
        const uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) mx = max(mx, max(a[e] & 0x7fffu, (a[e] >> 16) & 0x7fffu));
    };
    // four loads in flight per thread, then the remainder
    int64_t i = lo + threadIdx.x;
    for (; i + 3 * 256 < hi; i += 4 * 256) {
        const uint4 w0 = src[i], w1 = src[i + 256], w2 = src[i + 512], w3 = src[i + 768];
        fold(w0);
        fold(w1);
        fold(w2);
        fold(w3);
    }
    for (; i < hi; i += 256) fold(src[i]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
    __syncthreads();
    if (threadIdx.x == 0)
        vpart[(size_t)h * parts + gpart] = max(max(red[0], red[1]), max(red[2], red[3]));
}

// Power-of-two exponent e that puts the head's largest |v| (bfloat16 bits m)
// into [2^15, 2^16): v 2^e is then exact in fp16 for every |v| of the head
// down to 2^-30 of the largest (below that, fp16 subnormals round at an
// absolute 2^-25 of the scaled maximum), and nothing overflows.  e = 0 for an
// all-zero head.  The attention output is multiplied by 2^-e.
__device__ __forceinline__ int v_scale_exponent(uint32_t m) {
    if (m == 0) return 0;
    const int ex = (int)(m >> 7) & 0xff;  // biased exponent of the bfloat16
    // floor(log2 |v|): normal ex - 127; subnormal mantissa * 2^-133
    const int lg = ex ? ex - 127 : (31 - __builtin_clz(m & 0x7fu)) - 133;
    return 15 - lg;
}

// One workgroup per (head, block).  256 threads; thread tid owns the 16-byte
// chunk c = tid % (D/8) of rows w = tid / (D/8) + i * (256 / (D/8)).  PACK
// writes the packed K tile, PACKV also the packed V^T tile.
template <int D, bool POOL, bool PACK, bool PACKV = PACK>
__global__ __launch_bounds__(256) void pack_pool_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, Grid g, float *__restrict__ qp, float *__restrict__ kp,
    uint16_t *__restrict__ kt, uint16_t *__restrict__ vt, const uint32_t *__restrict__ vpart,
    int vparts, int32_t *__restrict__ vexp) {
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

    // the head's V exponent, from the partial maxima of vmax_kernel (one per
    // thread, kVmaxParts <= 256, then a workgroup max)
    __shared__ uint32_t vred[PACKV ? 4 : 1];
    int vsc = 0;
    if (PACKV) {
        uint32_t m = tid < vparts ? vpart[(size_t)h * vparts + tid] : 0u;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
        if ((tid & 63) == 0) vred[tid >> 6] = m;
        __syncthreads();
        vsc = v_scale_exponent(max(max(vred[0], vred[1]), max(vred[2], vred[3])));
        if (b == 0 && tid == 0) vexp[h] = vsc;
    }

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
                // v 2^vsc: exact in fp32, then rounded to fp16 (exact within
                // 2^30 of the head's largest |v|, which lands in [2^15, 2^16))
                const _Float16 lo = (_Float16)ldexpf(bf16_to_float(vw[e] & 0xffffu), vsc);
                const _Float16 hi = (_Float16)ldexpf(bf16_to_float(vw[e] >> 16), vsc);
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

// Pooled-logit entropy and radius.  The logits s = scale qbar . kbar of 16
// query blocks against 16 key blocks are one fp32 matrix-core product chain
// (v_mfma_f32_16x16x4_f32, D / 4 steps): the key tile is the A operand and
// the query tile the B operand, so that lane l ends with the logits of query
// block q0 + l % 16 against key blocks 4 (l / 16) + r, r = 0..3, of the tile.
// Step s takes dims kq D / 4 + s from lane group kq = l / 16 (the dot product
// does not depend on the order of the dims), so every lane reads one
// contiguous quarter row of its query and of its key.  The workgroup's waves
// take the key tiles round robin, each keeping an online (max, sum,
// weighted-log) state per lane in base 2 (x = s log2(e), sums of 2^(x - m):
// one v_exp_f32 per logit); the four lane groups and the waves are merged at
// the end, and H = ln Z - ln(2) A / Z.
constexpr int kEntWaves = 4;   // waves per workgroup
constexpr int kEntQB = 16;     // query blocks per workgroup

struct EntState {
    float m, Z, A;  // running max of x, sum 2^(x-m), sum 2^(x-m) (x-m)
};

__device__ __forceinline__ EntState ent_merge(EntState a, EntState b) {
    const float mn = fmaxf(a.m, b.m);
    const float ea = __builtin_amdgcn_exp2f(a.m - mn), eb = __builtin_amdgcn_exp2f(b.m - mn);
    EntState r;
    r.m = mn;
    r.Z = ea * a.Z + eb * b.Z;
    r.A = ea * (a.A + (a.m - mn) * a.Z) + eb * (b.A + (b.m - mn) * b.Z);
    return r;
}

template <int D>
__global__ __launch_bounds__(64 * kEntWaves) void entropy_kernel(
    const float *__restrict__ qp, const float *__restrict__ kp, Grid g, int r_min,
    int64_t R, int r_max, float inv_ln_nb, float scale, int32_t *__restrict__ radius,
    float *__restrict__ h_norm, float *__restrict__ logits) {
    constexpr int QD = D / 4;  // dims per lane group
    typedef float f32x4_t __attribute__((ext_vector_type(4)));
    __shared__ float red[3][kEntWaves][kEntQB];

    const float scale2 = scale * 1.4426950408889634f;
    const int h = blockIdx.y;
    const int q0 = blockIdx.x * kEntQB;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int col = lane & 15, kq = lane >> 4;
    const float *qh = qp + (size_t)h * g.nb * D;
    const float *kh = kp + (size_t)h * g.nb * D;

    // B operand: query block q0 + col, dims kq QD .. kq QD + QD (zeros past nb)
    float qv[QD];
    {
        const int qi = q0 + col;
        const float4 *src =
            reinterpret_cast<const float4 *>(qh + (size_t)min(qi, g.nb - 1) * D + kq * QD);
#pragma unroll
        for (int c = 0; c < QD / 4; ++c) {
            float4 t = src[c];
            if (qi >= g.nb) t = make_float4(0.f, 0.f, 0.f, 0.f);
            qv[4 * c] = t.x;
            qv[4 * c + 1] = t.y;
            qv[4 * c + 2] = t.z;
            qv[4 * c + 3] = t.w;
        }
    }

    const int ntiles = (g.nb + 15) / 16;
    EntState st{-1e30f, 0.f, 0.f};
    // A operand: key block 16 t + col, dims kq QD .. (rows past nb read the
    // last real row; their logits are left out below)
    float kv[QD];
    auto load_keys = [&](int t) {
        const float4 *src = reinterpret_cast<const float4 *>(
            kh + (size_t)min(16 * t + col, g.nb - 1) * D + kq * QD);
#pragma unroll
        for (int c = 0; c < QD / 4; ++c) {
            const float4 x = src[c];
            kv[4 * c] = x.x;
            kv[4 * c + 1] = x.y;
            kv[4 * c + 2] = x.z;
            kv[4 * c + 3] = x.w;
        }
    };
    if (wave < ntiles) load_keys(wave);
    for (int t = wave; t < ntiles; t += kEntWaves) {
        f32x4_t acc = {};
#pragma unroll
        for (int s = 0; s < QD; ++s)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(kv[s], qv[s], acc, 0, 0, 0);
        // the next tile's loads under this tile's VALU work
        if (t + kEntWaves < ntiles) load_keys(t + kEntWaves);
        const int key0 = 16 * t + 4 * kq;
        float sv[4];
        float mx = st.m;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            sv[r] = acc[r] * scale2;
            if (key0 + r < g.nb) mx = fmaxf(mx, sv[r]);
        }
        if (logits && q0 + col < g.nb) {
            float *row = logits + ((size_t)h * g.nb + q0 + col) * g.nb;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (key0 + r < g.nb) row[key0 + r] = acc[r] * scale;
        }
        if (mx > st.m) {
            const float a = __builtin_amdgcn_exp2f(st.m - mx);
            st.A = a * (st.A + (st.m - mx) * st.Z);
            st.Z *= a;
            st.m = mx;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if (key0 + r < g.nb) {
                const float x = sv[r] - st.m;
                const float e = __builtin_amdgcn_exp2f(x);
                st.Z += e;
                st.A += e * x;
            }
        }
    }
    // the four lane groups hold the same query block's other keys
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
        EntState o;
        o.m = __shfl_xor(st.m, off);
        o.Z = __shfl_xor(st.Z, off);
        o.A = __shfl_xor(st.A, off);
        st = ent_merge(st, o);
    }
    if (kq == 0) {
        red[0][wave][col] = st.m;
        red[1][wave][col] = st.Z;
        red[2][wave][col] = st.A;
    }
    __syncthreads();
    if (wave == 0 && kq == 0) {
        EntState acc{red[0][0][col], red[1][0][col], red[2][0][col]};
        for (int w = 1; w < kEntWaves; ++w)
            acc = ent_merge(acc, EntState{red[0][w][col], red[1][w][col], red[2][w][col]});
        const int b = q0 + col;
        if (b < g.nb) {
            const float Hb = logf(acc.Z) - 0.69314718055994531f * (acc.A / acc.Z);
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
                              uint16_t *kt, uint16_t *vt, const uint32_t *vpart, int vparts,
                              int32_t *vexp, hipStream_t s) {
    const dim3 grid(g.nb, heads), block(256);
    if (pool && pack)
        hipLaunchKernelGGL((pack_pool_kernel<D, true, true>), grid, block, 0, s, q, k, v, g, qp, kp,
                           kt, vt, vpart, vparts, vexp);
    else if (pool)
        hipLaunchKernelGGL((pack_pool_kernel<D, true, false>), grid, block, 0, s, q, k, v, g, qp,
                           kp, kt, vt, vpart, vparts, vexp);
    else if (pack)
        hipLaunchKernelGGL((pack_pool_kernel<D, false, true>), grid, block, 0, s, q, k, v, g, qp,
                           kp, kt, vt, vpart, vparts, vexp);
    return hipGetLastError();
}

}  // namespace

size_t packed_tile_elems(int D) { return (size_t)kBlockTokens * D; }

hipError_t launch_pack_k(int D, const uint16_t *k, const Grid &g, int heads, uint16_t *kt,
                         hipStream_t s) {
    const dim3 grid(g.nb, heads), block(256);
    if (D == 128)
        hipLaunchKernelGGL((pack_pool_kernel<128, false, true, false>), grid, block, 0, s, nullptr,
                           k, nullptr, g, nullptr, nullptr, kt, nullptr, nullptr, 0, nullptr);
    else if (D == 64)
        hipLaunchKernelGGL((pack_pool_kernel<64, false, true, false>), grid, block, 0, s, nullptr,
                           k, nullptr, g, nullptr, nullptr, kt, nullptr, nullptr, 0, nullptr);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

int vmax_parts(const Grid &g, int D) {
    // about 16 K elements per workgroup, at most kVmaxParts per head
    const int64_t n = (int64_t)g.T * g.H * g.W * D;
    const int64_t p = (n + 16383) / 16384;
    return (int)(p < 1 ? 1 : (p > kVmaxParts ? kVmaxParts : p));
}

hipError_t launch_vmax(int D, const uint16_t *v, const Grid &g, int heads, uint32_t *vpart,
                       int32_t *sched, hipStream_t s) {
    const int parts = vmax_parts(g, D);
    const int64_t n = (int64_t)g.T * g.H * g.W * D;
    hipLaunchKernelGGL(vmax_kernel, dim3((unsigned)parts, (unsigned)heads), dim3(256), 0, s, v, n,
                       parts, vpart, sched);
    return hipGetLastError();
}

hipError_t launch_pack_pool(int D, bool pool, bool pack, const uint16_t *q, const uint16_t *k,
                            const uint16_t *v, const Grid &g, int heads, float *qp, float *kp,
                            uint16_t *kt, uint16_t *vt, const uint32_t *vpart, int32_t *vexp,
                            hipStream_t s) {
    const int vparts = vmax_parts(g, D);
    if (D == 128)
        return pack_pool_dispatch<128>(pool, pack, q, k, v, g, heads, qp, kp, kt, vt, vpart, vparts,
                                       vexp, s);
    if (D == 64)
        return pack_pool_dispatch<64>(pool, pack, q, k, v, g, heads, qp, kp, kt, vt, vpart, vparts,
                                      vexp, s);
    return hipErrorInvalidValue;
}

hipError_t launch_entropy(int D, const float *qp, const float *kp, const Grid &g, int heads,
                          int r_min, int r_max, int32_t *radius, float *h_norm, hipStream_t s,
                          float *logits) {
    const dim3 grid((g.nb + kEntQB - 1) / kEntQB, heads), block(64 * kEntWaves);
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

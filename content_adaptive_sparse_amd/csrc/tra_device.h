// Device-side helpers shared by the matrix-core kernels (attention and the
// token-entropy warm-up): operand vector types, LDS operand loads, exact
// division by small constants, the lane-pair exchange of a wave64, s_waitcnt
// encodings and address-space casts for direct global -> LDS copies.
#pragma once

#include "tra_internal.h"

namespace tra {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

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
inline FastDiv make_fastdiv(int d) {
    FastDiv f;
    f.d = (uint32_t)d;
    f.m = (((uint64_t)1 << 39) + (uint64_t)d - 1) / (uint64_t)d;
    return f;
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

// s_waitcnt immediates for gfx9 (vmcnt bits [3:0] and [15:14], expcnt [6:4],
// lgkmcnt [11:8]); counters not waited on are left at their no-wait maxima.
constexpr int wait_vmcnt(int n) { return 0x0F70 | (n & 15) | (((n >> 4) & 3) << 14); }
constexpr int kWaitVmcnt0 = wait_vmcnt(0);

typedef __attribute__((address_space(3))) void lds_void_t;
// Arrays never written while a kernel runs (work orders, walk lengths) read
// through the constant address space give scalar loads.
typedef __attribute__((address_space(4))) const int32_t const_i32_t;

template <int N>
struct SlotTag {
    static constexpr int value = N;
};

// Key columns / rows of an edge tile that lie beyond the grid: a 64-key tile
// seen as two 32-key halves, register r of half hf holding key row 4 hf + r / 4
// and key column 4 hl + r % 4 (hl = lane / 32).  Masked logits become `fill`.
__device__ __forceinline__ void mask_edge_keys(f32x16_t (&sb)[2], int kny, int knx, int hl,
                                               float fill) {
    if (knx < kTileSide) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const bool bad = 4 * hl + c >= knx;
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int rg = 0; rg < 4; ++rg) sb[hf][4 * rg + c] = bad ? fill : sb[hf][4 * rg + c];
        }
    }
    if (kny < kTileSide) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg)
                if (4 * hf + rg >= kny)
#pragma unroll
                    for (int c = 0; c < 4; ++c) sb[hf][4 * rg + c] = fill;
    }
}

// Entropy of an attention row from its base-2 sums against a reference m,
// Z = sum 2^x and A = sum x 2^x with x = s log2(e) / sqrt(d) - m:
// H = ln Z - ln 2 A / Z (nats).  Token Radius Attention for Efficient Video
// Generation, "The TRA Pipeline: Entropy-to-Budget" and "Budget-to-Radius":
// the budget b = tau e^H keys, clamped to [1, T H W], and the base radius r0
// whose disks r0 e^(-gamma |t' - t|) over the T frames have a total area of b,
// r0 = sqrt(b / (pi sum_t' e^(-2 gamma |t' - t|))), with 2 gamma log2(e)
// passed in (formed once on the host).  Returns H, writes r0.
__device__ __forceinline__ float entropy_and_radius(float Z, float A, int t, const Grid &g,
                                                    float tau, float two_gamma_log2e, float *r0) {
    const float H = 0.69314718055994531f * (__builtin_amdgcn_logf(Z) - A / Z);
    const float N = (float)((int64_t)g.T * g.H * g.W);
    const float b = fminf(fmaxf(tau * __builtin_amdgcn_exp2f(H * 1.4426950408889634f), 1.0f), N);
    float S = 0.f;
    for (int tt = 0; tt < g.T; ++tt) S += __builtin_amdgcn_exp2f(-two_gamma_log2e * (float)abs(tt - t));
    *r0 = sqrtf(b / (3.14159265358979f * S));
    return H;
}

}  // namespace tra

// pip_attn.h -- pieces of the flash-style biased attention shared by the
// attention, fused and block-stack kernels.
//
// "Fusion 3" of the ml4sci_cms_e2e26 README ("How the Kernel Fusion Works"):
// softmax(Q K^T / sqrt(d) + bias) V with an online softmax.  Scores are
// computed transposed, S^T = K Q^T, so that lane l holds the scores of query
// l%16 against keys 4(l/16)+r: the row max / sum need an in-lane reduction
// over r and two cross-lane steps (l^16, l^32), and the probabilities are
// already the B operand of O^T += V^T P^T.  Scores are kept in base-2 units.
#pragma once

#include "pip_device.h"

namespace pip {

constexpr float kLog2e = 1.4426950408889634f;

// Reductions over the four lanes l, l^16, l^32, l^48 with the gfx950 row
// swaps: v_permlane16_swap of x with itself gives {x[l], x[l^16]} (in some
// order) and v_permlane32_swap {x[l], x[l^32]}; no LDS round trip.  Both
// lanes of a pair add the same two operands in the same order.
__device__ __forceinline__ float xmax16(float x) {
    const unsigned u = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const unsigned v = __float_as_uint(x);
    const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float xsum16(float x) {
    const unsigned u = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const unsigned v = __float_as_uint(x);
    const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Online-softmax update of one key block for the lane's query: s[r] are the
// base-2 scores (-inf for padded keys) and become the probabilities; m, l are
// the running max and sum; returns the factor that rescales the accumulator.
__device__ __forceinline__ float online_softmax(v4f &s, float &m, float &l) {
    float bm = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    bm = xmax16(bm);
    const float mn = fmaxf(m, bm);
    const float corr = __builtin_amdgcn_exp2f(m - mn);  // m = -inf on the first block -> 0
#pragma unroll
    for (int r = 0; r < 4; ++r) s[r] = __builtin_amdgcn_exp2f(s[r] - mn);
    float ps = (s[0] + s[1]) + (s[2] + s[3]);
    ps = xsum16(ps);
    l = l * corr + ps;
    m = mn;
    return corr;
}

__device__ __forceinline__ float bf2f(uint16_t b) {
    return __builtin_bit_cast(float, (uint32_t)b << 16);
}
__device__ __forceinline__ uint16_t f2bf(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}
__device__ __forceinline__ v4f mfma16bf(v4s a, v4s b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

}  // namespace pip

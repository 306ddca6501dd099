// pip_mlp.h -- the pair MLP as a chain of MFMA layers, weights read from LDS.
//
// The MLP is the pointwise 4 -> 64 -> 64 -> 64 -> 8 network of "Fusion 2"
// (ml4sci_cms_e2e26 README, "How the Kernel Fusion Works") with BatchNorm
// folded into the weights on the host.  One "pair block" is 16 pairs, the 16
// columns of a 16x16 MFMA tile; lane l's input is feature l/16 of pair l%16.
// Two pair blocks go through the chain together so that every weight operand
// read from LDS feeds two MFMAs and the two chains interleave.
#pragma once

#include "pip_device.h"

namespace pip {

// ------------------------------------------------------------ GELU
// GELU(x) = x Phi(x) = max(x, 0) - |x| Phi(-|x|) with Phi(-a) = 2^-Q(a) and Q
// a polynomial fitted by gen_gelu_coeffs.py (weighted least squares towards
// the minimax of the GELU error, a in [0, 7]).  Q has a positive leading
// coefficient and keeps growing beyond the fit range, so 2^-Q underflows to 0
// for large |x| and no clamp is needed.  max(x, 0) is taken on the bit
// pattern (an integer max), exact for every finite x, -0 included.
// Degree 5 (float32 path): |error| <= 8.9e-7 on [-40, 40]; degree 3 (bf16
// path): <= 9.6e-5.  Each costs its degree in FMAs, one v_exp_f32, one
// v_max_i32 and one FMA, with no branch.
constexpr float kGeluQ[6] = {1.000067353e+00f, 1.150599599e+00f, 4.603779614e-01f,
                             5.149073154e-02f, -6.955113262e-03f, 4.553909530e-04f};
constexpr float kGeluQ3[4] = {1.005338550e+00f, 1.122809887e+00f, 5.050402880e-01f,
                              2.316968702e-02f};

__device__ __forceinline__ float relu_bits(float x) {
    return __builtin_bit_cast(float, max(__builtin_bit_cast(int, x), 0));
}

__device__ __forceinline__ float gelu_f32(float x) {
    const float a = fabsf(x);
    float p = fmaf(kGeluQ[5], a, kGeluQ[4]);
    p = fmaf(p, a, kGeluQ[3]);
    p = fmaf(p, a, kGeluQ[2]);
    p = fmaf(p, a, kGeluQ[1]);
    p = fmaf(p, a, kGeluQ[0]);
    return fmaf(-a, __builtin_amdgcn_exp2f(-p), relu_bits(x));
}

__device__ __forceinline__ float gelu_lo(float x) {  // the bf16 path's GELU
    const float a = fabsf(x);
    float p = fmaf(kGeluQ3[3], a, kGeluQ3[2]);
    p = fmaf(p, a, kGeluQ3[1]);
    p = fmaf(p, a, kGeluQ3[0]);
    return fmaf(-a, __builtin_amdgcn_exp2f(-p), relu_bits(x));
}

// ------------------------------------------------------------ weight layout
// float32 operands are grouped by four: group q holds, for every lane, the
// operands 4q..4q+3 as one float4, so one ds_read_b128 fetches four MFMA A
// operands.  Groups: 0 = layer 1 (c = 0..3); 1 + co*4 + ci = layer 2 (r = 0..3);
// 17 + co*4 + ci = layer 3; 33 + ci = layer 4.  Operand (layer, co, ci, r) for
// lane l is W'[16co + l%16][16ci + 4(l/16) + r] (layer 1: W1'[16c + l%16][l/16];
// layer 4 rows >= 8 are zero).
constexpr int kW32Groups = 37;
constexpr int kW32Floats = kW32Groups * 64 * 4;  // 9,472
// bfloat16 operands (layers 2..4): 18 operands of 8 bf16 per lane, [op][lane].
constexpr int kW16Ops = 18;
constexpr int kW16Elems = kW16Ops * 64 * 8;      // 9,216
constexpr int kBiasFloats = 200;                 // b1' | b2' | b3' | b4

// Copy the packed weights and biases from global memory into LDS (all threads
// of the block; caller synchronises).
template <int kThreads>
__device__ inline void stage_weights(float4 *wl, float *bl, const float4 *__restrict__ w,
                                     const float *__restrict__ b, int nw4) {
    for (int i = threadIdx.x; i < nw4; i += kThreads) wl[i] = w[i];
    for (int i = threadIdx.x; i < kBiasFloats; i += kThreads) bl[i] = b[i];
}

__device__ __forceinline__ v4f bias4(const float *bl, int off) {
    return *(const v4f *)(bl + off);
}

// Two pair blocks through the float32 chain.  vA / vB are this lane's input
// features of blocks A and B; on return uA / uB hold U[head 4(l/16)+r][pair
// l%16] (meaningful for l < 32).
__device__ __forceinline__ void mlp2_f32(const float4 *__restrict__ wl,
                                         const float *__restrict__ bl, float vA, float vB,
                                         v4f &uA, v4f &uB) {
    const int lane = threadIdx.x & 63, g = lane >> 4;
    v4f hA[4], hB[4], tA[4], tB[4];
    {
        const float4 w = wl[lane];
        const float w1[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const v4f b = bias4(bl, 16 * c + 4 * g);
            hA[c] = mfma4(w1[c], vA, b);
            hB[c] = mfma4(w1[c], vB, b);
        }
    }
#pragma unroll
    for (int layer = 0; layer < 2; ++layer) {
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                hA[c][r] = gelu_f32(hA[c][r]);
                hB[c][r] = gelu_f32(hB[c][r]);
            }
#pragma unroll
        for (int co = 0; co < 4; ++co) {
            tA[co] = bias4(bl, 64 * (layer + 1) + 16 * co + 4 * g);
            tB[co] = tA[co];
        }
        const int gbase = 1 + 16 * layer;
#pragma unroll
        for (int ci = 0; ci < 4; ++ci)
#pragma unroll
            for (int co = 0; co < 4; ++co) {
                const float4 w = wl[(gbase + co * 4 + ci) * 64 + lane];
                const float wr[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    tA[co] = mfma4(wr[r], hA[ci][r], tA[co]);
                    tB[co] = mfma4(wr[r], hB[ci][r], tB[co]);
                }
            }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            hA[c] = tA[c];
            hB[c] = tB[c];
        }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            hA[c][r] = gelu_f32(hA[c][r]);
            hB[c][r] = gelu_f32(hB[c][r]);
        }
    v4f b4;
#pragma unroll
    for (int r = 0; r < 4; ++r) b4[r] = (4 * g + r < kHeads) ? bl[192 + 4 * g + r] : 0.0f;
    uA = b4;
    uB = b4;
#pragma unroll
    for (int ci = 0; ci < 4; ++ci) {
        const float4 w = wl[(33 + ci) * 64 + lane];
        const float wr[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            uA = mfma4(wr[r], hA[ci][r], uA);
            uB = mfma4(wr[r], hB[ci][r], uB);
        }
    }
}

// ------------------------------------------------------------ bf16 chain
__device__ __forceinline__ v4f mfma32bf(v8bf a, v8bf b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// bf16 B operand for K = 32: slots 0..3 from channel block lo, 4..7 from hi.
__device__ __forceinline__ v8bf pack_bf16(v4f lo, v4f hi) {
    v8bf o;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        o[r] = (__bf16)lo[r];
        o[r + 4] = (__bf16)hi[r];
    }
    return o;
}

// Two pair blocks through the bf16 chain: layer 1 in float32 (its inputs are
// the float32 features), layers 2..4 with bf16 operands on
// v_mfma_f32_16x16x32_bf16 and float32 accumulation.  wl holds the float32
// layer-1 group (64 float4), w16 the bf16 operands [op][lane].
__device__ __forceinline__ void mlp2_bf16(const float4 *__restrict__ wl,
                                          const v8bf *__restrict__ w16,
                                          const float *__restrict__ bl, float vA, float vB,
                                          v4f &uA, v4f &uB) {
    const int lane = threadIdx.x & 63, g = lane >> 4;
    v4f hA[4], hB[4], tA[4], tB[4];
    {
        const float4 w = wl[lane];
        const float w1[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const v4f b = bias4(bl, 16 * c + 4 * g);
            hA[c] = mfma4(w1[c], vA, b);
            hB[c] = mfma4(w1[c], vB, b);
        }
    }
#pragma unroll
    for (int layer = 0; layer < 2; ++layer) {
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                hA[c][r] = gelu_lo(hA[c][r]);
                hB[c][r] = gelu_lo(hB[c][r]);
            }
        const v8bf xA0 = pack_bf16(hA[0], hA[1]), xA1 = pack_bf16(hA[2], hA[3]);
        const v8bf xB0 = pack_bf16(hB[0], hB[1]), xB1 = pack_bf16(hB[2], hB[3]);
#pragma unroll
        for (int co = 0; co < 4; ++co) {
            const v4f b = bias4(bl, 64 * (layer + 1) + 16 * co + 4 * g);
            const v8bf w0 = w16[(layer * 8 + co * 2 + 0) * 64 + lane];
            const v8bf w1 = w16[(layer * 8 + co * 2 + 1) * 64 + lane];
            tA[co] = mfma32bf(w1, xA1, mfma32bf(w0, xA0, b));
            tB[co] = mfma32bf(w1, xB1, mfma32bf(w0, xB0, b));
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            hA[c] = tA[c];
            hB[c] = tB[c];
        }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            hA[c][r] = gelu_lo(hA[c][r]);
            hB[c][r] = gelu_lo(hB[c][r]);
        }
    v4f b4;
#pragma unroll
    for (int r = 0; r < 4; ++r) b4[r] = (4 * g + r < kHeads) ? bl[192 + 4 * g + r] : 0.0f;
    const v8bf w0 = w16[16 * 64 + lane], w1 = w16[17 * 64 + lane];
    uA = mfma32bf(w1, pack_bf16(hA[2], hA[3]), mfma32bf(w0, pack_bf16(hA[0], hA[1]), b4));
    uB = mfma32bf(w1, pack_bf16(hB[2], hB[3]), mfma32bf(w0, pack_bf16(hB[0], hB[1]), b4));
}

}  // namespace pip

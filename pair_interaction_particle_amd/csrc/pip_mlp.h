// pip_mlp.h -- the pair MLP as a chain of MFMA layers, weights read from LDS.
//
// The MLP is the pointwise 4 -> 64 -> 64 -> 64 -> 8 network of "Fusion 2"
// (ml4sci_cms_e2e26 README, "How the Kernel Fusion Works") with BatchNorm
// folded into the weights on the host.  One "pair block" is 16 pairs, the 16
// columns of a 16x16 MFMA tile; lane l's input is feature l/16 of pair l%16.
// Two pair blocks go through the chain together so that every weight operand
// read from LDS feeds two MFMAs and the two chains interleave.
#pragma once

#include <type_traits>

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
// 16-bit operands of layers 2..4 (bf16, or fp16 hi and lo halves): 18
// operands of 8 values per lane, [op][lane]; operand (layer 2 or 3, co, s) of
// lane l holds in slot j the weight W'[16co + l%16][32s + (j < 4 ? 0 : 16) +
// 4(l/16) + (j & 3)], operands 16 + s are layer 4 (rows >= 8 zero).
constexpr int kW16Ops = 18;
constexpr int kW16Elems = kW16Ops * 64 * 8;      // 9,216
constexpr int kBiasFloats = 200;                 // b1' | b2' | b3' | b4

// This thread's share of an N-element copy into LDS, split into a load step
// and a store step so that a caller can issue every load of several copies
// before the first store, and keep them in flight across other work.
template <int kThreads, int N, class T>
struct LdsCopy {
    static constexpr int kIt = (N + kThreads - 1) / kThreads;
    T v[kIt];
    __device__ __forceinline__ void load(const T *__restrict__ src) {
#pragma unroll
        for (int it = 0; it < kIt; ++it) v[it] = src[min((int)threadIdx.x + it * kThreads, N - 1)];
    }
    __device__ __forceinline__ void store(T *dst) const {
#pragma unroll
        for (int it = 0; it < kIt; ++it) {
            const int i = threadIdx.x + it * kThreads;
            if (i < N) dst[i] = v[it];
        }
    }
};

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


// ------------------------------------------------------------ fp16 x 2 chain
// Float32-faithful products on the fp16 matrix cores: every float32 operand x
// is carried as hi = fp16(x) and lo = fp16(x - hi) (11 + 11 significand
// bits, |x - hi - lo| <= 2^-22 |x| in the normal range), and
// x w = x_hi w_hi + x_hi w_lo + x_lo w_hi up to a dropped x_lo w_lo term of
// relative size 2^-22; accumulation is float32.  The weights are split on
// the host, the activations after every GELU.  An activation beyond the fp16
// range turns into inf and so into a non-finite U, which the caller detects
// and recomputes with the exact float32 chain.
// hi / lo fp16 B operands for K = 32 (slots 0..3 from channel block `lo_blk`,
// 4..7 from `hi_blk`, as in pack_bf16).
__device__ __forceinline__ void split_f16(v4f b0, v4f b1, v8h &hi, v8h &lo) {
    const v8f x = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
    split_f16<8>(x, hi, lo);
}

// t += W x over K = 64 (two K = 32 halves) with the three-term split.
__device__ __forceinline__ v4f mfma_x2(const v8h *__restrict__ wh, const v8h *__restrict__ wl,
                                       int op0, int lane, const v8h (&xh)[2],
                                       const v8h (&xl)[2], v4f t) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const v8h a = wh[(op0 + s) * 64 + lane], b = wl[(op0 + s) * 64 + lane];
        t = mfma32h(a, xl[s], t);
        t = mfma32h(b, xh[s], t);
        t = mfma32h(a, xh[s], t);
    }
    return t;
}

// Two pair blocks through the fp16 x 2 chain: layer 1 on the float32 MFMA
// (K = 4, float32 features), layers 2..4 as above.  wl holds the float32
// layer-1 group (64 float4); wh / wlo the fp16 hi / lo operands [op][lane].
__device__ __forceinline__ void mlp2_f16x2(const float4 *__restrict__ wl,
                                           const v8h *__restrict__ wh,
                                           const v8h *__restrict__ wlo,
                                           const float *__restrict__ bl, float vA, float vB,
                                           v4f &uA, v4f &uB) {
    const int lane = threadIdx.x & 63, g = lane >> 4;
    v4f hA[4], hB[4];
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
    for (int layer = 0; layer < 3; ++layer) {
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                hA[c][r] = gelu_f32(hA[c][r]);
                hB[c][r] = gelu_f32(hB[c][r]);
            }
        v8h xhA[2], xlA[2], xhB[2], xlB[2];
        split_f16(hA[0], hA[1], xhA[0], xlA[0]);
        split_f16(hA[2], hA[3], xhA[1], xlA[1]);
        split_f16(hB[0], hB[1], xhB[0], xlB[0]);
        split_f16(hB[2], hB[3], xhB[1], xlB[1]);
        if (layer < 2) {
#pragma unroll
            for (int co = 0; co < 4; ++co) {
                const v4f b = bias4(bl, 64 * (layer + 1) + 16 * co + 4 * g);
                const int op0 = layer * 8 + co * 2;
                hA[co] = mfma_x2(wh, wlo, op0, lane, xhA, xlA, b);
                hB[co] = mfma_x2(wh, wlo, op0, lane, xhB, xlB, b);
            }
        } else {
            v4f b4;
#pragma unroll
            for (int r = 0; r < 4; ++r) b4[r] = (4 * g + r < kHeads) ? bl[192 + 4 * g + r] : 0.0f;
            uA = mfma_x2(wh, wlo, 16, lane, xhA, xlA, b4);
            uB = mfma_x2(wh, wlo, 16, lane, xhB, xlB, b4);
        }
    }
}

// One pair block through the fp16 x 2 chain (as mlp2_f16x2, for kernels that
// give each wave a single block).
__device__ __forceinline__ v4f mlp1_f16x2(const float4 *__restrict__ wl,
                                          const v8h *__restrict__ wh,
                                          const v8h *__restrict__ wlo,
                                          const float *__restrict__ bl, float v) {
    const int lane = threadIdx.x & 63, g = lane >> 4;
    v4f h[4], u;
    {
        const float4 w = wl[lane];
        const float w1[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int c = 0; c < 4; ++c) h[c] = mfma4(w1[c], v, bias4(bl, 16 * c + 4 * g));
    }
#pragma unroll
    for (int layer = 0; layer < 3; ++layer) {
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r) h[c][r] = gelu_f32(h[c][r]);
        v8h xh[2], xl[2];
        split_f16(h[0], h[1], xh[0], xl[0]);
        split_f16(h[2], h[3], xh[1], xl[1]);
        if (layer < 2) {
#pragma unroll
            for (int co = 0; co < 4; ++co)
                h[co] = mfma_x2(wh, wlo, layer * 8 + co * 2, lane, xh, xl,
                                bias4(bl, 64 * (layer + 1) + 16 * co + 4 * g));
        } else {
            v4f b4;
#pragma unroll
            for (int r = 0; r < 4; ++r) b4[r] = (4 * g + r < kHeads) ? bl[192 + 4 * g + r] : 0.0f;
            u = mfma_x2(wh, wlo, 16, lane, xh, xl, b4);
        }
    }
    return u;
}

// One pair block through the bf16 chain (as mlp2_bf16).
__device__ __forceinline__ v4f mlp1_bf16(const float4 *__restrict__ wl,
                                         const v8bf *__restrict__ w16,
                                         const float *__restrict__ bl, float v) {
    const int lane = threadIdx.x & 63, g = lane >> 4;
    v4f h[4], t[4];
    {
        const float4 w = wl[lane];
        const float w1[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int c = 0; c < 4; ++c) h[c] = mfma4(w1[c], v, bias4(bl, 16 * c + 4 * g));
    }
#pragma unroll
    for (int layer = 0; layer < 2; ++layer) {
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r) h[c][r] = gelu_lo(h[c][r]);
        const v8bf x0 = pack_bf16(h[0], h[1]), x1 = pack_bf16(h[2], h[3]);
#pragma unroll
        for (int co = 0; co < 4; ++co) {
            const v4f b = bias4(bl, 64 * (layer + 1) + 16 * co + 4 * g);
            const v8bf w0 = w16[(layer * 8 + co * 2 + 0) * 64 + lane];
            const v8bf w1 = w16[(layer * 8 + co * 2 + 1) * 64 + lane];
            t[co] = mfma32bf(w1, x1, mfma32bf(w0, x0, b));
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) h[c] = t[c];
    }
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) h[c][r] = gelu_lo(h[c][r]);
    v4f b4;
#pragma unroll
    for (int r = 0; r < 4; ++r) b4[r] = (4 * g + r < kHeads) ? bl[192 + 4 * g + r] : 0.0f;
    const v8bf w0 = w16[16 * 64 + lane], w1 = w16[17 * 64 + lane];
    return mfma32bf(w1, pack_bf16(h[2], h[3]), mfma32bf(w0, pack_bf16(h[0], h[1]), b4));
}

// One pair block through the float32 chain (weights through any pointer):
// the exact fall back of the fp16 x 2 chain, which runs only for the rare
// block whose fp16 x 2 result was not finite.  One block at a time keeps its
// register footprint below that of the hot path it is inlined into.
__device__ inline v4f mlp1_f32(const float4 *__restrict__ wl, const float *__restrict__ bl,
                               float v) {
    const int lane = threadIdx.x & 63, g = lane >> 4;
    v4f h[4], t[4];
    {
        const float4 w = wl[lane];
        const float w1[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int c = 0; c < 4; ++c) h[c] = mfma4(w1[c], v, bias4(bl, 16 * c + 4 * g));
    }
    for (int layer = 0; layer < 2; ++layer) {
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r) h[c][r] = gelu_f32(h[c][r]);
#pragma unroll
        for (int co = 0; co < 4; ++co) t[co] = bias4(bl, 64 * (layer + 1) + 16 * co + 4 * g);
        const int gbase = 1 + 16 * layer;
#pragma unroll
        for (int ci = 0; ci < 4; ++ci)
#pragma unroll
            for (int co = 0; co < 4; ++co) {
                const float4 w = wl[(gbase + co * 4 + ci) * 64 + lane];
                t[co] = mfma4(w.x, h[ci][0], t[co]);
                t[co] = mfma4(w.y, h[ci][1], t[co]);
                t[co] = mfma4(w.z, h[ci][2], t[co]);
                t[co] = mfma4(w.w, h[ci][3], t[co]);
            }
#pragma unroll
        for (int c = 0; c < 4; ++c) h[c] = t[c];
    }
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) h[c][r] = gelu_f32(h[c][r]);
    v4f u;
#pragma unroll
    for (int r = 0; r < 4; ++r) u[r] = (4 * g + r < kHeads) ? bl[192 + 4 * g + r] : 0.0f;
#pragma unroll
    for (int ci = 0; ci < 4; ++ci) {
        const float4 w = wl[(33 + ci) * 64 + lane];
        u = mfma4(w.x, h[ci][0], u);
        u = mfma4(w.y, h[ci][1], u);
        u = mfma4(w.z, h[ci][2], u);
        u = mfma4(w.w, h[ci][3], u);
    }
    return u;
}

__device__ __forceinline__ bool all_finite(const v4f &a, const v4f &b) {
    bool ok = true;
#pragma unroll
    for (int r = 0; r < 4; ++r)
        ok = ok && __builtin_isfinite(a[r]) && __builtin_isfinite(b[r]);
    return ok;
}


// ------------------------------------------------------------ int8 chain
// Inputs of layers 2, 3, 4 quantised to int8 with a per-tensor zero point
// ("Economical Jet Taggers" summary, Methodologie, "Datatype Kwantisering"):
// q = clamp(rint(h / S) + Z, -128, 127); per-channel symmetric int8 weights
// Wq with scale sw; y = S sw (sum Wq q - Z sum Wq) + b' on
// v_mfma_i32_16x16x64_i8 with exact int32 sums.  Layer 1 and the GELUs are
// float32.  One K = 64 product per 16 output channels: lane group g's 16
// bytes hold the inputs 16c + 4g + r (byte 4c + r), which is where the
// float32 result registers of the previous layer already sit; the host packs
// the weight operands in the same order.
typedef int v4i __attribute__((ext_vector_type(4)));
constexpr int kW8Ops = 9;              // 4 + 4 output tiles of layers 2, 3 and 1 of layer 4
constexpr int kQ8Floats = 2 * 144;     // sw (136, padded to 144) | sum Wq (as floats)

__device__ __forceinline__ v4i mfma64i8(v4i a, v4i b, v4i c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// 16 activations (h[c][r] = input 16c + 4g + r) -> int8 codes, byte 4c + r:
// q = clamp(rint(h / S) + Z, -128, 127).  The clamp is one v_med3 (clamping
// before the rounding gives the same code: the bounds are integers); adding
// 1.5 * 2^23 rounds to the nearest integer, ties to even (the float32 sum
// has a unit ulp there), and leaves the code's two's complement in the low
// byte of the bit pattern; three byte permutes pack four codes.
__device__ __forceinline__ v4i quant16(const v4f (&h)[4], float inv_s, float zp) {
    v4i out;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        uint32_t b[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float x = __builtin_amdgcn_fmed3f(fmaf(h[c][r], inv_s, zp), -128.0f, 127.0f);
            b[r] = __builtin_bit_cast(uint32_t, x + 12582912.0f);
        }
        // perm(hi, lo, sel): byte k of the result is byte sel_k of {hi:lo}
        // (0..3 lo, 4..7 hi, 0x0c zero)
        const uint32_t lo = __builtin_amdgcn_perm(b[1], b[0], 0x0c0c0400u);
        const uint32_t hi = __builtin_amdgcn_perm(b[3], b[2], 0x0c0c0400u);
        out[c] = (int)__builtin_amdgcn_perm(hi, lo, 0x05040100u);
    }
    return out;
}

// Two pair blocks through the int8 chain.  wl: the float32 layer-1 group;
// w8: the int8 operands [op][lane]; deq / off: per channel S sw and
// b' - S sw Z sum Wq of layers 2 (0..63), 3 (64..127), 4 (128..143, rows >= 8
// zero), so that y = deq * sum + off.
__device__ __forceinline__ void mlp2_int8(const float4 *__restrict__ wl,
                                          const v4i *__restrict__ w8,
                                          const float *__restrict__ deq,
                                          const float *__restrict__ zs,
                                          const float *__restrict__ bl, const float (&inv_s)[3],
                                          const float (&zp)[3], float vA, float vB, v4f &uA,
                                          v4f &uB) {
    const int lane = threadIdx.x & 63, g = lane >> 4;
    v4f hA[4], hB[4];
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
    for (int layer = 0; layer < 3; ++layer) {
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                hA[c][r] = gelu_f32(hA[c][r]);
                hB[c][r] = gelu_f32(hB[c][r]);
            }
        const v4i xA = quant16(hA, inv_s[layer], zp[layer]);
        const v4i xB = quant16(hB, inv_s[layer], zp[layer]);
        const int nco = layer < 2 ? 4 : 1;
#pragma unroll
        for (int co = 0; co < nco; ++co) {
            const v4i w = w8[(layer * 4 + co) * 64 + lane];
            const v4i aA = mfma64i8(w, xA, (v4i){0, 0, 0, 0});
            const v4i aB = mfma64i8(w, xB, (v4i){0, 0, 0, 0});
            const int ch = 64 * layer + 16 * co + 4 * g;
            const v4f d = bias4(deq, ch), z = bias4(zs, ch);
            v4f yA, yB;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                yA[r] = fmaf(d[r], (float)aA[r], z[r]);
                yB[r] = fmaf(d[r], (float)aB[r], z[r]);
            }
            if (layer < 2) {
                hA[co] = yA;
                hB[co] = yB;
            } else {
                uA = yA;
                uB = yB;
            }
        }
    }
}

// Everything the int8 mode needs besides the float32 operands: the packed
// int8 weights, their scales and column sums (device), and the activation
// quantisation of the inputs of layers 2, 3, 4 (scale S, zero point Z).
struct Int8Args {
    const v4i *w8;
    const float *q8;
    float s[3], inv_s[3], zp[3];
};

// ------------------------------------------------------------ mode dispatch
// kMlpF32: every layer on the float32 MFMA (weights 37 KB in LDS).
// kMlpF16x2: layer 1 float32, layers 2..4 fp16 x 2 (float32-faithful), with
//   a per-block-pair fall back to the float32 chain (weights from global
//   memory) when an activation left the fp16 range.
// kMlpBf16: layer 1 float32, layers 2..4 bf16 operands, GELU degree 3.
// kMlpInt8: layer 1 float32, layers 2..4 int8 inputs and weights (above).
constexpr int kMlpF32 = 0, kMlpF16x2 = 1, kMlpBf16 = 2, kMlpInt8 = 3;

// U is stored as bfloat16 by the bf16 and int8 modes, as float32 otherwise.
template <int kMode>
using MlpOut = typename std::conditional<kMode == kMlpBf16 || kMode == kMlpInt8, uint16_t,
                                         float>::type;

template <int kMode>
struct MlpLds {
    static constexpr int kW4 = kMode == kMlpF32 ? kW32Groups * 64 : 64;
    static constexpr int kOps16 = kMode == kMlpF32 ? 1 : kW16Ops * 64;
    static constexpr bool kI8 = kMode == kMlpInt8;
    float4 *wl;
    v8h *wh;
    v8h *wlo;
    v8bf *wb;
    float *bl;
    v4i *w8;
    float *deq, *zs;
    float inv_s[3], zp[3];  // activation quantisation (int8 mode)

    __device__ MlpLds() {
        __shared__ float4 s_wl[kW4];
        __shared__ v8h s_wh[kMode == kMlpF16x2 ? kOps16 : 1];
        __shared__ v8h s_wlo[kMode == kMlpF16x2 ? kOps16 : 1];
        __shared__ v8bf s_wb[kMode == kMlpBf16 ? kOps16 : 1];
        __shared__ float s_bl[kBiasFloats];
        __shared__ v4i s_w8[kI8 ? kW8Ops * 64 : 1];
        __shared__ float s_dz[kI8 ? kQ8Floats : 1];
        wl = s_wl;
        wh = s_wh;
        wlo = s_wlo;
        wb = s_wb;
        bl = s_bl;
        w8 = s_w8;
        deq = s_dz;
        zs = s_dz + kQ8Floats / 2;
#pragma unroll
        for (int l = 0; l < 3; ++l) inv_s[l] = zp[l] = 0.f;
    }
    __device__ void set_act(const Int8Args &ia) {
#pragma unroll
        for (int l = 0; l < 3; ++l) {
            inv_s[l] = ia.inv_s[l];
            zp[l] = ia.zp[l];
        }
    }

    // Copy this mode's operands and the biases into LDS (all threads; the
    // caller synchronises before use).
    // This thread's share of the staging as a load step and a store step
    // (the caller synchronises before the weights are used).
    template <int kThreads>
    struct Staging {
        LdsCopy<kThreads, kW4, float4> c32;
        LdsCopy<kThreads, kBiasFloats, float> cb;
        LdsCopy<kThreads, kMode == kMlpF16x2 ? kOps16 : 1, v8h> chi, clo;
        LdsCopy<kThreads, kMode == kMlpBf16 ? kOps16 : 1, v8bf> c16;
        LdsCopy<kThreads, kI8 ? kW8Ops * 64 : 1, v4i> c8;
        LdsCopy<kThreads, kI8 ? kQ8Floats : 1, float> cq;
        float qs[3], qz[3];
        // for the offset entries (second half of q8): the channel's sw and bias
        float qw[decltype(cq)::kIt], qb[decltype(cq)::kIt];
        __device__ __forceinline__ void load(const float4 *__restrict__ w32,
                                             const v8bf *__restrict__ w16,
                                             const v8h *__restrict__ wx2,
                                             const float *__restrict__ bias,
                                             const Int8Args *ia = nullptr) {
            c32.load(w32);
            cb.load(bias);
            if constexpr (kMode == kMlpF16x2) {
                chi.load(wx2);
                clo.load(wx2 + kOps16);
            }
            if constexpr (kMode == kMlpBf16) c16.load(w16);
            if constexpr (kI8) {
                c8.load(ia->w8);
                cq.load(ia->q8);
#pragma unroll
                for (int l = 0; l < 3; ++l) {
                    qs[l] = ia->s[l];
                    qz[l] = ia->zp[l];
                }
                // channel ch's folded bias is b' at 64 + ch (b2' | b3' | b4
                // sit at 64..199), 0 for the unused layer-4 rows >= 8
#pragma unroll
                for (int it = 0; it < decltype(cq)::kIt; ++it) {
                    const int ch = (threadIdx.x + it * kThreads) % (kQ8Floats / 2);
                    qw[it] = ia->q8[ch];
                    qb[it] = ch < 136 ? bias[64 + ch] : 0.0f;
                }
            }
        }
        __device__ __forceinline__ void store(const MlpLds &M) const {
            c32.store(M.wl);
            cb.store(M.bl);
            if constexpr (kMode == kMlpF16x2) {
                chi.store(M.wh);
                clo.store(M.wlo);
            }
            if constexpr (kMode == kMlpBf16) c16.store(M.wb);
            if constexpr (kI8) {
                c8.store(M.w8);
                // deq = S sw and off = b' - S sw Z sum Wq per output channel
                // (channels 0..63 layer 2, 64..127 layer 3, 128.. layer 4)
#pragma unroll
                for (int it = 0; it < decltype(cq)::kIt; ++it) {
                    const int i = threadIdx.x + it * kThreads;
                    if (i >= kQ8Floats) continue;
                    const int ch = i % (kQ8Floats / 2), l = ch < 64 ? 0 : (ch < 128 ? 1 : 2);
                    M.deq[i] = i < kQ8Floats / 2
                                   ? cq.v[it] * qs[l]
                                   : fmaf(-(qw[it] * qs[l]), cq.v[it] * qz[l], qb[it]);
                }
            }
        }
    };
    template <int kThreads>
    __device__ void stage(const float4 *__restrict__ w32, const v8bf *__restrict__ w16,
                          const v8h *__restrict__ wx2, const float *__restrict__ bias,
                          const Int8Args *ia = nullptr) {
        Staging<kThreads> st;
        st.load(w32, w16, wx2, bias, ia);
        st.store(*this);
    }

    // Two pair blocks through this mode's chain.  Returns false (for the
    // whole wave) when the fp16 x 2 chain produced a non-finite value, i.e.
    // an activation may have left the fp16 range: the caller then redoes its
    // work with run_exact.  The other modes always return true.
    __device__ __forceinline__ bool run(float fA, float fB, v4f &uA, v4f &uB) const {
        if constexpr (kMode == kMlpF32) {
            mlp2_f32(wl, bl, fA, fB, uA, uB);
            return true;
        } else if constexpr (kMode == kMlpF16x2) {
            mlp2_f16x2(wl, wh, wlo, bl, fA, fB, uA, uB);
            return __ballot(!all_finite(uA, uB)) == 0;
        } else if constexpr (kMode == kMlpBf16) {
            mlp2_bf16(wl, wb, bl, fA, fB, uA, uB);
            return true;
        } else {
            mlp2_int8(wl, w8, deq, zs, bl, inv_s, zp, fA, fB, uA, uB);
            return true;
        }
    }

    // The exact float32 chain with the float32 operands w32 in global memory.
    __device__ __forceinline__ void run_exact(const float4 *__restrict__ w32, float fA, float fB,
                                              v4f &uA, v4f &uB) const {
        uA = mlp1_f32(w32, bl, fA);
        uB = mlp1_f32(w32, bl, fB);
    }

    // One pair block through this mode's chain (float32, fp16 x 2 or bf16),
    // with run()'s meaning of the return value.
    __device__ __forceinline__ bool run1(float f, v4f &u) const {
        static_assert(kMode != kMlpInt8, "the int8 chain runs two blocks");
        if constexpr (kMode == kMlpF32) {
            u = mlp1_f32(wl, bl, f);
            return true;
        } else if constexpr (kMode == kMlpF16x2) {
            u = mlp1_f16x2(wl, wh, wlo, bl, f);
            bool ok = true;
#pragma unroll
            for (int r = 0; r < 4; ++r) ok = ok && __builtin_isfinite(u[r]);
            return __ballot(!ok) == 0;
        } else {
            u = mlp1_bf16(wl, wb, bl, f);
            return true;
        }
    }
};

}  // namespace pip

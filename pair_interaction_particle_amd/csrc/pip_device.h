// pip_device.h -- device-side helpers shared by the HIP kernels of libpip.
//
// Register layouts used throughout (gfx950 MFMA, wave64, lane l, g = l / 16):
//   v_mfma_f32_16x16x4_f32   A: lane l holds A[l%16][g]      (16 x 4)
//                            B: lane l holds B[g][l%16]      (4 x 16)
//                            D: lane l, reg r holds D[4g+r][l%16]
//   v_mfma_f32_16x16x16_bf16 A: lane l holds A[l%16][4g..4g+3]; B: B[4g..4g+3][l%16]
//   v_mfma_f32_16x16x32_bf16 A: lane l holds A[l%16][8g..8g+7]; B: B[8g..8g+7][l%16]
// A reduction over k only needs A and B to agree on which (lane group, slot)
// carries which k, so the weights are packed on the host with the reduction
// index permuted to match the D layout of the previous layer: the output
// registers of one MFMA layer are, after the activation, directly the B
// operand of the next.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pip {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v4bf __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef float v8f __attribute__((ext_vector_type(8)));

constexpr int kHid = 64;
constexpr int kHeads = 8;
constexpr int kTile = 16;
constexpr int kMaxP = 256;
// ln(1e-8) and 1e-8: the feature clamp (PIP_FEATURE_EPS).
constexpr double kEps = 1e-8;
constexpr float kLnEps = -18.420680743952367f;
constexpr double kPi = 3.141592653589793238462643383279502884;
constexpr double kTwoPi = 6.283185307179586476925286766559005768;
constexpr double kRapFloor = 1e-300;

__device__ __forceinline__ v4f mfma4(float a, float b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v4f mfma32bf(v8bf a, v8bf b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v4f mfma32h(v8h a, v8h b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// x = hi + lo with hi = fp16(x), lo = fp16(x - hi), both rounded to nearest:
// 22 significand bits, |x - hi - lo| <= 2^-22 |x| while x and x - hi stay in
// the normal fp16 range (|x| <= 65504; below 2^-14 the error is absolute,
// at most 2^-25).
// The residual x - hi is formed as fma(hi, -1, x) with the -1 in a scalar
// register the optimiser cannot see through: the FMA then stays an FMA and
// reads its fp16 operand in place (v_fma_mix_f32), one instruction instead of
// a conversion and a subtraction.  The value is the same: x - hi is exact.
__device__ __forceinline__ float opaque_neg_one() {
    float m;
    __asm__("s_mov_b32 %0, -1.0" : "=s"(m));
    return m;
}
template <int N>
__device__ __forceinline__ void split_f16(const float __attribute__((ext_vector_type(N))) &x,
                                          _Float16 __attribute__((ext_vector_type(N))) &hi,
                                          _Float16 __attribute__((ext_vector_type(N))) &lo) {
    typedef float VF __attribute__((ext_vector_type(N)));
    hi = __builtin_convertvector(x, _Float16 __attribute__((ext_vector_type(N))));
    const float m1 = opaque_neg_one();
    VF r;
#pragma unroll
    for (int j = 0; j < N; ++j) r[j] = fmaf((float)hi[j], m1, x[j]);
    lo = __builtin_convertvector(r, _Float16 __attribute__((ext_vector_type(N))));
}
__device__ __forceinline__ void split4_f16(float4 x, v4h &hi, v4h &lo) {
    const v4f v = {x.x, x.y, x.z, x.w};
    split_f16<4>(v, hi, lo);
}

// ------------------------------------------------------------ kinematics
// Per-particle record staged in LDS (struct of arrays, one slot per particle).
template <int N>
struct PartLds {
    double E[N], px[N], py[N], pz[N], y[N], phi[N];
    float lnpt[N], pt[N];
    int real[N];
};

// Fill LDS slot `s` from the energy-first 4-vector (E, px, py, pz):
// pT = sqrt(px^2 + py^2), y = 1/2 ln((E+pz)/(E-pz)) with both arguments
// floored at 1e-300, phi = atan2(py, px); all in float64.
template <class PL>
__device__ inline void stage_particle(PL& L, int s, float4 p, int real) {
    double E = p.x, px = p.y, py = p.z, pz = p.w;
    double num = E + pz, den = E - pz;
    num = (num > kRapFloor) ? num : kRapFloor;
    den = (den > kRapFloor) ? den : kRapFloor;
    double pt = sqrt(px * px + py * py);
    L.E[s] = E;
    L.px[s] = px;
    L.py[s] = py;
    L.pz[s] = pz;
    L.y[s] = 0.5 * log(num / den);
    L.phi[s] = atan2(py, px);
    L.pt[s] = (float)pt;
    L.lnpt[s] = (float)log(pt);
    L.real[s] = real;
}

// Squared angular distance dy^2 + dphi^2 (dphi wrapped into (-pi, pi]; only
// its square enters, and 2pi - |d| equals the wrapped |d| exactly) and the
// pair's invariant mass squared (E_a+E_b)^2 - |p_a+p_b|^2, in float64 with
// every product and difference rounded separately (no contraction), so that
// near-collinear pairs, where m^2 cancels, are reproducible bit for bit.
template <class PL>
__device__ __forceinline__ void pair_geometry(const PL& L, int ia, int ib, double& dr2,
                                              double& m2) {
#pragma clang fp contract(off)
    double dy = L.y[ia] - L.y[ib];
    double dphi = fabs(L.phi[ia] - L.phi[ib]);
    dphi = (dphi > kPi) ? (kTwoPi - dphi) : dphi;
    dr2 = dy * dy + dphi * dphi;
    double es = L.E[ia] + L.E[ib];
    double xs = L.px[ia] + L.px[ib];
    double ys = L.py[ia] + L.py[ib];
    double zs = L.pz[ia] + L.pz[ib];
    m2 = es * es - xs * xs - ys * ys - zs * zs;
}

// Feature k (0 ln kT, 1 ln z, 2 ln dR, 3 ln m2) of the pair (ia, ib), each
// the log of its argument clamped at eps, written with one log per feature:
//   ln kT = max(ln ptmin + ln(dR^2)/2, ln eps)
//   ln z  = max(ln ptmin - ln max(pT_a + pT_b, eps), ln eps)
//   ln dR = max(ln(dR^2)/2, ln eps)
//   ln m2 = ln max(m2, eps)
template <class PL>
__device__ __forceinline__ float pair_feature(const PL& L, int ia, int ib, int k) {
    double dr2, m2;
    pair_geometry(L, ia, ib, dr2, m2);
    float lnptmin = fminf(L.lnpt[ia], L.lnpt[ib]);
    float ptsum = fmaxf(L.pt[ia] + L.pt[ib], (float)kEps);
    float m2c = (float)((m2 > kEps) ? m2 : kEps);
    float arg = (k == 1) ? ptsum : ((k == 3) ? m2c : (float)dr2);
    float lg = logf(arg);
    float v;
    if (k == 0) v = lnptmin + 0.5f * lg;
    else if (k == 1) v = lnptmin - lg;
    else if (k == 2) v = 0.5f * lg;
    else v = lg;
    return fmaxf(v, kLnEps);
}

}  // namespace pip

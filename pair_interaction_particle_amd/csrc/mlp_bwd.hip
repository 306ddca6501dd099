// mlp_bwd.hip -- gradient of the pair MLP's folded parameters, float32.
//
// The pair MLP is the pointwise 4 -> 64 -> 64 -> 64 -> 8 network of
// "Fusion 2" (ml4sci_cms_e2e26 README, "How the Kernel Fusion Works"); its
// backward is what a training step of the "Train" column of the README's
// end-to-end benchmarks needs once the attention backward has produced dU.
// With BatchNorm folded (W', b'), the MLP is y_l = W'_l h_{l-1} + b'_l,
// h_l = GELU(y_l) (l = 1..3), u = W4 h3 + b4.  U[a, c] and U[c, a] are the
// same evaluation (the features are symmetric), so every unique real pair
// contributes the backward of its evaluation for g = dU[a, c] + dU[c, a]
// (g = dU[a, a] on the diagonal):
//   dW4 += g h3^T, db4 += g;  dy3 = (W4^T g) o GELU'(y3);
//   dW'_l += dy_l h_{l-1}^T, db'_l += dy_l;  dy_{l-1} = (W'_l^T dy_l) o GELU'(y_{l-1}).
// GELU is the erf form x Phi(x), GELU'(x) = Phi(x) + x phi(x), with Phi from a
// fitted exponent (absolute error <= 7.5e-8).
//
// One 256-thread workgroup per (jet, row tile I) of 16 particles; its pair
// blocks (row i of tile (I, J < I): 16 pairs; the diagonal tile: 136 pairs
// in 9 blocks) go round-robin to the 4 waves.  Per block a wave recomputes
// the forward on the float32 matrix cores (v_mfma_f32_16x16x4_f32, hidden
// states in registers, feature-major: lane l holds features 4(l/16)+r of
// pair l%16), runs the backward chain with W'^T operands read from a
// row-major LDS copy of the weights, then forms the weight gradients as
// products over the 16 pairs: both factors are transposed through a
// wave-private LDS tile into the pair-major operand layout, and the 16x16
// results accumulate in registers across all of the wave's blocks.  At the
// end the 4 waves merge their sums into LDS in a fixed order (no atomics),
// each workgroup writes one slot of the workspace, and two more kernels add
// the slots in a fixed order: the result is the same bit for bit on every run.
#include "pip_internal.h"
#include "pip_mlp.h"

namespace pip {

constexpr int kMbWaves = 4;
constexpr int kMbThreads = 64 * kMbWaves;
constexpr int kGradFloats = 64 * 4 + 2 * 64 * 64 + 8 * 64 + 3 * 64 + 8;  // 9,160
constexpr int kGW1 = 0, kGW2 = 256, kGW3 = 4352, kGW4 = 8448;
constexpr int kGB1 = 8960, kGB2 = 9024, kGB3 = 9088, kGB4 = 9152;

// Phi(x) = x > 0 ? 1 - t : t with t = Phi(-|x|) = 2^-R(|x|), R a degree-8
// polynomial fitted by gen_gelu_coeffs.py (kPhiR): |Phi error| <= 7.5e-8 on
// [-40, 40], no clamp (R keeps growing, so t underflows to 0).  GELU(x) =
// x Phi(x) and GELU'(x) = Phi(x) + x phi(x), phi(x) = exp(-x^2/2) / sqrt(2 pi).
constexpr float kPhiR[9] = {1.000000000e+00f, 1.151105046e+00f, 4.592107534e-01f,
                            5.248672515e-02f, -7.048579864e-03f, 1.256083196e-04f,
                            1.904473174e-04f, -4.009847908e-05f, 2.873645371e-06f};
__device__ __forceinline__ float normal_cdf(float x) {
    const float a = fabsf(x);
    float p = kPhiR[8];
#pragma unroll
    for (int k = 7; k >= 0; --k) p = fmaf(p, a, kPhiR[k]);
    const float t = __builtin_amdgcn_exp2f(-p);
    return x > 0.f ? 1.f - t : t;
}
__device__ __forceinline__ float gelu_exact(float x) { return x * normal_cdf(x); }
__device__ __forceinline__ float gelu_grad(float x) {
    // 1 / (2 ln 2) = 0.72134752..., 1 / sqrt(2 pi) = 0.39894228...
    return fmaf(x * 0.39894228040143268f, __builtin_amdgcn_exp2f(-0.72134752044448170f * x * x),
                normal_cdf(x));
}

// Pair (i, j), i >= j, of lane `lane` in block k of a diagonal tile.
__device__ __forceinline__ bool tri_pair(int k, int lane, int &i, int &j) {
    int p = 16 * k + (lane & 15);
    const bool valid = p < 136;
    p = valid ? p : 0;
    int r = (int)((sqrtf(8.0f * (float)p + 1.0f) - 1.0f) * 0.5f);
    while ((r + 1) * (r + 2) / 2 <= p) ++r;
    while (r * (r + 1) / 2 > p) --r;
    i = r;
    j = p - r * (r + 1) / 2;
    return valid;
}

// X (64 features x 16 pairs, feature-major registers: X[t][r] is feature
// 16t + 4g + r of pair c) into an LDS tile [feature][pair].
__device__ __forceinline__ void to_tile(float (*Tb)[17], const v4f (&X)[4]) {
    const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) Tb[16 * t + 4 * g + r][c] = X[t][r];
}

// A[ot kNi + it] += sum over the 16 pairs of TA[o][pair] TB[i][pair]: the
// weight-gradient product of one block of pairs, accumulated in registers
// across a wave's blocks.  Output tile (ot, it): lane (g, c) holds rows
// 16 ot + 4g + r, column 16 it + c.  Tile rows >= rmax and columns >= cmax
// read as 0 (tile rows the block did not write).
template <int kNo, int kNi>
__device__ __forceinline__ void outer_reg(v4f (&A)[kNo * kNi], v4f (&R)[kNo],
                                          const float (*TA)[17], const float (*TB)[17], int rmax,
                                          int cmax) {
    const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
    float a[kNo][4], b[kNi][4];
#pragma unroll
    for (int t = 0; t < kNo; ++t)
#pragma unroll
        for (int s = 0; s < 4; ++s) a[t][s] = 16 * t + c < rmax ? TA[16 * t + c][4 * s + g] : 0.f;
#pragma unroll
    for (int t = 0; t < kNi; ++t)
#pragma unroll
        for (int s = 0; s < 4; ++s) b[t][s] = 16 * t + c < cmax ? TB[16 * t + c][4 * s + g] : 0.f;
#pragma unroll
    for (int ot = 0; ot < kNo; ++ot) {
#pragma unroll
        for (int it = 0; it < kNi; ++it)
#pragma unroll
            for (int s = 0; s < 4; ++s)
                A[kNi * ot + it] = mfma4(a[ot][s], b[it][s], A[kNi * ot + it]);
        // the row sums over the pairs (the bias gradient): the same A
        // operands against a column of ones; every column of R holds them
#pragma unroll
        for (int s = 0; s < 4; ++s) R[ot] = mfma4(a[ot][s], 1.0f, R[ot]);
    }
}

// acc (row stride ld) += the register tiles of outer_reg, rows < rmax and
// columns < cmax: a plain read-add-write, so the caller makes sure no other
// wave writes the same region meanwhile.
template <int kNo, int kNi>
__device__ __forceinline__ void flush_reg(float *acc, int ld, const v4f (&A)[kNo * kNi], int rmax,
                                          int cmax) {
    const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
#pragma unroll
    for (int ot = 0; ot < kNo; ++ot)
#pragma unroll
        for (int it = 0; it < kNi; ++it)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * ot + 4 * g + r, col = 16 * it + c;
                if (row < rmax && col < cmax) acc[row * ld + col] += A[kNi * ot + it][r];
            }
}

// acc[16 t + 4g + r] += R[t][r] for rows < rmax, from the lanes of column 0
// (every column of the row-sum tiles of outer_reg holds the same sums)
template <int kN>
__device__ __forceinline__ void flush_rows(float *acc, const v4f (&R)[kN], int rmax) {
    const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
    if (c != 0) return;
#pragma unroll
    for (int t = 0; t < kN; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (16 * t + 4 * g + r < rmax) acc[16 * t + 4 * g + r] += R[t][r];
}

template <int kPP>
__global__ __launch_bounds__(kMbThreads) __attribute__((amdgpu_waves_per_eu(1))) void
mlp_bwd_kernel(const float4 *__restrict__ p4, const uint8_t *__restrict__ mask, int P,
               const float *__restrict__ wplain, const float *__restrict__ bias,
               const float *__restrict__ dU, float *__restrict__ partial) {
    // W2', W3' row-major and transposed (rows padded to 68 floats: 16-byte
    // aligned, so each lane reads its four k-steps of an operand at once)
    __shared__ float4 Wl4[2][64][17];
    __shared__ float4 WlT4[2][64][17];
    __shared__ float W4s[8][65];
    __shared__ float W1s[64][4];
    __shared__ float bs[200];
    __shared__ float acc[kGradFloats];
    __shared__ PartLds<kPP> L;
    __shared__ float tr[kMbWaves][2][64][17];

    const int T = P / kTile;
    // the largest row tiles of every jet first (longest workgroups start early)
    const int nj = (int)(gridDim.x / T);
    const int jet = (int)(blockIdx.x % nj), I = T - 1 - (int)(blockIdx.x / nj);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, c = lane & 15;

    for (int e = tid; e < 64 * 64; e += kMbThreads) {
        float *w0 = (float *)Wl4[0][e >> 6], *w1 = (float *)Wl4[1][e >> 6];
        float *t0 = (float *)WlT4[0][e & 63], *t1 = (float *)WlT4[1][e & 63];
        const float a = wplain[256 + e], b = wplain[4352 + e];
        w0[e & 63] = a;
        w1[e & 63] = b;
        t0[e >> 6] = a;
        t1[e >> 6] = b;
    }
    for (int e = tid; e < 8 * 64; e += kMbThreads) W4s[e >> 6][e & 63] = wplain[8448 + e];
    if (tid < 256) W1s[tid >> 2][tid & 3] = wplain[tid];
    if (tid < 200) bs[tid] = bias[tid];
    for (int e = tid; e < kGradFloats; e += kMbThreads) acc[e] = 0.f;
    const int ncols = (I + 1) * kTile;
    if (tid < ncols) {
        const size_t idx = (size_t)jet * P + tid;
        const float4 pv = p4[idx];
        const int real = mask[idx] != 0;
        stage_particle(L, tid, real ? pv : make_float4(0.f, 0.f, 0.f, 0.f), real);
    }
    __syncthreads();

    const float *dUj = dU + (size_t)jet * kHeads * P * P;
    const size_t plane = (size_t)P * P;
    float (*T0)[17] = tr[wave][0];
    float (*T1)[17] = tr[wave][1];
    const int nb = 16 * I + 9;
    // the gradients summed over this wave's blocks, in registers: weight
    // tiles of every layer, per-lane partial sums of the bias gradients
    v4f gw1[4], gw2[16], gw3[16], gw4[4], gb1[4], gb2[4], gb3[4], gb4[1];
#pragma unroll
    for (int t = 0; t < 16; ++t) gw2[t] = gw3[t] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 4; ++t)
        gw1[t] = gw4[t] = gb1[t] = gb2[t] = gb3[t] = (v4f){0.f, 0.f, 0.f, 0.f};
    gb4[0] = (v4f){0.f, 0.f, 0.f, 0.f};
    for (int blk = wave; blk < nb; blk += kMbWaves) {
        int i, j;
        bool valid;
        if (blk < 16 * I) {
            i = blk & 15;
            j = (blk >> 4) * kTile + c;
            i += I * kTile;
            valid = true;
        } else {
            int ti, tj;
            valid = tri_pair(blk - 16 * I, lane, ti, tj);
            i = I * kTile + ti;
            j = I * kTile + tj;
        }
        valid = valid && L.real[i] && L.real[j];
        if (!__any(valid)) continue;
        // g = dU[a][c] + dU[c][a] for heads 4t + (l/16), t = 0, 1
        float gv[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int h = 4 * t + g;
            const float x = dUj[h * plane + (size_t)i * P + j];
            const float y = dUj[h * plane + (size_t)j * P + i];
            gv[t] = valid ? (i != j ? x + y : x) : 0.f;
        }
        const float f = valid ? pair_feature(L, i, j, g) : 0.f;

        // ---- forward, feature-major
        v4f y1[4], y2[4], y3[4], hh[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            v4f b;
#pragma unroll
            for (int r = 0; r < 4; ++r) b[r] = bs[16 * t + 4 * g + r];
            y1[t] = mfma4(W1s[16 * t + c][g], f, b);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) hh[t][r] = gelu_exact(y1[t][r]);
#pragma unroll
        for (int co = 0; co < 4; ++co) {
#pragma unroll
            for (int r = 0; r < 4; ++r) y2[co][r] = bs[64 + 16 * co + 4 * g + r];
#pragma unroll
            for (int ci = 0; ci < 4; ++ci) {
                const float4 w = Wl4[0][16 * co + c][4 * ci + g];
                y2[co] = mfma4(w.x, hh[ci][0], y2[co]);
                y2[co] = mfma4(w.y, hh[ci][1], y2[co]);
                y2[co] = mfma4(w.z, hh[ci][2], y2[co]);
                y2[co] = mfma4(w.w, hh[ci][3], y2[co]);
            }
        }
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) hh[t][r] = gelu_exact(y2[t][r]);
#pragma unroll
        for (int co = 0; co < 4; ++co) {
#pragma unroll
            for (int r = 0; r < 4; ++r) y3[co][r] = bs[128 + 16 * co + 4 * g + r];
#pragma unroll
            for (int ci = 0; ci < 4; ++ci) {
                const float4 w = Wl4[1][16 * co + c][4 * ci + g];
                y3[co] = mfma4(w.x, hh[ci][0], y3[co]);
                y3[co] = mfma4(w.y, hh[ci][1], y3[co]);
                y3[co] = mfma4(w.z, hh[ci][2], y3[co]);
                y3[co] = mfma4(w.w, hh[ci][3], y3[co]);
            }
        }
        // ---- layer 4: dW4 += g h3^T, db4 += g; dy3 = (W4^T g) o GELU'(y3)
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) hh[t][r] = gelu_exact(y3[t][r]);
        to_tile(T1, hh);
#pragma unroll
        for (int t = 0; t < 2; ++t) T0[4 * t + g][c] = gv[t];
        __builtin_amdgcn_wave_barrier();
        outer_reg<1, 4>(gw4, gb4, T0, T1, 8, 64);
        v4f dy[4];
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            v4f d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < 2; ++t) d = mfma4(W4s[4 * t + g][16 * it + c], gv[t], d);
#pragma unroll
            for (int r = 0; r < 4; ++r) dy[it][r] = d[r] * gelu_grad(y3[it][r]);
        }
        __builtin_amdgcn_wave_barrier();
        // ---- layers 3 and 2: dW' += dy h^T, db' += dy; dy <- (W'^T dy) o GELU'(y)
#pragma unroll
        for (int l = 1; l >= 0; --l) {
            v4f (&yp)[4] = l == 1 ? y2 : y1;
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) hh[t][r] = gelu_exact(yp[t][r]);
            to_tile(T0, dy);
            to_tile(T1, hh);
            __builtin_amdgcn_wave_barrier();
            if (l == 1) outer_reg<4, 4>(gw3, gb3, T0, T1, 64, 64);
            else outer_reg<4, 4>(gw2, gb2, T0, T1, 64, 64);
            v4f nd[4];
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                v4f d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ot = 0; ot < 4; ++ot) {
                    // W'^T[16 it + c][16 ot + 4g + r] = W'[16 ot + 4g + r][16 it + c]
                    const float4 w = WlT4[l][16 * it + c][4 * ot + g];
                    d = mfma4(w.x, dy[ot][0], d);
                    d = mfma4(w.y, dy[ot][1], d);
                    d = mfma4(w.z, dy[ot][2], d);
                    d = mfma4(w.w, dy[ot][3], d);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) nd[it][r] = d[r] * gelu_grad(yp[it][r]);
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) dy[t] = nd[t];
            __builtin_amdgcn_wave_barrier();
        }
        // ---- layer 1: dW1' += dy1 f^T, db1' += dy1
        to_tile(T0, dy);
        T1[g][c] = f;
        __builtin_amdgcn_wave_barrier();
        outer_reg<4, 1>(gw1, gb1, T0, T1, 64, 4);
        __builtin_amdgcn_wave_barrier();
    }
    // Merge the waves' register sums into acc without atomics: the gradient
    // is cut into kMbWaves disjoint parts, and in phase j wave w adds part
    // (j + w) mod kMbWaves, so no two waves touch the same floats at once and
    // every float receives the waves' sums in a fixed order.
    static_assert(kMbWaves == 4, "four gradient parts, one per wave and phase");
#pragma unroll
    for (int j = 0; j < kMbWaves; ++j) {
        const int part = (j + wave) & 3;
        if (part == 0) {
            flush_reg<4, 4>(acc + kGW2, 64, gw2, 64, 64);
        } else if (part == 1) {
            flush_reg<4, 4>(acc + kGW3, 64, gw3, 64, 64);
        } else if (part == 2) {
            flush_reg<4, 1>(acc + kGW1, 4, gw1, 64, 4);
            flush_reg<1, 4>(acc + kGW4, 64, gw4, 8, 64);
        } else {
            flush_rows<4>(acc + kGB1, gb1, 64);
            flush_rows<4>(acc + kGB2, gb2, 64);
            flush_rows<4>(acc + kGB3, gb3, 64);
            flush_rows<1>(acc + kGB4, gb4, 8);
        }
        __syncthreads();
    }
    float *out = partial + (size_t)blockIdx.x * kGradFloats;
    for (int e = tid; e < kGradFloats; e += kMbThreads) out[e] = acc[e];
}

// grad[e] = sum over the workgroup slots w = 0 .. nslots-1 of partial[w][e],
// in a fixed order: chunk k = blockIdx.y of kRedChunk consecutive slots is
// summed in slot order (its loads issued together) into chunk[k][e], then the
// chunk sums are added in chunk order.  The chunk sums have their own region
// after the slots.
constexpr int kRedChunk = 32;
__global__ __launch_bounds__(256) void mlp_bwd_reduce_kernel(const float *__restrict__ partial,
                                                             int nslots,
                                                             float *__restrict__ chunk) {
    const int e = blockIdx.x * 256 + threadIdx.x;
    const int w0 = blockIdx.y * kRedChunk;
    if (e >= kGradFloats) return;
    float v[kRedChunk];
#pragma unroll
    for (int w = 0; w < kRedChunk; ++w)
        v[w] = w0 + w < nslots ? partial[(size_t)(w0 + w) * kGradFloats + e] : 0.f;
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < kRedChunk; ++w) s += v[w];
    chunk[(size_t)blockIdx.y * kGradFloats + e] = s;
}

__global__ __launch_bounds__(256) void mlp_bwd_final_kernel(const float *__restrict__ partial,
                                                            int nchunks,
                                                            float *__restrict__ grad) {
    const int e = blockIdx.x * 256 + threadIdx.x;
    if (e >= kGradFloats) return;
    float s = 0.f;
    for (int k = 0; k < nchunks; ++k) s += partial[(size_t)k * kGradFloats + e];
    grad[e] = s;
}

// one slot per (jet, row tile) workgroup, then one chunk sum per kRedChunk slots
size_t mlp_bwd_workspace(int B, int P) {
    const size_t nslots = (size_t)B * (P / kTile);
    return (nslots + (nslots + kRedChunk - 1) / kRedChunk) * kGradFloats * sizeof(float);
}

hipError_t launch_mlp_bwd_f32(const float *p4, const uint8_t *mask, int B, int P,
                              const pip_pair_mlp *m, const float *dU, float *grad, void *ws,
                              hipStream_t s) {
    const int T = P / kTile;
    float *partial = (float *)ws;
    const dim3 rg((kGradFloats + 255) / 256);
    if (B == 0) {  // no pair: the sum over no chunk writes zeros
        hipLaunchKernelGGL(mlp_bwd_final_kernel, rg, dim3(256), 0, s, partial, 0, grad);
        return hipGetLastError();
    }
    if (P <= 128)
        hipLaunchKernelGGL(mlp_bwd_kernel<128>, dim3((unsigned)(B * T)), dim3(kMbThreads), 0, s,
                           (const float4 *)p4, mask, P, m->wplain, m->bias, dU, partial);
    else
        hipLaunchKernelGGL(mlp_bwd_kernel<256>, dim3((unsigned)(B * T)), dim3(kMbThreads), 0, s,
                           (const float4 *)p4, mask, P, m->wplain, m->bias, dU, partial);
    const int nslots = B * T, nchunks = (nslots + kRedChunk - 1) / kRedChunk;
    float *chunk = partial + (size_t)nslots * kGradFloats;
    hipLaunchKernelGGL(mlp_bwd_reduce_kernel, dim3(rg.x, (unsigned)nchunks), dim3(256), 0, s,
                       (const float *)partial, nslots, chunk);
    hipLaunchKernelGGL(mlp_bwd_final_kernel, rg, dim3(256), 0, s, (const float *)chunk, nchunks,
                       grad);
    return hipGetLastError();
}

}  // namespace pip

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
// GELU is the exact erf form here, GELU'(x) = Phi(x) + x phi(x).
//
// One 512-thread workgroup per (jet, row tile I) of 16 particles; its pair
// blocks (row i of tile (I, J < I): 16 pairs; the diagonal tile: 136 pairs
// in 9 blocks) go round-robin to the 8 waves.  Per block a wave recomputes
// the forward on the float32 matrix cores (v_mfma_f32_16x16x4_f32, hidden
// states in registers, feature-major: lane l holds features 4(l/16)+r of
// pair l%16), runs the backward chain with W'^T operands read from a
// row-major LDS copy of the weights, then forms the weight gradients as
// products over the 16 pairs: both factors are transposed through a
// wave-private LDS tile into the pair-major operand layout, and the 16x16
// results are added to the workgroup's LDS accumulators (float atomics, so
// the last bits depend on the order in which the waves add).  Each workgroup
// writes its accumulators to one slot of the workspace; a second kernel adds
// the slots in a fixed order.
#include "pip_internal.h"
#include "pip_mlp.h"

namespace pip {

constexpr int kMbWaves = 8;
constexpr int kMbThreads = 64 * kMbWaves;
constexpr int kGradFloats = 64 * 4 + 2 * 64 * 64 + 8 * 64 + 3 * 64 + 8;  // 9,160
constexpr int kGW1 = 0, kGW2 = 256, kGW3 = 4352, kGW4 = 8448;
constexpr int kGB1 = 8960, kGB2 = 9024, kGB3 = 9088, kGB4 = 9152;

__device__ __forceinline__ float normal_cdf(float x) {
    return 0.5f * erfcf(-x * 0.70710678118654752f);
}
__device__ __forceinline__ float gelu_exact(float x) { return x * normal_cdf(x); }
__device__ __forceinline__ float gelu_grad(float x) {
    return normal_cdf(x) + x * 0.39894228040143268f * __expf(-0.5f * x * x);
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

// acc[o][i] (row stride ld) += sum over the 16 pairs of A[o][pair] B[i][pair]
// for the 16-row output tiles ot < no and 16-column tiles it < ni, from the
// tiles TA and TB; rows >= rmax and columns >= cmax are not accumulated.
template <int kNo, int kNi>
__device__ __forceinline__ void outer_acc(float *acc, int ld, const float (*TA)[17],
                                          const float (*TB)[17], int rmax, int cmax) {
    const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
    float a[kNo][4], b[kNi][4];
#pragma unroll
    for (int ot = 0; ot < kNo; ++ot)
#pragma unroll
        for (int s = 0; s < 4; ++s) a[ot][s] = 16 * ot + c < rmax ? TA[16 * ot + c][4 * s + g] : 0.f;
#pragma unroll
    for (int it = 0; it < kNi; ++it)
#pragma unroll
        for (int s = 0; s < 4; ++s) b[it][s] = 16 * it + c < cmax ? TB[16 * it + c][4 * s + g] : 0.f;
#pragma unroll
    for (int ot = 0; ot < kNo; ++ot)
#pragma unroll
        for (int it = 0; it < kNi; ++it) {
            v4f d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) d = mfma4(a[ot][s], b[it][s], d);
            const int col = 16 * it + c;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * ot + 4 * g + r;
                if (row < rmax && col < cmax) atomicAdd(acc + row * ld + col, d[r]);
            }
        }
}

// acc[f] += sum over the 16 pairs of tile row f, f < rows (one lane per row)
__device__ __forceinline__ void row_sums(float *acc, const float (*Tb)[17], int rows) {
    const int lane = threadIdx.x & 63;
    if (lane < rows) {
        float s = 0.f;
#pragma unroll
        for (int p = 0; p < 16; ++p) s += Tb[lane][p];
        atomicAdd(acc + lane, s);
    }
}

template <int kPP>
__global__ __launch_bounds__(kMbThreads) __attribute__((amdgpu_waves_per_eu(2))) void
mlp_bwd_kernel(const float4 *__restrict__ p4, const uint8_t *__restrict__ mask, int P,
               const float *__restrict__ wplain, const float *__restrict__ bias,
               const float *__restrict__ dU, float *__restrict__ partial) {
    __shared__ float Wl[2][64][65];  // W2', W3' row-major
    __shared__ float W4s[8][65];
    __shared__ float W1s[64][4];
    __shared__ float bs[200];
    __shared__ float acc[kGradFloats];
    __shared__ PartLds<kPP> L;
    __shared__ float tr[kMbWaves][2][64][17];

    const int T = P / kTile;
    const int jet = blockIdx.x / T, I = T - 1 - (int)(blockIdx.x % T);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, c = lane & 15;

    for (int e = tid; e < 64 * 64; e += kMbThreads) {
        Wl[0][e >> 6][e & 63] = wplain[256 + e];
        Wl[1][e >> 6][e & 63] = wplain[4352 + e];
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
            for (int ci = 0; ci < 4; ++ci)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    y2[co] = mfma4(Wl[0][16 * co + c][16 * ci + 4 * g + r], hh[ci][r], y2[co]);
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
            for (int ci = 0; ci < 4; ++ci)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    y3[co] = mfma4(Wl[1][16 * co + c][16 * ci + 4 * g + r], hh[ci][r], y3[co]);
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
        outer_acc<1, 4>(acc + kGW4, 64, T0, T1, 8, 64);
        row_sums(acc + kGB4, T0, 8);
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
            outer_acc<4, 4>(acc + (l == 1 ? kGW3 : kGW2), 64, T0, T1, 64, 64);
            row_sums(acc + (l == 1 ? kGB3 : kGB2), T0, 64);
            v4f nd[4];
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                v4f d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ot = 0; ot < 4; ++ot)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        d = mfma4(Wl[l][16 * ot + 4 * g + r][16 * it + c], dy[ot][r], d);
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
        outer_acc<4, 1>(acc + kGW1, 4, T0, T1, 64, 4);
        row_sums(acc + kGB1, T0, 64);
        __builtin_amdgcn_wave_barrier();
    }
    __syncthreads();
    float *out = partial + (size_t)blockIdx.x * kGradFloats;
    for (int e = tid; e < kGradFloats; e += kMbThreads) out[e] = acc[e];
}

// grad[e] = sum over the workgroup slots w = 0 .. nslots-1 of partial[w][e]
__global__ __launch_bounds__(256) void mlp_bwd_reduce_kernel(const float *__restrict__ partial,
                                                             int nslots,
                                                             float *__restrict__ grad) {
    const int e = blockIdx.x * 256 + threadIdx.x;
    if (e >= kGradFloats) return;
    float s = 0.f;
    for (int w = 0; w < nslots; ++w) s += partial[(size_t)w * kGradFloats + e];
    grad[e] = s;
}

size_t mlp_bwd_workspace(int B, int P) {
    return (size_t)B * (P / kTile) * kGradFloats * sizeof(float);
}

hipError_t launch_mlp_bwd_f32(const float *p4, const uint8_t *mask, int B, int P,
                              const pip_pair_mlp *m, const float *dU, float *grad, void *ws,
                              hipStream_t s) {
    const int T = P / kTile;
    float *partial = (float *)ws;
    if (B == 0) {  // no pair: the reduction over no slot writes zeros
        hipLaunchKernelGGL(mlp_bwd_reduce_kernel, dim3((kGradFloats + 255) / 256), dim3(256), 0,
                           s, partial, 0, grad);
        return hipGetLastError();
    }
    if (P <= 128)
        hipLaunchKernelGGL(mlp_bwd_kernel<128>, dim3((unsigned)(B * T)), dim3(kMbThreads), 0, s,
                           (const float4 *)p4, mask, P, m->wplain, m->bias, dU, partial);
    else
        hipLaunchKernelGGL(mlp_bwd_kernel<256>, dim3((unsigned)(B * T)), dim3(kMbThreads), 0, s,
                           (const float4 *)p4, mask, P, m->wplain, m->bias, dU, partial);
    hipLaunchKernelGGL(mlp_bwd_reduce_kernel, dim3((kGradFloats + 255) / 256), dim3(256), 0, s,
                       partial, B * T, grad);
    return hipGetLastError();
}

}  // namespace pip

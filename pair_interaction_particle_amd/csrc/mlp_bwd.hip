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
// Two kernels compute it.  The fp16 x 2 kernel further down (every large
// product on the fp16 matrix cores with split operands, a balanced share of
// all blocks per compute unit) is the one that runs; the float32 kernel
// described next takes over when the folded weights leave the fp16 range or
// the fp16 x 2 sums come out non-finite.
//
// Float32 kernel: one 256-thread workgroup per (jet, row tile I) of 16 particles; its pair
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
#include <algorithm>

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
mlp_bwd_kernel(const float4 *__restrict__ p4, const uint8_t *__restrict__ mask, int B, int P,
               const float *__restrict__ wplain, const float *__restrict__ bias,
               const float *__restrict__ dU, float *__restrict__ partial,
               const int *__restrict__ flags, int nflags) {
    // after the fp16 x 2 kernel: runs only if one of its workgroups flagged
    // a non-finite sum
    if (flags) {
        bool any = false;
        for (int k = (int)(threadIdx.x & 63); k < nflags; k += 64) any = any || flags[k] != 0;
        if (!__any(any)) return;
    }
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
    // slot = jet + B (T - 1 - I): the largest row tiles of every jet first
    const int slot = blockIdx.x, jet = slot % B, I = T - 1 - slot / B;
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
    float *out = partial + (size_t)slot * kGradFloats;
    for (int e = tid; e < kGradFloats; e += kMbThreads) out[e] = acc[e];
}

// ---------------------------------------------------------------- block plan
// The blocks of slot (jet, I) holding a real pair are the off-diagonal blocks
// (row i of tile I, column tile J < I) whose row is real and whose column tile
// holds a real particle, and those of the diagonal tile's 9 blocks (its 136
// pairs (a, c), a >= c, in order) with a pair of two real particles.
// diag_row_blocks: the diagonal blocks that row a of a tile with real bits R
// puts a real pair into.  Row a's pairs are p = a(a+1)/2 + c, c <= a, at most
// 16 of them, so they fall into one block or two neighbouring ones.
__device__ __forceinline__ uint32_t diag_row_blocks(uint32_t R, int a) {
    if (!((R >> a) & 1u)) return 0u;
    const int p0 = a * (a + 1) / 2, k0 = p0 >> 4, k1 = (p0 + a) >> 4;
    const uint32_t cols = R & ((2u << a) - 1u);               // real c <= a
    const uint32_t low = (1u << (16 * (k0 + 1) - p0)) - 1u;   // the columns of block k0
    return ((cols & low) ? 1u << k0 : 0u) | ((k1 != k0 && (cols & ~low)) ? 1u << k1 : 0u);
}

// start[s] = blocks of the slots before s (s = jet * T + I), start[nslots] =
// all blocks N; share k of G is the blocks [bpos[k], bpos[k + 1]) (equal in
// cost, kSlotCost above), and first[k] the slot holding block bpos[k].  One workgroup, jets in chunks of kPlanJets: each wave takes
// the real bits of eight jets at a time (all loads issued first, then one
// ballot per 64 particles) into LDS; then one thread per slot counts its
// blocks.  The counts stay in LDS (in start[] beyond kPlanLds slots); each
// thread then sums a run of slots, the run totals are scanned, and the runs
// are written out as prefix sums.
constexpr int kPlanThreads = 1024;
// A workgroup's time follows its rounds: a slot's blocks in rounds of 8 plus
// one round to drain the pipeline, and the slot's particle staging.  The
// shares are equal in cost, a slot costing its blocks plus kSlotCost: with
// equal block counts, a share cut into many slot pieces took up to 27 rounds
// where the mean was 19 (kernel workload, 256 workgroups); with a slot cost
// of 8 the largest takes 21.  Measured: 275.7 us with equal block counts,
// 246.2, 234.4, 233.1, 237.1, 239.3 and 250.5 us for slot costs 4, 6, 8, 10,
// 12 and 16.
constexpr int kSlotCost = 8;
__host__ __device__ constexpr int slot_cost(int blocks) { return blocks > 0 ? blocks + kSlotCost : 0; }
constexpr int kPlanLds = 8192;   // slot counts kept in LDS up to this many slots
constexpr int kPlanJets = 1024;  // jets whose real bits are in LDS at once
__global__ __launch_bounds__(kPlanThreads) void mlp_bwd_plan_kernel(
    const uint8_t *__restrict__ mask, int B, int P, int G, int *__restrict__ start,
    int *__restrict__ first, int *__restrict__ bpos) {
    __shared__ int wsum[kPlanThreads / 64];
    __shared__ int total;
    __shared__ int lcnt[kPlanLds];
    __shared__ uint32_t bits[kPlanJets][8];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int T = P / kTile, nslots = B * T;
    int *cnt = nslots <= kPlanLds ? lcnt : start;
    for (int c0 = 0; c0 < B; c0 += kPlanJets) {
        const int nj = min(kPlanJets, B - c0);
        for (int j0 = 8 * wave; j0 < nj; j0 += 8 * (kPlanThreads / 64)) {
            uint8_t mb[8][4];  // unconditional loads of clamped addresses
#pragma unroll
            for (int q = 0; q < 8; ++q)
#pragma unroll
                for (int ch = 0; ch < 4; ++ch)
                    mb[q][ch] = mask[(size_t)(c0 + min(j0 + q, nj - 1)) * P +
                                     min(64 * ch + lane, P - 1)];
#pragma unroll
            for (int q = 0; q < 8; ++q)
#pragma unroll
                for (int ch = 0; ch < 4; ++ch) {
                    const uint64_t m = __ballot(mb[q][ch] != 0 && 64 * ch + lane < P);
                    if (lane == 0 && j0 + q < nj) {
                        bits[j0 + q][2 * ch] = (uint32_t)m;
                        bits[j0 + q][2 * ch + 1] = (uint32_t)(m >> 32);
                    }
                }
        }
        __syncthreads();
        for (int s = c0 * T + tid; s < (c0 + nj) * T; s += kPlanThreads) {
            const int jl = s / T - c0, I = s % T;
            const uint32_t R = (bits[jl][I >> 1] >> (16 * (I & 1))) & 0xffffu;
            int tiles = 0;
            for (int J = 0; J < I; ++J) tiles += ((bits[jl][J >> 1] >> (16 * (J & 1))) & 0xffffu) != 0;
            uint32_t dv = 0;
#pragma unroll
            for (int a = 0; a < kTile; ++a) dv |= diag_row_blocks(R, a);
            cnt[s] = __popc(R) * tiles + __popc(dv);
        }
        __syncthreads();
    }
    const int per = (nslots + kPlanThreads - 1) / kPlanThreads;
    const int s0 = min(tid * per, nslots), s1 = min(s0 + per, nslots);
    // exclusive prefix of the run totals and the grand total: within the
    // wave, then across waves (two passes: blocks, then costs)
    auto scan = [&](int mine, int &excl) {
        int inc = mine;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int v = __shfl_up(inc, o);
            if (lane >= o) inc += v;
        }
        if (lane == 63) wsum[wave] = inc;
        __syncthreads();
        if (wave == 0) {
            int w = lane < kPlanThreads / 64 ? wsum[lane] : 0;
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) {
                const int v = __shfl_up(w, o);
                if (lane >= o) w += v;
            }
            if (lane < kPlanThreads / 64) wsum[lane] = w;  // inclusive wave totals
            if (lane == kPlanThreads / 64 - 1) total = w;
        }
        __syncthreads();
        excl = inc - mine + (wave > 0 ? wsum[wave - 1] : 0);
        const int t = total;
        __syncthreads();  // wsum and total are reused by the next pass
        return t;
    };
    int mine = 0, minec = 0;
    for (int s = s0; s < s1; ++s) {
        mine += cnt[s];
        minec += slot_cost(cnt[s]);
    }
    int acc, accc;
    const int N = scan(mine, acc), Ct = scan(minec, accc);
    for (int s = s0; s < s1; ++s) {
        const int c = cnt[s];
        start[s] = acc;
        if (c > 0) {
            // the shares whose cost position floor(k Ct / G) falls inside this
            // slot's cost range [accc, accc + kSlotCost + c): they begin at
            // the slot's first block while inside its overhead, else in it
            int k = (int)(((unsigned long long)accc * G + Ct - 1) / (unsigned)Ct);
            for (; k < G; ++k) {
                const int ck = (int)((unsigned long long)k * Ct / (unsigned)G);
                if (ck >= accc + slot_cost(c)) break;
                first[k] = s;
                bpos[k] = acc + max(0, ck - accc - kSlotCost);
            }
        }
        acc += c;
        accc += slot_cost(c);
    }
    if (Ct == 0)  // no block at all: every share is empty
        for (int k = tid; k < G; k += kPlanThreads) bpos[k] = 0;
    if (tid == 0) {
        start[nslots] = N;
        bpos[G] = N;
    }
}

// ---------------------------------------------------------------- fp16 x 2 kernel
// The same gradient with every large product on the fp16 matrix cores
// (v_mfma_f32_16x16x32_f16), each float32 factor carried as hi = fp16(x),
// lo = fp16(x - hi) and x w = x_hi w_hi + x_hi w_lo + x_lo w_hi (relative
// error ~2^-22 per product, float32 accumulation), as in the forward chain.
// One 512-thread workgroup per compute unit takes an equal-cost share of the
// flattened list of all slots' blocks with a real pair (mlp_bwd_plan_kernel
// lays it out), slot by slot; the blocks go out in rounds, one per wave.
// Per round:
//   * every wave runs its block's forward (hidden states feature-major in
//     registers) and the backward chain dy3 -> dy2 -> dy1 (W'^T operands
//     packed on the host like the forward ones);
//   * each activation the weight gradients need (h1, h2, h3, dy1, dy2, dy3,
//     g, the features) is staged in LDS pair-major as fp16 hi / lo halves,
//     so a lane reads 8 consecutive pairs of one feature as an MFMA operand
//     with the round's 128 pairs as the K dimension;
//   * the gradient tiles are split among the waves (two or three 16x16 tiles
//     of dW3' and of dW2', one of dW1' or dW4, the bias tiles as products
//     against a column of ones), so each wave keeps only its own tiles.
// g is scaled per round by a power of two 2^e so that max |g| lies in [1, 2)
// (the backward chain is linear in g, so every dy carries the same factor);
// the accumulators hold their sums in units of 2^e and are rescaled exactly
// when e changes.  Each workgroup writes one partial sum.  If any of them
// comes out non-finite (an activation or a dy beyond the fp16 range), the
// workgroup raises its flag and the float32 kernel above recomputes every
// slot.  Every sum has a fixed order: the result is the same bit for bit on
// every run.
constexpr int kXWaves = 8;
constexpr int kXThreads = 64 * kXWaves;
constexpr int kXPairs = 16 * kXWaves;  // pairs per round: one block per wave
constexpr int kXPitch = kXPairs + 8;   // halves per staged row (272 bytes: rows 4 banks apart)
constexpr int kXOps = 16;              // fp16 operands of layers 2 and 3 (per half)

// The staged activations come first: every read of them is then one base
// register plus an immediate offset below 64 KiB.
template <int kPP>
struct XLds {
    _Float16 xa[2][64][kXPitch];  // staged activations: [hi | lo][feature][pair]
    _Float16 xb[2][64][kXPitch];
    _Float16 gs[2][8][kXPitch];  // g per head
    _Float16 fs[2][4][kXPitch];  // the pair features
    v8h wf[2][kXOps * 64];  // W' of layers 2, 3 as forward operands, hi | lo, [op][lane]
    v8h wt[2][kXOps * 64];  // W'^T of layers 2, 3 as operands of the backward chain
    float4 w1[64];          // layer 1 (float32, K = 4)
    float w4[8][64];        // layer 4 (float32)
    float bias[200];
    float emax[kXWaves];
    int bad;
    uint8_t blk[256];
    PartLds<kPP> part;
};
static_assert(sizeof(XLds<256>) <= 160 * 1024, "one workgroup's LDS");

// h = GELU(y) and d = GELU'(y), sharing Phi
__device__ __forceinline__ void gelu_both(const v4f (&y)[4], v4f (&h)[4], v4f (&d)[4]) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float x = y[t][r], ph = normal_cdf(x);
            h[t][r] = x * ph;
            d[t][r] = fmaf(x * 0.39894228040143268f,
                           __builtin_amdgcn_exp2f(-0.72134752044448170f * x * x), ph);
        }
}

// the hi / lo operands of 16 feature-major values (slot j of half s holds
// feature 16 (2s + j/4) + 4g + j%4, the order of the chain's B operands)
__device__ __forceinline__ void split16(const v4f (&x)[4], v8h (&hi)[2], v8h (&lo)[2]) {
    split_f16(x[0], x[1], hi[0], lo[0]);
    split_f16(x[2], x[3], hi[1], lo[1]);
}

// X[hi | lo][feature][pair p] = this lane's 16 split values
__device__ __forceinline__ void stage16(_Float16 (*X)[64][kXPitch], const v8h (&hi)[2],
                                        const v8h (&lo)[2], int p, int g) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int f = 16 * (2 * s + (j >> 2)) + 4 * g + (j & 3);
            X[0][f][p] = hi[s][j];
            X[1][f][p] = lo[s][j];
        }
}

// operand of K step q: row `row`, pairs 32q + 8g .. 32q + 8g + 7
__device__ __forceinline__ v8h xop(const _Float16 (*X)[kXPitch], int row, int q, int g) {
    return *(const v8h *)&X[row][32 * q + 8 * g];
}

// acc += A B^T over the round's pairs with the three-term split
__device__ __forceinline__ v4f mfma_x3(v8h ah, v8h al, v8h bh, v8h bl, v4f acc) {
    acc = mfma32h(ah, bl, acc);
    acc = mfma32h(al, bh, acc);
    return mfma32h(ah, bh, acc);
}

__device__ __forceinline__ void scale_tile(v4f &a, int e) {
#pragma unroll
    for (int r = 0; r < 4; ++r) a[r] = __builtin_amdgcn_ldexpf(a[r], e);
}

__device__ __forceinline__ bool tile_finite(const v4f &a) {
    bool ok = true;
#pragma unroll
    for (int r = 0; r < 4; ++r) ok = ok && __builtin_isfinite(a[r]);
    return ok;
}

template <int kPP>
__global__ __launch_bounds__(kXThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void
mlp_bwd_x2_kernel(const float4 *__restrict__ p4, const uint8_t *__restrict__ mask, int B, int P,
                  const v8h *__restrict__ wx2, const v8h *__restrict__ wtx2,
                  const float4 *__restrict__ w32, const float *__restrict__ wplain,
                  const float *__restrict__ bias, const float *__restrict__ dU,
                  const int *__restrict__ start, const int *__restrict__ first,
                  const int *__restrict__ bpos, float *__restrict__ partial,
                  int *__restrict__ flags) {
    __shared__ XLds<kPP> L;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int T = P / kTile, nslots = B * T;
    const size_t plane = (size_t)P * P;

    // weights, once per workgroup (wx2: 18 hi operands then 18 lo ones)
    for (int e = tid; e < 2 * kXOps * 64; e += kXThreads) {
        const int h = e / (kXOps * 64), k = e % (kXOps * 64);
        L.wf[h][k] = wx2[h * 18 * 64 + k];
        L.wt[h][k] = wtx2[e];
    }
    if (tid < 64) L.w1[tid] = w32[tid];
    for (int e = tid; e < 8 * 64; e += kXThreads) L.w4[e >> 6][e & 63] = wplain[8448 + e];
    if (tid < 200) L.bias[tid] = bias[tid];

    const v8h ones = {1, 1, 1, 1, 1, 1, 1, 1}, zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
    // the gradient tiles this wave owns (see the write-out at the end)
    const int ro = wave >> 1, ci0 = 2 * (wave & 1);
    const bool odd = (wave & 1) != 0;

    // this workgroup's share [lo, hi) of the flattened list of every slot's
    // blocks with a real pair (slots s = jet * T + I in order; start[s] is
    // the first block of slot s, first[k] the slot where share k begins)
    const long long lo = bpos[blockIdx.x], hi = bpos[blockIdx.x + 1];

    v4f a3[2], a2[2], b3, b2, ax, b4;
    a3[0] = a3[1] = a2[0] = a2[1] = b3 = b2 = ax = b4 = (v4f){0.f, 0.f, 0.f, 0.f};
    int ecur = 0;
    // the block state carried from one round's preparation to its phases
    v8h h1h[2], h1l[2], h2h[2], h2l[2], h3h[2], h3l[2];
    v4f d1[4], d2[4], dy[4];
    float gv[2], fv;
    if (tid == 0) L.bad = 0;

    long long pos = lo;
    int s = lo < hi ? __builtin_amdgcn_readfirstlane(first[blockIdx.x]) : nslots;
    while (pos < hi) {
        const int sb = __builtin_amdgcn_readfirstlane(start[s]);
        const int se = __builtin_amdgcn_readfirstlane(start[s + 1]);
        if (se == sb) {  // a slot without a real pair
            ++s;
            continue;
        }
        const int jet = s / T, I = s - jet * T;
        const int from = (int)(pos - sb), to = (int)(min(hi, (long long)se) - sb);
        const int ncols = (I + 1) * kTile;
        if (tid < ncols) {
            const size_t idx = (size_t)jet * P + tid;
            const float4 pv = p4[idx];
            const int real = mask[idx] != 0;
            stage_particle(L.part, tid, real ? pv : make_float4(0.f, 0.f, 0.f, 0.f), real);
        }
        __syncthreads();
        // the slot's blocks with a real pair, in order (the plan's test)
        if (wave == 0) {
            const uint32_t rows = (uint32_t)__ballot(lane < 16 && L.part.real[I * kTile + lane]);
            uint32_t tany = 0;
            for (int ch = 0; ch < 4; ++ch) {
                const int t = 64 * ch + lane;
                const uint64_t m = __ballot(t < I * kTile && L.part.real[t]);
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if ((m >> (16 * q)) & 0xffffull) tany |= 1u << (4 * ch + q);
            }
            // diagonal tile: lane a < 16 marks the blocks of its real pairs (a, c)
            uint32_t dv = lane < 16 ? diag_row_blocks(rows, lane) : 0u;
#pragma unroll
            for (int o = 8; o > 0; o >>= 1) dv |= __shfl_xor(dv, o);
            dv = __builtin_amdgcn_readfirstlane(dv);
            const int nb = 16 * I + 9;
            int base = 0;
            for (int ch = 0; ch < 4; ++ch) {
                const int b = 64 * ch + lane;
                const bool v = b < 16 * I ? ((rows >> (b & 15)) & (tany >> (b >> 4)) & 1u) != 0
                                          : (b < nb && ((dv >> (b - 16 * I)) & 1u) != 0);
                const uint64_t m = __ballot(v);
                if (v) L.blk[base + __popcll(m & ((1ull << lane) - 1))] = (uint8_t)b;
                base += __popcll(m);
            }
        }
        __syncthreads();
        const int nr = (to - from + kXWaves - 1) / kXWaves;
        const float *dUj = dU + (size_t)jet * kHeads * plane;


        for (int r = 0; r <= nr; ++r) {
            // lane-dependent addresses are recomputed every round rather than
            // held in registers across the loop
            int ln = lane;
            asm volatile("" : "+v"(ln));
            const int gq = ln >> 4, cq = ln & 15, pq = 16 * wave + cq;
            // round r's block and its dU values, loaded a round ahead of use
            int ni = I * kTile, nj = I * kTile;
            bool nvalid = false;
            float nx[2], ny[2];
            if (r < nr) {
                const int kb = from + kXWaves * r + wave;
                const int bi = kb < to ? L.blk[kb] : -1;
                if (bi >= 0 && bi < 16 * I) {
                    ni = I * kTile + (bi & 15);
                    nj = (bi >> 4) * kTile + cq;
                    nvalid = true;
                } else if (bi >= 0) {
                    int ti, tj;
                    nvalid = tri_pair(bi - 16 * I, ln, ti, tj);
                    ni = I * kTile + ti;
                    nj = I * kTile + tj;
                }
                nvalid = nvalid && L.part.real[ni] && L.part.real[nj];
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int h = 4 * t + gq;
                    nx[t] = dUj[h * plane + (size_t)ni * P + nj];
                    ny[t] = dUj[h * plane + (size_t)nj * P + ni];
                }
            }
            if (r > 0) {
                // [A] the round's scale; stage dy3 and h2
                float M = L.emax[0];
#pragma unroll
                for (int k = 1; k < kXWaves; ++k) M = fmaxf(M, L.emax[k]);
                int e = 0;
                if (M > 0.f && M <= 3.0e38f) e = 1 - __builtin_amdgcn_frexp_expf(M);
                if (e != ecur) {
                    const int de = e - ecur;
                    scale_tile(a3[0], de), scale_tile(a3[1], de), scale_tile(a2[0], de);
                    scale_tile(a2[1], de), scale_tile(b3, de), scale_tile(b2, de);
                    scale_tile(ax, de), scale_tile(b4, de);
                    ecur = e;
                }
#pragma unroll
                for (int t = 0; t < 4; ++t) scale_tile(dy[t], e);
                gv[0] = __builtin_amdgcn_ldexpf(gv[0], e);
                gv[1] = __builtin_amdgcn_ldexpf(gv[1], e);
                v8h dh[2], dl[2];
                split16(dy, dh, dl);
                stage16(L.xa, dh, dl, pq, gq);
                stage16(L.xb, h2h, h2l, pq, gq);
                __syncthreads();
                // [D] dW3' (rows ro, column tiles ci0, ci0 + 1), db3' (odd waves); dy2
#pragma unroll
                for (int q = 0; q < kXPairs / 32; ++q) {
                    const v8h ah = xop(L.xa[0], 16 * ro + cq, q, gq), al = xop(L.xa[1], 16 * ro + cq, q, gq);
#pragma unroll
                    for (int k = 0; k < 2; ++k)
                        a3[k] = mfma_x3(ah, al, xop(L.xb[0], 16 * (ci0 + k) + cq, q, gq),
                                        xop(L.xb[1], 16 * (ci0 + k) + cq, q, gq), a3[k]);
                    if (odd) b3 = mfma32h(al, ones, mfma32h(ah, ones, b3));
                }
#pragma unroll
                for (int it = 0; it < 4; ++it) {
                    const v4f t = mfma_x2(L.wt[0], L.wt[1], 8 + 2 * it, ln, dh, dl,
                                          (v4f){0.f, 0.f, 0.f, 0.f});
#pragma unroll
                    for (int k = 0; k < 4; ++k) dy[it][k] = t[k] * d2[it][k];
                }
                split16(dy, dh, dl);
                __syncthreads();
                // [E] stage dy2 and h1
                stage16(L.xa, dh, dl, pq, gq);
                stage16(L.xb, h1h, h1l, pq, gq);
                __syncthreads();
                // [F] dW2', db2'; dy1
#pragma unroll
                for (int q = 0; q < kXPairs / 32; ++q) {
                    const v8h ah = xop(L.xa[0], 16 * ro + cq, q, gq), al = xop(L.xa[1], 16 * ro + cq, q, gq);
#pragma unroll
                    for (int k = 0; k < 2; ++k)
                        a2[k] = mfma_x3(ah, al, xop(L.xb[0], 16 * (ci0 + k) + cq, q, gq),
                                        xop(L.xb[1], 16 * (ci0 + k) + cq, q, gq), a2[k]);
                    if (odd) b2 = mfma32h(al, ones, mfma32h(ah, ones, b2));
                }
#pragma unroll
                for (int it = 0; it < 4; ++it) {
                    const v4f t = mfma_x2(L.wt[0], L.wt[1], 2 * it, ln, dh, dl,
                                          (v4f){0.f, 0.f, 0.f, 0.f});
#pragma unroll
                    for (int k = 0; k < 4; ++k) dy[it][k] = t[k] * d1[it][k];
                }
                split16(dy, dh, dl);
                __syncthreads();
                // [G] stage dy1, h3, g and the features
                stage16(L.xa, dh, dl, pq, gq);
                stage16(L.xb, h3h, h3l, pq, gq);
                {
                    v4h qh, ql;
                    split4_f16(make_float4(gv[0], gv[1], fv, 0.f), qh, ql);
                    L.gs[0][gq][pq] = qh[0], L.gs[1][gq][pq] = ql[0];
                    L.gs[0][4 + gq][pq] = qh[1], L.gs[1][4 + gq][pq] = ql[1];
                    L.fs[0][gq][pq] = qh[2], L.fs[1][gq][pq] = ql[2];
                }
                __syncthreads();
                // [H] dW1' | db1' (waves 4..7: rows 16 (wave - 4)), dW4 (waves 0..3:
                // column tile `wave`), db4 (wave 0)
                if (wave >= 4) {
                    const int rw = 16 * (wave - 4) + cq, fr = min(cq, 3);
#pragma unroll
                    for (int q = 0; q < kXPairs / 32; ++q) {
                        v8h fh = xop(L.fs[0], fr, q, gq), fl = xop(L.fs[1], fr, q, gq);
                        if (cq >= 4) fh = (cq == 4) ? ones : zero8, fl = zero8;
                        ax = mfma_x3(xop(L.xa[0], rw, q, gq), xop(L.xa[1], rw, q, gq), fh, fl, ax);
                    }
                } else {
                    const int gr = min(cq, 7);
#pragma unroll
                    for (int q = 0; q < kXPairs / 32; ++q) {
                        v8h gh = xop(L.gs[0], gr, q, gq), gl = xop(L.gs[1], gr, q, gq);
                        if (cq >= 8) gh = zero8, gl = zero8;
                        ax = mfma_x3(gh, gl, xop(L.xb[0], 16 * wave + cq, q, gq),
                                     xop(L.xb[1], 16 * wave + cq, q, gq), ax);
                        if (wave == 0) b4 = mfma32h(gl, ones, mfma32h(gh, ones, b4));
                    }
                }
            }
            if (r < nr) {
                // prepare round r: g, the features, the forward and dy3
#pragma unroll
                for (int t = 0; t < 2; ++t)
                    gv[t] = nvalid ? (ni != nj ? nx[t] + ny[t] : nx[t]) : 0.f;
                fv = nvalid ? pair_feature(L.part, ni, nj, gq) : 0.f;
                float m = fmaxf(fabsf(gv[0]), fabsf(gv[1]));
#pragma unroll
                for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
                if (lane == 0) L.emax[wave] = m;

                v4f y[4], h[4];
                {
                    const float4 w = L.w1[ln];
                    const float w1[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                    for (int t = 0; t < 4; ++t) y[t] = mfma4(w1[t], fv, bias4(L.bias, 16 * t + 4 * gq));
                }
                gelu_both(y, h, d1);
                split16(h, h1h, h1l);
#pragma unroll
                for (int co = 0; co < 4; ++co)
                    y[co] = mfma_x2(L.wf[0], L.wf[1], 2 * co, ln, h1h, h1l,
                                    bias4(L.bias, 64 + 16 * co + 4 * gq));
                gelu_both(y, h, d2);
                split16(h, h2h, h2l);
#pragma unroll
                for (int co = 0; co < 4; ++co)
                    y[co] = mfma_x2(L.wf[0], L.wf[1], 8 + 2 * co, ln, h2h, h2l,
                                    bias4(L.bias, 128 + 16 * co + 4 * gq));
                v4f d3[4];
                gelu_both(y, h, d3);
                split16(h, h3h, h3l);
                // dy3 = (W4^T g) o GELU'(y3), before the round's scale
#pragma unroll
                for (int it = 0; it < 4; ++it) {
                    v4f d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int t = 0; t < 2; ++t) d = mfma4(L.w4[4 * t + gq][16 * it + cq], gv[t], d);
#pragma unroll
                    for (int k = 0; k < 4; ++k) dy[it][k] = d[k] * d3[it][k];
                }
            }
            __syncthreads();
        }

        pos = sb + to;
        ++s;
    }

    // write this wave's tiles (sums back to unit scale) and flag non-finite ones
    float *out = partial + (size_t)blockIdx.x * kGradFloats;
    const int ue = -ecur;
    int lo_ = lane;
    asm volatile("" : "+v"(lo_));
    const int go = lo_ >> 4, co_ = lo_ & 15;
    bool ok = tile_finite(a3[0]) && tile_finite(a3[1]) && tile_finite(a2[0]) &&
              tile_finite(a2[1]) && tile_finite(ax);
    if (odd) ok = ok && tile_finite(b3) && tile_finite(b2);
    if (wave == 0) ok = ok && tile_finite(b4);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int row = 16 * ro + 4 * go + r;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            out[kGW3 + row * 64 + 16 * (ci0 + k) + co_] = __builtin_amdgcn_ldexpf(a3[k][r], ue);
            out[kGW2 + row * 64 + 16 * (ci0 + k) + co_] = __builtin_amdgcn_ldexpf(a2[k][r], ue);
        }
        if (odd && co_ == 0) {
            out[kGB3 + row] = __builtin_amdgcn_ldexpf(b3[r], ue);
            out[kGB2 + row] = __builtin_amdgcn_ldexpf(b2[r], ue);
        }
        if (wave >= 4) {
            const int o = 16 * (wave - 4) + 4 * go + r;
            if (co_ < 4) out[kGW1 + o * 4 + co_] = __builtin_amdgcn_ldexpf(ax[r], ue);
            else if (co_ == 4) out[kGB1 + o] = __builtin_amdgcn_ldexpf(ax[r], ue);
        } else if (go < 2) {
            out[kGW4 + (4 * go + r) * 64 + 16 * wave + co_] = __builtin_amdgcn_ldexpf(ax[r], ue);
            if (wave == 0 && co_ == 0) out[kGB4 + 4 * go + r] = __builtin_amdgcn_ldexpf(b4[r], ue);
        }
    }
    if (!__all(ok) && lane == 0) L.bad = 1;
    __syncthreads();
    if (tid == 0) flags[blockIdx.x] = L.bad;
}

// grad[e] = the sum over n partial sums w of partial[w][e] in a fixed order:
// chunk k = blockIdx.y of kRedChunk consecutive partials is summed in order
// (its loads issued together) into chunk[k][e], then the chunk sums are added
// in chunk order.  The partials are the fp16 x 2 kernel's (nx2 of them) unless
// that kernel did not run (flags null) or one of its workgroups raised its
// flag; then they are the float32 kernel's (n32, one per slot).  Both kernels
// take the same decision from the flags.
constexpr int kRedChunk = 32;
__global__ __launch_bounds__(256) void mlp_bwd_reduce_kernel(
    const float *__restrict__ p32, int n32, const float *__restrict__ px2, int nx2,
    const int *__restrict__ flags, float *__restrict__ chunk) {
    bool use32 = flags == nullptr;
    if (!use32) {
        bool any = false;
        for (int k = (int)(threadIdx.x & 63); k < nx2; k += 64) any = any || flags[k] != 0;
        use32 = __any(any);
    }
    const float *partial = use32 ? p32 : px2;
    const int n = use32 ? n32 : nx2;
    const int e = blockIdx.x * 256 + threadIdx.x;
    const int w0 = blockIdx.y * kRedChunk;
    if (e >= kGradFloats || w0 >= n) return;  // the final sum stops before this chunk
    float v[kRedChunk];
#pragma unroll
    for (int w = 0; w < kRedChunk; ++w)
        v[w] = w0 + w < n ? partial[(size_t)(w0 + w) * kGradFloats + e] : 0.f;
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < kRedChunk; ++w) sum += v[w];
    chunk[(size_t)blockIdx.y * kGradFloats + e] = sum;
}

__global__ __launch_bounds__(256) void mlp_bwd_final_kernel(
    const float *__restrict__ partial, int n32, int nx2, const int *__restrict__ flags,
    float *__restrict__ grad) {
    bool use32 = flags == nullptr;
    if (!use32) {
        bool any = false;
        for (int k = (int)(threadIdx.x & 63); k < nx2; k += 64) any = any || flags[k] != 0;
        use32 = __any(any);
    }
    const int nchunks = ((use32 ? n32 : nx2) + kRedChunk - 1) / kRedChunk;
    const int e = blockIdx.x * 256 + threadIdx.x;
    if (e >= kGradFloats) return;
    float sum = 0.f;
    for (int k0 = 0; k0 < nchunks; k0 += 8) {  // eight loads in flight, added in order
        float v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k)
            v[k] = k0 + k < nchunks ? partial[(size_t)(k0 + k) * kGradFloats + e] : 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) sum += v[k];
    }
    grad[e] = sum;
}

// workgroups of the fp16 x 2 kernel (at most; fewer on a smaller device)
static int x2_groups(int nslots) { return nslots < 16 ? 16 * nslots : 256; }

// Workspace, in order: one float32 partial per (jet, row tile) slot; one per
// fp16 x 2 workgroup; the reduction's chunk sums; then ints: the fp16 x 2
// workgroups' flags, the block plan's start (nslots + 1) and first (one per
// workgroup).
size_t mlp_bwd_workspace(int B, int P) {
    const size_t nslots = (size_t)B * (P / kTile), gx = (size_t)x2_groups((int)nslots);
    const size_t nchunks = (std::max(nslots, gx) + kRedChunk - 1) / kRedChunk;
    return (nslots + gx + nchunks) * kGradFloats * sizeof(float) +
           (gx + nslots + 1 + gx + gx + 1) * sizeof(int);
}

hipError_t launch_mlp_bwd_f32(const float *p4, const uint8_t *mask, int B, int P,
                              const pip_pair_mlp *m, const float *dU, float *grad, void *ws,
                              hipStream_t s) {
    const int T = P / kTile;
    float *p32 = (float *)ws;
    const dim3 rg((kGradFloats + 255) / 256);
    if (B == 0) {  // no pair: the sum over no chunk writes zeros
        hipLaunchKernelGGL(mlp_bwd_final_kernel, rg, dim3(256), 0, s, p32, 0, 0,
                           (const int *)nullptr, grad);
        return hipGetLastError();
    }
    const int nslots = B * T, gx = x2_groups(nslots);
    const int nchunks = (std::max(nslots, gx) + kRedChunk - 1) / kRedChunk;
    float *px2 = p32 + (size_t)nslots * kGradFloats;
    float *chunk = px2 + (size_t)gx * kGradFloats;
    int *flags = (int *)(chunk + (size_t)nchunks * kGradFloats);
    int *start = flags + gx, *first = start + nslots + 1, *bpos = first + gx;
    // the fp16 x 2 path needs well-scaled weights and a block count within int
    const bool x2 = m->f16ok && (long long)nslots * slot_cost(16 * kTile + 9) < (1ll << 31);
    const int G = std::min(gx, cu_count());
    if (x2) {
        hipLaunchKernelGGL(mlp_bwd_plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, mask, B, P, G,
                           start, first, bpos);
        if (P <= 128)
            hipLaunchKernelGGL(mlp_bwd_x2_kernel<128>, dim3((unsigned)G), dim3(kXThreads), 0, s,
                               (const float4 *)p4, mask, B, P, (const v8h *)m->wx2,
                               (const v8h *)m->wtx2, (const float4 *)m->w32, m->wplain, m->bias,
                               dU, (const int *)start, (const int *)first, (const int *)bpos,
                               px2, flags);
        else
            hipLaunchKernelGGL(mlp_bwd_x2_kernel<256>, dim3((unsigned)G), dim3(kXThreads), 0, s,
                               (const float4 *)p4, mask, B, P, (const v8h *)m->wx2,
                               (const v8h *)m->wtx2, (const float4 *)m->w32, m->wplain, m->bias,
                               dU, (const int *)start, (const int *)first, (const int *)bpos,
                               px2, flags);
    }
    const int *fl = x2 ? flags : nullptr;
    const dim3 g32((unsigned)nslots);
    if (P <= 128)
        hipLaunchKernelGGL(mlp_bwd_kernel<128>, g32, dim3(kMbThreads), 0, s, (const float4 *)p4,
                           mask, B, P, m->wplain, m->bias, dU, p32, fl, G);
    else
        hipLaunchKernelGGL(mlp_bwd_kernel<256>, g32, dim3(kMbThreads), 0, s, (const float4 *)p4,
                           mask, B, P, m->wplain, m->bias, dU, p32, fl, G);
    hipLaunchKernelGGL(mlp_bwd_reduce_kernel, dim3(rg.x, (unsigned)nchunks), dim3(256), 0, s,
                       (const float *)p32, nslots, (const float *)px2, G, fl, chunk);
    hipLaunchKernelGGL(mlp_bwd_final_kernel, rg, dim3(256), 0, s, (const float *)chunk, nslots,
                       G, fl, grad);
    return hipGetLastError();
}

}  // namespace pip

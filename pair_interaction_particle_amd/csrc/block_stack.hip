// block_stack.hip -- L masked biased-attention layers that reuse one pair
// bias U: the attention sublayer of the ParT encoder blocks ("Architecture
// Comparison" of the ml4sci_cms_e2e26 README: 8 ParT blocks, 8 heads; the
// bias enters every block's attention as in "Fusion 3").
//
// Per layer two kernels:
//  A, one workgroup per (jet, head h): K_h = X Wk[:, h], V_h = X Wv[:, h] for
//    every real row block go to LDS, then each wave takes query blocks,
//    forms Q_h^T and runs the online-softmax attention over the real key
//    blocks with U[jet, h]; O_h goes to the workspace (B, P, C) at columns
//    16h..16h+15 (padded query rows store 0).
//  B, one workgroup per (jet, row block): X[rows] += O[rows] Wo.
// MFMA operand choice makes every product land in the layout its consumer
// wants: K^T and Q^T come out of A = W^T, B = X^T (lane l holds row l%16,
// d = 4(l/16)+r: the A/B layouts of the score MFMA), V out of A = X, B = W
// (lane l holds V[4(l/16)+r][d = l%16]: the A layout of O^T += V^T P^T).  The
// reduction over the C input columns uses the slot map c = 16t + 4(l/16) + u
// for step 4t + u, so each lane reads X with float4 loads.
#include "pip_attn.h"
#include "pip_internal.h"

namespace pip {

constexpr int kStackThreads = 256;

// Does row block rb of the jet hold a real row?
__device__ __forceinline__ bool block_real(const int *real, int rb) {
    int a = 0;
#pragma unroll
    for (int i = 0; i < kTile; ++i) a |= real[rb * kTile + i];
    return a != 0;
}

// One 16x16 MFMA product tile with a reduction over the C columns of X.
// Xrow points at this lane's row (l%16) of X, Wcol at column (l%16) of a
// (C, C) row-major weight; for input slot c = 16t + 4g + u the lane supplies
// x = X[row][c] and w = W[c][col].  w_first: D = W^T X^T, so lane l receives
// (X W)[row l%16][col 4g + r]; otherwise D = X W and lane l receives
// (X W)[row 4g + r][col l%16].
__device__ __forceinline__ v4f proj_tile(const float *__restrict__ Xrow,
                                         const float *__restrict__ Wcol, int C, bool w_first) {
    const int g = (threadIdx.x & 63) >> 4;
    v4f acc = {0.f, 0.f, 0.f, 0.f};
    for (int t = 0; t < C / 16; ++t) {
        const float4 xv = *(const float4 *)(Xrow + 16 * t + 4 * g);
        const float x[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float w = Wcol[(size_t)(16 * t + 4 * g + u) * C];
            acc = w_first ? mfma4(w, x[u], acc) : mfma4(x[u], w, acc);
        }
    }
    return acc;
}

__global__ __launch_bounds__(kStackThreads) void stack_attention_kernel(
    const float *__restrict__ X, const float *__restrict__ Wq, const float *__restrict__ Wk,
    const float *__restrict__ Wv, const float *__restrict__ U, const uint8_t *__restrict__ mask,
    int H, int P, int C, float *__restrict__ Ows) {
    __shared__ float Ks[kMaxP * 16], Vs[kMaxP * 16];
    __shared__ int realS[kMaxP];
    __shared__ int blkAny[kMaxP / kTile];
    const int jet = blockIdx.x / H, h = blockIdx.x - jet * H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, c = lane & 15;
    const int T = P / kTile;
    for (int i = tid; i < P; i += kStackThreads) realS[i] = mask[(size_t)jet * P + i] != 0;
    __syncthreads();
    if (tid < T) blkAny[tid] = block_real(realS, tid);
    __syncthreads();

    const float *Xj = X + (size_t)jet * P * C;
    // phase 1: K and V of every real row block
    for (int rb = wave; rb < T; rb += kStackThreads / 64) {
        if (!blkAny[rb]) continue;
        const float *Xrow = Xj + (size_t)(rb * kTile + c) * C;
        const v4f kt = proj_tile(Xrow, Wk + 16 * h + c, C, true);   // K[row c][4g + r]
        *(float4 *)(Ks + (rb * kTile + c) * 16 + 4 * g) = make_float4(kt[0], kt[1], kt[2], kt[3]);
        const v4f vt = proj_tile(Xrow, Wv + 16 * h + c, C, false);  // V[4g + r][d = c]
#pragma unroll
        for (int r = 0; r < 4; ++r) Vs[(rb * kTile + 4 * g + r) * 16 + c] = vt[r];
    }
    __syncthreads();

    // phase 2: attention of every query block
    const float *Uh = U + ((size_t)jet * H + h) * P * P;
    for (int qb = wave; qb < T; qb += kStackThreads / 64) {
        const int q0 = qb * kTile, q = q0 + c;
        float *orow = Ows + ((size_t)jet * P + q) * C + 16 * h + 4 * g;
        if (!blkAny[qb]) {
            *(float4 *)orow = make_float4(0.f, 0.f, 0.f, 0.f);
            continue;
        }
        const v4f qt = proj_tile(Xj + (size_t)q * C, Wq + 16 * h + c, C, true);  // Q[q][4g+r]
        float m = -INFINITY, l = 0.f;
        v4f acc = {0.f, 0.f, 0.f, 0.f};
        for (int kb = 0; kb < T; ++kb) {
            if (!blkAny[kb]) continue;
            const int k0 = kb * kTile;
            const float4 kv = *(const float4 *)(Ks + (k0 + c) * 16 + 4 * g);
            v4f s = {0.f, 0.f, 0.f, 0.f};
            s = mfma4(kv.x, qt[0], s);
            s = mfma4(kv.y, qt[1], s);
            s = mfma4(kv.z, qt[2], s);
            s = mfma4(kv.w, qt[3], s);
            const float4 u = *(const float4 *)(Uh + (size_t)q * P + k0 + 4 * g);
            const float uu[4] = {u.x, u.y, u.z, u.w};
            int kreal[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                kreal[r] = realS[k0 + 4 * g + r];
                s[r] = kreal[r] ? fmaf(s[r], kQkScale2, uu[r] * kLog2e) : -INFINITY;
            }
            const float corr = online_softmax(s, m, l);
            acc *= corr;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float vv = kreal[r] ? Vs[(k0 + 4 * g + r) * 16 + c] : 0.f;
                acc = mfma4(vv, s[r], acc);
            }
        }
        const bool rq = realS[q];
        const float inv = rq ? 1.0f / l : 0.0f;
        const v4f o = rq ? acc * inv : (v4f){0.f, 0.f, 0.f, 0.f};
        *(float4 *)orow = make_float4(o[0], o[1], o[2], o[3]);
    }
}

// X[rows] += O[rows] Wo for one (jet, row block); wave w takes output column
// tiles w, w+4, ...
__global__ __launch_bounds__(kStackThreads) void stack_out_proj_kernel(
    float *__restrict__ X, const float *__restrict__ Wo, const float *__restrict__ Ows,
    const uint8_t *__restrict__ mask, int P, int C) {
    const int T = P / kTile;
    const int jet = blockIdx.x / T, rb = blockIdx.x - jet * T;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, c = lane & 15;
    int any = 0;
    for (int i = 0; i < kTile; ++i) any |= mask[(size_t)jet * P + rb * kTile + i];
    if (!any) return;  // padded rows keep X; their O is 0 anyway
    const size_t row0 = (size_t)jet * P + rb * kTile;
    const float *Orow = Ows + (row0 + c) * C;
    for (int ct = wave; ct < C / 16; ct += kStackThreads / 64) {
        // D[row 4g + r][col 16 ct + c] = sum_k O[row][k] Wo[k][col]
        const v4f d = proj_tile(Orow, Wo + 16 * ct + c, C, false);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if (!mask[row0 + 4 * g + r]) continue;  // padded rows keep their bits
            float *x = X + (row0 + 4 * g + r) * C + 16 * ct + c;
            *x += d[r];
        }
    }
}

hipError_t launch_block_stack(float *X, const float *Wq, const float *Wk, const float *Wv,
                              const float *Wo, const float *U, const uint8_t *mask, int B,
                              int P, int C, int H, int L, float *ws, hipStream_t s) {
    const int T = P / kTile;
    for (int l = 0; l < L; ++l) {
        const size_t wo = (size_t)l * C * C;
        hipLaunchKernelGGL(stack_attention_kernel, dim3(B * H), dim3(kStackThreads), 0, s, X,
                           Wq + wo, Wk + wo, Wv + wo, U, mask, H, P, C, ws);
        hipLaunchKernelGGL(stack_out_proj_kernel, dim3(B * T), dim3(kStackThreads), 0, s, X,
                           Wo + wo, ws, mask, P, C);
    }
    return hipGetLastError();
}

}  // namespace pip

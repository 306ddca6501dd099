// attention.hip -- masked multi-head attention with an additive pair bias.
//
// "Event Classification with Masked Transformer Autoencoders"
// (ml4sci_cms_e2e26 README), "How the Kernel Fusion Works", Fusion 3:
// softmax(Q K^T / sqrt(d) + bias) V in one pass with a FlashAttention-style
// online softmax, never materialising the (B*H, P, P) score matrix.
//
// gfx950 design: one 256-thread workgroup per (jet, head); wave w owns query
// blocks w, w+4, ... of 16 queries.  For each key block of 16 keys that holds
// a real key, the scores are computed transposed, S^T = K Q^T, with MFMA so
// that lane l ends up with the 4 scores of query l%16 against keys 4(l/16)+r:
// the row max / row sum need an in-lane reduction over r plus two cross-lane
// steps (lanes l^16 and l^32), and the probabilities are already the B operand
// of O^T += V^T P^T.  The U tile is read with one 16-byte load per lane
// (query row, 4 consecutive keys).  Key blocks without a real key and query
// blocks without a real query are skipped; padded query rows store 0.
#include "pip_device.h"
#include "pip_internal.h"

namespace pip {

__device__ __forceinline__ float xmax16(float x) {
    x = fmaxf(x, __shfl_xor(x, 16));
    return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float xsum16(float x) {
    x += __shfl_xor(x, 16);
    return x + __shfl_xor(x, 32);
}

// log2(e) / sqrt(16) and log2(e): scores are kept in base-2 units.
constexpr float kLog2e = 1.4426950408889634f;

// Online-softmax update of one key block for the lane's query (l%16).  s[r]
// are base-2 scores for keys 4(l/16)+r (-inf for padded keys); returns the
// probabilities p[r] and updates m (running max), l (running sum) and the
// rescale factor of the accumulator.
__device__ __forceinline__ float online_softmax(v4f &s, float &m, float &l) {
    float bm = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    bm = xmax16(bm);
    const float mn = fmaxf(m, bm);
    const float corr = exp2f(m - mn);  // m = -inf on the first block -> 0
#pragma unroll
    for (int r = 0; r < 4; ++r) s[r] = exp2f(s[r] - mn);
    float ps = (s[0] + s[1]) + (s[2] + s[3]);
    ps = xsum16(ps);
    l = l * corr + ps;
    m = mn;
    return corr;
}

__global__ __launch_bounds__(256) void attention_f32_kernel(
    const float *__restrict__ Q, const float *__restrict__ K, const float *__restrict__ V,
    const float *__restrict__ U, const uint8_t *__restrict__ mask, int H, int P,
    float *__restrict__ O) {
    __shared__ int realS[kTile * 16];
    __shared__ int blkAny[16];
    const int bh = blockIdx.x, jet = bh / H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, c = lane & 15;
    const int T = P / kTile;
    for (int i = tid; i < P; i += 256) realS[i] = mask[(size_t)jet * P + i] != 0;
    __syncthreads();
    if (tid < T) {
        int a = 0;
        for (int i = 0; i < kTile; ++i) a |= realS[tid * kTile + i];
        blkAny[tid] = a;
    }
    __syncthreads();

    const size_t base = (size_t)bh * P;
    const float qk_scale = kLog2e * 0.25f;  // log2(e) / sqrt(16)
    for (int qb = wave; qb < T; qb += 4) {
        const int q = qb * kTile + c;
        float4 *orow = (float4 *)(O + (base + q) * 16 + 4 * g);
        if (!blkAny[qb]) {
            *orow = make_float4(0.f, 0.f, 0.f, 0.f);
            continue;
        }
        const float4 qv = *(const float4 *)(Q + (base + q) * 16 + 4 * g);
        float m = -INFINITY, l = 0.f;
        v4f acc = {0.f, 0.f, 0.f, 0.f};
        for (int kb = 0; kb < T; ++kb) {
            if (!blkAny[kb]) continue;
            const int k0 = kb * kTile;
            const float4 kv = *(const float4 *)(K + (base + k0 + c) * 16 + 4 * g);
            v4f s = {0.f, 0.f, 0.f, 0.f};
            s = mfma4(kv.x, qv.x, s);
            s = mfma4(kv.y, qv.y, s);
            s = mfma4(kv.z, qv.z, s);
            s = mfma4(kv.w, qv.w, s);
            const float4 u = *(const float4 *)(U + (base + q) * P + k0 + 4 * g);
            const float uu[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int r = 0; r < 4; ++r)
                s[r] = realS[k0 + 4 * g + r] ? fmaf(s[r], qk_scale, uu[r] * kLog2e) : -INFINITY;
            const float corr = online_softmax(s, m, l);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] *= corr;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                // select, not multiply: a NaN in a padded V row must not meet p = 0
                const float vv = realS[k0 + 4 * g + r] ? V[(base + k0 + 4 * g + r) * 16 + c] : 0.f;
                acc = mfma4(vv, s[r], acc);
            }
        }
        const float inv = realS[q] ? 1.0f / l : 0.0f;
        float4 o;
        o.x = realS[q] ? acc[0] * inv : 0.f;
        o.y = realS[q] ? acc[1] * inv : 0.f;
        o.z = realS[q] ? acc[2] * inv : 0.f;
        o.w = realS[q] ? acc[3] * inv : 0.f;
        *orow = o;
    }
}

// ------------------------------------------------------------ bf16
__device__ __forceinline__ float bf2f(uint16_t b) {
    return __builtin_bit_cast(float, (uint32_t)b << 16);
}
__device__ __forceinline__ uint16_t f2bf(float x) {
    __bf16 h = (__bf16)x;
    return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ v4f mfma16bf(v4s a, v4s b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__global__ __launch_bounds__(256) void attention_bf16_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const uint16_t *__restrict__ U,
    const uint8_t *__restrict__ mask, int H, int P, uint16_t *__restrict__ O) {
    __shared__ int realS[kTile * 16];
    __shared__ int blkAny[16];
    const int bh = blockIdx.x, jet = bh / H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, c = lane & 15;
    const int T = P / kTile;
    for (int i = tid; i < P; i += 256) realS[i] = mask[(size_t)jet * P + i] != 0;
    __syncthreads();
    if (tid < T) {
        int a = 0;
        for (int i = 0; i < kTile; ++i) a |= realS[tid * kTile + i];
        blkAny[tid] = a;
    }
    __syncthreads();

    const size_t base = (size_t)bh * P;
    const float qk_scale = kLog2e * 0.25f;
    for (int qb = wave; qb < T; qb += 4) {
        const int q = qb * kTile + c;
        uint2 *orow = (uint2 *)(O + (base + q) * 16 + 4 * g);
        if (!blkAny[qb]) {
            *orow = make_uint2(0u, 0u);
            continue;
        }
        const v4s qv = *(const v4s *)(Q + (base + q) * 16 + 4 * g);
        float m = -INFINITY, l = 0.f;
        v4f acc = {0.f, 0.f, 0.f, 0.f};
        for (int kb = 0; kb < T; ++kb) {
            if (!blkAny[kb]) continue;
            const int k0 = kb * kTile;
            const v4s kv = *(const v4s *)(K + (base + k0 + c) * 16 + 4 * g);
            v4f s = {0.f, 0.f, 0.f, 0.f};
            s = mfma16bf(kv, qv, s);
            const uint2 uw = *(const uint2 *)(U + (base + q) * P + k0 + 4 * g);
            const float uu[4] = {bf2f(uw.x & 0xffff), bf2f(uw.x >> 16), bf2f(uw.y & 0xffff),
                                 bf2f(uw.y >> 16)};
#pragma unroll
            for (int r = 0; r < 4; ++r)
                s[r] = realS[k0 + 4 * g + r] ? fmaf(s[r], qk_scale, uu[r] * kLog2e) : -INFINITY;
            const float corr = online_softmax(s, m, l);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] *= corr;
            v4s vv, pv;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                vv[r] = realS[k0 + 4 * g + r] ? (short)V[(base + k0 + 4 * g + r) * 16 + c] : 0;
                pv[r] = (short)f2bf(s[r]);
            }
            acc = mfma16bf(vv, pv, acc);
        }
        const bool rq = realS[q];
        const float inv = rq ? 1.0f / l : 0.0f;
        uint2 o;
        o.x = rq ? ((uint32_t)f2bf(acc[0] * inv) | ((uint32_t)f2bf(acc[1] * inv) << 16)) : 0u;
        o.y = rq ? ((uint32_t)f2bf(acc[2] * inv) | ((uint32_t)f2bf(acc[3] * inv) << 16)) : 0u;
        *orow = o;
    }
}

hipError_t launch_attention_f32(const float *Q, const float *K, const float *V,
                                const float *U, const uint8_t *mask, int B, int H, int P,
                                float *O, hipStream_t s) {
    hipLaunchKernelGGL(attention_f32_kernel, dim3(B * H), dim3(256), 0, s, Q, K, V, U, mask, H,
                       P, O);
    return hipGetLastError();
}

hipError_t launch_attention_bf16(const uint16_t *Q, const uint16_t *K, const uint16_t *V,
                                 const uint16_t *U, const uint8_t *mask, int B, int H, int P,
                                 uint16_t *O, hipStream_t s) {
    hipLaunchKernelGGL(attention_bf16_kernel, dim3(B * H), dim3(256), 0, s, Q, K, V, U, mask,
                       H, P, O);
    return hipGetLastError();
}

}  // namespace pip

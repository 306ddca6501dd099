// pair_embed.hip -- pair features and the fused features + pair-MLP kernels.
//
// "Event Classification with Masked Transformer Autoencoders"
// (ml4sci_cms_e2e26 README), "How the Kernel Fusion Works", Fusion 2: the
// four pair features and the whole 4-layer MLP run in one launch, hidden
// states stay on chip, and only the (B, H, P, P) bias is written.
//
// Work decomposition (gfx950): one 256-thread workgroup per (jet, 16x16 tile
// (I, J) with I >= J).  U is symmetric in (a, b) because every feature is, so
// only the lower triangle of tiles is computed and each off-diagonal tile is
// written twice (direct and transposed) from an LDS staging buffer.  Inside a
// tile the unit of work is a "pair block" of 16 pairs = the 16 columns of one
// 16x16 MFMA: off-diagonal tiles have 16 of them (one per row), diagonal
// tiles pack their 136 unique pairs into 9.  Each wave pushes its pair blocks
// through the layer chain with MFMA, the hidden activations never leaving
// registers.  Tiles that hold no real pair only write zeros.
#include "pip_device.h"
#include "pip_internal.h"

namespace pip {

// largest i with i (i + 1) / 2 <= t
__device__ __forceinline__ int tri_row(int t) {
    int i = (int)((sqrtf(8.0f * (float)t + 1.0f) - 1.0f) * 0.5f);
    while ((i + 1) * (i + 2) / 2 <= t) ++i;
    while (i * (i + 1) / 2 > t) --i;
    return i;
}

// Stage the 16 particles of block I into LDS slots 0..15 and those of block J
// into slots 16..31 (threads 0..31).  Padded slots are staged as zero vectors:
// their values never reach an output.
__device__ inline void stage_tile(PartLds &L, const float4 *__restrict__ p4,
                                  const uint8_t *__restrict__ mask, int jet, int P, int I,
                                  int J) {
    int t = threadIdx.x;
    if (t < 32) {
        int part = (t < 16) ? (I * kTile + t) : (J * kTile + t - 16);
        size_t idx = (size_t)jet * P + part;
        int real = mask[idx] != 0;
        float4 p = real ? p4[idx] : make_float4(0.f, 0.f, 0.f, 0.f);
        stage_particle(L, t, p, real);
    }
}

// ------------------------------------------------------------ features
__global__ __launch_bounds__(256) void pair_features_kernel(const float4 *__restrict__ p4,
                                                            const uint8_t *__restrict__ mask,
                                                            int P, float *__restrict__ F) {
    __shared__ PartLds L;
    const int T = P / kTile;
    const int jet = blockIdx.x / (T * T);
    const int I = (blockIdx.x / T) % T, J = blockIdx.x % T;
    stage_tile(L, p4, mask, jet, P, I, J);
    __syncthreads();
    const int i = threadIdx.x >> 4, j = threadIdx.x & 15;
    const bool real = L.real[i] && L.real[16 + j];
    for (int k = 0; k < 4; ++k) {
        float v = real ? pair_feature(L, i, 16 + j, k) : 0.0f;
        F[(((size_t)jet * 4 + k) * P + I * kTile + i) * P + J * kTile + j] = v;
    }
}

hipError_t launch_pair_features(const float *p4, const uint8_t *mask, int B, int P, float *F,
                                hipStream_t s) {
    const int T = P / kTile;
    hipLaunchKernelGGL(pair_features_kernel, dim3(B * T * T), dim3(256), 0, s,
                       (const float4 *)p4, mask, P, F);
    return hipGetLastError();
}

// ------------------------------------------------------------ MLP cores
// float32 chain: every layer on v_mfma_f32_16x16x4_f32.
struct MlpW32 {
    float w1[4], w2[64], w3[64], w4[16];
    v4f b1[4], b2[4], b3[4], b4;

    __device__ inline void load(const float *__restrict__ wp, const float *__restrict__ bias,
                                int lane) {
        const int g = lane >> 4;
#pragma unroll
        for (int c = 0; c < 4; ++c) w1[c] = wp[kW32L1 + c * 64 + lane];
#pragma unroll
        for (int o = 0; o < 64; ++o) w2[o] = wp[kW32L2 + o * 64 + lane];
#pragma unroll
        for (int o = 0; o < 64; ++o) w3[o] = wp[kW32L3 + o * 64 + lane];
#pragma unroll
        for (int o = 0; o < 16; ++o) w4[o] = wp[kW32L4 + o * 64 + lane];
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                b1[c][r] = bias[kBiasL1 + 16 * c + 4 * g + r];
                b2[c][r] = bias[kBiasL2 + 16 * c + 4 * g + r];
                b3[c][r] = bias[kBiasL3 + 16 * c + 4 * g + r];
            }
#pragma unroll
        for (int r = 0; r < 4; ++r) b4[r] = (4 * g + r < kHeads) ? bias[kBiasL4 + 4 * g + r] : 0.f;
    }
};

// One pair block: v is this lane's input feature (feature l/16 of pair l%16).
// Returns lane l's U values U[head 4(l/16) + r][pair l%16] (valid for l < 32).
__device__ __forceinline__ v4f mlp_chain_f32(const MlpW32 &W, float v) {
    v4f h[4], t[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) h[c] = mfma4(W.w1[c], v, W.b1[c]);
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) h[c][r] = gelu(h[c][r]);
#pragma unroll
    for (int co = 0; co < 4; ++co) t[co] = W.b2[co];
#pragma unroll
    for (int ci = 0; ci < 4; ++ci)
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int co = 0; co < 4; ++co)
                t[co] = mfma4(W.w2[(co * 4 + ci) * 4 + r], h[ci][r], t[co]);
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) h[c][r] = gelu(t[c][r]);
#pragma unroll
    for (int co = 0; co < 4; ++co) t[co] = W.b3[co];
#pragma unroll
    for (int ci = 0; ci < 4; ++ci)
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int co = 0; co < 4; ++co)
                t[co] = mfma4(W.w3[(co * 4 + ci) * 4 + r], h[ci][r], t[co]);
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) h[c][r] = gelu(t[c][r]);
    v4f u = W.b4;
#pragma unroll
    for (int ci = 0; ci < 4; ++ci)
#pragma unroll
        for (int r = 0; r < 4; ++r) u = mfma4(W.w4[ci * 4 + r], h[ci][r], u);
    return u;
}

// bfloat16 chain: layer 1 stays float32 (its inputs are the float32
// features), layers 2..4 take bf16 operands on v_mfma_f32_16x16x32_bf16 with
// float32 accumulation; GELU runs in float32.
struct MlpW16 {
    float w1[4];
    v8bf w2[8], w3[8], w4[2];
    v4f b1[4], b2[4], b3[4], b4;

    __device__ inline void load(const float *__restrict__ wp, const uint16_t *__restrict__ wp16,
                                const float *__restrict__ bias, int lane) {
        const int g = lane >> 4;
#pragma unroll
        for (int c = 0; c < 4; ++c) w1[c] = wp[kW32L1 + c * 64 + lane];
        const v8bf *q = (const v8bf *)wp16;
#pragma unroll
        for (int o = 0; o < 8; ++o) w2[o] = q[(kW16L2 / 8) + o * 64 + lane];
#pragma unroll
        for (int o = 0; o < 8; ++o) w3[o] = q[(kW16L3 / 8) + o * 64 + lane];
#pragma unroll
        for (int o = 0; o < 2; ++o) w4[o] = q[(kW16L4 / 8) + o * 64 + lane];
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                b1[c][r] = bias[kBiasL1 + 16 * c + 4 * g + r];
                b2[c][r] = bias[kBiasL2 + 16 * c + 4 * g + r];
                b3[c][r] = bias[kBiasL3 + 16 * c + 4 * g + r];
            }
#pragma unroll
        for (int r = 0; r < 4; ++r) b4[r] = (4 * g + r < kHeads) ? bias[kBiasL4 + 4 * g + r] : 0.f;
    }
};

__device__ __forceinline__ v8bf pack_bf16(v4f lo, v4f hi) {
    v8bf o;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        o[r] = (__bf16)lo[r];
        o[r + 4] = (__bf16)hi[r];
    }
    return o;
}

__device__ __forceinline__ v4f mfma32bf(v8bf a, v8bf b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v4f mlp_chain_bf16(const MlpW16 &W, float v) {
    v4f h[4], t[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) h[c] = mfma4(W.w1[c], v, W.b1[c]);
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) h[c][r] = gelu(h[c][r]);
    v8bf x0 = pack_bf16(h[0], h[1]), x1 = pack_bf16(h[2], h[3]);
#pragma unroll
    for (int co = 0; co < 4; ++co) {
        t[co] = mfma32bf(W.w2[co * 2 + 0], x0, W.b2[co]);
        t[co] = mfma32bf(W.w2[co * 2 + 1], x1, t[co]);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) h[c][r] = gelu(t[c][r]);
    x0 = pack_bf16(h[0], h[1]);
    x1 = pack_bf16(h[2], h[3]);
#pragma unroll
    for (int co = 0; co < 4; ++co) {
        t[co] = mfma32bf(W.w3[co * 2 + 0], x0, W.b3[co]);
        t[co] = mfma32bf(W.w3[co * 2 + 1], x1, t[co]);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) h[c][r] = gelu(t[c][r]);
    x0 = pack_bf16(h[0], h[1]);
    x1 = pack_bf16(h[2], h[3]);
    v4f u = mfma32bf(W.w4[0], x0, W.b4);
    return mfma32bf(W.w4[1], x1, u);
}

// ------------------------------------------------------------ U stores
__device__ __forceinline__ void store4(float *U, size_t off, float a, float b, float c, float d) {
    *(float4 *)(U + off) = make_float4(a, b, c, d);
}
__device__ __forceinline__ uint16_t bf16_bits(float x) {
    __bf16 h = (__bf16)x;
    return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ void store4(uint16_t *U, size_t off, float a, float b, float c,
                                       float d) {
    uint2 w;
    w.x = (uint32_t)bf16_bits(a) | ((uint32_t)bf16_bits(b) << 16);
    w.y = (uint32_t)bf16_bits(c) | ((uint32_t)bf16_bits(d) << 16);
    *(uint2 *)(U + off) = w;
}

// Write tile (I, J) of every head and, if I != J, its transpose (J, I), from
// the LDS tile us[h][i][j]; pairs with a padded end are written as 0.
template <typename OutT>
__device__ inline void write_tile(const PartLds &L, const float (*us)[16][17], OutT *U, int P,
                                  int I, int J, bool zero) {
    const int tid = threadIdx.x;
    for (int idx = tid; idx < 512; idx += 256) {
        const int h = idx >> 6, i = (idx >> 2) & 15, j0 = (idx & 3) * 4;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            v[e] = (!zero && L.real[i] && L.real[16 + j0 + e]) ? us[h][i][j0 + e] : 0.0f;
        store4(U, ((size_t)h * P + I * kTile + i) * P + J * kTile + j0, v[0], v[1], v[2], v[3]);
    }
    if (I == J) return;
    for (int idx = tid; idx < 512; idx += 256) {
        const int h = idx >> 6, j = (idx >> 2) & 15, i0 = (idx & 3) * 4;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            v[e] = (!zero && L.real[16 + j] && L.real[i0 + e]) ? us[h][i0 + e][j] : 0.0f;
        store4(U, ((size_t)h * P + J * kTile + j) * P + I * kTile + i0, v[0], v[1], v[2], v[3]);
    }
}

// ------------------------------------------------------------ pair embed
template <bool kBf16>
__global__ __launch_bounds__(256) void pair_embed_kernel(const float4 *__restrict__ p4,
                                                         const uint8_t *__restrict__ mask, int P,
                                                         int ntri,
                                                         const float *__restrict__ wp,
                                                         const uint16_t *__restrict__ wp16,
                                                         const float *__restrict__ bias,
                                                         void *__restrict__ Uout) {
    __shared__ PartLds L;
    __shared__ float us[kHeads][16][17];
    const int jet = blockIdx.x / ntri;
    const int t = blockIdx.x - jet * ntri;
    const int I = tri_row(t), J = t - I * (I + 1) / 2;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    stage_tile(L, p4, mask, jet, P, I, J);
    __syncthreads();

    int anyI = 0, anyJ = 0;
#pragma unroll
    for (int s = 0; s < 16; ++s) {
        anyI |= L.real[s];
        anyJ |= L.real[16 + s];
    }
    typedef typename std::conditional<kBf16, uint16_t, float>::type OutT;
    OutT *U = (OutT *)Uout + (size_t)jet * kHeads * P * P;
    if (!(anyI && anyJ)) {  // tile without a real pair: zeros only
        write_tile<OutT>(L, us, U, P, I, J, true);
        return;
    }

    const bool diag = (I == J);
    const int nblk = diag ? 9 : 16;
    typename std::conditional<kBf16, MlpW16, MlpW32>::type W;
    if constexpr (kBf16) W.load(wp, wp16, bias, lane);
    else W.load(wp, bias, lane);

    for (int k = wave; k < nblk; k += 4) {
        int i, j;
        bool valid = true;
        if (!diag) {
            i = k;
            j = lane & 15;
        } else {
            int p = 16 * k + (lane & 15);
            valid = p < 136;
            p = valid ? p : 0;
            i = tri_row(p);
            j = p - i * (i + 1) / 2;
        }
        const bool real = valid && L.real[i] && L.real[16 + j];
        if (__ballot(real) == 0) continue;
        float v = pair_feature(L, i, 16 + j, lane >> 4);
        v = real ? v : 0.0f;
        v4f u;
        if constexpr (kBf16) u = mlp_chain_bf16(W, v);
        else u = mlp_chain_f32(W, v);
        if (lane < 32 && valid) {
            const int h0 = (lane >> 4) * 4;
#pragma unroll
            for (int r = 0; r < 4; ++r) us[h0 + r][i][j] = u[r];
            if (diag) {
#pragma unroll
                for (int r = 0; r < 4; ++r) us[h0 + r][j][i] = u[r];
            }
        }
    }
    __syncthreads();
    write_tile<OutT>(L, us, U, P, I, J, false);
}

hipError_t launch_pair_embed_f32(const float *p4, const uint8_t *mask, int B, int P,
                                 const pip_pair_mlp *m, float *U, hipStream_t s) {
    const int T = P / kTile, ntri = T * (T + 1) / 2;
    hipLaunchKernelGGL(pair_embed_kernel<false>, dim3(B * ntri), dim3(256), 0, s,
                       (const float4 *)p4, mask, P, ntri, m->w32, m->w16, m->bias, (void *)U);
    return hipGetLastError();
}

hipError_t launch_pair_embed_bf16(const float *p4, const uint8_t *mask, int B, int P,
                                  const pip_pair_mlp *m, uint16_t *U, hipStream_t s) {
    const int T = P / kTile, ntri = T * (T + 1) / 2;
    hipLaunchKernelGGL(pair_embed_kernel<true>, dim3(B * ntri), dim3(256), 0, s,
                       (const float4 *)p4, mask, P, ntri, m->w32, m->w16, m->bias, (void *)U);
    return hipGetLastError();
}

}  // namespace pip

// pair_embed.hip -- pair features and the fused features + pair-MLP kernels.
//
// "Event Classification with Masked Transformer Autoencoders"
// (ml4sci_cms_e2e26 README), "How the Kernel Fusion Works", Fusion 2: the
// four pair features and the whole 4-layer MLP run in one launch, hidden
// states stay on chip, and only the (B, H, P, P) bias is written.
//
// Work decomposition (gfx950).  U is symmetric in (a, b) because every
// feature is, so only the lower triangle of 16x16 tiles (I >= J) is computed
// and every off-diagonal tile is written twice (direct and transposed) from
// an LDS staging buffer.  A 512-thread workgroup owns a chunk of consecutive
// tiles of one jet (triangle order t = I(I+1)/2 + J): it stages the jet's
// particle kinematics (float64) and the packed MLP weights in LDS once, then
// walks its tiles.  Inside a tile the unit of work is a pair block of 16 pairs
// = the 16 columns of one 16x16 MFMA: off-diagonal tiles have 16 (one per
// row), diagonal tiles pack their 136 unique pairs into 9.  Each of the 8
// waves pushes two pair blocks at a time through the MFMA layer chain; hidden
// activations never leave registers.  Tiles without a real pair only write
// zeros; rows of padded particles are skipped.
#include <type_traits>

#include "pip_internal.h"
#include "pip_mlp.h"

namespace pip {

// largest i with i (i + 1) / 2 <= t
__device__ __forceinline__ int tri_row(int t) {
    int i = (int)((sqrtf(8.0f * (float)t + 1.0f) - 1.0f) * 0.5f);
    while ((i + 1) * (i + 2) / 2 <= t) ++i;
    while (i * (i + 1) / 2 > t) --i;
    return i;
}

// ------------------------------------------------------------ features
// Stage block I into LDS slots 0..15 and block J into 16..31 (threads 0..31).
// Padded slots are staged as zero vectors: their values never reach an output.
__device__ inline void stage_tile(PartLds<32> &L, const float4 *__restrict__ p4,
                                  const uint8_t *__restrict__ mask, int jet, int P, int I,
                                  int J) {
    const int t = threadIdx.x;
    if (t < 32) {
        const int part = (t < 16) ? (I * kTile + t) : (J * kTile + t - 16);
        const size_t idx = (size_t)jet * P + part;
        const int real = mask[idx] != 0;
        stage_particle(L, t, real ? p4[idx] : make_float4(0.f, 0.f, 0.f, 0.f), real);
    }
}

__global__ __launch_bounds__(256) void pair_features_kernel(const float4 *__restrict__ p4,
                                                            const uint8_t *__restrict__ mask,
                                                            int P, float *__restrict__ F) {
    __shared__ PartLds<32> L;
    const int T = P / kTile;
    const int jet = blockIdx.x / (T * T);
    const int I = (blockIdx.x / T) % T, J = blockIdx.x % T;
    stage_tile(L, p4, mask, jet, P, I, J);
    __syncthreads();
    const int i = threadIdx.x >> 4, j = threadIdx.x & 15;
    const bool real = L.real[i] && L.real[16 + j];
    for (int k = 0; k < 4; ++k) {
        const float v = real ? pair_feature(L, i, 16 + j, k) : 0.0f;
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

// ------------------------------------------------------------ U stores
__device__ __forceinline__ void store4(float *U, size_t off, const float (&v)[4]) {
    *(float4 *)(U + off) = make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint32_t bf16_pair(float a, float b) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)a) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)b) << 16);
}
__device__ __forceinline__ void store4(uint16_t *U, size_t off, const float (&v)[4]) {
    *(uint2 *)(U + off) = make_uint2(bf16_pair(v[0], v[1]), bf16_pair(v[2], v[3]));
}

constexpr int kEmbedThreads = 512;
constexpr int kEmbedWaves = kEmbedThreads / 64;

// Write tile (I, J) of every head and, if I != J, its transpose (J, I), from
// the LDS tile us[h][i][j]; pairs with a padded end are written as 0 (select).
template <typename OutT, class PL>
__device__ inline void write_tile(const PL &L, const float (*us)[16][17], OutT *U, int P, int I,
                                  int J, bool zero) {
    const int tid = threadIdx.x;
    const int r0 = I * kTile, c0 = J * kTile;
    {
        const int h = tid >> 6, i = (tid >> 2) & 15, j0 = (tid & 3) * 4;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            v[e] = (!zero && L.real[r0 + i] && L.real[c0 + j0 + e]) ? us[h][i][j0 + e] : 0.0f;
        store4(U, ((size_t)h * P + r0 + i) * P + c0 + j0, v);
    }
    if (I == J) return;
    {
        const int h = tid >> 6, j = (tid >> 2) & 15, i0 = (tid & 3) * 4;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            v[e] = (!zero && L.real[c0 + j] && L.real[r0 + i0 + e]) ? us[h][i0 + e][j] : 0.0f;
        store4(U, ((size_t)h * P + c0 + j) * P + r0 + i0, v);
    }
}

// Pair (i, j) (tile-local) that lane `lane` of pair block k computes.
__device__ __forceinline__ bool block_pair(bool diag, int k, int nblk, int lane, int &i, int &j) {
    if (k >= nblk) {
        i = j = 0;
        return false;
    }
    if (!diag) {
        i = k;
        j = lane & 15;
        return true;
    }
    int p = 16 * k + (lane & 15);
    const bool valid = p < 136;
    p = valid ? p : 0;
    i = tri_row(p);
    j = p - i * (i + 1) / 2;
    return valid;
}

template <bool kBf16>
__global__ __launch_bounds__(kEmbedThreads) __attribute__((amdgpu_waves_per_eu(4)))
void pair_embed_kernel(const float4 *__restrict__ p4, const uint8_t *__restrict__ mask, int P,
                       int ntri, int nchunk, int G, const float4 *__restrict__ w32,
                       const v8bf *__restrict__ w16, const float *__restrict__ bias,
                       void *__restrict__ Uout) {
    constexpr int kW4 = kBf16 ? 64 : kW32Groups * 64;  // float4 operand groups in LDS
    __shared__ float4 wl[kW4];
    __shared__ v8bf wl16[kBf16 ? kW16Ops * 64 : 1];
    __shared__ float bl[kBiasFloats];
    __shared__ PartLds<kMaxP> L;
    __shared__ float us[kHeads][16][17];
    __shared__ int blkAny[kMaxP / kTile];

    const int jet = blockIdx.x / nchunk;
    const int t0 = (blockIdx.x - jet * nchunk) * G;
    const int t1 = min(t0 + G, ntri);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    for (int s = tid; s < P; s += kEmbedThreads) {
        const size_t idx = (size_t)jet * P + s;
        const int real = mask[idx] != 0;
        stage_particle(L, s, real ? p4[idx] : make_float4(0.f, 0.f, 0.f, 0.f), real);
    }
    stage_weights<kEmbedThreads>(wl, bl, w32, bias, kW4);
    if constexpr (kBf16)
        for (int i = tid; i < kW16Ops * 64; i += kEmbedThreads) wl16[i] = w16[i];
    __syncthreads();
    if (tid < P / kTile) {
        int a = 0;
        for (int i = 0; i < kTile; ++i) a |= L.real[tid * kTile + i];
        blkAny[tid] = a;
    }
    __syncthreads();

    typedef typename std::conditional<kBf16, uint16_t, float>::type OutT;
    OutT *U = (OutT *)Uout + (size_t)jet * kHeads * P * P;
    for (int t = t0; t < t1; ++t) {
        const int I = tri_row(t), J = t - I * (I + 1) / 2;
        if (!(blkAny[I] && blkAny[J])) {  // no real pair: zeros only
            write_tile<OutT>(L, us, U, P, I, J, true);
            continue;
        }
        const bool diag = (I == J);
        const int nblk = diag ? 9 : 16;
        const int r0 = I * kTile, c0 = J * kTile;
        int iA, jA, iB, jB;
        const bool vA = block_pair(diag, 2 * wave, nblk, lane, iA, jA);
        const bool vB = block_pair(diag, 2 * wave + 1, nblk, lane, iB, jB);
        const bool realA = vA && L.real[r0 + iA] && L.real[c0 + jA];
        const bool realB = vB && L.real[r0 + iB] && L.real[c0 + jB];
        if (__ballot(realA || realB) != 0) {
            const int k = lane >> 4;
            const float fA = realA ? pair_feature(L, r0 + iA, c0 + jA, k) : 0.0f;
            const float fB = realB ? pair_feature(L, r0 + iB, c0 + jB, k) : 0.0f;
            v4f uA, uB;
            if constexpr (kBf16) mlp2_bf16(wl, wl16, bl, fA, fB, uA, uB);
            else mlp2_f32(wl, bl, fA, fB, uA, uB);
            if (lane < 32) {
                const int h0 = (lane >> 4) * 4;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if (vA) {
                        us[h0 + r][iA][jA] = uA[r];
                        if (diag) us[h0 + r][jA][iA] = uA[r];
                    }
                    if (vB) {
                        us[h0 + r][iB][jB] = uB[r];
                        if (diag) us[h0 + r][jB][iB] = uB[r];
                    }
                }
            }
        }
        __syncthreads();
        write_tile<OutT>(L, us, U, P, I, J, false);
        __syncthreads();
    }
}

// Tiles per workgroup: enough workgroups to fill 256 CUs twice over, few
// enough that staging the jet and the weights is amortised.
static int chunk_tiles(int B, int ntri) {
    int G = 4;
    while (G > 1 && (long)B * ((ntri + G - 1) / G) < 2048) --G;
    return G;
}

template <bool kBf16>
static hipError_t launch_embed(const float *p4, const uint8_t *mask, int B, int P,
                               const pip_pair_mlp *m, void *U, hipStream_t s) {
    const int T = P / kTile, ntri = T * (T + 1) / 2;
    const int G = chunk_tiles(B, ntri), nchunk = (ntri + G - 1) / G;
    hipLaunchKernelGGL(pair_embed_kernel<kBf16>, dim3(B * nchunk), dim3(kEmbedThreads), 0, s,
                       (const float4 *)p4, mask, P, ntri, nchunk, G, (const float4 *)m->w32,
                       (const v8bf *)m->w16, m->bias, U);
    return hipGetLastError();
}

hipError_t launch_pair_embed_f32(const float *p4, const uint8_t *mask, int B, int P,
                                 const pip_pair_mlp *m, float *U, hipStream_t s) {
    return launch_embed<false>(p4, mask, B, P, m, U, s);
}

hipError_t launch_pair_embed_bf16(const float *p4, const uint8_t *mask, int B, int P,
                                  const pip_pair_mlp *m, uint16_t *U, hipStream_t s) {
    return launch_embed<true>(p4, mask, B, P, m, U, s);
}

}  // namespace pip

// attention_bwd.hip -- gradients of the masked biased attention, float32.
//
// "Event Classification with Masked Transformer Autoencoders"
// (ml4sci_cms_e2e26 README), "How the Kernel Fusion Works", Fusion 3: the
// attention with an additive bias has a forward and a backward kernel.  For
// a loss with dL/dO = dO, per head and real query a (real keys c only):
//   p = softmax_c(s),  s_c = scale q_a . k_c + U[a, c],  O_a = sum_c p_c v_c
//   dS_c = p_c (dO_a . v_c - dO_a . O_a),   dU[a, c] = dS_c
//   dQ_a = scale sum_c dS_c k_c,  dK_c = scale sum_a dS_c q_a,  dV_c = sum_a p_c dO_a.
// Everything that involves a padded slot is exactly 0.
//
// One 512-thread workgroup per (jet, head).  K and V are staged in LDS
// (float32, padded rows 0).  Each wave owns
// query blocks of 16 queries and recomputes the forward of its rows from
// the U strip: scores S^T = K Q^T (lane l: query l%16 against keys
// 4(l/16)+r), an exact two-pass softmax, O^T = V^T P^T and D = dO . O; then
// per key block dP^T = V dO^T, dS, the dU strip (one 16-byte store per lane
// and block, the forward's U read layout), dQ^T += K^T dS^T in registers, and
// P and dS transposed through a wave-private LDS tile into the operand layout
// of dV = P^T dO and dK = dS^T Q, whose 16x16 tiles stay in registers for
// two key blocks at a time.  The waves then merge their tiles into the LDS
// accumulators in 8 barrier-separated phases (wave w adds key block
// (j + w) mod 8 in phase j when it holds that block's tile): plain
// read-add-write, no atomics (LDS float atomics cost several cycles per
// lane here), and a fixed order of additions, so dK and dV are the same bit
// for bit on every run.  All products are float32 MFMA
// (v_mfma_f32_16x16x4_f32), so the gradients are float32 results of the
// same definition.
#include "pip_attn.h"
#include "pip_internal.h"

namespace pip {

constexpr int kBwdWaves = 8;

// x where keep, else +0 (component selects: a select between two float4
// objects is lowered through a stack copy)
__device__ __forceinline__ float4 keep4(bool keep, float4 x) {
    return make_float4(keep ? x.x : 0.f, keep ? x.y : 0.f, keep ? x.z : 0.f, keep ? x.w : 0.f);
}

constexpr int kBwdThreads = 64 * kBwdWaves;
// key blocks whose dK / dV tiles a wave holds between two merges (2: 16
// registers, so that the P <= 128 kernel fits in 128 VGPRs without a spill
// and two workgroups share a CU; 4 spilled 32 bytes, 8 held one per CU)
constexpr int kMg = 2;
static_assert(kBwdWaves == 8 && kMg <= 8, "merge phases map 8 waves onto key blocks mod 8");

template <int kT>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(kT <= 8 ? 4 : 2))) void attention_bwd_kernel(
    const float *__restrict__ Q, const float *__restrict__ K, const float *__restrict__ V,
    const float *__restrict__ U, const uint8_t *__restrict__ mask,
    const float *__restrict__ dO, int B, int H, int P, float scale, float *__restrict__ dQ,
    float *__restrict__ dK, float *__restrict__ dV, float *__restrict__ dU) {
    constexpr int kP = kT * 16;
    __shared__ float Ks[kP][16];
    __shared__ float Vs[kP][16];
    __shared__ float dKs[kP][16];
    __shared__ float dVs[kP][16];
    __shared__ float Tp[kBwdWaves][16][17];   // P tile, [query][key]
    __shared__ float Tds[kBwdWaves][16][17];  // dS tile, [query][key]
    __shared__ uint8_t rs[kP];                // real slots

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, c = lane & 15;
    // workgroup i runs on XCD i % 8; XCD x takes the H workgroups of jets x,
    // x + 8, ... (the grid is rounded up to 8 jets), so a jet's mask row is
    // fetched from HBM once and hit in that XCD's L2 by its other heads
    const int xcd = blockIdx.x & 7, t8 = blockIdx.x >> 3;
    const int jet = xcd + 8 * (t8 / H), bh = jet * H + t8 % H;
    if (jet >= B) return;  // uniform: a slot of the rounding
    const int T = P / kTile;
    const size_t base = (size_t)bh * P;
    const float *Qh = Q + base * 16, *Kh = K + base * 16, *Vh = V + base * 16;
    const float *dOh = dO + base * 16;
    const float *Ub = U + base * P;
    float *dUb = dU + base * P;

    // ---- K, V, the mask into LDS (one pass: each thread reads its row's
    // mask byte with its K and V pieces); accumulators to 0
    for (int i = tid; i < P * 4; i += kBwdThreads) {
        const int k = i >> 2, d0 = (i & 3) * 4;
        const bool rk = mask[(size_t)jet * P + k] != 0;
        const float4 kv = *(const float4 *)(Kh + (size_t)k * 16 + d0);
        const float4 vv = *(const float4 *)(Vh + (size_t)k * 16 + d0);
        const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
        if (d0 == 0) rs[k] = rk;
        *(float4 *)&Ks[k][d0] = keep4(rk, kv);
        *(float4 *)&Vs[k][d0] = keep4(rk, vv);
        *(float4 *)&dKs[k][d0] = z;
        *(float4 *)&dVs[k][d0] = z;
    }
    __syncthreads();

    // Rounds of up to 8 query blocks, one per wave; every wave runs every
    // round (the dK / dV merge below has barriers).
    for (int q8 = 0; q8 < T; q8 += kBwdWaves) {
        const int qb = q8 + wave, q0 = qb * kTile;
        bool act = qb < T;
        const bool rq = act && rs[q0 + c];
        if (act) {
            bool anyq = false;
            for (int i = 0; i < kTile; ++i) anyq |= rs[q0 + i] != 0;
            if (!anyq) {
                // no real query: zero dU strip, dQ rows
                for (int kb = 0; kb < T; ++kb)
                    *(float4 *)(dUb + (size_t)(q0 + c) * P + kb * kTile + 4 * g) =
                        make_float4(0.f, 0.f, 0.f, 0.f);
                *(float4 *)(dQ + (base + q0 + c) * 16 + 4 * g) = make_float4(0.f, 0.f, 0.f, 0.f);
                act = false;
            }
        }
        // operands of this query block: Q[q0+c][4s+g] and dO[q0+c][4s+g]
        // (B operands of the K = 4 slices), Q[q0+4s+g][c] and dO[q0+4s+g][c]
        // (B operands of dK and dV), dO[q0+c][4g..] for D; padded queries 0
        float qB[4], gB[4], qT[4], gT[4];
        float s[kT][4];
        float Dq = 0.f;
        if (act) {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const float a = Qh[(size_t)(q0 + c) * 16 + 4 * t + g];
                const float b = dOh[(size_t)(q0 + c) * 16 + 4 * t + g];
                qB[t] = rq ? a : 0.f;
                gB[t] = rq ? b : 0.f;
                const int qr = q0 + 4 * t + g;
                const bool rr = rs[qr];
                const float a2 = Qh[(size_t)qr * 16 + c];
                const float b2 = dOh[(size_t)qr * 16 + c];
                qT[t] = rr ? a2 : 0.f;
                gT[t] = rr ? b2 : 0.f;
            }
            const float4 gr4 = *(const float4 *)(dOh + (size_t)(q0 + c) * 16 + 4 * g);
            // ---- pass 1: scores and the row max.  The whole U strip is
            // loaded first, every load issued before any is waited for (key
            // blocks past T re-read block 0, unused), into the registers the
            // scores take.
#pragma unroll
            for (int kb = 0; kb < kT; ++kb) {
                const int col = (kb < T ? kb * kTile : 0) + 4 * g;
                const float4 uv = *(const float4 *)(Ub + (size_t)(q0 + c) * P + col);
                s[kb][0] = uv.x, s[kb][1] = uv.y, s[kb][2] = uv.z, s[kb][3] = uv.w;
            }
            float m = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < kT; ++kb) {
                if (kb >= T) continue;
                v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int t = 0; t < 4; ++t) acc = mfma4(Ks[kb * kTile + c][4 * t + g], qB[t], acc);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const bool rk = rs[kb * kTile + 4 * g + r];
                    s[kb][r] = rk ? fmaf(acc[r], scale, s[kb][r]) : -INFINITY;
                    m = fmaxf(m, s[kb][r]);
                }
            }
            m = xmax16(m);
            // ---- probabilities (0 for padded queries and keys)
            float l = 0.f;
#pragma unroll
            for (int kb = 0; kb < kT; ++kb) {
                if (kb >= T) continue;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float e = __expf(s[kb][r] - m);
                    s[kb][r] = e;
                    l += e;
                }
            }
            l = xsum16(l);
            const float il = 1.0f / l;
#pragma unroll
            for (int kb = 0; kb < kT; ++kb) {
                if (kb >= T) continue;
#pragma unroll
                for (int r = 0; r < 4; ++r) s[kb][r] = rq ? s[kb][r] * il : 0.f;
            }
            // ---- pass 2: O^T = V^T P^T, then D = dO . O per query
            v4f o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < kT; ++kb) {
                if (kb >= T) continue;
#pragma unroll
                for (int r = 0; r < 4; ++r) o = mfma4(Vs[kb * kTile + 4 * g + r][c], s[kb][r], o);
            }
            // lane (g, c) holds O[query c][4g + r]
            Dq = xsum16(o[0] * gr4.x + o[1] * gr4.y + o[2] * gr4.z + o[3] * gr4.w);
        }
        // ---- pass 3, kMg key blocks at a time: dP, dS, dU, dQ, and this
        // query block's dK / dV tiles, kept in registers, then merged into
        // LDS without atomics: in merge phase j (of 8) wave w adds its tile
        // of key block (j + w) mod 8 when that is below kMg, so no two waves
        // touch one tile in a phase and each wave visits each tile once.
        v4f dq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int h0 = 0; h0 < kT; h0 += kMg) {
            v4f avs[kMg], aks[kMg];
#pragma unroll
            for (int kl = 0; kl < kMg; ++kl) {
                const int kb = h0 + kl, k0 = kb * kTile;
                avs[kl] = aks[kl] = (v4f){0.f, 0.f, 0.f, 0.f};
                if (!act || kb >= T) continue;
                v4f dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int t = 0; t < 4; ++t) dp = mfma4(Vs[k0 + c][4 * t + g], gB[t], dp);
                // (a select, not the product: a padded pair is +0.0 bit for bit)
                float ds[4];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    ds[r] = rq && rs[k0 + 4 * g + r] ? s[kb][r] * (dp[r] - Dq) : 0.f;
                *(float4 *)(dUb + (size_t)(q0 + c) * P + k0 + 4 * g) =
                    make_float4(ds[0], ds[1], ds[2], ds[3]);
#pragma unroll
                for (int r = 0; r < 4; ++r) dq = mfma4(Ks[k0 + 4 * g + r][c], ds[r], dq);
                // P and dS of the tile, transposed through LDS: [query c][key 4g+r]
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    Tp[wave][c][4 * g + r] = s[kb][r];
                    Tds[wave][c][4 * g + r] = ds[r];
                }
                __builtin_amdgcn_wave_barrier();
                // dV[key c'][d] += sum_q P[q][key] dO[q][d]: lane (g, c) supplies
                // A = P[q0+4t+g][k0+c], B = dO[q0+4t+g][c]; D row = key 4g+r
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    avs[kl] = mfma4(Tp[wave][4 * t + g][c], gT[t], avs[kl]);
                    aks[kl] = mfma4(Tds[wave][4 * t + g][c], qT[t], aks[kl]);
                }
                __builtin_amdgcn_wave_barrier();
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int kl_w = (j + wave) & 7;
#pragma unroll
                for (int kl = 0; kl < kMg; ++kl) {
                    const int kb = h0 + kl, k0 = kb * kTile;
                    if (kl != kl_w || !act || kb >= T) continue;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        dVs[k0 + 4 * g + r][c] += avs[kl][r];
                        dKs[k0 + 4 * g + r][c] += aks[kl][r];
                    }
                }
                __syncthreads();
            }
        }
        if (act)
            *(float4 *)(dQ + (base + q0 + c) * 16 + 4 * g) =
                keep4(rq, make_float4(dq[0] * scale, dq[1] * scale, dq[2] * scale, dq[3] * scale));
    }
    __syncthreads();
    for (int i = tid; i < P * 4; i += kBwdThreads) {
        const int k = i >> 2, d0 = (i & 3) * 4;
        const bool rk = rs[k];
        const float4 a = *(const float4 *)&dKs[k][d0], b = *(const float4 *)&dVs[k][d0];
        *(float4 *)(dK + (base + k) * 16 + d0) =
            keep4(rk, make_float4(a.x * scale, a.y * scale, a.z * scale, a.w * scale));
        *(float4 *)(dV + (base + k) * 16 + d0) = keep4(rk, b);
    }
}

hipError_t launch_attention_bwd_f32(const float *Q, const float *K, const float *V,
                                    const float *U, const uint8_t *mask, const float *dO, int B,
                                    int H, int P, float scale, float *dQ, float *dK, float *dV,
                                    float *dU, hipStream_t s) {
    const dim3 grid((unsigned)(attention_jet_slots(B) * H));
    if (P <= 128)
        hipLaunchKernelGGL(attention_bwd_kernel<8>, grid, dim3(kBwdThreads), 0, s, Q, K, V, U,
                           mask, dO, B, H, P, scale, dQ, dK, dV, dU);
    else
        hipLaunchKernelGGL(attention_bwd_kernel<16>, grid, dim3(kBwdThreads), 0, s, Q, K, V, U,
                           mask, dO, B, H, P, scale, dQ, dK, dV, dU);
    return hipGetLastError();
}

}  // namespace pip

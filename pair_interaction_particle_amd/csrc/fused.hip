// fused.hip -- pair embedding and biased attention in one kernel: U only ever
// lives on chip ("Fusion 2" and "Fusion 3" of the ml4sci_cms_e2e26 README,
// "How the Kernel Fusion Works", composed).
//
// Jet kernel (P <= 128).  One 1024-thread workgroup per jet walks the lower
// triangle of 16x16 tiles in rounds.  In each round the 16 waves push the
// tile's pair blocks (one each) through the MFMA MLP chain into an LDS tile
// of U (8 heads); then the two waves of head h apply head h of that tile:
// wave h to query block I against key block J, wave h + 8 (transposed) to
// query block J against key block I.  So every unique pair goes through the
// MLP once, as in pair_embed.  The online-softmax state (O, running max,
// running sum) of every (head, query block) is kept in LDS; within a round
// no two waves update the same state, and the round's barrier orders the
// updates of consecutive rounds (the U tile is double buffered).  One pair
// block per wave keeps the kernel within 128 registers, so 16 waves (4 per
// SIMD) share a CU; with two blocks per wave (8 waves, 238 registers) the
// same kernel ran at 2 waves per SIMD.  Jets are taken largest first: every workgroup ranks the jets
// by real multiplicity (from the mask) and takes the one whose rank is its
// block index, so the hardware dispatcher schedules longest-job-first.
//
// Row kernel (any P <= 256).  One 512-thread workgroup per (jet, query block
// I) computes the U tiles (I, J) for every key block J and consumes them at
// once; each of its 8 waves computes two rows of every tile and owns one
// head.  It recomputes the MLP for the mirrored
// pairs and is used where the jet kernel's LDS state does not fit (P > 128)
// and for batches of at most half as many jets as CUs.
#include <type_traits>

#include "pip_attn.h"
#include "pip_internal.h"
#include "pip_mlp.h"

namespace pip {

__device__ __forceinline__ int tri_row_f(int t) {
    int i = (int)((sqrtf(8.0f * (float)t + 1.0f) - 1.0f) * 0.5f);
    while ((i + 1) * (i + 2) / 2 <= t) ++i;
    while (i * (i + 1) / 2 > t) --i;
    return i;
}

__device__ __forceinline__ bool block_pair_f(bool diag, int k, int nblk, int lane, int &i,
                                             int &j) {
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
    i = tri_row_f(p);
    j = p - i * (i + 1) / 2;
    return valid;
}

// number of nonzero bytes in a 32-bit word
__device__ __forceinline__ int nz_bytes(uint32_t w) {
    uint32_t t = w | (w >> 4);
    t |= t >> 2;
    t |= t >> 1;
    return __popc(t & 0x01010101u);
}

// Element type of Q/K/V/O.
template <bool kBf16>
using QkvT = typename std::conditional<kBf16, uint16_t, float>::type;

// The Q, K and V values one attention unit (query block q0 against key block
// k0) needs in this lane, loaded ahead of the round's MLP so that their L2
// latency overlaps it.  Every load is unconditional (rows < P); padded keys
// are selected to 0 only when used.
template <bool kBf16>
struct UnitIn {
    using Q4 = typename std::conditional<kBf16, v4s, float4>::type;
    Q4 q, k;
    QkvT<kBf16> v[4];

    __device__ __forceinline__ void load(const QkvT<kBf16> *__restrict__ Qh,
                                         const QkvT<kBf16> *__restrict__ Kh,
                                         const QkvT<kBf16> *__restrict__ Vh, int q0, int k0) {
        const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
        q = *(const Q4 *)(Qh + (size_t)(q0 + c) * 16 + 4 * g);
        k = *(const Q4 *)(Kh + (size_t)(k0 + c) * 16 + 4 * g);
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = Vh[(size_t)(k0 + 4 * g + r) * 16 + c];
    }
    // S^T tile (keys x queries): lane l gets the scores of query q0 + l%16
    // against keys k0 + 4(l/16) + r; the reduction over d pairs lane group g,
    // step s with d = 4g + s
    __device__ __forceinline__ v4f scores() const {
        if constexpr (kBf16) {
            return mfma16bf(k, q, (v4f){0.f, 0.f, 0.f, 0.f});
        } else {
            v4f s = {0.f, 0.f, 0.f, 0.f};
            s = mfma4(k.x, q.x, s);
            s = mfma4(k.y, q.y, s);
            s = mfma4(k.z, q.z, s);
            return mfma4(k.w, q.w, s);
        }
    }
    // acc (O^T: lane l holds O[q0 + l%16][4(l/16) + r]) += V^T P^T for key
    // block k0, p[r] the probability of key k0 + 4(l/16) + r; V of padded keys
    // is selected to 0 (a NaN there must not meet p = 0 inside the MFMA)
    __device__ __forceinline__ v4f pv(const v4f &p, const int (&kreal)[4], v4f acc) const {
        if constexpr (kBf16) {
            v4s vv, pp;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                vv[r] = kreal[r] ? (short)v[r] : (short)0;
                pp[r] = (short)f2bf(p[r]);
            }
            return mfma16bf(vv, pp, acc);
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) acc = mfma4(kreal[r] ? v[r] : 0.f, p[r], acc);
            return acc;
        }
    }
};

template <bool kBf16>
__device__ __forceinline__ void store_o(QkvT<kBf16> *Orow, const v4f &o) {
    if constexpr (kBf16)
        *(uint2 *)Orow = make_uint2((uint32_t)f2bf(o[0]) | ((uint32_t)f2bf(o[1]) << 16),
                                    (uint32_t)f2bf(o[2]) | ((uint32_t)f2bf(o[3]) << 16));
    else *(float4 *)Orow = make_float4(o[0], o[1], o[2], o[3]);
}

// Two pair blocks through the chain of mode kMode; a non-finite fp16 x 2
// result (an activation beyond fp16) is recomputed with the exact chain.
template <int kMode>
__device__ __forceinline__ void mlp_pair_blocks(const MlpLds<kMode> &M,
                                                const float4 *__restrict__ w32, float fA,
                                                float fB, v4f &uA, v4f &uB) {
    if (!M.run(fA, fB, uA, uB)) M.run_exact(w32, fA, fB, uA, uB);
}

// ------------------------------------------------------------ jet kernel
constexpr int kJetThreads = 1024;
constexpr int kJetMaxP = 128;
constexpr int kJetMaxT = kJetMaxP / kTile;
constexpr int kSortMaxB = 2048;

template <int kMode, bool kBf16 = (kMode == kMlpBf16)>
__global__ __launch_bounds__(kJetThreads) void embed_attention_jet_kernel(
    const float4 *__restrict__ p4, const uint8_t *__restrict__ mask, int B, int P, int sort,
    const float4 *__restrict__ w32, const v8bf *__restrict__ w16, const v8h *__restrict__ wx2,
    const float *__restrict__ bias, const QkvT<kBf16> *__restrict__ Q,
    const QkvT<kBf16> *__restrict__ K, const QkvT<kBf16> *__restrict__ V, float qk2,
    QkvT<kBf16> *__restrict__ O) {
    MlpLds<kMode> M;
    __shared__ PartLds<kJetMaxP> L;
    __shared__ float us[2][kHeads][16][17];
    __shared__ float4 Ost[kHeads][kJetMaxT][64];  // O^T accumulators, lane layout
    __shared__ float mst[kHeads][kJetMaxT][16], lst[kHeads][kJetMaxT][16];
    __shared__ int blkAny[kJetMaxT];
    __shared__ uint16_t nj[kSortMaxB];
    __shared__ int hist[kJetMaxP + 2];
    __shared__ int scanbuf[kJetThreads];
    __shared__ int jetSel;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, c = lane & 15;
    const int T = P / kTile;

    // ---- which jet: rank blockIdx.x in the order (n descending, index ascending)
    if (sort) {
        for (int i = tid; i <= P + 1; i += kJetThreads) hist[i] = 0;
        __syncthreads();
        for (int b = tid; b < B; b += kJetThreads) {
            // every load of the row issued before the first is used
            // (addresses clamped into the row; blocks past P / 16 not counted)
            const uint4 *row = (const uint4 *)(mask + (size_t)b * P);
            uint4 v[kJetMaxT];
#pragma unroll
            for (int w = 0; w < kJetMaxT; ++w) v[w] = row[min(w, P / 16 - 1)];
            int n = 0;
#pragma unroll
            for (int w = 0; w < kJetMaxT; ++w)
                n += w < P / 16
                         ? nz_bytes(v[w].x) + nz_bytes(v[w].y) + nz_bytes(v[w].z) + nz_bytes(v[w].w)
                         : 0;
            nj[b] = (uint16_t)n;
            atomicAdd(&hist[n], 1);
        }
        __syncthreads();
        if (tid == 0) {
            // bin of rank r: bins in descending n; find n* and the rank within it
            int r = blockIdx.x, n = P;
            while (r >= hist[n]) {
                r -= hist[n];
                --n;
            }
            hist[P + 1] = n;  // n*
            scanbuf[0] = r;   // k: position among the jets with n == n*
        }
        __syncthreads();
        const int nstar = hist[P + 1], k = scanbuf[0];
        // k-th jet (index order) with n == nstar: contiguous ranges per thread
        const int per = (B + kJetThreads - 1) / kJetThreads;
        const int b0 = tid * per, b1 = min(b0 + per, B);
        int cnt = 0;
        for (int b = b0; b < b1; ++b) cnt += nj[b] == nstar;
        __syncthreads();
        scanbuf[tid] = cnt;
        __syncthreads();
        for (int off = 1; off < kJetThreads; off <<= 1) {  // inclusive scan
            const int v = (tid >= off) ? scanbuf[tid - off] : 0;
            __syncthreads();
            scanbuf[tid] += v;
            __syncthreads();
        }
        const int excl = scanbuf[tid] - cnt;
        if (k >= excl && k < excl + cnt) {
            int seen = excl;
            for (int b = b0; b < b1; ++b)
                if (nj[b] == nstar) {
                    if (seen == k) jetSel = b;
                    ++seen;
                }
        }
        __syncthreads();
    } else if (tid == 0) {
        jetSel = blockIdx.x;
    }
    if (!sort) __syncthreads();
    const int jet = jetSel;

    // ---- stage particles, weights, state
    for (int s = tid; s < P; s += kJetThreads) {
        const size_t idx = (size_t)jet * P + s;
        const float4 pv = p4[idx];  // both loads issued before either is used
        const uint8_t mb = mask[idx];
        __asm__ volatile("" ::: "memory");
        const int real = mb != 0;
        stage_particle(L, s, real ? pv : make_float4(0.f, 0.f, 0.f, 0.f), real);
    }
    M.template stage<kJetThreads>(w32, w16, wx2, bias);
    for (int i = tid; i < kHeads * T * 64; i += kJetThreads)
        (&Ost[0][0][0])[(i / (T * 64)) * kJetMaxT * 64 + i % (T * 64)] =
            make_float4(0.f, 0.f, 0.f, 0.f);
    for (int i = tid; i < kHeads * kJetMaxT * 16; i += kJetThreads) {
        (&mst[0][0][0])[i] = -INFINITY;
        (&lst[0][0][0])[i] = 0.0f;
    }
    __syncthreads();
    if (tid < T) {
        int a = 0;
        for (int i = 0; i < kTile; ++i) a |= L.real[tid * kTile + i];
        blkAny[tid] = a;
    }
    __syncthreads();

    // this wave's head; the two waves of a head take the two attention units
    // of a round (half 0: query block I, half 1: query block J)
    static_assert(kJetThreads == 64 * 2 * kHeads, "two waves per head");
    const int h = wave & 7, half = wave >> 3;
    const size_t hb = ((size_t)jet * kHeads + h) * P;
    const QkvT<kBf16> *Qh = Q + hb * 16, *Kh = K + hb * 16, *Vh = V + hb * 16;

    // one attention unit: query block qb against key block kb of head h, U
    // element (query q, key k) = Ut[q][k] (or Ut[k][q] when transposed)
    auto unit = [&](const float (*Ut)[17], bool transposed, int qb, int kb,
                    const UnitIn<kBf16> &in) {
        const int k0 = kb * kTile;
        v4f s = in.scores();
        int kreal[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            kreal[r] = L.real[k0 + 4 * g + r];
            const float u = transposed ? Ut[4 * g + r][c] : Ut[c][4 * g + r];
            s[r] = kreal[r] ? fmaf(s[r], qk2, u * kLog2e) : -INFINITY;
        }
        float m = mst[h][qb][c], l = lst[h][qb][c];
        const float corr = online_softmax(s, m, l);
        const float4 a4 = Ost[h][qb][lane];
        v4f acc = {a4.x * corr, a4.y * corr, a4.z * corr, a4.w * corr};
        acc = in.pv(s, kreal, acc);
        Ost[h][qb][lane] = make_float4(acc[0], acc[1], acc[2], acc[3]);
        if (g == 0) {
            mst[h][qb][c] = m;
            lst[h][qb][c] = l;
        }
    };

    const int ntri = T * (T + 1) / 2;
    int round = 0;
    for (int t = 0; t < ntri; ++t) {
        const int I = tri_row_f(t), J = t - I * (I + 1) / 2;
        if (!(blkAny[I] && blkAny[J])) continue;
        const int buf = round & 1;
        ++round;
        const bool diag = (I == J);
        const int nblk = diag ? 9 : 16;
        const int r0 = I * kTile, c0 = J * kTile;
        // this round's Q, K, V (the wave's unit), in flight during the MLP
        UnitIn<kBf16> in;
        if (half == 0) in.load(Qh, Kh, Vh, r0, c0);
        else in.load(Qh, Kh, Vh, c0, r0);
        // one pair block per wave
        int iA, jA;
        const bool vA = block_pair_f(diag, wave, nblk, lane, iA, jA);
        const bool realA = vA && L.real[r0 + iA] && L.real[c0 + jA];
        if (__ballot(realA) != 0) {
            const float fA = realA ? pair_feature(L, r0 + iA, c0 + jA, lane >> 4) : 0.0f;
            v4f uA;
            if (!M.run1(fA, uA)) uA = mlp1_f32(w32, M.bl, fA);  // fp16 x 2 left its range
            if (lane < 32 && vA) {
                const int h0 = (lane >> 4) * 4;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    us[buf][h0 + r][iA][jA] = uA[r];
                    if (diag) us[buf][h0 + r][jA][iA] = uA[r];
                }
            }
        }
        __syncthreads();
        if (half == 0) unit(us[buf][h], false, I, J, in);
        else if (!diag) unit(us[buf][h], true, J, I, in);
    }

    // ---- finalise this head's query blocks of this half: O = acc / l on
    // real queries, exact 0 elsewhere (the other wave of the head may have
    // updated one of them in the last round: wait for it)
    __syncthreads();
    for (int qb = half; qb < T; qb += 2) {
        const int q = qb * kTile + c;
        const bool rq = blkAny[qb] && L.real[q];
        v4f o = {0.f, 0.f, 0.f, 0.f};
        if (rq) {
            const float4 a4 = Ost[h][qb][lane];
            const float inv = 1.0f / lst[h][qb][c];
            o = (v4f){a4.x * inv, a4.y * inv, a4.z * inv, a4.w * inv};
        }
        store_o<kBf16>(O + (hb + q) * 16 + 4 * g, o);
    }
}

// ------------------------------------------------------------ row kernel
constexpr int kRowThreads = 512;  // 8 waves: two rows of the tile and one head each

template <int kMode, bool kBf16 = (kMode == kMlpBf16)>
__global__ __launch_bounds__(kRowThreads) __attribute__((amdgpu_waves_per_eu(4))) void
embed_attention_row_kernel(
    const float4 *__restrict__ p4, const uint8_t *__restrict__ mask, int P,
    const float4 *__restrict__ w32, const v8bf *__restrict__ w16, const v8h *__restrict__ wx2,
    const float *__restrict__ bias, const QkvT<kBf16> *__restrict__ Q,
    const QkvT<kBf16> *__restrict__ K, const QkvT<kBf16> *__restrict__ V, float qk2,
    QkvT<kBf16> *__restrict__ O) {
    MlpLds<kMode> M;
    __shared__ PartLds<kMaxP> L;
    __shared__ float us[kHeads][16][17];
    __shared__ int blkAny[kMaxP / kTile];

    const int T = P / kTile;
    const int jet = blockIdx.x / T, I = blockIdx.x - jet * T;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, c = lane & 15;
    const int r0 = I * kTile;

    for (int s = tid; s < P; s += kRowThreads) {
        const size_t idx = (size_t)jet * P + s;
        const float4 pv = p4[idx];  // both loads issued before either is used
        const uint8_t mb = mask[idx];
        __asm__ volatile("" ::: "memory");
        const int real = mb != 0;
        stage_particle(L, s, real ? pv : make_float4(0.f, 0.f, 0.f, 0.f), real);
    }
    __syncthreads();
    if (tid < T) {
        int a = 0;
        for (int i = 0; i < kTile; ++i) a |= L.real[tid * kTile + i];
        blkAny[tid] = a;
    }
    __syncthreads();
    if (!blkAny[I]) {  // no real query in this block: zeros
        for (int i = tid; i < kHeads * 16 * 4; i += kRowThreads) {
            const int hh = i >> 6, q = (i >> 2) & 15, d4 = (i & 3) * 4;
            store_o<kBf16>(O + ((((size_t)jet * kHeads + hh) * P) + r0 + q) * 16 + d4,
                           (v4f){0.f, 0.f, 0.f, 0.f});
        }
        return;
    }
    M.template stage<kRowThreads>(w32, w16, wx2, bias);
    __syncthreads();

    static_assert(kRowThreads == 64 * kHeads, "one head per wave");
    const int h = wave;
    const size_t hb = ((size_t)jet * kHeads + h) * P;
    float m = -INFINITY, l = 0.f;
    v4f acc = {0.f, 0.f, 0.f, 0.f};
    for (int J = 0; J < T; ++J) {
        if (!blkAny[J]) continue;
        const int c0 = J * kTile;
        // this key block's Q, K, V for the wave's head, in flight during the MLP
        UnitIn<kBf16> in;
        in.load(Q + hb * 16, K + hb * 16, V + hb * 16, r0, c0);
        {  // rows 2 wave and 2 wave + 1 of tile (I, J)
            const int iA = 2 * wave, iB = iA + 1, j = lane & 15;
            const bool realA = L.real[r0 + iA] && L.real[c0 + j];
            const bool realB = L.real[r0 + iB] && L.real[c0 + j];
            if (__ballot(realA || realB) != 0) {
                const int k = lane >> 4;
                if constexpr (kMode == kMlpBf16) {  // both blocks at once (102 registers)
                    const float fA = realA ? pair_feature(L, r0 + iA, c0 + j, k) : 0.0f;
                    const float fB = realB ? pair_feature(L, r0 + iB, c0 + j, k) : 0.0f;
                    v4f uA, uB;
                    mlp_pair_blocks<kMode>(M, w32, fA, fB, uA, uB);
                    if (lane < 32) {
                        const int h0 = (lane >> 4) * 4;
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            us[h0 + r][iA][j] = uA[r];
                            us[h0 + r][iB][j] = uB[r];
                        }
                    }
                } else {  // float32 chains: one block at a time (two do not fit 128 registers)
#pragma unroll 1
                    for (int t = 0; t < 2; ++t) {
                        const int i = iA + t;
                        const bool rl = t ? realB : realA;
                        const float f = rl ? pair_feature(L, r0 + i, c0 + j, k) : 0.0f;
                        v4f u;
                        if (!M.run1(f, u)) u = mlp1_f32(w32, M.bl, f);  // fp16 x 2 left its range
                        if (lane < 32) {
                            const int h0 = (lane >> 4) * 4;
#pragma unroll
                            for (int r = 0; r < 4; ++r) us[h0 + r][i][j] = u[r];
                        }
                    }
                }
            }
        }
        __syncthreads();
        {
            v4f sc = in.scores();
            int kreal[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                kreal[r] = L.real[c0 + 4 * g + r];
                sc[r] = kreal[r] ? fmaf(sc[r], qk2, us[h][c][4 * g + r] * kLog2e) : -INFINITY;
            }
            const float corr = online_softmax(sc, m, l);
            acc *= corr;
            acc = in.pv(sc, kreal, acc);
        }
        __syncthreads();
    }
    {
        const int q = r0 + c;
        const bool rq = L.real[q];
        const float inv = rq ? 1.0f / l : 0.0f;
        const v4f o = rq ? acc * inv : (v4f){0.f, 0.f, 0.f, 0.f};
        store_o<kBf16>(O + (hb + q) * 16 + 4 * g, o);
    }
}

template <int kMode, bool kBf16 = (kMode == kMlpBf16)>
static hipError_t launch_fused(const float *p4, const uint8_t *mask, int B, int P,
                               const pip_pair_mlp *m, const QkvT<kBf16> *Q,
                               const QkvT<kBf16> *K, const QkvT<kBf16> *V, float scale,
                               QkvT<kBf16> *O, hipStream_t s) {
    const float qk2 = scale * kLog2e;  // scores in base-2 units
    // The jet kernel gives each jet one CU for all its rounds: with at most
    // half as many jets as CUs, half the chip idles and the largest jet sets
    // the time (about 250 us at P = 128 whatever the batch).  The row kernel
    // spreads a jet over its query blocks, at twice the MLP work.  Measured
    // crossover at P = 128: row 212 us against jet 249 at B = 128, 283
    // against 253 at B = 192 (identical O).
    if (P <= kJetMaxP && 2 * B > cu_count()) {
        const int sort = B <= kSortMaxB ? 1 : 0;
        hipLaunchKernelGGL(embed_attention_jet_kernel<kMode>, dim3(B), dim3(kJetThreads), 0, s,
                           (const float4 *)p4, mask, B, P, sort, (const float4 *)m->w32,
                           (const v8bf *)m->w16, (const v8h *)m->wx2, m->bias, Q, K, V, qk2, O);
    } else {
        hipLaunchKernelGGL(embed_attention_row_kernel<kMode>, dim3(B * (P / kTile)),
                           dim3(kRowThreads), 0, s, (const float4 *)p4, mask, P,
                           (const float4 *)m->w32, (const v8bf *)m->w16, (const v8h *)m->wx2,
                           m->bias, Q, K, V, qk2, O);
    }
    return hipGetLastError();
}

hipError_t launch_embed_attention_f32(const float *p4, const uint8_t *mask, int B, int P,
                                      const pip_pair_mlp *m, const float *Q, const float *K,
                                      const float *V, float scale, float *O, hipStream_t s) {
    return m->f16ok ? launch_fused<kMlpF16x2>(p4, mask, B, P, m, Q, K, V, scale, O, s)
                    : launch_fused<kMlpF32>(p4, mask, B, P, m, Q, K, V, scale, O, s);
}

hipError_t launch_embed_attention_bf16(const float *p4, const uint8_t *mask, int B, int P,
                                       const pip_pair_mlp *m, const uint16_t *Q,
                                       const uint16_t *K, const uint16_t *V, float scale,
                                       uint16_t *O, hipStream_t s) {
    return launch_fused<kMlpBf16>(p4, mask, B, P, m, Q, K, V, scale, O, s);
}

}  // namespace pip

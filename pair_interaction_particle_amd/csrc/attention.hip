// attention.hip -- masked multi-head attention with an additive pair bias.
//
// "Event Classification with Masked Transformer Autoencoders"
// (ml4sci_cms_e2e26 README), "How the Kernel Fusion Works", Fusion 3:
// softmax(Q K^T / sqrt(d) + bias) V in one pass, never materialising the
// (B*H, P, P) score matrix in HBM.
//
// The kernel reads U once and is bound by HBM, so the design is about bytes in
// flight: every workgroup of the launch should be resident at once, issue all
// of its loads early and have little work left once the data is there.  One
// workgroup per (jet, head, group of up to 4 (P <= 128) or 8 query blocks of 16
// queries); each
// wave owns one query block.
//   1. Each wave takes the jet's real-slot bits with ballots (wave-uniform,
//      no LDS), then issues the loads of its U strips (16 queries x every key
//      block that holds a real key) and of its Q rows into registers.
//   2. While those are in flight the workgroup stages K and V in LDS for
//      the key blocks up to an even count; padded key rows and blocks without
//      a real key are written as 0 (a NaN there must not meet a zero
//      probability inside the MFMA).
//   3. One barrier, then per query block: U of padded keys is replaced by
//      -inf; scores S^T = K Q^T on the matrix cores, transposed so that lane l
//      holds query l%16 against keys 4(l/16)+r, over pairs of key blocks.
//      float32: an exact two-pass softmax over the scores held in registers;
//      bfloat16: a running max and sum per pair of key blocks (the rescale
//      costs one exp2 per pair and keeps no score array, so the kernel stays
//      within 64 registers at P = 256).  Row max and row sum take an in-lane
//      reduction and two cross-lane swaps.  Then O^T += V^T P^T with one
//      K = 32 product per pair of key blocks, the probabilities already in
//      the B-operand layout.  V is staged row-major with 8-byte stores and
//      read as V^T by the gfx950 LDS transpose load (ds_read_b64_tr_b16).
// Query blocks without a real query store zeros; padded queries store 0.
//
// float32 inputs run on the fp16 matrix cores with split operands: every
// float32 x is carried as hi + lo (two fp16, 22 significand bits).  Scores
// take all four products, (K_hi + K_lo)(Q_hi + Q_lo), in two 16x16x32 MFMAs
// whose reduction index runs over [hi | lo] x d; P V takes three
// (V_hi P_hi + V_hi P_lo + V_lo P_hi).  The products are exact in fp32 and
// accumulated in fp32, so the result is float32-faithful (relative product
// error about 2^-22).  K and V are split once when staged.  When a real Q, K
// or V value is beyond the fp16 range (or not finite) the query block takes a
// float32 MFMA path instead.  bfloat16 inputs use the bf16 matrix cores.
#include "pip_attn_core.h"
#include "pip_internal.h"

namespace pip {

// Query blocks per workgroup: 4 for P <= 128 (a jet of at most 64 real
// slots then leaves its second workgroup nothing to do, and it ends at once,
// instead of holding four idle waves), 8 beyond (the larger register
// strips would lower the occupancy with 4).
__host__ __device__ constexpr int attn_qblocks(int kT) { return kT <= 8 ? 4 : 8; }
// ------------------------------------------------------------ float32
// One query block (rows q0 .. q0+15) of a float32 head.  u is the U strip
// (-inf for key blocks without a real key), qa / qc are this lane's Q row
// entries 8(g&1) .. +3 and +4 .. +7 (0 for padded queries).  K and V sit in
// LDS scaled by the head's powers of two (kinv, vinv undo them); each query
// row is scaled here by its own power of two before the split, so a row of
// any magnitude keeps 22 significand bits against K of any magnitude.
template <int kT, int kWords>
__device__ __forceinline__ void attend_f32(float4 (&u)[kT], float4 qa, float4 qc, bool rq,
                                           bool wr, float qk_mul, float vinv,
                                           const SlotBits<kWords> &real, int T,
                                           const uint16_t *Ks, const uint16_t *Vsh,
                                           const uint16_t *Vsl, float *__restrict__ orow) {
    float qsc, qinv;
    pow2_scale(xmax16(fmaxf(absmax4(qa), absmax4(qc))), qsc, qinv);
    v8h qh, ql;
    {
        v4h h0, l0, h1, l1;
        split4_f16(make_float4(qa.x * qsc, qa.y * qsc, qa.z * qsc, qa.w * qsc), h0, l0);
        split4_f16(make_float4(qc.x * qsc, qc.y * qsc, qc.z * qsc, qc.w * qsc), h1, l1);
        qh = __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7);
        ql = __builtin_shufflevector(l0, l1, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    v4f o;
    float lsum;
    attend_split<kT>(u, qh, ql, qk_mul * qinv, real, T, Ks, Vsh, Vsl, o, lsum);
    const float inv = vinv / lsum;
    if (wr)
        *(float4 *)orow = rq ? make_float4(o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv)
                             : make_float4(0.f, 0.f, 0.f, 0.f);
}

// ------------------------------------------------------------ bfloat16
// One query block of a bf16 head.  u holds bf16 pairs (-inf for key blocks
// without a real key), qv this lane's Q row entries 4g .. 4g+3.
template <int kT, int kWords>
__device__ __forceinline__ void attend_bf16(uint2 (&u)[kT], v4s qv, bool rq, bool wr, float scale,
                                            const SlotBits<kWords> &real, int T,
                                            const uint16_t *Ks, const uint16_t *Vsh,
                                            uint16_t *__restrict__ orow) {
    const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
    // U of padded keys -> -inf (bit patterns), so that every score is an FMA result
#pragma unroll
    for (int kb = 0; kb < kT; kb += 2) {
        const uint32_t bits = real.pair(kb >> 1);
        if (kb < T && bits != 0 && bits != 0xffffffffu) {
            const uint32_t lb = bits >> (8 * g);
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const uint32_t kbits = lb >> (4 * t);
                const uint32_t k0 = ((kbits & 1) ? 0xffffu : 0u) | ((kbits & 2) ? 0xffff0000u : 0u);
                const uint32_t k1 = ((kbits & 4) ? 0xffffu : 0u) | ((kbits & 8) ? 0xffff0000u : 0u);
                u[kb + t].x = (u[kb + t].x & k0) | (kBf16NegInf & ~k0);
                u[kb + t].y = (u[kb + t].y & k1) | (kBf16NegInf & ~k1);
            }
        }
    }
    // online softmax over pairs of key blocks: the running max m is the same
    // in the 4 lane groups of a query (cross-lane max per pair)
    float m = -INFINITY, lsum = 0.f;
    v4f o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < kT; kb += 2) {
        if (!pair_real(real, kb, T)) continue;
        const v4s k0 = *(const v4s *)(Ks + (kb * kTile + c) * 16 + 4 * g);
        const v4s k1 = *(const v4s *)(Ks + ((kb + 1) * kTile + c) * 16 + 4 * g);
        const v4f a0 = mfma16bf(k0, qv, (v4f){0.f, 0.f, 0.f, 0.f});
        const v4f a1 = mfma16bf(k1, qv, (v4f){0.f, 0.f, 0.f, 0.f});
        float s0[4], s1[4];
        s0[0] = fmaf(a0[0], scale, bf2f(u[kb].x & 0xffff));
        s0[1] = fmaf(a0[1], scale, bf2f(u[kb].x >> 16));
        s0[2] = fmaf(a0[2], scale, bf2f(u[kb].y & 0xffff));
        s0[3] = fmaf(a0[3], scale, bf2f(u[kb].y >> 16));
        s1[0] = fmaf(a1[0], scale, bf2f(u[kb + 1].x & 0xffff));
        s1[1] = fmaf(a1[1], scale, bf2f(u[kb + 1].x >> 16));
        s1[2] = fmaf(a1[2], scale, bf2f(u[kb + 1].y & 0xffff));
        s1[3] = fmaf(a1[3], scale, bf2f(u[kb + 1].y >> 16));
        const float mn = fmaxf(m, xmax16(max8(s0, s1)));
        const float corr = __builtin_amdgcn_exp2f((m - mn) * kLog2e);
        m = mn;
        const float mb = mn * kLog2e;
        v8f p;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            p[r] = __builtin_amdgcn_exp2f(fmaf(s0[r], kLog2e, -mb));
            p[4 + r] = __builtin_amdgcn_exp2f(fmaf(s1[r], kLog2e, -mb));
        }
        lsum = fmaf(lsum, corr, ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7])));
        o = o * corr;
        const v8bf vt = __builtin_bit_cast(v8bf, v_operand<true>(Vsh, kb * kTile));
        o = mfma32bf(vt, __builtin_convertvector(p, v8bf), o);
    }
    const float inv = 1.0f / xsum16(lsum);
    if (wr)
        *(uint2 *)orow =
            rq ? make_uint2((uint32_t)f2bf(o[0] * inv) | ((uint32_t)f2bf(o[1] * inv) << 16),
                            (uint32_t)f2bf(o[2] * inv) | ((uint32_t)f2bf(o[3] * inv) << 16))
               : make_uint2(0u, 0u);
}

// ------------------------------------------------------------ kernel
// Padded layout (kPacked false): Q, K, V, O (B, H, P, 16), U (B, H, P, P),
// mask (B, P).  Packed layout (kPacked true): jet b owns rows cu[b] ..
// cu[b+1]-1 of Q, K, V, O (H, N, 16); its bias is (H, n_b, ld_b) at element
// H u_off[b], ld_b = n_b rounded up to 8; every row < n_b is real and rows
// of other jets are never read or written.  A packed jet with inconsistent
// cu / u_off entries is skipped (its O rows are not written).
// (float32 at P <= 128: held to 6 waves per SIMD, i.e. at most 80 VGPRs, so
// that three workgroups stay resident per CU)
template <bool kBf16, int kT, int kQ, bool kPacked>
__global__ __launch_bounds__(64 * attn_qblocks(kT) / kQ)
__attribute__((amdgpu_waves_per_eu(!kBf16 && kT == 8 ? 6 : 1))) void attention_kernel(
    const AttnElt<kBf16> *__restrict__ Q, const AttnElt<kBf16> *__restrict__ K,
    const AttnElt<kBf16> *__restrict__ V, const AttnElt<kBf16> *__restrict__ U,
    const uint8_t *__restrict__ mask, int B, int H, int P, int chunks, float scale,
    AttnElt<kBf16> *__restrict__ O, const int *__restrict__ cu,
    const int64_t *__restrict__ uoff, int N, int64_t u_elems) {
    using E = AttnElt<kBf16>;
    constexpr int kQB = attn_qblocks(kT);
    constexpr int kWaves = kQB / kQ, kThreads = 64 * kWaves;
    constexpr int kWords = (kT * 16 + 63) / 64;
    // fp32: K rows as 32 fp16 [hi d0..15 | lo d0..15], V hi and lo;
    // bf16: K rows of 16 bf16 and V.  K rows in key order (fp32) or key_row
    // order (bf16), V row-major in key order (read transposed as the P V
    // operand).
    constexpr int kKRow = kBf16 ? 16 : 32;
    __shared__ __attribute__((aligned(16))) uint16_t Ks[kT * 16 * kKRow];
    __shared__ __attribute__((aligned(16))) uint16_t Vsh[kT * 16 * kVRow];
    __shared__ __attribute__((aligned(16))) uint16_t Vsl[kBf16 ? 1 : kT * 16 * kVRow];
    __shared__ float kvmax[2][kWaves];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, c = lane & 15;
    // Workgroup i runs on XCD i % 8; XCD x takes the H * chunks workgroups of
    // jets x, x + 8, ..., so a jet's mask row (or cu / u_off entries), the
    // first load of every chain, is fetched from HBM once and then hit in
    // that XCD's L2.  The grid is rounded up to 8 jets.
    const int per_jet = H * chunks;
    const int xcd = blockIdx.x & 7, t8 = blockIdx.x >> 3;
    const int jet = xcd + 8 * (t8 / per_jet), sub = t8 - (t8 / per_jet) * per_jet;
    if (jet >= B) return;  // uniform: a slot of the rounding
    const int chunk = sub % chunks, bh = jet * H + sub / chunks;
    // rows: rows of this (jet, head) that exist (P, or n in the packed
    // layout); ld: U row stride; T: blocks of 16 rows
    int rows, ld, T;
    const E *Qh, *Kh, *Vh, *Ub;
    E *Oh;
    SlotBits<kWords> real;
    if constexpr (!kPacked) {
        rows = ld = P;
        T = P / kTile;
        const size_t base = (size_t)bh * P;
        Qh = Q + base * 16;
        Kh = K + base * 16;
        Vh = V + base * 16;
        Oh = O + base * 16;
        Ub = U + base * P;
    } else {
        const int h = bh - jet * H;
        const int start = __builtin_amdgcn_readfirstlane(cu[jet]);
        const int end = __builtin_amdgcn_readfirstlane(cu[jet + 1]);
        const int64_t a0 = uoff[jet], a1 = uoff[jet + 1];
        int n = end - start;
        const int lp = (n + 7) & ~7;
        const bool ok = start >= 0 && n >= 0 && n <= P && end <= N && a0 >= 0 &&
                        a1 - a0 == (int64_t)n * lp && a1 <= u_elems / H;
        n = ok ? n : 0;
        rows = n;
        ld = lp;
        T = (n + kTile - 1) / kTile;
        if (chunk * kQB >= T) return;  // uniform: nothing of this jet here
        const size_t base = (size_t)h * N + start;
        Qh = Q + base * 16;
        Kh = K + base * 16;
        Vh = V + base * 16;
        Oh = O + base * 16;
        Ub = U + (size_t)H * a0 + (size_t)h * n * lp;
    }

    // ---- 1. K and V rows this thread stages, issued before the mask is known
    // (blocks below an even block count; the mask only decides what is kept),
    // then the mask, then the U strips and Q rows of this wave's query blocks.
    // The wait counter drains in issue order, so the barrier waits for K and V
    // alone.  Nothing else loaded here is looked at before the barrier.
    constexpr int kItems = (kT * 16 * 4 + kThreads - 1) / kThreads;
    using KVec = typename std::conditional<kBf16, uint2, float4>::type;
    const int nst = 16 * (T + (T & 1));
    KVec kk[kItems], vv[kItems];
#pragma unroll
    for (int it = 0; it < kItems; ++it) {
        const int i = tid + it * kThreads, k = i >> 2, d0 = (i & 3) * 4;
        const size_t off = (i < nst * 4 && k < rows) ? (size_t)k * 16 + d0 : 0;
        kk[it] = *(const KVec *)(Kh + off);
        vv[it] = *(const KVec *)(Vh + off);
    }

    if constexpr (!kPacked) real.load(mask + (size_t)jet * P, P);
    else real.first(rows);

    using UVec = typename std::conditional<kBf16, uint2, float4>::type;
    UVec u[kQ][kT];
    float4 qa[kQ], qc[kQ];  // fp32: Q[q0 + c][8(g & 1) .. + 7]
    v4s qb16[kQ];           // bf16: Q[q0 + c][4g .. 4g + 3]
    // a zero the compiler cannot see (P <= 256): the unneeded strip loads
    // read the row start, and must not be merged with the load of block 0
    const int zero = P >> 16;
#pragma unroll
    for (int j = 0; j < kQ; ++j) {
        const int qb = chunk * kQB + wave + j * kWaves;
        const bool act = qb < T && real.block_rt(qb) != 0;
        const int qr = act && qb * kTile + c < rows ? qb * kTile + c : 0;  // query row read
        const E *urow = Ub + (size_t)qr * ld;
#pragma unroll
        for (int kb = 0; kb < kT; kb += 2) {
            // lane group g's 8 keys of the pair: one contiguous run
            // (a pair past an odd block count is half outside the row:
            // clamped, and those keys are masked)
            const bool need = act && kb < T && real.pair(kb >> 1) != 0;
            if constexpr (kBf16) {
                const int off = min(need ? u_col(kb, g) : u_col(kb, g) * zero, ld - 8);
                const uint4 v = *(const uint4 *)(urow + off);
                u[j][kb] = make_uint2(v.x, v.y);
                u[j][kb + 1] = make_uint2(v.z, v.w);
            } else {
                // natural order: 4 keys 16 kb + 4g .. of each block
                const int o0 = 16 * kb + 4 * g, o1 = o0 + 16;
                u[j][kb] = *(const float4 *)(urow + min(need ? o0 : o0 * zero, ld - 4));
                u[j][kb + 1] = *(const float4 *)(urow + min(need ? o1 : o1 * zero, ld - 4));
            }
        }
        if constexpr (kBf16) {
            qb16[j] = *(const v4s *)(Qh + (size_t)qr * 16 + 4 * g);
        } else {
            const float4 *qp = (const float4 *)(Qh + (size_t)qr * 16 + 8 * (g & 1));
            qa[j] = qp[0];
            qc[j] = qp[1];
        }
    }

    // ---- 2. K and V into LDS.  float32: the head's largest |K| and |V| over
    // real keys first (one barrier), then K and V scaled by powers of two
    // into [2^13, 2^14) and split into fp16 hi / lo.
    float ksc = 1.f, kinv = 1.f, vsc = 1.f, vinv = 1.f;
    if constexpr (!kBf16) {
        float kmx = 0.f, vmx = 0.f;
#pragma unroll
        for (int it = 0; it < kItems; ++it) {
            const int i = tid + it * kThreads, k = i >> 2;
            if (i >= nst * 4 || !(k < P && real.slot(k))) continue;
            kmx = fmaxf(kmx, absmax4(kk[it]));
            vmx = fmaxf(vmx, absmax4(vv[it]));
        }
        kmx = wave_max(kmx);
        vmx = wave_max(vmx);
        if (lane == 0) {
            kvmax[0][wave] = kmx;
            kvmax[1][wave] = vmx;
        }
        __syncthreads();
        float km = 0.f, vm = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            km = fmaxf(km, kvmax[0][w]);
            vm = fmaxf(vm, kvmax[1][w]);
        }
        pow2_scale(km, ksc, kinv);
        pow2_scale(vm, vsc, vinv);
    }
#pragma unroll
    for (int it = 0; it < kItems; ++it) {
        const int i = tid + it * kThreads, k = i >> 2, d0 = (i & 3) * 4;
        if (i >= nst * 4) continue;
        const bool rk = k < rows && real.slot(k);
        const int kr = kBf16 ? key_row(k) : k;
        if constexpr (kBf16) {
            const uint2 kz = rk ? kk[it] : make_uint2(0u, 0u);
            const uint2 vz = rk ? vv[it] : make_uint2(0u, 0u);
            *(uint2 *)(Ks + kr * 16 + d0) = kz;
            *(uint2 *)(Vsh + k * kVRow + d0) = vz;
        } else {
            const float4 zero = make_float4(0.f, 0.f, 0.f, 0.f);
            const float4 a = kk[it], b = vv[it];
            const float4 kz = rk ? make_float4(a.x * ksc, a.y * ksc, a.z * ksc, a.w * ksc) : zero;
            const float4 vz = rk ? make_float4(b.x * vsc, b.y * vsc, b.z * vsc, b.w * vsc) : zero;
            v4h kh, kl, vh, vl;
            split4_f16(kz, kh, kl);
            split4_f16(vz, vh, vl);
            *(v4h *)(Ks + kr * 32 + d0) = kh;
            *(v4h *)(Ks + kr * 32 + 16 + d0) = kl;
            *(v4h *)(Vsh + k * kVRow + d0) = vh;
            *(v4h *)(Vsl + k * kVRow + d0) = vl;
        }
    }
    __syncthreads();

    // ---- 3. per query block
#pragma unroll
    for (int j = 0; j < kQ; ++j) {
        const int qb = chunk * kQB + wave + j * kWaves;
        const int q0 = qb * kTile;
        if (qb >= T) continue;
        E *orow = Oh + (size_t)(q0 + c) * 16 + 4 * g;
        const bool wr = !kPacked || q0 + c < rows;  // packed: rows past n are another jet's
        if (real.block_rt(qb) == 0) {
            if constexpr (kBf16) *(uint2 *)orow = make_uint2(0u, 0u);
            else *(float4 *)orow = make_float4(0.f, 0.f, 0.f, 0.f);
            continue;
        }
        // U of key blocks without a real key -> -inf, Q rows of padded
        // queries -> 0 (only now: a select on a loaded value before the
        // barrier would wait for every load)
#pragma unroll
        for (int kb = 0; kb < kT; ++kb) {
            if (pair_real(real, kb & ~1, T)) continue;
            if constexpr (kBf16) u[j][kb] = make_uint2(kBf16NegInf, kBf16NegInf);
            else u[j][kb] = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
        }
        const bool rq = real.slot(q0 + c);
        if constexpr (kBf16) {
            attend_bf16<kT>(u[j], rq ? qb16[j] : (v4s){0, 0, 0, 0}, rq, wr, scale, real, T, Ks,
                            Vsh, orow);
        } else {
            const float4 zero = make_float4(0.f, 0.f, 0.f, 0.f);
            attend_f32<kT>(u[j], rq ? qa[j] : zero, rq ? qc[j] : zero, rq, wr, scale * kinv,
                           vinv, real, T, Ks, Vsh, Vsl, orow);
        }
    }
}

// workgroups per (jet, head) (P rounded up to 16)
int attention_chunks(int P) {
    const int T = P / kTile, qb = attn_qblocks(T <= 8 ? 8 : 16);
    return (T + qb - 1) / qb;
}

// jets the grid covers: B rounded up to the 8 XCDs
int64_t attention_jet_slots(int64_t B) { return (B + 7) / 8 * 8; }

template <bool kBf16>
static hipError_t launch_attention(const AttnElt<kBf16> *Q, const AttnElt<kBf16> *K,
                                   const AttnElt<kBf16> *V, const AttnElt<kBf16> *U,
                                   const uint8_t *mask, int B, int H, int P, float scale,
                                   AttnElt<kBf16> *O, hipStream_t s) {
    const int chunks = attention_chunks(P);
    const dim3 grid((unsigned)(attention_jet_slots(B) * H * chunks));
    if (P <= 128)
        hipLaunchKernelGGL((attention_kernel<kBf16, 8, 1, false>), grid, dim3(64 * attn_qblocks(8)),
                           0, s, Q, K, V, U, mask, B, H, P, chunks, scale, O, nullptr, nullptr,
                           0, (int64_t)0);
    else
        hipLaunchKernelGGL((attention_kernel<kBf16, 16, 1, false>), grid,
                           dim3(64 * attn_qblocks(16)), 0, s, Q, K, V, U, mask, B, H, P, chunks,
                           scale, O, nullptr, nullptr, 0, (int64_t)0);
    return hipGetLastError();
}

hipError_t launch_attention_f32(const float *Q, const float *K, const float *V,
                                const float *U, const uint8_t *mask, int B, int H, int P,
                                float scale, float *O, hipStream_t s) {
    return launch_attention<false>(Q, K, V, U, mask, B, H, P, scale, O, s);
}

hipError_t launch_attention_bf16(const uint16_t *Q, const uint16_t *K, const uint16_t *V,
                                 const uint16_t *U, const uint8_t *mask, int B, int H, int P,
                                 float scale, uint16_t *O, hipStream_t s) {
    return launch_attention<true>(Q, K, V, U, mask, B, H, P, scale, O, s);
}

// Packed layout: max_n plays the part of P (the largest jet; jets beyond it
// are skipped).
template <bool kBf16>
static hipError_t launch_attention_packed(const AttnElt<kBf16> *Q, const AttnElt<kBf16> *K,
                                          const AttnElt<kBf16> *V, const AttnElt<kBf16> *U,
                                          const int *cu, const int64_t *uoff, int B, int H,
                                          int N, int max_n, int64_t u_elems, float scale,
                                          AttnElt<kBf16> *O, hipStream_t s) {
    const int chunks = attention_chunks((max_n + 15) & ~15);
    if (chunks == 0) return hipSuccess;
    const dim3 grid((unsigned)(attention_jet_slots(B) * H * chunks));
    if (max_n <= 128)
        hipLaunchKernelGGL((attention_kernel<kBf16, 8, 1, true>), grid, dim3(64 * attn_qblocks(8)),
                           0, s, Q, K, V, U, nullptr, B, H, max_n, chunks, scale, O, cu, uoff,
                           N, u_elems);
    else
        hipLaunchKernelGGL((attention_kernel<kBf16, 16, 1, true>), grid,
                           dim3(64 * attn_qblocks(16)), 0, s, Q, K, V, U, nullptr, B, H, max_n,
                           chunks, scale, O, cu, uoff, N, u_elems);
    return hipGetLastError();
}

hipError_t launch_attention_packed_f32(const float *Q, const float *K, const float *V,
                                       const float *U, const int *cu, const int64_t *uoff, int B,
                                       int H, int N, int max_n, int64_t u_elems, float scale,
                                       float *O, hipStream_t s) {
    return launch_attention_packed<false>(Q, K, V, U, cu, uoff, B, H, N, max_n, u_elems, scale,
                                          O, s);
}

hipError_t launch_attention_packed_bf16(const uint16_t *Q, const uint16_t *K,
                                        const uint16_t *V, const uint16_t *U, const int *cu,
                                        const int64_t *uoff, int B, int H, int N, int max_n,
                                        int64_t u_elems, float scale, uint16_t *O,
                                        hipStream_t s) {
    return launch_attention_packed<true>(Q, K, V, U, cu, uoff, B, H, N, max_n, u_elems, scale,
                                         O, s);
}

}  // namespace pip

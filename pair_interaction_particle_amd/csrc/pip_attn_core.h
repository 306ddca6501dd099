// pip_attn_core.h -- the query-block core of the biased attention on split
// fp16 operands, shared by the attention kernel and the block stack.
//
// "Fusion 3" of the ml4sci_cms_e2e26 README ("How the Kernel Fusion Works"):
// softmax(Q K^T / sqrt(d) + bias) V.  K (as [key][hi d0..15 | lo d0..15]
// fp16) and V (hi and lo, row-major in key order) sit in LDS; the bias rows
// of one query block (the "U strip") sit in registers.  Scores are computed
// transposed, S^T = K Q^T, so that lane l holds query l%16 against keys
// 4(l/16)+r; the softmax is exact (two passes over the strip); P V takes one
// K = 32 product per pair of key blocks, the probabilities already in the
// B-operand layout.
#pragma once

#include "pip_attn.h"

namespace pip {

constexpr uint32_t kBf16NegInf = 0xff80ff80u;  // two bf16 -inf

template <bool kBf16>
using AttnElt = typename std::conditional<kBf16, uint16_t, float>::type;

// Real-slot bits of one jet: bit k of word k/64, the same in every lane.
template <int kWords>
struct SlotBits {
    uint64_t w[kWords];

    // every byte load is issued (address clamped into the row) before the
    // first ballot, so the loads overlap
    __device__ __forceinline__ void load(const uint8_t *__restrict__ mrow, int P) {
        const int lane = threadIdx.x & 63;
        uint8_t b[kWords];
#pragma unroll
        for (int i = 0; i < kWords; ++i) b[i] = mrow[min(64 * i + lane, P - 1)];
#pragma unroll
        for (int i = 0; i < kWords; ++i) w[i] = __ballot(64 * i + lane < P && b[i] != 0);
    }
    // the first n slots real, the rest not (n wave-uniform)
    __device__ __forceinline__ void first(int n) {
#pragma unroll
        for (int i = 0; i < kWords; ++i)
            w[i] = n >= 64 * (i + 1) ? ~0ull : (n > 64 * i ? (1ull << (n - 64 * i)) - 1 : 0ull);
    }
    // word i for a run-time i.  The words pass through readfirstlane (free:
    // they are wave-uniform) so that the selects act on values; a select
    // between two fields would otherwise be folded into an indexed load,
    // which keeps the struct in memory (moved to LDS or scratch).
    __device__ __forceinline__ uint64_t word(int i) const {
        uint64_t r = uniform(w[0]);
#pragma unroll
        for (int j = 1; j < kWords; ++j) r = i == j ? uniform(w[j]) : r;
        return r;
    }
    static __device__ __forceinline__ uint64_t uniform(uint64_t x) {
        const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
        const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
        return ((uint64_t)hi << 32) | lo;
    }
    // the 16 bits of block kb (compile-time kb)
    __device__ __forceinline__ uint32_t block(int kb) const {
        return (uint32_t)(w[kb >> 2] >> (16 * (kb & 3))) & 0xffffu;
    }
    __device__ __forceinline__ uint32_t block_rt(int kb) const {
        return (uint32_t)(word(kb >> 2) >> (16 * (kb & 3))) & 0xffffu;
    }
    __device__ __forceinline__ bool slot(int k) const { return (word(k >> 6) >> (k & 63)) & 1; }
    // the 32 bits of key-block pair p (keys 32p .. 32p+31; compile-time p)
    __device__ __forceinline__ uint32_t pair(int p) const {
        return (uint32_t)(w[p >> 1] >> (32 * (p & 1)));
    }
    __device__ __forceinline__ uint32_t pair_rt(int p) const {
        return (uint32_t)(word(p >> 1) >> (32 * (p & 1)));
    }
};

// V in LDS: row-major, one row of kVRow 16-bit elements (d = 0 .. 15) per
// key, written with one 8-byte store per 4 values.
constexpr int kVRow = 16;

// The P V A operand (V^T: row d = lane % 16, reduction slots 8 (lane / 16) ..
// + 7, k0 = 32 p for pair p) from row-major V with two gfx950 LDS transpose
// reads.  In the pair key order (kPairOrder) the slots of lane group g are the
// keys k0 + 8g .. + 7; in the natural order they are k0 + 4g .. + 3 and
// k0 + 16 + 4g .. + 3 (the keys that group's probabilities hold).  Within a 16-lane group,
// ds_read_b64_tr_b16 gives lane 4c + d, slot e, element d of the 4-element
// block addressed by lane 4e + c; so lane j addresses V[k + j / 4][4 (j % 4)]
// and lane i receives V[k .. k + 3][i].
template <bool kPairOrder>
__device__ __forceinline__ v8h v_operand(const uint16_t *Vr, int k0) {
    const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
    typedef __attribute__((address_space(3))) v4s *LdsV4s;
    const int row = kPairOrder ? k0 + 8 * g : k0 + 4 * g, step = kPairOrder ? 4 : 16;
    const uint16_t *p = Vr + (row + (c >> 2)) * kVRow + 4 * (c & 3);
    const v4s r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LdsV4s)p);
    const v4s r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LdsV4s)(p + step * kVRow));
    return __builtin_bit_cast(v8h, __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Key orders of the score MFMA (D row 4g + r of key block kb lands in lane
// group g, register r).
// * Natural (the float32 paths): K row = key, so block kb puts key
//   16 kb + 4g + r in lane group g, register r.  A lane's U entries of a block
//   are 4 consecutive floats: one 16-byte load per lane and block, and each
//   load instruction reads 64 contiguous bytes of every row of the strip.
// * Pair order (bfloat16): inside a pair of key blocks (keys 32p .. 32p+31)
//   block t = 0, 1 puts key 32p + 8g + 4t + r in lane group g, register r.
//   Lane group g's keys of both blocks are then the 8 consecutive keys
//   32p + 8g .. +7: one 16-byte U read per lane and pair.  key_row(k) is the
//   K row (score A-operand row 16 (2p + t) + 4g + r) that holds key k.
__device__ __forceinline__ int key_row(int k) {
    return (k & ~31) | (((k >> 2) & 1) << 4) | (((k >> 3) & 3) << 2) | (k & 3);
}
// Offset inside a U row of lane group g's 4 keys of key block kb (pair order).
__device__ __forceinline__ int u_col(int kb, int g) {
    return 32 * (kb >> 1) + 8 * g + 4 * (kb & 1);
}

__device__ __forceinline__ float absmax4(float4 x) {
    return fmaxf(fmaxf(fabsf(x.x), fabsf(x.y)), fmaxf(fabsf(x.z), fabsf(x.w)));
}

// Power-of-two scale s (and 1/s) that puts amax into [2^13, 2^14); 1 for
// zero, inf or NaN.  A float32 value scaled this way is split into fp16
// hi + lo with 22 significand bits whatever its magnitude: the largest
// element sits just below fp16's maximum, and an element 2^k times smaller
// keeps relative error 2^-22 down to k = 16, below which its error is at
// most 2^-25 of the largest element, absolute.  Scaling by a power of two
// is exact and undone exactly.
__device__ __forceinline__ void pow2_scale(float amax, float &s, float &inv) {
    const int eb = (int)((__float_as_uint(amax) >> 23) & 0xff);
    if (!(amax > 0.f) || eb == 255) {
        s = inv = 1.f;
        return;
    }
    int e = 13 - (eb - 127);
    e = min(max(e, -126), 126);
    s = __uint_as_float((uint32_t)(e + 127) << 23);
    inv = __uint_as_float((uint32_t)(127 - e) << 23);
}

// Maximum over the 64 lanes of a wave.
__device__ __forceinline__ float wave_max(float x) {
    x = xmax16(x);
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}

__device__ __forceinline__ float max8(const float (&a)[4], const float (&b)[4]) {
    return fmaxf(fmaxf(fmaxf(a[0], a[1]), fmaxf(a[2], a[3])),
                 fmaxf(fmaxf(b[0], b[1]), fmaxf(b[2], b[3])));
}

// Does the pair of key blocks (kb, kb + 1) (kb even) hold a real key?  (Bits
// of slots at or past P are 0.)
template <int kWords>
__device__ __forceinline__ bool pair_real(const SlotBits<kWords> &real, int kb, int T) {
    return kb < T && real.pair(kb >> 1) != 0;
}

// Scores, exact softmax and P V of one query block:
//   s = qk_mul (k . q) + u   (u = -inf for keys to exclude),
//   p = exp(s - max s),  o = sum_k p v_k (lane layout of O^T), l = sum_k p.
// qh / ql are this lane's split Q entries 8(g&1) .. +7 of query l%16; u is
// the strip in the natural key order (U of padded keys inside
// a pair with a real key is replaced here; pairs without a real key must
// already hold -inf).  K and V rows of keys that are not real must be 0 in LDS
// for every pair below an even block count.  V hi / lo are row-major (kVRow).
template <int kT, int kWords>
__device__ __forceinline__ void attend_split(float4 (&u)[kT], v8h qh, v8h ql, float qk_mul,
                                             const SlotBits<kWords> &real, int T,
                                             const uint16_t *Ks, const uint16_t *Vh,
                                             const uint16_t *Vl, v4f &o, float &l) {
    const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
    // U of padded keys -> -inf, so that every score is an FMA result
#pragma unroll
    for (int kb = 0; kb < kT; kb += 2) {
        const uint32_t bits = real.pair(kb >> 1);
        if (kb < T && bits != 0 && bits != 0xffffffffu) {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const uint32_t kbits = bits >> (16 * t + 4 * g);
                u[kb + t].x = (kbits & 1) ? u[kb + t].x : -INFINITY;
                u[kb + t].y = (kbits & 2) ? u[kb + t].y : -INFINITY;
                u[kb + t].z = (kbits & 4) ? u[kb + t].z : -INFINITY;
                u[kb + t].w = (kbits & 8) ? u[kb + t].w : -INFINITY;
            }
        }
    }
    // scores over pairs of key blocks; a block without a real key has zero K
    // rows in LDS and U = -inf, so its scores are -inf
    float s[kT][4];
    float m = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < kT; kb += 2) {
        if (!pair_real(real, kb, T)) {
#pragma unroll
            for (int r = 0; r < 4; ++r) s[kb][r] = s[kb + 1][r] = -INFINITY;
            continue;
        }
        // lane group g holds reduction entries [hi | lo][8(g & 1) .. + 7]
        const v8h ka0 = *(const v8h *)(Ks + (kb * kTile + c) * 32 + 8 * g);
        const v8h ka1 = *(const v8h *)(Ks + ((kb + 1) * kTile + c) * 32 + 8 * g);
        v4f a0 = mfma32h(ka0, qh, (v4f){0.f, 0.f, 0.f, 0.f});
        v4f a1 = mfma32h(ka1, qh, (v4f){0.f, 0.f, 0.f, 0.f});
        a0 = mfma32h(ka0, ql, a0);
        a1 = mfma32h(ka1, ql, a1);
        s[kb][0] = fmaf(a0[0], qk_mul, u[kb].x);
        s[kb][1] = fmaf(a0[1], qk_mul, u[kb].y);
        s[kb][2] = fmaf(a0[2], qk_mul, u[kb].z);
        s[kb][3] = fmaf(a0[3], qk_mul, u[kb].w);
        s[kb + 1][0] = fmaf(a1[0], qk_mul, u[kb + 1].x);
        s[kb + 1][1] = fmaf(a1[1], qk_mul, u[kb + 1].y);
        s[kb + 1][2] = fmaf(a1[2], qk_mul, u[kb + 1].z);
        s[kb + 1][3] = fmaf(a1[3], qk_mul, u[kb + 1].w);
        m = fmaxf(m, max8(s[kb], s[kb + 1]));
    }
    m = xmax16(m);
    const float mb = m * kLog2e;
    float lsum = 0.f;
    o = (v4f){0.f, 0.f, 0.f, 0.f};
    // P V over the same pairs; V rows of blocks without a real key are 0
#pragma unroll
    for (int kb = 0; kb < kT; kb += 2) {
        if (!pair_real(real, kb, T)) continue;
        v8f p;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            p[r] = __builtin_amdgcn_exp2f(fmaf(s[kb][r], kLog2e, -mb));
            p[4 + r] = __builtin_amdgcn_exp2f(fmaf(s[kb + 1][r], kLog2e, -mb));
        }
        lsum += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
        const v8h vh = v_operand<false>(Vh, kb * kTile);
        const v8h vl = v_operand<false>(Vl, kb * kTile);
        v8h ph, pl;
        split_f16<8>(p, ph, pl);
        o = mfma32h(vh, pl, o);
        o = mfma32h(vl, ph, o);
        o = mfma32h(vh, ph, o);
    }
    l = xsum16(lsum);
}

}  // namespace pip

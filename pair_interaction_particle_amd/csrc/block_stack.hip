// block_stack.hip -- L masked biased-attention layers that reuse one pair
// bias U: the attention sublayer of the ParT encoder blocks ("Architecture
// Comparison" of the ml4sci_cms_e2e26 README: 8 ParT blocks, 8 heads; the
// bias enters every block's attention as in "Fusion 3").
//
// Per call:
//   prep   once: every layer's Wq, Wk, Wv, Wo becomes fp16 hi / lo MFMA A
//          operands (W^T tiles, 16 output columns x 32 inputs per operand),
//          each output column scaled by an exact power of two so that its
//          largest |w| lies in [2^13, 2^14); the inverse scales are kept.
//   per layer l:
//   attention  per (jet, head): Q_h, K_h, V_h = X W of the jet's rows on the
//          matrix cores, straight into the attention's LDS / register
//          layouts, then the biased attention with U -> O (B, H, P, 16);
//   out    X += O Wo[l] per block of rows.
// Q, K and V never reach HBM.
//
// Products run on the fp16 matrix cores with split operands (x = hi + lo and
// w = hi + lo, products hi.hi + hi.lo + lo.hi accumulated in fp32, relative
// product error ~2^-22).  Each input row is scaled by its own power of two
// (largest |x| into [2^13, 2^14)) before the split, so any magnitude keeps its
// relative accuracy, and the scale is undone exactly on the result.  Padded
// rows of X are never written.
#include "pip_attn_core.h"
#include "pip_internal.h"

namespace pip {

constexpr int kStackWaves = 4;
constexpr int kStackThreads = 64 * kStackWaves;
constexpr int kMaxC = 256;  // channels (C % 16 == 0, C <= 256)

// ------------------------------------------------------------ prep
// One workgroup per (layer, matrix, column tile nt).  Packed operand index:
// (((layer * 4 + m) * NT + nt) * KS + s) * 64 + lane, 8 halves each; slot j
// of lane l holds W[k = 32 s + 8 (l / 16) + j][n = 16 nt + l % 16] (0 for
// k >= C).
__global__ __launch_bounds__(kStackThreads) void stack_prep_kernel(
    const float *__restrict__ Wq, const float *__restrict__ Wk, const float *__restrict__ Wv,
    const float *__restrict__ Wo, int C, uint16_t *__restrict__ Ahi, uint16_t *__restrict__ Alo,
    float *__restrict__ colinv) {
    // Thread t converts operand elements idx = t + 256 i (i < KS * 2): all of
    // them in column c = (t / 8) % 16, so one round of loads (every load
    // issued before the first is used) gives both the column maximum and the
    // values to convert.
    constexpr int kMaxKS = kMaxC / 32, kPer = kMaxKS * 512 / kStackThreads;
    __shared__ float part[kStackThreads];
    __shared__ int partnan[kStackThreads];
    __shared__ float cs[16];
    const int NT = C / 16, KS = (C + 31) / 32;
    const int nt = blockIdx.x % NT, lm = blockIdx.x / NT, m = lm & 3, layer = lm >> 2;
    const float *W = (m == 0 ? Wq : m == 1 ? Wk : m == 2 ? Wv : Wo) + (size_t)layer * C * C;
    const int tid = threadIdx.x, col = (tid >> 3) & 15;
    const int n = KS * 512 / kStackThreads;  // elements of this thread (<= kPer)
    float w[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int idx = tid + kStackThreads * i;
        const int s = idx >> 9, lane = (idx >> 3) & 63, j = idx & 7;
        const int k = 32 * s + 8 * (lane >> 4) + j;
        w[i] = (i < n && k < C) ? W[(size_t)k * C + 16 * nt + col] : 0.f;
    }
    float mx = 0.f;
    int nan = 0;  // fmaxf drops NaN: a NaN column keeps scale 1
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        mx = fmaxf(mx, fabsf(w[i]));
        nan |= w[i] != w[i];
    }
    part[tid] = mx;
    partnan[tid] = nan;
    __syncthreads();
    if (tid < 16) {  // column tid: threads t with (t / 8) % 16 == tid
        float a = 0.f;
        int anynan = 0;
        for (int t = 8 * tid; t < kStackThreads; t += 128)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                a = fmaxf(a, part[t + e]);
                anynan |= partnan[t + e];
            }
        float sc, inv;
        pow2_scale(anynan ? __uint_as_float(0x7fc00000u) : a, sc, inv);
        cs[tid] = sc;
        colinv[(size_t)lm * C + 16 * nt + tid] = inv;
    }
    __syncthreads();
    const size_t base = ((size_t)lm * NT + nt) * KS * 512;
    const float sc = cs[col];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        if (i >= n) break;
        const int idx = tid + kStackThreads * i;
        const float x = w[i] * sc;
        const _Float16 hi = (_Float16)x;
        const _Float16 lo = (_Float16)(x - (float)hi);
        Ahi[base + idx] = __builtin_bit_cast(uint16_t, hi);
        Alo[base + idx] = __builtin_bit_cast(uint16_t, lo);
    }
}

// ------------------------------------------------------------ rows
// The workgroup's rows of one GEMM input live in LDS as float32 (row stride
// kXs); rsc holds each row's power-of-two scale.
template <int kKS>
struct RowsLds {
    static constexpr int kXs = kKS * 32 + 4;
};

// Split B operand of row block i at k-step s: lane (c, g) takes row c's
// inputs k = 32 s + 8 g .. + 7, scaled by the row's power of two.
template <int kKS>
__device__ __forceinline__ void b_operand(const float *Xs, const float *rsc, int i, int s,
                                          v8h &bh, v8h &bl) {
    constexpr int kXs = RowsLds<kKS>::kXs;
    const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
    const float *src = Xs + (16 * i + c) * kXs + 32 * s + 8 * g;
    const float4 a = *(const float4 *)src, b = *(const float4 *)(src + 4);
    const float sc = rsc[16 * i + c];
    const v8f x = {a.x * sc, a.y * sc, a.z * sc, a.w * sc, b.x * sc, b.y * sc, b.z * sc, b.w * sc};
    split_f16<8>(x, bh, bl);
}

// Row scales of the kRows rows in Xs (all kStackThreads threads; the caller
// synchronises before and after).  part is kStackThreads floats of scratch.
template <int kKS, int kRows>
__device__ __forceinline__ void row_scales(const float *Xs, float *part, float *rsc, float *rinv,
                                           int C) {
    constexpr int kXs = RowsLds<kKS>::kXs;
    constexpr int kPer = kStackThreads / kRows;  // threads per row
    const int tid = threadIdx.x, r = tid / kPer, q = tid % kPer;
    float mx = 0.f;
    for (int k = 4 * q; k < C; k += 4 * kPer) {
        const float4 v = *(const float4 *)(Xs + r * kXs + k);
        mx = fmaxf(mx, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    }
    part[tid] = mx;
    __syncthreads();
    if (tid < kRows) {
        float a = 0.f;
        for (int t = 0; t < kPer; ++t) a = fmaxf(a, part[tid * kPer + t]);
        float sc, inv;
        pow2_scale(a, sc, inv);
        rsc[tid] = sc;
        rinv[tid] = inv;
    }
}

// acc[j][i] (output tile j of this wave, row block i) = sum over k-steps of
// the split products; tile j is column tile tile0 + kStackWaves j of the
// packed matrix block starting at operand op0 (NT tiles).  The W operands of
// the next k-step load while the current step's MFMAs run.
template <int kKS, int kRB, int kJ>
__device__ __forceinline__ void first_operands(const v8h *__restrict__ Ahi,
                                               const v8h *__restrict__ Alo, size_t op0, int tile0,
                                               int ntiles, int KS, v8h (&ch)[kJ], v8h (&cl)[kJ]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
        const int t = tile0 + kStackWaves * j;
        const size_t o = (op0 + (size_t)(t < ntiles ? t : tile0) * KS) * 64 + lane;
        ch[j] = Ahi[o];
        cl[j] = Alo[o];
    }
}

// The W operands of every k-step (C <= 128: 64 registers), loaded together
// with the rows, so that the product never waits on L2.
template <int kKS, int kJ>
__device__ __forceinline__ void all_operands(const v8h *__restrict__ Ahi,
                                             const v8h *__restrict__ Alo, size_t op0, int tile0,
                                             int ntiles, int KS, v8h (&ch)[kJ][kKS],
                                             v8h (&cl)[kJ][kKS]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
        const int t = tile0 + kStackWaves * j;
#pragma unroll
        for (int s = 0; s < kKS; ++s) {
            const size_t o =
                (op0 + (size_t)(t < ntiles ? t : tile0) * KS + min(s, KS - 1)) * 64 + lane;
            ch[j][s] = Ahi[o];
            cl[j][s] = Alo[o];
        }
    }
}

// gemm_rows with every k-step's operands already in registers (all_operands).
template <int kKS, int kRB, int kJ>
__device__ __forceinline__ void gemm_rows_pre(int tile0, int ntiles, int KS, const float *Xs,
                                              const float *rsc, const bool (&any)[kRB],
                                              const v8h (&ch)[kJ][kKS],
                                              const v8h (&cl)[kJ][kKS], v4f (&acc)[kJ][kRB]) {
#pragma unroll
    for (int j = 0; j < kJ; ++j)
#pragma unroll
        for (int i = 0; i < kRB; ++i) acc[j][i] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kKS; ++s) {
        if (s >= KS) break;
#pragma unroll
        for (int i = 0; i < kRB; ++i) {
            if (!any[i]) continue;
            v8h bh, bl;
            b_operand<kKS>(Xs, rsc, i, s, bh, bl);
#pragma unroll
            for (int j = 0; j < kJ; ++j) {
                if (tile0 + kStackWaves * j >= ntiles) continue;
                acc[j][i] = mfma32h(ch[j][s], bl, acc[j][i]);
                acc[j][i] = mfma32h(cl[j][s], bh, acc[j][i]);
                acc[j][i] = mfma32h(ch[j][s], bh, acc[j][i]);
            }
        }
    }
}

// ch / cl: the operands of step 0 (first_operands), consumed.
template <int kKS, int kRB, int kJ>
__device__ __forceinline__ void gemm_rows(const v8h *__restrict__ Ahi, const v8h *__restrict__ Alo,
                                          size_t op0, int tile0, int ntiles, int KS,
                                          const float *Xs, const float *rsc, const bool (&any)[kRB],
                                          v8h (&ch)[kJ], v8h (&cl)[kJ], v4f (&acc)[kJ][kRB]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int j = 0; j < kJ; ++j)
#pragma unroll
        for (int i = 0; i < kRB; ++i) acc[j][i] = (v4f){0.f, 0.f, 0.f, 0.f};
    // operand index of tile j, step s (tiles past ntiles re-read tile0: never used)
    auto opi = [&](int j, int s) {
        const int t = tile0 + kStackWaves * j;
        return (op0 + (size_t)(t < ntiles ? t : tile0) * KS + s) * 64 + lane;
    };
#pragma unroll
    for (int s = 0; s < kKS; ++s) {
        if (s >= KS) break;
        v8h nh[kJ], nl[kJ];
        const int sn = s + 1 < KS ? s + 1 : s;
#pragma unroll
        for (int j = 0; j < kJ; ++j) {
            nh[j] = Ahi[opi(j, sn)];
            nl[j] = Alo[opi(j, sn)];
        }
#pragma unroll
        for (int i = 0; i < kRB; ++i) {
            if (!any[i]) continue;
            v8h bh, bl;
            b_operand<kKS>(Xs, rsc, i, s, bh, bl);
#pragma unroll
            for (int j = 0; j < kJ; ++j) {
                if (tile0 + kStackWaves * j >= ntiles) continue;
                acc[j][i] = mfma32h(ch[j], bl, acc[j][i]);
                acc[j][i] = mfma32h(cl[j], bh, acc[j][i]);
                acc[j][i] = mfma32h(ch[j], bh, acc[j][i]);
            }
        }
#pragma unroll
        for (int j = 0; j < kJ; ++j) {
            ch[j] = nh[j];
            cl[j] = nl[j];
        }
    }
}

// Cooperative float4 load of the workgroup's rows of a (rows, C) matrix,
// issued into registers (load) and stored to LDS later (store), so that the
// loads of several matrices overlap.  Zeros for rows past R and for the
// columns C .. 32 KS - 1 that the last k-step reads (there the packed W is 0
// too; the zero keeps 0 * NaN out).  head_major: the source is (B, H, P, 16)
// and row r's column k lives at ((b H + k / 16) P + p) 16 + k % 16.
template <int kKS, int kRows>
struct RowLoad {
    static constexpr int kXs = RowsLds<kKS>::kXs;
    static constexpr int kPer = 8 * kKS;  // float4 chunks per row
    static constexpr int kIt = (kRows * kPer + kStackThreads - 1) / kStackThreads;
    float4 v[kIt];

    // Every load is issued, at an address clamped into the matrix; what is
    // out of range is replaced by 0 only when stored (a conditional load
    // would make the compiler wait for it on the spot).
    __device__ __forceinline__ void load(const float *__restrict__ src, bool head_major, int row0,
                                         int R, int P, int C, int H) {
#pragma unroll
        for (int it = 0; it < kIt; ++it) {
            const int idx = threadIdx.x + it * kStackThreads;
            const int r = idx / kPer, row = min(row0 + r, R - 1);
            const int k = min(4 * (idx - r * kPer), C - 4);
            if (head_major) {
                const int b = row / P, p = row - b * P;
                v[it] = *(const float4 *)(src + (((size_t)b * H + (k >> 4)) * P + p) * 16 +
                                          (k & 15));
            } else {
                v[it] = *(const float4 *)(src + (size_t)row * C + k);
            }
        }
    }
    __device__ __forceinline__ void store(float *Xs, int row0, int R, int C) const {
#pragma unroll
        for (int it = 0; it < kIt; ++it) {
            const int idx = threadIdx.x + it * kStackThreads;
            const int r = idx / kPer, k = 4 * (idx - r * kPer);
            const bool in = row0 + r < R && k < C;
            if (idx < kRows * kPer)
                *(float4 *)(Xs + r * kXs + k) = in ? v[it] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
};

// X += O Wo for the workgroup's 16 kRB rows (O head-major (B, H, P, 16)).
template <int kKS, int kRB>
__global__ __launch_bounds__(kStackThreads)
__attribute__((amdgpu_waves_per_eu(kKS <= 4 ? 4 : 1))) void stack_out_kernel(
    float *__restrict__ X, const float *__restrict__ O, const v8h *__restrict__ Awhi,
    const v8h *__restrict__ Awlo, const float *__restrict__ ciw,
    const uint8_t *__restrict__ mask, int R, int P, int C, int H) {
    constexpr int kRows = 16 * kRB;
    constexpr int kXs = RowsLds<kKS>::kXs;
    constexpr int kJw = (2 * kKS + kStackWaves - 1) / kStackWaves;  // Wo tiles per wave
    __shared__ __attribute__((aligned(16))) float Xs[kRows * kXs];  // O rows
    __shared__ __attribute__((aligned(16))) float Xo[kRows * kXs];  // X rows
    __shared__ float part[kStackThreads], rsc[kRows], rinv[kRows];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, c = lane & 15;
    const int NT = C / 16, KS = (C + 31) / 32;
    const int row0 = blockIdx.x * kRows;

    // W operands of the first k-step, the mask bytes (address clamped: every
    // load issued before the first wait), the O and X rows
    // (C <= 128: every k-step's operands at once; beyond, one step ahead)
    constexpr bool kPre = kKS <= 4;
    v8h wh[kJw], wl[kJw], ah[kJw][kKS], al[kJw][kKS];
    if constexpr (kPre)
        all_operands<kKS, kJw>(Awhi, Awlo, (size_t)3 * NT * KS, wave, NT, KS, ah, al);
    else
        first_operands<kKS, kRB, kJw>(Awhi, Awlo, (size_t)3 * NT * KS, wave, NT, KS, wh, wl);
    int row[kRB];
    uint8_t mb[kRB];
#pragma unroll
    for (int i = 0; i < kRB; ++i) {
        row[i] = row0 + 16 * i + c;
        mb[i] = mask[min(row[i], R - 1)];
    }
    RowLoad<kKS, kRows> in0, in1;
    in0.load(O, true, row0, R, P, C, H);
    in1.load(X, false, row0, R, P, C, H);
    in0.store(Xs, row0, R, C);  // (the stores wait for every load)
    in1.store(Xo, row0, R, C);
    bool real[kRB], any[kRB];
#pragma unroll
    for (int i = 0; i < kRB; ++i) {
        real[i] = row[i] < R && mb[i] != 0;
        any[i] = __ballot(real[i]) != 0;
    }
    __syncthreads();
    row_scales<kKS, kRows>(Xs, part, rsc, rinv, C);
    __syncthreads();
    v4f acc[kJw][kRB];
    if constexpr (kPre)
        gemm_rows_pre<kKS, kRB, kJw>(wave, NT, KS, Xs, rsc, any, ah, al, acc);
    else
        gemm_rows<kKS, kRB, kJw>(Awhi, Awlo, (size_t)3 * NT * KS, wave, NT, KS, Xs, rsc, any, wh,
                                 wl, acc);
#pragma unroll
    for (int j = 0; j < kJw; ++j) {
        const int nt = wave + kStackWaves * j;
        if (nt >= NT) continue;
        const float4 ci = *(const float4 *)(ciw + 3 * C + 16 * nt + 4 * g);
#pragma unroll
        for (int i = 0; i < kRB; ++i) {
            if (!real[i]) continue;  // padded rows keep their bits
            float4 x = *(const float4 *)(Xo + (16 * i + c) * kXs + 16 * nt + 4 * g);
            const float ri = rinv[16 * i + c];
            x.x += acc[j][i][0] * ri * ci.x;
            x.y += acc[j][i][1] * ri * ci.y;
            x.z += acc[j][i][2] * ri * ci.z;
            x.w += acc[j][i][3] * ri * ci.w;
            *(float4 *)(X + (size_t)row[i] * C + 16 * nt + 4 * g) = x;
        }
    }
}

// ------------------------------------------------------------ attention
// One workgroup per (jet, head, group of 8 query blocks), 8 waves; the H x
// chunks workgroups of a jet share one XCD (block index modulo 8), so the
// jet's X rows are read from HBM once per layer.
//   1. The head's packed Q/K/V weight operands go to LDS (one load round
//      for the workgroup); wave w loads the X rows of row blocks w and w + 8
//      (every block below an even block count that holds a real row).
//   2. K_h, V_h (and Q_h of its own query block) of those rows on the fp16
//      matrix cores with split operands, every X row scaled by its own power
//      of two first.  Padded rows give 0.
//   3. The largest |K| and |V| of the head (and |Q| of each query block) pick
//      power-of-two scales that put them into [2^13, 2^14): the split fp16
//      operands of the attention can then neither overflow nor lose
//      relative accuracy, and the scales are undone exactly on the scores
//      and the output.  K and V go to LDS, Q through LDS into the
//      B-operand layout.
//   4. The U strip of the wave's query block is loaded once the projections
//      no longer hold registers; the attention core of pair_bias_attention
//      runs on it; O goes to the
//      head-major (B, H, P, 16) buffer the Wo step reads.
constexpr int kSaWaves = 8;
constexpr int kSaThreads = 64 * kSaWaves;

template <int kT, int kKS>
__global__ __launch_bounds__(kSaThreads) void stack_attention_kernel(
    const float *__restrict__ X, const v8h *__restrict__ Ahi, const v8h *__restrict__ Alo,
    const float *__restrict__ ci, const float *__restrict__ U, const uint8_t *__restrict__ mask,
    int B, int H, int P, int C, int chunks, float *__restrict__ O) {
    constexpr int kWords = (kT * 16 + 63) / 64;
    constexpr int kRbw = (kT + kSaWaves - 1) / kSaWaves;  // row blocks per wave
    // LDS: during the projections the head's packed Q/K/V weight operands
    // ([m][hi, lo][s][lane], read by all 8 waves); afterwards, in the same
    // bytes, K, V and the Q tiles of the attention.
    constexpr int kKsB = kT * 16 * 32 * 2, kVtB = kT * 16 * kVRow * 2, kQsB = kSaWaves * 16 * 20 * 4;
    constexpr int kWB = 3 * 2 * kKS * 64 * 16;
    constexpr int kAttnB = kKsB + 2 * kVtB + kQsB;
    static_assert(kKsB % 16 == 0 && kVtB % 16 == 0, "LDS sections stay 16-byte aligned");
    __shared__ __attribute__((aligned(16))) unsigned char smem[kAttnB > kWB ? kAttnB : kWB];
    __shared__ float kvmax[2][kSaWaves];
    uint16_t *Ks = (uint16_t *)smem;
    uint16_t *Vsh = (uint16_t *)(smem + kKsB);  // V hi / lo, row-major
    uint16_t *Vsl = (uint16_t *)(smem + kKsB + kVtB);
    float (*Qs)[16][20] = (float (*)[16][20])(smem + kKsB + 2 * kVtB);
    v8h *Ws = (v8h *)smem;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, c = lane & 15;
    // XCD-aware decode: block i runs on XCD i % 8; XCD x takes jets x, x+8, ...
    const int per_jet = H * chunks;
    const int xcd = blockIdx.x & 7, t = blockIdx.x >> 3;
    const int jet = xcd + 8 * (t / per_jet), sub = t - (t / per_jet) * per_jet;
    if (jet >= B) return;
    const int h = sub / chunks, chunk = sub - h * chunks;
    const int T = P / kTile, NT = C / 16, KS = (C + 31) / 32;
    const size_t base = ((size_t)jet * H + h) * P;

    SlotBits<kWords> real;
    real.load(mask + (size_t)jet * P, P);
    const int nst = T + (T & 1);  // key blocks staged (zeros past the real ones)

    // ---- 1. X rows of this wave's row blocks, then the U strip
    float xv[kRbw][kKS][8];
#pragma unroll
    for (int t2 = 0; t2 < kRbw; ++t2) {
        const int rb = wave + kSaWaves * t2;
        const bool need = rb < T && real.block_rt(rb) != 0;
        const float *xr = X + ((size_t)jet * P + (need ? rb * kTile + c : 0)) * C;
#pragma unroll
        for (int s = 0; s < kKS; ++s) {
            const int k0 = 32 * s + 8 * g;
            const int off = (s < KS && k0 < C) ? k0 : 0;  // in range; unused when not needed
            const float4 a = *(const float4 *)(xr + off), b = *(const float4 *)(xr + off + 4);
            xv[t2][s][0] = a.x; xv[t2][s][1] = a.y; xv[t2][s][2] = a.z; xv[t2][s][3] = a.w;
            xv[t2][s][4] = b.x; xv[t2][s][5] = b.y; xv[t2][s][6] = b.z; xv[t2][s][7] = b.w;
        }
    }
    const int qb = chunk * kSaWaves + wave, q0 = qb * kTile;
    const bool qact = qb < T && real.block_rt(qb) != 0;

    // the head's weight operands into LDS, every load issued before the first
    // store (one L2 round trip per workgroup instead of one per K step and wave)
    {
        constexpr int kW = 3 * 2 * kKS * 64;  // v8h operands
        constexpr int kIt = (kW + kSaThreads - 1) / kSaThreads;
        v8h wv[kIt];
#pragma unroll
        for (int it = 0; it < kIt; ++it) {
            const int i = min(tid + it * kSaThreads, kW - 1);
            const int m = i / (2 * kKS * 64), hl = (i / (kKS * 64)) & 1;
            const int s = (i / 64) % kKS, l = i & 63;
            const size_t o = ((size_t)(m * NT + h) * KS + min(s, KS - 1)) * 64 + l;
            wv[it] = hl ? Alo[o] : Ahi[o];
        }
#pragma unroll
        for (int it = 0; it < kIt; ++it)
            if (tid + it * kSaThreads < kW) Ws[tid + it * kSaThreads] = wv[it];
    }
    __syncthreads();
    // operand (m, hi / lo, s) of this lane
    auto wop = [&](int m, int hl, int s) { return Ws[((m * 2 + hl) * kKS + s) * 64 + lane]; };

    // ---- 2. projections
    v4f kt[kRbw], vt[kRbw], qt = {0.f, 0.f, 0.f, 0.f};
    float kmx = 0.f, vmx = 0.f;
#pragma unroll
    for (int t2 = 0; t2 < kRbw; ++t2) {
        const int rb = wave + kSaWaves * t2;
        kt[t2] = vt[t2] = (v4f){0.f, 0.f, 0.f, 0.f};
        if (!(rb < T && real.block_rt(rb) != 0)) continue;
        const bool isq = rb == qb;
        // this row's power of two, then the split operands
        float amax = 0.f;
#pragma unroll
        for (int s = 0; s < kKS; ++s)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (s < KS && 32 * s + 8 * g + j < C) amax = fmaxf(amax, fabsf(xv[t2][s][j]));
        amax = xmax16(amax);
        float rs, ri;
        pow2_scale(amax, rs, ri);
        v4f ak = {0.f, 0.f, 0.f, 0.f}, av = ak, aq = ak;
#pragma unroll
        for (int s = 0; s < kKS; ++s) {
            if (s >= KS) break;
            v8f x;
#pragma unroll
            for (int j = 0; j < 8; ++j) x[j] = 32 * s + 8 * g + j < C ? xv[t2][s][j] * rs : 0.f;
            v8h bh, bl;
            split_f16<8>(x, bh, bl);
            const v8h kh = wop(1, 0, s), kl = wop(1, 1, s), vh = wop(2, 0, s), vl = wop(2, 1, s);
            ak = mfma32h(kh, bl, ak);
            av = mfma32h(vh, bl, av);
            ak = mfma32h(kl, bh, ak);
            av = mfma32h(vl, bh, av);
            ak = mfma32h(kh, bh, ak);
            av = mfma32h(vh, bh, av);
            if (isq) {
                const v8h qh = wop(0, 0, s), ql = wop(0, 1, s);
                aq = mfma32h(qh, bl, aq);
                aq = mfma32h(ql, bh, aq);
                aq = mfma32h(qh, bh, aq);
            }
        }
        // lane (c, g) holds row c, head columns 4g .. 4g+3; padded rows -> 0
        const bool rr = real.slot(rb * kTile + c);
        const float4 ck = *(const float4 *)(ci + C + 16 * h + 4 * g);
        const float4 cv = *(const float4 *)(ci + 2 * C + 16 * h + 4 * g);
        const float cka[4] = {ck.x, ck.y, ck.z, ck.w}, cva[4] = {cv.x, cv.y, cv.z, cv.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            kt[t2][r] = rr ? ak[r] * ri * cka[r] : 0.f;
            vt[t2][r] = rr ? av[r] * ri * cva[r] : 0.f;
            kmx = fmaxf(kmx, fabsf(kt[t2][r]));
            vmx = fmaxf(vmx, fabsf(vt[t2][r]));
        }
        if (isq) {
            const float4 cq = *(const float4 *)(ci + 16 * h + 4 * g);
            const float cqa[4] = {cq.x, cq.y, cq.z, cq.w};
#pragma unroll
            for (int r = 0; r < 4; ++r) qt[r] = rr ? aq[r] * ri * cqa[r] : 0.f;
        }
    }
    // the U strip, issued once the projections no longer need registers
    float4 u[kT];
    {
        const int zero = P >> 16;  // 0, opaque to the compiler (P <= 256)
        const float *urow = U + (base + (qact ? q0 + c : 0)) * P;
#pragma unroll
        for (int kb = 0; kb < kT; kb += 2) {
            // (half a pair lies past an odd block count: clamped, masked)
            const bool need = qact && kb < T && real.pair(kb >> 1) != 0;
            // natural key order: 4 keys 16 kb + 4g .. of each block
            const int o0 = 16 * kb + 4 * g, o1 = o0 + 16;
            u[kb] = *(const float4 *)(urow + min(need ? o0 : o0 * zero, P - 4));
            u[kb + 1] = *(const float4 *)(urow + min(need ? o1 : o1 * zero, P - 4));
        }
    }

    kmx = wave_max(kmx);
    vmx = wave_max(vmx);
    if (lane == 0) {
        kvmax[0][wave] = kmx;
        kvmax[1][wave] = vmx;
    }
    __syncthreads();

    // ---- 3. head scales; K, V to LDS; Q through LDS
    float km = 0.f, vm = 0.f;
#pragma unroll
    for (int w = 0; w < kSaWaves; ++w) {
        km = fmaxf(km, kvmax[0][w]);
        vm = fmaxf(vm, kvmax[1][w]);
    }
    float ksc, kinv, vsc, vinv;
    pow2_scale(km, ksc, kinv);
    pow2_scale(vm, vsc, vinv);
#pragma unroll
    for (int t2 = 0; t2 < kRbw; ++t2) {
        const int rb = wave + kSaWaves * t2;
        if (rb >= nst) continue;
        const int k = rb * kTile + c;
        const float4 kk = make_float4(kt[t2][0] * ksc, kt[t2][1] * ksc, kt[t2][2] * ksc,
                                      kt[t2][3] * ksc);
        const float4 vv = make_float4(vt[t2][0] * vsc, vt[t2][1] * vsc, vt[t2][2] * vsc,
                                      vt[t2][3] * vsc);
        v4h kh, kl, vh, vl;
        split4_f16(kk, kh, kl);
        split4_f16(vv, vh, vl);
        *(v4h *)(Ks + k * 32 + 4 * g) = kh;
        *(v4h *)(Ks + k * 32 + 16 + 4 * g) = kl;
        *(v4h *)(Vsh + k * kVRow + 4 * g) = vh;
        *(v4h *)(Vsl + k * kVRow + 4 * g) = vl;
    }
    float qinv = 1.f;
    if (qact) {
        float qsc;
        pow2_scale(wave_max(fmaxf(fmaxf(fabsf(qt[0]), fabsf(qt[1])),
                                  fmaxf(fabsf(qt[2]), fabsf(qt[3])))),
                   qsc, qinv);
        *(float4 *)&Qs[wave][c][4 * g] =
            make_float4(qt[0] * qsc, qt[1] * qsc, qt[2] * qsc, qt[3] * qsc);
    }
    __syncthreads();

    // ---- 4. attention of this wave's query block
    if (qb >= T) return;
    float *orow = O + (base + q0 + c) * 16 + 4 * g;
    if (!qact) {
        *(float4 *)orow = make_float4(0.f, 0.f, 0.f, 0.f);
        return;
    }
#pragma unroll
    for (int kb = 0; kb < kT; ++kb)
        if (!pair_real(real, kb & ~1, T)) u[kb] = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
    v8h qh, ql;
    {
        const float4 a = *(const float4 *)&Qs[wave][c][8 * (g & 1)];
        const float4 b = *(const float4 *)&Qs[wave][c][8 * (g & 1) + 4];
        v4h h0, l0, h1, l1;
        split4_f16(a, h0, l0);
        split4_f16(b, h1, l1);
        qh = __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7);
        ql = __builtin_shufflevector(l0, l1, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    v4f o;
    float l;
    attend_split<kT>(u, qh, ql, 0.25f * kinv * qinv, real, T, Ks, Vsh, Vsl, o, l);
    const float inv = vinv / l;
    *(float4 *)orow = real.slot(q0 + c)
                          ? make_float4(o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv)
                          : make_float4(0.f, 0.f, 0.f, 0.f);
}

// ------------------------------------------------------------ launch
static size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// Workspace: O (B, H, P, 16) floats, then the hi and lo operands of every
// layer, then the column scales, each section 256-byte aligned.
size_t block_stack_workspace(int B, int P, int C, int L) {
    const size_t act = align256((size_t)B * P * C * sizeof(float));
    const size_t ops = align256((size_t)L * 4 * (C / 16) * ((C + 31) / 32) * 512 * 2);
    const size_t sc = align256((size_t)L * 4 * C * sizeof(float));
    return act + 2 * ops + sc;
}

// Operands of one layer inside the packed buffers.
struct StackOps {
    const v8h *hi, *lo;
    const float *ci;
};

hipError_t launch_block_stack(float *X, const float *Wq, const float *Wk, const float *Wv,
                              const float *Wo, const float *U, const uint8_t *mask, int B,
                              int P, int C, int H, int L, void *ws, hipStream_t s) {
    const int NT = C / 16, KS = (C + 31) / 32, R = B * P;
    const size_t act = align256((size_t)B * P * C * sizeof(float));
    const size_t ops = align256((size_t)L * 4 * NT * KS * 512 * 2);
    char *w = (char *)ws;
    float *O = (float *)w;
    uint16_t *Ahi = (uint16_t *)(w + act), *Alo = (uint16_t *)(w + act + ops);
    float *ci = (float *)(w + act + 2 * ops);

    hipLaunchKernelGGL(stack_prep_kernel, dim3(L * 4 * NT), dim3(kStackThreads), 0, s, Wq, Wk,
                       Wv, Wo, C, Ahi, Alo, ci);
    const size_t lop = (size_t)4 * NT * KS * 64;  // v8h operands per layer
    auto layer_ops = [&](int l) {
        return StackOps{(const v8h *)Ahi + (size_t)l * lop, (const v8h *)Alo + (size_t)l * lop,
                        ci + (size_t)l * 4 * C};
    };
    const int chunks = (P / kTile + kSaWaves - 1) / kSaWaves;
    const unsigned sa_grid = (unsigned)(8 * ((B + 7) / 8) * H * chunks);
    for (int l = 0; l < L; ++l) {
        const StackOps o = layer_ops(l);
        if (P <= 128 && KS <= 4)
            hipLaunchKernelGGL((stack_attention_kernel<8, 4>), dim3(sa_grid), dim3(kSaThreads), 0,
                               s, X, o.hi, o.lo, o.ci, U, mask, B, H, P, C, chunks, O);
        else if (KS <= 4)
            hipLaunchKernelGGL((stack_attention_kernel<16, 4>), dim3(sa_grid), dim3(kSaThreads),
                               0, s, X, o.hi, o.lo, o.ci, U, mask, B, H, P, C, chunks, O);
        else if (P <= 128)
            hipLaunchKernelGGL((stack_attention_kernel<8, 8>), dim3(sa_grid), dim3(kSaThreads), 0,
                               s, X, o.hi, o.lo, o.ci, U, mask, B, H, P, C, chunks, O);
        else
            hipLaunchKernelGGL((stack_attention_kernel<16, 8>), dim3(sa_grid), dim3(kSaThreads),
                               0, s, X, o.hi, o.lo, o.ci, U, mask, B, H, P, C, chunks, O);
        // X += O Wo[l]
        if (KS <= 4)
            hipLaunchKernelGGL((stack_out_kernel<4, 1>), dim3((unsigned)((R + 15) / 16)),
                               dim3(kStackThreads), 0, s, X, O, o.hi, o.lo, o.ci, mask, R, P, C,
                               H);
        else
            hipLaunchKernelGGL((stack_out_kernel<8, 1>), dim3((unsigned)((R + 15) / 16)),
                               dim3(kStackThreads), 0, s, X, O, o.hi, o.lo, o.ci, mask, R, P, C,
                               H);
    }
    return hipGetLastError();
}

}  // namespace pip

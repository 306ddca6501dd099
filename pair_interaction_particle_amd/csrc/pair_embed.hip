// pair_embed.hip -- pair features and the fused features + pair-MLP kernels.
//
// "Event Classification with Masked Transformer Autoencoders"
// (ml4sci_cms_e2e26 README), "How the Kernel Fusion Works", Fusion 2: the
// four pair features and the whole 4-layer MLP run in one launch, hidden
// states stay on chip, and only the (B, H, P, P) bias is written.
//
// Work decomposition (gfx950).  U is symmetric in (a, b) because every
// feature is, so only the lower triangle of 16x16 tiles (I >= J) is computed
// and every value is written twice (U[a][b] and U[b][a]) straight from
// registers.  The kernel is persistent: two 512-thread workgroups per CU, each
// staging the packed MLP weights in LDS once and taking an equal share of the
// batch's estimated work (counted from the mask in-kernel); the first
// workgroup of each CU also takes a share of the all-padding tiles, which only
// get zeros.  A workgroup stages the
// particle kinematics (float64) of the jets its share touches in LDS, two jets
// at a time.  Inside a tile the unit of work is a pair block of 16 pairs = the
// 16 columns of one 16x16 MFMA: off-diagonal tiles have 16 (one per row),
// diagonal tiles pack their 136 unique pairs into 9 (plus an empty 10th).
// Each of the 8 waves pushes two pair blocks at a time through the MFMA layer
// chain; hidden activations never leave registers.
//
// The same kernel takes a packed batch (jets back to back, no padding: the
// layout of packed_embed.hip).  A packed jet of n particles has exactly
// ceil(n/16) active blocks with its real slots first, so the work estimate
// is exact; U is written into the jet's (8, n, ld) block, guarded to its n
// rows and ld columns, and there are no zero tiles.  (The earlier packed
// kernel dealt single tiles with one barrier per tile: 70.6 us against
// 57.6 us here on the kernel workload's jets, bit-identical U.)
#include <algorithm>
#include <type_traits>

#include "pip_internal.h"
#include "pip_mlp.h"
#include "pip_packed.h"

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
        const float4 pv = p4[idx];  // both loads issued before either is used
        const uint8_t mb = mask[idx];
        __asm__ volatile("" ::: "memory");
        const int real = mb != 0;
        stage_particle(L, t, real ? pv : make_float4(0.f, 0.f, 0.f, 0.f), real);
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
__device__ __forceinline__ void store4(float *U, uint32_t off, const float (&v)[4]) {
    *(float4 *)(U + off) = make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint32_t bf16_pair(float a, float b) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)a) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)b) << 16);
}
__device__ __forceinline__ void store4(uint16_t *U, uint32_t off, const float (&v)[4]) {
    *(uint2 *)(U + off) = make_uint2(bf16_pair(v[0], v[1]), bf16_pair(v[2], v[3]));
}

constexpr int kEmbedThreads = 512;
constexpr int kEmbedWaves = kEmbedThreads / 64;
constexpr int kWgPerCu = 1024 / kEmbedThreads;
static_assert((kEmbedWaves & (kEmbedWaves - 1)) == 0, "the sweep rotates waves modulo a power of two");

// Zero tile (I, J) of every head and, if I != J, its transpose (J, I), by
// 512 threads (t = 0 .. 511): one 16-byte store per thread and direction.
template <typename OutT>
__device__ inline void zero_tile(OutT *U, int P, int I, int J, int tid) {
    const float z[4] = {0.f, 0.f, 0.f, 0.f};
    const int h = tid >> 6, i = (tid >> 2) & 15, j0 = (tid & 3) * 4;
    store4(U, ((uint32_t)h * P + I * kTile + i) * P + J * kTile + j0, z);
    if (I != J) store4(U, ((uint32_t)h * P + J * kTile + i) * P + I * kTile + j0, z);
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

// Bit t set when 16-block t of a mask row holds a real particle (row 16-byte
// aligned, read as T 16-byte vectors).  All loads are issued before the
// first is looked at (addresses clamped into the row): one memory round trip
// instead of T.
__device__ __forceinline__ uint32_t jet_activity(const uint8_t *__restrict__ mrow, int T) {
    constexpr int kMaxT = kMaxP / kTile;
    uint4 v[kMaxT];
#pragma unroll
    for (int t = 0; t < kMaxT; ++t) v[t] = ((const uint4 *)mrow)[min(t, T - 1)];
    uint32_t act = 0;
#pragma unroll
    for (int t = 0; t < kMaxT; ++t)
        if (t < T && (v[t].x | v[t].y | v[t].z | v[t].w)) act |= 1u << t;
    return act;
}

// index of the k-th set bit of act (k < popcount(act))
__device__ __forceinline__ int nth_bit(uint32_t act, int k) {
    for (int i = 0; i < k; ++i) act &= act - 1;
    return __builtin_ctz(act);
}

// Pair blocks of a jet's active-tile triangle, in tile order: tile (ia, ja)
// of the active blocks (ja <= ia) has 16 blocks off the diagonal and 10 on
// it (9 hold its 136 unique pairs, the 10th is empty so that every tile has
// an even count and a wave's two blocks are always rows 2m, 2m+1 of one
// tile), so the blocks before row ia number 8 ia (ia - 1) + 10 ia.
__device__ __forceinline__ int blocks_before_row(int ia) { return 8 * ia * (ia - 1) + 10 * ia; }
__device__ __forceinline__ int blocks_before(int kt) {
    const int ia = tri_row(kt), ja = kt - ia * (ia + 1) / 2;
    return blocks_before_row(ia) + 16 * ja;
}

// Flat pair block q of the jet with activity act -> tile (I, J) and the pair
// (i, j) lane `lane` computes; false for the unused slots of a diagonal tile.
__device__ __forceinline__ bool flat_pair(uint32_t act, int q, int lane, int &I, int &J, int &i,
                                          int &j) {
    int ia = (int)((sqrtf(4.0f + 32.0f * (float)q) - 2.0f) * 0.0625f);
    while (blocks_before_row(ia + 1) <= q) ++ia;
    while (blocks_before_row(ia) > q) --ia;
    const int rem = q - blocks_before_row(ia);
    const int ja = min(rem / 16, ia);
    I = nth_bit(act, ia);
    J = nth_bit(act, ja);
    return block_pair(ia == ja, rem - 16 * ja, ia == ja ? 10 : 16, lane, i, j);
}

constexpr uint8_t kNoPair = 0x0f;

// Active block indices of a jet, 4 bits each (entry k = k-th set bit of act).
__device__ __forceinline__ uint64_t active_index(uint32_t act) {
    uint64_t idx = 0;
    for (int k = 0; act; ++k, act &= act - 1) idx |= (uint64_t)__builtin_ctz(act) << (4 * k);
    return idx;
}
__device__ __forceinline__ int nth_active(uint64_t idx, int k) { return (int)(idx >> (4 * k)) & 15; }

__device__ __forceinline__ int active_tiles(uint32_t act) {
    const int a = __popc(act);
    return a * (a + 1) / 2;
}

// Offsets inside one jet's U block (8 P^2 <= 2^19 elements) are 32-bit, so
// the stores take the jet base from scalar registers plus a 32-bit lane offset.
__device__ __forceinline__ void store_u(float *U, uint32_t off, float v) { U[off] = v; }
__device__ __forceinline__ void store_u(uint16_t *U, uint32_t off, float v) {
    U[off] = __builtin_bit_cast(uint16_t, (__bf16)v);
}

// Write the result of one pair block from registers: lane l < 32 holds the
// values of heads 4(l/16) + q for the pair (i, j) of tile (I, J); each value
// goes to U[h][a][b] and to its mirror U[h][b][a] (once when a == b), as
// exact 0 when a or b is padded.
template <typename OutT, class PL>
__device__ __forceinline__ void write_block(const PL &L, OutT *U, int P, int I, int J, bool valid,
                                           int i, int j, const v4f &u, bool zero) {
    const int lane = threadIdx.x & 63;
    if (lane >= 32 || !valid) return;
    const int a = I * kTile + i, b = J * kTile + j;
    const bool real = !zero && L.real[a] && L.real[b];
    const uint32_t pp = (uint32_t)P * P;
    const uint32_t h0 = (lane >> 4) * 4 * pp;
    const uint32_t oab = h0 + (uint32_t)a * P + b, oba = h0 + (uint32_t)b * P + a;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float v = real ? u[q] : 0.0f;
        store_u(U, oab + q * pp, v);
        if (a != b) store_u(U, oba + q * pp, v);
    }
}

__device__ __forceinline__ void store_u2(float *U, uint32_t off, float a, float b) {
    *(float2 *)(U + off) = make_float2(a, b);
}
__device__ __forceinline__ void store_u2(uint16_t *U, uint32_t off, float a, float b) {
    *(uint32_t *)(U + off) = bf16_pair(a, b);
}

// Write two blocks that are rows a0 = I*16 + 2m and a0 + 1 of off-diagonal
// tile (I, J): lane l < 32 holds heads 4(l/16) + q for column b = J*16 + l%16.
// Direct rows are 64-byte segments across the lanes; the mirrored pair
// U[h][b][a0..a0+1] is one 8-byte store per lane.
template <typename OutT, class PL>
__device__ __forceinline__ void write_row_pair(const PL &L, OutT *U, int P, int a0, int b,
                                              const v4f &uA, const v4f &uB, bool zero) {
    const int lane = threadIdx.x & 63;
    if (lane >= 32) return;
    const bool rb = !zero && L.real[b];
    const bool rA = rb && L.real[a0], rB = rb && L.real[a0 + 1];
    const uint32_t pp = (uint32_t)P * P;
    const uint32_t h0 = (lane >> 4) * 4 * pp;
    const uint32_t oab = h0 + (uint32_t)a0 * P + b, oba = h0 + (uint32_t)b * P + a0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float vA = rA ? uA[q] : 0.0f, vB = rB ? uB[q] : 0.0f;
        store_u(U, oab + q * pp, vA);
        store_u(U, oab + q * pp + P, vB);
        store_u2(U, oba + q * pp, vA, vB);
    }
}

// ---- packed batches (jets back to back, no padding)
// The padded kernel below also takes a packed batch (PackedArgs.cu set): jet
// b's particles are rows cu[b] .. cu[b+1]-1 of p4, all real, and its bias is
// the (8, n, ld) block at element 8 u_off[b], ld = n rounded up to 8.  A jet
// whose entries are inconsistent (packed_jet_ok) counts as empty: it gets no
// pair blocks and nothing of it is written.
struct PackedArgs {
    const int *cu;
    const int64_t *uoff;
    int N, max_n;
    int64_t u_elems;
};
// real count n of packed jet b (0 when inconsistent), first row, U offset
__device__ __forceinline__ int packed_jet(const PackedArgs &pk, int b, int &start, int64_t &u0) {
    int n;
    const bool ok = packed_jet_ok(pk.cu, pk.uoff, b, pk.N, pk.max_n, pk.u_elems, kHeads, n);
    start = pk.cu[b];
    u0 = pk.uoff[b];
    return ok ? n : 0;
}

// The packed forms of write_row_pair / write_block: rows are n long with
// stride ld and planes of n ld elements; nothing is written in row a >= n
// (the next jet's) or column >= ld, and the columns n .. ld-1 of a row get
// zeros (their pairs are not real).  ld is a multiple of 8 and a0 even, so
// a mirrored pair (a0, a0 + 1) lies inside a row whenever a0 < ld.
template <typename OutT, class PL>
__device__ __forceinline__ void write_row_pair_packed(const PL &L, OutT *U, int n, int ld,
                                                     uint32_t plane, int a0, int b,
                                                     const v4f &uA, const v4f &uB, bool zero) {
    const int lane = threadIdx.x & 63;
    if (lane >= 32) return;
    const bool rb = !zero && L.real[b];
    const bool rA = rb && L.real[a0], rB = rb && L.real[a0 + 1];
    const bool dA = a0 < n && b < ld, dB = a0 + 1 < n && b < ld, mir = b < n && a0 < ld;
    const uint32_t h0 = (lane >> 4) * 4 * plane;
    const uint32_t oab = h0 + (uint32_t)a0 * ld + b, oba = h0 + (uint32_t)b * ld + a0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float vA = rA ? uA[q] : 0.0f, vB = rB ? uB[q] : 0.0f;
        if (dA) store_u(U, oab + q * plane, vA);
        if (dB) store_u(U, oab + q * plane + ld, vB);
        if (mir) store_u2(U, oba + q * plane, vA, vB);
    }
}
template <typename OutT, class PL>
__device__ __forceinline__ void write_block_packed(const PL &L, OutT *U, int n, int ld,
                                                  uint32_t plane, int I, int J, bool valid,
                                                  int i, int j, const v4f &u, bool zero) {
    const int lane = threadIdx.x & 63;
    if (lane >= 32 || !valid) return;
    const int a = I * kTile + i, b = J * kTile + j;
    const bool real = !zero && L.real[a] && L.real[b];
    const bool d = a < n && b < ld, mir = a != b && b < n && a < ld;
    const uint32_t h0 = (lane >> 4) * 4 * plane;
    const uint32_t oab = h0 + (uint32_t)a * ld + b, oba = h0 + (uint32_t)b * ld + a;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float v = real ? u[q] : 0.0f;
        if (d) store_u(U, oab + q * plane, v);
        if (mir) store_u(U, oba + q * plane, v);
    }
}

// ---- work estimate for the balanced split
// A CU's time follows the wave iterations (pairs of blocks) it runs and the
// jets it starts: an iteration that holds a real pair runs the MLP, an
// all-padding one only walks the tile and stores zeros, and every jet costs
// a staging round (particles, barriers).  The weights below are a least-
// squares fit of per-CU end times (s_memtime) to those counts: float32
// 0.51 us per real iteration, ~0 per padding one and 1.6 us per jet; bf16
// 0.63, 0.15 and 0.67 us.  The estimate takes the real slots of a jet to
// come first (the usual layout):
// the ia-th active block then holds r = min(16, n - 16 ia) real rows (at least
// 1), an off-diagonal tile of its rows has ceil(r / 2) real iterations of 8,
// and its diagonal tile min(5, ceil(r (r + 1) / 64)) of 5.  Any other layout
// only moves the split points; every iteration is still done exactly once.
template <int kMode>
struct WorkCost {  // relative cost of a real and an all-padding iteration, and of a jet
    static constexpr bool kLow = kMode == kMlpBf16 || kMode == kMlpInt8;
    static constexpr int kReal = kLow ? 4 : 5, kPad = 1, kJet = kLow ? 4 : 15;
};

struct JetInfo {
    uint32_t act;  // bit t: block t holds a real slot
    int n;         // real slots
};
// a packed jet of n real slots (all first): blocks 0 .. ceil(n/16)-1 active
__device__ __forceinline__ JetInfo packed_info(int n) {
    const int T = (n + kTile - 1) / kTile;  // <= 16
    return JetInfo{(1u << T) - 1u, n};
}
// bit k set when byte k of x is nonzero (k < 4)
__device__ __forceinline__ uint32_t nonzero_bytes(uint32_t x) {
    x |= x >> 4;
    x |= x >> 2;
    x |= x >> 1;
    x &= 0x01010101u;
    return (x | (x >> 7) | (x >> 14) | (x >> 21)) & 0xfu;
}
// Every load is issued before the first is looked at (addresses clamped into
// the row): one memory round trip.
__device__ __forceinline__ JetInfo jet_info(const uint8_t *__restrict__ mrow, int T) {
    constexpr int kMaxT = kMaxP / kTile;
    uint4 v[kMaxT];
#pragma unroll
    for (int t = 0; t < kMaxT; ++t) v[t] = ((const uint4 *)mrow)[min(t, T - 1)];
    JetInfo j = {0u, 0};
#pragma unroll
    for (int t = 0; t < kMaxT; ++t) {
        const int c = __popc(nonzero_bytes(v[t].x) | nonzero_bytes(v[t].y) << 4 |
                             nonzero_bytes(v[t].z) << 8 | nonzero_bytes(v[t].w) << 12);
        if (t < T && c) {
            j.act |= 1u << t;
            j.n += c;
        }
    }
    return j;
}
// The jet of a 16-lane group: lane t of the group holds 16-byte block t of the
// mask row (t < T); every lane of the group returns the jet's info.  Call with
// the whole wave active.
__device__ __forceinline__ JetInfo jet_info16(uint4 v, int T) {
    const int lane = threadIdx.x & 63, t = lane & 15;
    // (computed for every lane and then scaled, so that the load it depends on
    // is not sunk into a branch, which would make the wait counter drain)
    const int c = __popc(nonzero_bytes(v.x) | nonzero_bytes(v.y) << 4 | nonzero_bytes(v.z) << 8 |
                         nonzero_bytes(v.w) << 12) *
                  (int)(t < T);
    JetInfo j;
    j.act = (uint32_t)(__ballot(c != 0) >> (lane & ~15)) & 0xffffu;
    int n = c;
    n += __shfl_xor(n, 1);
    n += __shfl_xor(n, 2);
    n += __shfl_xor(n, 4);
    n += __shfl_xor(n, 8);
    j.n = n;
    return j;
}
__device__ __forceinline__ int est_rows(int n, int ia) { return max(1, min(16, n - 16 * ia)); }
__device__ __forceinline__ int est_diag_real(int r) { return min(5, (r * (r + 1) / 2 + 31) >> 5); }
template <class C>
__device__ __forceinline__ int est_off_cost(int r) {
    return 8 * C::kPad + (C::kReal - C::kPad) * ((r + 1) >> 1);
}
template <class C>
__device__ __forceinline__ int est_diag_cost(int r) {
    return 5 * C::kPad + (C::kReal - C::kPad) * est_diag_real(r);
}
template <class C>
__device__ __forceinline__ int est_row_cost(int n, int ia) {
    const int r = est_rows(n, ia);
    return ia * est_off_cost<C>(r) + est_diag_cost<C>(r);
}
template <class C>
__device__ __forceinline__ int jet_cost(JetInfo j) {
    int c = 0;
    const int a = __popc(j.act);
    for (int ia = 0; ia < a; ++ia) c += est_row_cost<C>(j.n, ia);
    return a ? c + C::kJet : 0;
}
// The flat block index (even) of the first iteration of the jet whose cost
// prefix reaches tl (0 <= tl < jet_cost(j); the jet's own cost comes first).
template <class C>
__device__ __forceinline__ int jet_split(JetInfo j, int tl) {
    tl = max(tl - C::kJet, 0);
    int ia = 0, acc = 0;
    for (;; ++ia) {
        const int rc = est_row_cost<C>(j.n, ia);
        if (tl < acc + rc) break;
        acc += rc;
    }
    const int r = est_rows(j.n, ia), oc = est_off_cost<C>(r);
    int rem = tl - acc, first, n;
    bool diag;
    if (rem < ia * oc) {
        const int ja = rem / oc;
        rem -= ja * oc;
        first = blocks_before_row(ia) + 16 * ja;
        n = 8;
        diag = false;
    } else {
        rem -= ia * oc;
        first = blocks_before_row(ia) + 16 * ia;
        n = 5;
        diag = true;
    }
    // the smallest iteration whose cost prefix inside the tile reaches rem
    const int dr = est_diag_real(r);
    int k = 0, pre = 0;
    while (k < n && pre < rem) {
        pre += (diag ? k < dr : 2 * k < r) ? C::kReal : C::kPad;
        ++k;
    }
    return first + 2 * k;
}
// The tile row ia that holds flat pair block q.
__device__ __forceinline__ int block_row(int q) {
    int ia = (int)((sqrtf(4.0f + 32.0f * (float)q) - 2.0f) * 0.0625f);
    while (blocks_before_row(ia + 1) <= q) ++ia;
    while (ia > 0 && blocks_before_row(ia) > q) --ia;
    return ia;
}
// Pair blocks of a jet (the blocks before the row past its last active tile).
__device__ __forceinline__ int jet_blocks(uint32_t act) { return blocks_before_row(__popc(act)); }

// Persistent pair-embed kernel.  The work of every jet (its pair blocks in
// tile order, weighted by the estimate above) is counted from the mask; one
// wave scans the per-jet costs and gives every workgroup an equal contiguous
// share, split at pair-block granularity (the two workgroups of a CU then
// carry a like load).  All-padding tiles are split evenly over the first
// workgroup of each CU (the older one, which finishes its share first) and
// only get zeros.  The 8 waves
// claim the iterations (pairs of blocks) of each jet from a counter in LDS and
// run them alone (no barrier between iterations, none between the first two
// jets), writing U straight from registers.  Workgroup w is remapped so
// that the workgroups of one XCD (dispatch is round-robin over 8 XCDs) hold
// adjacent ranges and thus write neighbouring parts of U.
// kPacked: a packed batch (PackedArgs above; mask unused, P = 16 times the
// largest jet's block count); its jets have no padded tiles, so there are no
// zero tiles.
template <int kMode, bool kPacked>
__global__ __launch_bounds__(kEmbedThreads) __attribute__((amdgpu_waves_per_eu(4)))
void pair_embed_kernel(const float4 *__restrict__ p4, const uint8_t *__restrict__ mask, int B,
                       int P, const float4 *__restrict__ w32, const v8bf *__restrict__ w16,
                       const v8h *__restrict__ wx2, const float *__restrict__ bias,
                       void *__restrict__ Uout, int wz, Int8Args ia, PackedArgs pk) {
    MlpLds<kMode> M;
    if constexpr (kMode == kMlpInt8) M.set_act(ia);
    __shared__ PartLds<kMaxP> Ls[2];  // the particles of two jets
    __shared__ int scan[kEmbedThreads];
    __shared__ JetInfo jinfo[kEmbedThreads];
    __shared__ int work_next[2];  // next unclaimed iteration of the jet in each slot
    __shared__ int work_fail;     // a wave's fp16 x 2 results were not all finite
    __shared__ int split_out[4];  // first and end jet, first and end pair block
    __shared__ JetInfo split_jet[2];

    // pair (i, j), j <= i, of slot p of a diagonal tile's triangle packing
    // as i << 4 | j; the unused slots 136..159 hold kNoPair (i = 0, j = 15),
    // which no valid entry can equal since j <= i
    __shared__ uint8_t diagPair[160];

    typedef MlpOut<kMode> OutT;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (tid < 160) {
        const int i = tri_row(tid);
        diagPair[tid] = tid < 136 ? (uint8_t)(i << 4 | (tid - i * (i + 1) / 2)) : kNoPair;
    }
    const int T = P / kTile, ntri = T * (T + 1) / 2;
    const int W = gridDim.x;
    const int w = (W % 8 == 0) ? (blockIdx.x % 8) * (W / 8) + blockIdx.x / 8 : blockIdx.x;

    // ---- this workgroup's equal share of the estimated work: a block scan of
    // the per-jet costs (each thread sums the jets of its range), split at
    // iteration granularity
    // Per-jet info from the mask by 16-lane groups (group g of the block takes
    // jets g, g + 32, ..., four per round with every load of a round issued
    // first; each load instruction reads four whole rows).  With one jet per
    // thread (per == 1) the info goes to jinfo[jet]; else the costs are summed
    // per thread range in scan[].  The MLP weight loads are issued right after
    // the first round's mask loads (the wait counter drains in order, so the
    // mask values need not wait for them) and stored to LDS after the split.
    typename MlpLds<kMode>::template Staging<kEmbedThreads> wst;
    const int per = (B + kEmbedThreads - 1) / kEmbedThreads;
    jinfo[tid] = JetInfo{0u, 0};
    scan[tid] = 0;
    __syncthreads();
    if constexpr (kPacked) {
        wst.load(w32, w16, wx2, bias, &ia);
        for (int b = tid; b < B; b += kEmbedThreads) {
            int st;
            int64_t u0;
            const JetInfo ji = packed_info(packed_jet(pk, b, st, u0));
            if (per == 1) jinfo[b] = ji;
            else atomicAdd(&scan[b / per], jet_cost<WorkCost<kMode>>(ji));
        }
    } else {
        constexpr int kJ = 4;
        constexpr int kGroups = kEmbedThreads / 16;
        const int grp = tid >> 4;  // 0 .. kGroups - 1
        auto round_loads = [&](int r0, uint4 (&v)[kJ]) {
#pragma unroll
            for (int k = 0; k < kJ; ++k) {
                const int b = min(r0 + grp + kGroups * k, B - 1);
                v[k] = ((const uint4 *)(mask + (size_t)b * P))[min(lane & 15, T - 1)];
            }
        };
        auto round_info = [&](int r0, const uint4 (&v)[kJ]) {
#pragma unroll
            for (int k = 0; k < kJ; ++k) {
                const int b = r0 + grp + kGroups * k;
                const JetInfo ji = jet_info16(v[k], T);
                if ((lane & 15) == 0 && b < B) {
                    if (per == 1) jinfo[b] = ji;
                    else atomicAdd(&scan[b / per], jet_cost<WorkCost<kMode>>(ji));
                }
            }
        };
        uint4 v[kJ];
        round_loads(0, v);
        __asm__ volatile("" ::: "memory");  // (issue order: mask rows, then weights)
        wst.load(w32, w16, wx2, bias, &ia);
        round_info(0, v);
        for (int r0 = kGroups * kJ; r0 < B; r0 += kGroups * kJ) {
            round_loads(r0, v);
            round_info(r0, v);
        }
    }
    __syncthreads();
    // the cost of each thread's entry (its jet, or its range of jets)
    if (per == 1) scan[tid] = jet_cost<WorkCost<kMode>>(jinfo[tid]);
    __syncthreads();
    // Wave 0 scans the kEmbedThreads entry costs (kPerLane per lane) and finds
    // both split points; the other waves store the MLP weights meanwhile.
    // Split point i: the first iteration whose cost prefix reaches
    // floor(totw (w + i) / W), as the jet and the cost left inside it (jet B
    // at the end).  With totw = W qt + rt that floor is qt (w + i) +
    // floor(rt (w + i) / W), exact in 32 bits (a 64-bit division costs a long
    // scalar sequence and a register spill whose reload waits for every load
    // in flight).
    // the info of jet b (b < B), read again from the mask or the packed entries
    auto info_of = [&](int b) -> JetInfo {
        if constexpr (kPacked) {
            int st;
            int64_t u0;
            return packed_info(packed_jet(pk, b, st, u0));
        } else {
            return jet_info(mask + (size_t)b * P, T);
        }
    };
    if (wv == 0) {
        constexpr int kPerLane = kEmbedThreads / 64;
        int cst[kPerLane], sum = 0;
#pragma unroll
        for (int e = 0; e < kPerLane; ++e) {
            cst[e] = scan[kPerLane * lane + e];
            sum += cst[e];
        }
        int inc = sum;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int v = __shfl_up(inc, off);
            inc += lane >= off ? v : 0;
        }
        // (readlane: a uniform source lane needs no LDS round trip)
        const int totw = __builtin_amdgcn_readlane(inc, 63), excl = inc - sum;
        const int qt = totw / W, rt = totw - qt * W;
        int sb[2], st[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int t = qt * (w + i) + rt * (w + i) / W;
            // entries of this lane whose inclusive prefix is at most t (the
            // prefix does not decrease, so they come first), and the prefix
            // before the next one
            int k = 0, pre = excl, run = excl;
#pragma unroll
            for (int e = 0; e < kPerLane; ++e) {
                run += cst[e];
                const bool below = run <= t;
                k += below;
                pre = below ? run : pre;
            }
            // the first lane whose inclusive prefix exceeds t holds the entry
            const int L = __popcll(__ballot(inc <= t));
            sb[i] = B;
            st[i] = 0;
            if (t < totw) {
                sb[i] = (kPerLane * L + __builtin_amdgcn_readlane(k, L)) * per;
                st[i] = t - __builtin_amdgcn_readlane(pre, L);
            }
        }
        // the jets at the split points: from LDS when every thread has one
        // jet, else walked from the first jet of the split entry's range
        JetInfo js = {0u, 0}, je = {0u, 0};
        if (per == 1) {
            if (sb[0] < B) js = jinfo[sb[0]];
            if (sb[1] < B) je = jinfo[sb[1]];
        } else {
            js = sb[0] < B ? info_of(sb[0]) : JetInfo{0u, 0};
            je = sb[1] < B ? info_of(sb[1]) : JetInfo{0u, 0};
            for (int jc = jet_cost<WorkCost<kMode>>(js); sb[0] < B && st[0] >= jc;
                 jc = jet_cost<WorkCost<kMode>>(js)) {
                st[0] -= jc;
                ++sb[0];
                js = info_of(min(sb[0], B - 1));
            }
            for (int jc = jet_cost<WorkCost<kMode>>(je); sb[1] < B && st[1] >= jc;
                 jc = jet_cost<WorkCost<kMode>>(je)) {
                st[1] -= jc;
                ++sb[1];
                je = info_of(min(sb[1], B - 1));
            }
        }
        if (lane == 0) {
            split_out[0] = sb[0];
            split_out[1] = sb[1];
            split_out[2] = sb[0] < B ? jet_split<WorkCost<kMode>>(js, st[0]) : 0;
            split_out[3] = sb[1] < B ? jet_split<WorkCost<kMode>>(je, st[1]) : 0;
            split_jet[0] = js;
            split_jet[1] = je;
        }
    }
    wst.store(M);
    __syncthreads();
    const int bS = split_out[0], bE = split_out[1], qS = split_out[2], qE = split_out[3];
    const JetInfo js = split_jet[0], je = split_jet[1];
    const int nj = bE - bS + (qE > 0 ? 1 : 0);  // jets this workgroup visits

    // the particles of jet j of the range into slot j & 1 (all threads)
    auto stage_jet = [&](int j) {
        const int b = bS + j;
        PartLds<kMaxP> &Lj = Ls[j & 1];
        if constexpr (kPacked) {  // rows 0 .. n-1 real, the rest of the last block padding
            int st;
            int64_t u0;
            const int n = packed_jet(pk, b, st, u0), ns = (n + kTile - 1) / kTile * kTile;
            for (int s = tid; s < ns; s += kEmbedThreads) {
                const bool real = s < n;
                stage_particle(Lj, s, real ? p4[(size_t)st + s] : make_float4(0.f, 0.f, 0.f, 0.f),
                               real);
            }
            return;
        }
        for (int s = tid; s < P; s += kEmbedThreads) {
            const size_t idx = (size_t)b * P + s;
            // both loads issued before either is used (a load under the mask
            // test would be a second round trip)
            const float4 pv = p4[idx];
            const uint8_t mb = mask[idx];
            __asm__ volatile("" ::: "memory");
            const int real = mb != 0;
            stage_particle(Lj, s, real ? pv : make_float4(0.f, 0.f, 0.f, 0.f), real);
        }
    };
    if (tid == 0) {
        work_next[0] = work_next[1] = kEmbedWaves;  // iteration w opens wave w's claims
        work_fail = 0;
    }
    // the first two jets at once, so that no barrier separates them: thread t
    // takes particle t % kMaxP of jet t / kMaxP
    static_assert(kEmbedThreads >= 2 * kMaxP, "one particle per thread for two jets");
    if constexpr (kPacked) {
        const int j = tid / kMaxP, sl = tid % kMaxP;
        if (j < min(nj, 2)) {
            int st;
            int64_t u0;
            const int n = packed_jet(pk, bS + j, st, u0);
            if (sl < (n + kTile - 1) / kTile * kTile) {
                const bool real = sl < n;
                stage_particle(Ls[j], sl,
                               real ? p4[(size_t)st + sl] : make_float4(0.f, 0.f, 0.f, 0.f), real);
            }
        }
    } else {
        const int j = tid / kMaxP, sl = tid % kMaxP;
        if (j < min(nj, 2) && sl < P) {
            const size_t idx = (size_t)(bS + j) * P + sl;
            const float4 pv = p4[idx];  // both loads issued before either is used
            const uint8_t mb = mask[idx];
            __asm__ volatile("" ::: "memory");
            const int real = mb != 0;
            stage_particle(Ls[j], sl, real ? pv : make_float4(0.f, 0.f, 0.f, 0.f), real);
        }
    }
    __syncthreads();

    // One jet of the range: its pair blocks [q0, q1), flattened into wave
    // iterations of two blocks; the tile walk is wave-uniform (scalar
    // registers).  Fast pass (fp16 x 2 or bf16): iterations claimed from the
    // slot's counter, so the waves finish together; exact pass: a fixed deal
    // in which round r gives wave w iteration kEmbedWaves r + (w - r) mod
    // kEmbedWaves.
    auto run_jet = [&](int j, auto exact_t) {
        constexpr bool kExact = decltype(exact_t)::value;
        const int b = bS + j;
        const PartLds<kMaxP> &L = Ls[j & 1];
        uint32_t act;
        if (b == bS) act = js.act;
        else if (b == bE) act = je.act;
        else if (per == 1) act = jinfo[b].act;
        else if constexpr (kPacked) act = info_of(b).act;
        else act = jet_activity(mask + (size_t)b * P, T);
        const int q0 = b == bS ? qS : 0, q1 = b == bE ? qE : jet_blocks(act);
        const int nit = max(0, (q1 - q0) >> 1);
        OutT *U = (OutT *)Uout + (size_t)b * kHeads * P * P;
        int pn = 0, pld = 0;  // packed: the jet's rows and row stride
        uint32_t pplane = 0;
        if constexpr (kPacked) {
            int st;
            int64_t u0;
            pn = packed_jet(pk, b, st, u0);
            pld = packed_ld(pn);
            pplane = (uint32_t)(pn * pld);
            U = (OutT *)Uout + (size_t)kHeads * u0;
        }
        const uint64_t aidx = active_index(act);
        bool ok = true;
        int ia = block_row(max(q0, 0));
        int it = wv, r = 0;
        while (kExact ? kEmbedWaves * r < nit : it < nit) {
            int itn = 0;
            if constexpr (kExact) {
                it = kEmbedWaves * r + ((wv - r) & (kEmbedWaves - 1));
                ++r;
                if (it >= nit) continue;
            } else if (lane == 0) {
                itn = atomicAdd(&work_next[j & 1], 1);  // the next claim, early
            }
            const int q = q0 + 2 * it;
            int rem = q - blocks_before_row(ia);
            // Compiler-only memory barrier (emits nothing): keeps the
            // loop-invariant LDS weight reads inside the loop instead of
            // hoisting 144+ registers of operands out of it.
            __asm__ volatile("" ::: "memory");
            while (rem >= 16 * ia + 10) {  // rows have 16 ia + 10 blocks
                rem -= 16 * ia + 10;
                ++ia;
            }
            const int ja = min(rem >> 4, ia), kb = rem - 16 * ja;
            const int I = nth_active(aidx, ia), J = nth_active(aidx, ja);
            const bool diag = ia == ja;
            // this lane's pairs (tile-local rows / columns) of blocks kb, kb+1
            int iA = kb, jA = lane & 15, iB = kb + 1, jB = lane & 15;
            bool vA = true, vB = true;
            if (diag) {
                const int eA = diagPair[16 * kb + (lane & 15)];
                const int eB = diagPair[16 * kb + 16 + (lane & 15)];
                vA = eA != kNoPair;
                vB = eB != kNoPair;
                iA = vA ? eA >> 4 : 0;
                jA = vA ? eA & 15 : 0;
                iB = vB ? eB >> 4 : 0;
                jB = vB ? eB & 15 : 0;
            }
            const int aA = I * kTile + iA, bA = J * kTile + jA;
            const int aB = I * kTile + iB, bB = J * kTile + jB;
            const bool realA = vA && L.real[aA] && L.real[bA];
            const bool realB = vB && L.real[aB] && L.real[bB];
            v4f uA = {0.f, 0.f, 0.f, 0.f}, uB = uA;
            const bool any = __ballot(realA || realB) != 0;
            if (any) {
                const int f = lane >> 4;
                const float fA = realA ? pair_feature(L, aA, bA, f) : 0.0f;
                const float fB = realB ? pair_feature(L, aB, bB, f) : 0.0f;
                if constexpr (kExact) M.run_exact(w32, fA, fB, uA, uB);
                else ok = M.run(fA, fB, uA, uB) && ok;
            }
            if constexpr (kPacked) {
                if (!diag) {
                    write_row_pair_packed<OutT>(L, U, pn, pld, pplane, aA, bA, uA, uB, !any);
                } else {
                    write_block_packed<OutT>(L, U, pn, pld, pplane, I, J, vA, iA, jA, uA, !any);
                    write_block_packed<OutT>(L, U, pn, pld, pplane, I, J, vB, iB, jB, uB, !any);
                }
            } else if (!diag) {  // rows kb, kb + 1 of one off-diagonal tile
                write_row_pair<OutT>(L, U, P, aA, bA, uA, uB, !any);
            } else {
                write_block<OutT>(L, U, P, I, J, vA, iA, jA, uA, !any);
                write_block<OutT>(L, U, P, I, J, vB, iB, jB, uB, !any);
            }
            if constexpr (!kExact) it = __builtin_amdgcn_readfirstlane(itn);
        }
        return ok;
    };
    bool ok = true;
    for (int j = 0; j < nj; ++j) {
        if (j >= 2) {  // a third jet reuses slot j & 1: wait for jet j - 2
            __syncthreads();
            stage_jet(j);
            if (tid == 0) work_next[j & 1] = kEmbedWaves;
            __syncthreads();
        }
        ok = run_jet(j, std::false_type{}) && ok;
    }
    // When a wave's fp16 x 2 results were not all finite, the workgroup redoes
    // its range exactly (the later stores replace the earlier ones).
    if (!ok && lane == 0) work_fail = 1;
    __syncthreads();
    if (work_fail) {
        for (int j = 0; j < nj; ++j) {
            __syncthreads();
            stage_jet(j);
            __syncthreads();
            run_jet(j, std::true_type{});
        }
    }

    // ---- tiles without a real pair: zeros (after the real tiles, so these
    // stores overlap the other workgroups' work; jet activity read once per
    // jet).  Only the first wz workgroups (one per CU: workgroups i and
    // i + wz share a CU, and the older one finishes first) write them.
    if (!kPacked && (int)blockIdx.x < wz) {
        // tiles [tot zw / wz, tot (zw + 1) / wz), floors taken in 32 bits as above
        const int zw = blockIdx.x;
        const int tot = B * ntri, qz = tot / wz, rz = tot - qz * wz;
        const int z1 = qz * (zw + 1) + rz * (zw + 1) / wz;
        // each 512 threads take one tile per step (the half is wave-uniform)
        constexpr int kZPar = kEmbedThreads / 512;
        static_assert(kEmbedThreads % 512 == 0, "zero tiles are written by 512 threads");
        int bz = -1;
        uint32_t actz = 0;
        for (int z0 = qz * zw + rz * zw / wz; z0 < z1; z0 += kZPar) {
            const int z = z0 + tid / 512;
            if (z >= z1) continue;
            const int bb = z / ntri, t = z - bb * ntri;
            if (bb != bz) {
                bz = bb;
                actz = per == 1 ? jinfo[bb].act : jet_activity(mask + (size_t)bb * P, T);
            }
            const int I = tri_row(t), J = t - I * (I + 1) / 2;
            if ((actz >> I & 1) && (actz >> J & 1)) continue;
            zero_tile<OutT>((OutT *)Uout + (size_t)bb * kHeads * P * P, P, I, J, tid % 512);
        }
    }
}

// Compute units of the current device (cached per device).
int cu_count() {
    static int cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    if (cus[dev] <= 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cus[dev] = n;
    }
    return cus[dev];
}

// kWgPerCu resident workgroups per CU (16 waves: 4 per SIMD at the kernel's
// register budget).
static int persistent_grid(int B, int P) {
    const long T = P / kTile, tiles = (long)B * T * (T + 1) / 2;
    return (int)std::min<long>((long)kWgPerCu * cu_count(), std::max<long>(tiles, 1));
}

// Batches are cut into segments of at most 65,536 jets so that tile counts
// stay far inside int range.
template <int kMode>
static hipError_t launch_embed(const float *p4, const uint8_t *mask, int B, int P,
                               const pip_pair_mlp *m, void *U, hipStream_t s,
                               const Int8Args &ia = Int8Args{}) {
    typedef MlpOut<kMode> OutT;
    constexpr int kSeg = 65536;
    for (int b0 = 0; b0 < B; b0 += kSeg) {
        const int nb = std::min(kSeg, B - b0);
        const int grid = persistent_grid(nb, P);
        // zero tiles: the workgroups that are first on their CU
        const int wz = std::max(1, std::min(grid, cu_count()));
        hipLaunchKernelGGL((pair_embed_kernel<kMode, false>), dim3(grid), dim3(kEmbedThreads), 0,
                           s, (const float4 *)p4 + (size_t)b0 * P, mask + (size_t)b0 * P, nb, P,
                           (const float4 *)m->w32, (const v8bf *)m->w16, (const v8h *)m->wx2,
                           m->bias, (void *)((OutT *)U + (size_t)b0 * kHeads * P * P), wz, ia,
                           PackedArgs{nullptr, nullptr, 0, 0, 0});
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// A packed batch: the same kernel over the jets' real blocks (P = 16 times
// the largest block count), cut into segments of at most 65,536 jets (cu and
// u_off of a segment are the batch's, offset; rows and U offsets stay
// absolute).
template <int kMode>
static hipError_t launch_embed_packed(const float *p4, const int *cu, const int64_t *uoff, int B,
                                      int N, int max_n, const pip_pair_mlp *m, void *U,
                                      int64_t u_elems, hipStream_t s) {
    const int P = (max_n + kTile - 1) / kTile * kTile;
    if (P == 0) return hipSuccess;
    constexpr int kSeg = 65536;
    for (int b0 = 0; b0 < B; b0 += kSeg) {
        const int nb = std::min(kSeg, B - b0);
        const int grid = persistent_grid(nb, P);
        const int wz = std::max(1, std::min(grid, cu_count()));
        hipLaunchKernelGGL((pair_embed_kernel<kMode, true>), dim3(grid), dim3(kEmbedThreads), 0, s,
                           (const float4 *)p4, (const uint8_t *)nullptr, nb, P,
                           (const float4 *)m->w32, (const v8bf *)m->w16, (const v8h *)m->wx2,
                           m->bias, U, wz, Int8Args{},
                           PackedArgs{cu + b0, uoff + b0, N, max_n, u_elems});
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_pair_embed_packed_f32(const float *p4, const int *cu, const int64_t *uoff,
                                        int B, int N, int max_n, const pip_pair_mlp *m, float *U,
                                        int64_t u_elems, hipStream_t s) {
    return m->f16ok
               ? launch_embed_packed<kMlpF16x2>(p4, cu, uoff, B, N, max_n, m, U, u_elems, s)
               : launch_embed_packed<kMlpF32>(p4, cu, uoff, B, N, max_n, m, U, u_elems, s);
}

hipError_t launch_pair_embed_packed_bf16(const float *p4, const int *cu, const int64_t *uoff,
                                         int B, int N, int max_n, const pip_pair_mlp *m,
                                         uint16_t *U, int64_t u_elems, hipStream_t s) {
    return launch_embed_packed<kMlpBf16>(p4, cu, uoff, B, N, max_n, m, U, u_elems, s);
}

hipError_t launch_pair_embed_f32(const float *p4, const uint8_t *mask, int B, int P,
                                 const pip_pair_mlp *m, float *U, hipStream_t s) {
    return m->f16ok ? launch_embed<kMlpF16x2>(p4, mask, B, P, m, U, s)
                    : launch_embed<kMlpF32>(p4, mask, B, P, m, U, s);
}

hipError_t launch_pair_embed_bf16(const float *p4, const uint8_t *mask, int B, int P,
                                  const pip_pair_mlp *m, uint16_t *U, hipStream_t s) {
    return launch_embed<kMlpBf16>(p4, mask, B, P, m, U, s);
}

hipError_t launch_pair_embed_int8(const float *p4, const uint8_t *mask, int B, int P,
                                  const pip_pair_mlp *m, const float *act_scale,
                                  const int *act_zero, uint16_t *U, hipStream_t s) {
    Int8Args ia;
    ia.w8 = (const v4i *)m->w8;
    ia.q8 = m->q8;
    for (int l = 0; l < 3; ++l) {
        ia.s[l] = act_scale[l];
        ia.inv_s[l] = 1.0f / act_scale[l];
        ia.zp[l] = (float)act_zero[l];
    }
    return launch_embed<kMlpInt8>(p4, mask, B, P, m, U, s, ia);
}

}  // namespace pip

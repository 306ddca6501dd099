// packed_embed.hip -- the pair embedding on jets packed back to back
// (variable length, no padding), and the offsets of their U blocks.
//
// Layout.  Particles of all jets are concatenated: p4 is (N, 4), jet b owns
// rows cu[b] .. cu[b+1]-1 (cu_seqlens, the `ptr` of the lloca
// transformer_v2.Transformer.forward documentation), n_b = cu[b+1] - cu[b].
// Jet b's bias is one (8, n_b, ld_b) block, ld_b = n_b rounded up to a
// multiple of 8 (rows start 16-byte aligned for the attention's vector
// loads; the <= 7 columns past n_b in each row are written as 0), starting at
// element 8 u_off[b] with u_off[b] = sum_{j<b} n_j ld_j.  There are no padded
// rows, no padded tiles and no zero tiles.
//
// What is computed is "Fusion 2" of the ml4sci_cms_e2e26 README ("How the
// Kernel Fusion Works"): the four pair features and the whole MLP per pair,
// the bias written once per head.
//
// Work decomposition.  One 512-thread workgroup per (jet, row tile I), row
// tiles of 16 particles; the grid runs the largest I first so that the long
// workgroups start early.  The workgroup stages its MLP weights and the
// jet's particles 0 .. 16(I+1)-1 in LDS, then walks the tiles (I, J), J <= I,
// of the lower triangle (U is symmetric): each wave pushes two 16-pair blocks
// through the MFMA chain (off-diagonal tile: rows w and w+8; diagonal tile:
// its 136 unique pairs in blocks 2w, 2w+1), the results go to a 16x16 LDS
// tile per head, and after one barrier the workgroup writes the tile and its
// transpose as contiguous row segments (both directions are full 64-byte
// rows; the padded kernel's mirror is an 8-byte scatter).  The tile buffer
// is double-buffered so one barrier per tile suffices.
//
// A jet whose cu / u_off entries are inconsistent (n < 0, n > max_n, rows
// past N, a U block of the wrong size or past u_elems) is skipped: nothing
// of it is written.
#include <algorithm>
#include <type_traits>

#include "pip_internal.h"
#include "pip_mlp.h"

namespace pip {

constexpr int kPkThreads = 512;
constexpr int kPkWaves = kPkThreads / 64;

__device__ __forceinline__ int packed_ld(int n) { return (n + 7) & ~7; }

// Is jet b of a packed batch consistent (the check PackedJet::load makes),
// and its size n: per lane, b may differ from lane to lane.
__device__ __forceinline__ bool packed_jet_ok(const int *__restrict__ cu,
                                              const int64_t *__restrict__ uoff, int b, int N,
                                              int max_n, int64_t u_elems, int heads, int &n) {
    const int start = cu[b], end = cu[b + 1];
    const int64_t a0 = uoff[b], a1 = uoff[b + 1];
    n = end - start;
    return start >= 0 && n >= 0 && n <= max_n && n <= kMaxP && end <= N && a0 >= 0 &&
           a1 - a0 == (int64_t)n * packed_ld(n) && a1 <= u_elems / heads;
}

// Jet b of a packed batch, read and checked (b and so every value here is
// wave-uniform).
struct PackedJet {
    int start, n, ld;
    int64_t u0;
    bool ok;
    __device__ __forceinline__ void load(const int *__restrict__ cu,
                                         const int64_t *__restrict__ uoff, int b, int N,
                                         int max_n, int64_t u_elems, int heads) {
        start = __builtin_amdgcn_readfirstlane(cu[b]);
        const int end = __builtin_amdgcn_readfirstlane(cu[b + 1]);
        const int64_t a0 = uoff[b], a1 = uoff[b + 1];
        n = end - start;
        ld = packed_ld(n);
        u0 = a0;
        ok = start >= 0 && n >= 0 && n <= max_n && n <= kMaxP && end <= N && a0 >= 0 &&
             a1 - a0 == (int64_t)n * ld && a1 <= u_elems / heads;
    }
};

__device__ __forceinline__ void store_one(float *U, size_t off, float v) { U[off] = v; }
__device__ __forceinline__ void store_one(uint16_t *U, size_t off, float v) {
    U[off] = __builtin_bit_cast(uint16_t, (__bf16)v);
}

// Tile-local pair (i, j), i >= j, of lane `lane` in block k of a diagonal
// tile (136 pairs, blocks of 16 in row-major order of the lower triangle).
__device__ __forceinline__ bool diag_pair(int k, int lane, int &i, int &j) {
    int p = 16 * k + (lane & 15);
    const bool valid = p < 136;
    p = valid ? p : 0;
    int r = (int)((sqrtf(8.0f * (float)p + 1.0f) - 1.0f) * 0.5f);
    while ((r + 1) * (r + 2) / 2 <= p) ++r;
    while (r * (r + 1) / 2 > p) --r;
    i = r;
    j = p - r * (r + 1) / 2;
    return valid;
}

// The tiles (I, J <= I) of one workgroup.  kExact: every pair block through
// the exact float32 chain (weights from global memory).  Otherwise this
// mode's chain; returns true when a wave of the fp16 x 2 chain produced a
// non-finite value (an activation left the fp16 range), after which the
// caller runs the whole row of tiles again exactly.
template <int kMode, bool kExact, typename OutT>
__device__ __forceinline__ bool packed_tiles(const MlpLds<kMode> &M, const PartLds<kMaxP> &L,
                                             float (*Ut)[kHeads][16][17],
                                             const float4 *__restrict__ w32, OutT *Ub, int I,
                                             int n, int ld) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, c = lane & 15;
    const size_t plane = (size_t)n * ld;
    bool failed = false;
    for (int J = 0; J <= I; ++J) {
        const int buf = J & 1;
        const bool diag = J == I;
        // this wave's two pair blocks
        int iA, jA, iB, jB;
        bool vA, vB, work;
        if (!diag) {
            iA = wave;
            iB = wave + 8;
            jA = jB = c;
            vA = I * kTile + iA < n;
            vB = I * kTile + iB < n;
            work = vA || vB;
        } else {
            vA = diag_pair(2 * wave, lane, iA, jA) && I * kTile + iA < n;
            vB = diag_pair(2 * wave + 1, lane, iB, jB) && I * kTile + iB < n;
            work = wave < 5 && __any(vA || vB);
        }
        if (work) {
            const int aA = I * kTile + iA, cA = J * kTile + jA;
            const int aB = I * kTile + iB, cB = J * kTile + jB;
            const float fA = vA ? pair_feature(L, aA, cA, g) : 0.0f;
            const float fB = vB ? pair_feature(L, aB, cB, g) : 0.0f;
            v4f uA, uB;
            if constexpr (kExact) M.run_exact(w32, fA, fB, uA, uB);
            else failed |= !M.run(fA, fB, uA, uB);
            // (only valid pairs: an unused lane of the last diagonal block
            // names pair (0, 0), which another lane owns)
            if (lane < 32) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int h = 4 * g + r;
                    if (vA) {
                        Ut[buf][h][iA][jA] = uA[r];
                        if (diag) Ut[buf][h][jA][iA] = uA[r];
                    }
                    if (vB) {
                        Ut[buf][h][iB][jB] = uB[r];
                        if (diag) Ut[buf][h][jB][iB] = uB[r];
                    }
                }
            }
        }
        __syncthreads();
        // tile (I, J) and, off the diagonal, its transpose (J, I): wave w
        // writes head w, lane (row l/16 + 4k, column l%16) for k = 0..3, so
        // each store instruction writes four 16-element row segments
        {
            const int h = wave;
            OutT *Uh = Ub + h * plane;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int r = g + 4 * k;
                const int a = I * kTile + r, col = J * kTile + c;
                if (a < n && col < n) store_one(Uh, (size_t)a * ld + col, Ut[buf][h][r][c]);
                if (!diag) {
                    const int a2 = J * kTile + r, col2 = I * kTile + c;
                    if (col2 < n) store_one(Uh, (size_t)a2 * ld + col2, Ut[buf][h][c][r]);
                }
            }
        }
    }
    return failed;
}

template <int kMode, typename OutT>
__global__ __launch_bounds__(kPkThreads) __attribute__((amdgpu_waves_per_eu(4))) void
pair_embed_packed_kernel(const float4 *__restrict__ p4, const int *__restrict__ cu,
                         const int64_t *__restrict__ uoff, int B, int N, int Tmax, int max_n,
                         int64_t u_elems, const float4 *__restrict__ w32,
                         const v8bf *__restrict__ w16, const v8h *__restrict__ wx2,
                         const float *__restrict__ bias, OutT *__restrict__ U) {
    MlpLds<kMode> M;
    __shared__ PartLds<kMaxP> L;
    __shared__ float Ut[2][kHeads][16][17];
    __shared__ int redo;

    // row tile I of jet b; the grid runs the largest I first
    const int I = Tmax - 1 - (int)(blockIdx.x / (unsigned)B);
    const int b = (int)(blockIdx.x % (unsigned)B);
    PackedJet jt;
    jt.load(cu, uoff, b, N, max_n, u_elems, kHeads);
    if (!jt.ok || I * kTile >= jt.n) return;  // uniform over the workgroup
    const int n = jt.n, ld = jt.ld;
    const int tid = threadIdx.x;

    // weights and the particles 0 .. ncols-1 (all real) into LDS
    {
        typename MlpLds<kMode>::template Staging<kPkThreads> st;
        st.load(w32, w16, wx2, bias);
        const int ncols = min((I + 1) * kTile, n);
        const float4 pv =
            tid < ncols ? p4[(size_t)jt.start + tid] : make_float4(0.f, 0.f, 0.f, 0.f);
        st.store(M);
        if (tid < ncols) stage_particle(L, tid, pv, 1);
    }
    if (tid == 0) redo = 0;
    OutT *Ub = U + (size_t)kHeads * jt.u0;
    // the <= 7 columns past n of this workgroup's rows: zeros
    {
        const int pad = ld - n;
        const size_t plane = (size_t)n * ld;
        for (int e = tid; e < kHeads * kTile * 8; e += kPkThreads) {
            const int h = e >> 7, r = (e >> 3) & 15, q = e & 7;
            const int a = I * kTile + r;
            if (q < pad && a < n) store_one(Ub, h * plane + (size_t)a * ld + n + q, 0.0f);
        }
    }
    __syncthreads();
    const bool failed = packed_tiles<kMode, false>(M, L, Ut, w32, Ub, I, n, ld);
    if constexpr (kMode == kMlpF16x2) {
        if (failed && (tid & 63) == 0) redo = 1;
        __syncthreads();
        if (redo) packed_tiles<kMode, true>(M, L, Ut, w32, Ub, I, n, ld);
    }
}

// ---- persistent form: single tiles dealt round-robin -------------------
// A row of tiles holds up to 16 tiles, so one workgroup per row leaves the
// longest rows to set the end of the launch.  Here a persistent grid (two
// workgroups per CU) stages the MLP weights once, builds the prefix sums of
// every jet's tile count T(T+1)/2 (T = ceil(n/16), 0 for a skipped jet) in
// LDS, and takes tiles t = w, w + G, w + 2G, ... of the flattened list (jet,
// row tile I, column tile J <= I): about the same number of tiles per
// workgroup.  Each tile's 32 particles (16 rows, 16 columns) are staged
// into one of two LDS slot buffers while the previous tile runs, so one
// barrier per tile separates the MLP work from the stores.  Batches of
// more than kPkMaxJets jets (the LDS prefix) take the row kernel above.
constexpr int kPkMaxJets = 4096;

template <int kMode, bool kExact, typename OutT>
__device__ __forceinline__ bool packed_tile(const MlpLds<kMode> &M, const PartLds<32> &L,
                                            float (*Ut)[16][17], const float4 *__restrict__ w32,
                                            int I, int J, int n) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, c = lane & 15;
    const bool diag = J == I;
    int iA, jA, iB, jB;
    bool vA, vB, work;
    if (!diag) {
        iA = wave;
        iB = wave + 8;
        jA = jB = c;
        vA = I * kTile + iA < n;
        vB = I * kTile + iB < n;
        work = vA || vB;
    } else {
        vA = diag_pair(2 * wave, lane, iA, jA) && I * kTile + iA < n;
        vB = diag_pair(2 * wave + 1, lane, iB, jB) && I * kTile + iB < n;
        work = wave < 5 && __any(vA || vB);
    }
    bool failed = false;
    if (work) {
        // rows sit in slots 0..15; columns in 16..31 (the rows again on the diagonal)
        const int cs = diag ? 0 : 16;
        const float fA = vA ? pair_feature(L, iA, cs + jA, g) : 0.0f;
        const float fB = vB ? pair_feature(L, iB, cs + jB, g) : 0.0f;
        v4f uA, uB;
        if constexpr (kExact) M.run_exact(w32, fA, fB, uA, uB);
        else failed = !M.run(fA, fB, uA, uB);
        if (lane < 32) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int h = 4 * g + r;
                if (vA) {
                    Ut[h][iA][jA] = uA[r];
                    if (diag) Ut[h][jA][iA] = uA[r];
                }
                if (vB) {
                    Ut[h][iB][jB] = uB[r];
                    if (diag) Ut[h][jB][iB] = uB[r];
                }
            }
        }
    }
    return failed;
}

// Tile t of the flattened list: jet b, row tile I, column tile J <= I.
struct PackedTile {
    int b, I, J;
    __device__ __forceinline__ void decode(const int *pre, int B, int t) {
        int lo = 0, hi = B;  // pre[lo] <= t < pre[hi]: jets with no tile are skipped
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (pre[mid] <= t) lo = mid;
            else hi = mid;
        }
        b = lo;
        const int q = t - pre[b];
        int i = (int)((sqrtf(8.0f * (float)q + 1.0f) - 1.0f) * 0.5f);
        while ((i + 1) * (i + 2) / 2 <= q) ++i;
        while (i * (i + 1) / 2 > q) --i;
        I = i;
        J = q - i * (i + 1) / 2;
    }
};

// Stage tile t's particles into slot buffer L (wave kStageWave: rows I*16..
// into slots 0..15, columns J*16.. into 16..31 off the diagonal); t >= S
// stages nothing.
constexpr int kStageWave = kPkWaves - 1;  // idle on diagonal tiles (waves 5..7)
__device__ __forceinline__ void stage_tile_particles(PartLds<32> &L, const int *pre, int B, int S,
                                                     int t, const float4 *__restrict__ p4,
                                                     const int *__restrict__ cu) {
    const int tid = threadIdx.x, lane = tid & 63;
    if (t >= S || (tid >> 6) != kStageWave || lane >= 32) return;
    PackedTile tl;
    tl.decode(pre, B, t);
    if (lane >= 16 && tl.J == tl.I) return;
    const int start = cu[tl.b], n = cu[tl.b + 1] - start;
    const int a = (lane < 16 ? tl.I : tl.J) * kTile + (lane & 15);
    const bool real = a < n;
    stage_particle(L, lane, real ? p4[(size_t)start + a] : make_float4(0.f, 0.f, 0.f, 0.f), real);
}

// This workgroup's tiles t = blockIdx.x, + gridDim.x, ... of the flattened
// list; returns true when a wave of the fp16 x 2 chain produced a non-finite
// value.  One barrier per tile: the slot buffers and result tiles are
// double-buffered, and the particles of the next tile are staged (by one
// wave) while the others run the MLP of the current one.
template <int kMode, bool kExact, typename OutT>
__device__ __forceinline__ bool packed_tiles_sweep(const MlpLds<kMode> &M, PartLds<32> (&L)[2],
                                                   float (*Ut)[kHeads][16][17], const int *pre,
                                                   const float4 *__restrict__ p4,
                                                   const int *__restrict__ cu,
                                                   const int64_t *__restrict__ uoff, int B, int S,
                                                   const float4 *__restrict__ w32,
                                                   OutT *__restrict__ U) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    bool failed = false;
    stage_tile_particles(L[0], pre, B, S, blockIdx.x, p4, cu);
    __syncthreads();
    int it = 0;
    for (int t = blockIdx.x; t < S; t += gridDim.x, ++it) {
        const int buf = it & 1;
        PackedTile tl;
        tl.decode(pre, B, t);
        const int I = tl.I, J = tl.J;
        const int start = __builtin_amdgcn_readfirstlane(cu[tl.b]);
        const int n = __builtin_amdgcn_readfirstlane(cu[tl.b + 1]) - start;
        failed |= packed_tile<kMode, kExact, OutT>(M, L[buf], Ut[buf], w32, I, J, n);
        // the next tile's particles into the other slot buffer (its last
        // reader, the previous tile's MLP, finished before the last barrier)
        stage_tile_particles(L[buf ^ 1], pre, B, S, t + gridDim.x, p4, cu);
        __syncthreads();
        // tile (I, J) and, off the diagonal, its transpose (J, I): wave w
        // writes head w, four 16-element row segments per store instruction
        const int ld = packed_ld(n);
        const size_t plane = (size_t)n * ld;
        OutT *Uh = U + (size_t)kHeads * uoff[tl.b] + wave * plane;
        const bool diag = J == I;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int r = (lane >> 4) + 4 * k, c = lane & 15;
            const int a = I * kTile + r, col = J * kTile + c;
            if (a < n && col < n) store_one(Uh, (size_t)a * ld + col, Ut[buf][wave][r][c]);
            if (!diag) {
                const int a2 = J * kTile + r, col2 = I * kTile + c;
                if (col2 < n) store_one(Uh, (size_t)a2 * ld + col2, Ut[buf][wave][c][r]);
            }
        }
        // the diagonal tile also zeroes its rows' <= 7 columns past n
        if (diag) {
            const int pad = ld - n;
            for (int e = lane; e < kTile * 8; e += 64) {
                const int r = e >> 3, qq = e & 7, a = I * kTile + r;
                if (qq < pad && a < n) store_one(Uh, (size_t)a * ld + n + qq, 0.0f);
            }
        }
    }
    return failed;
}

template <int kMode, typename OutT>
__global__ __launch_bounds__(kPkThreads) __attribute__((amdgpu_waves_per_eu(4))) void
pair_embed_packed_tiles_kernel(const float4 *__restrict__ p4, const int *__restrict__ cu,
                               const int64_t *__restrict__ uoff, int B, int N, int max_n,
                               int64_t u_elems, const float4 *__restrict__ w32,
                               const v8bf *__restrict__ w16, const v8h *__restrict__ wx2,
                               const float *__restrict__ bias, OutT *__restrict__ U) {
    MlpLds<kMode> M;
    __shared__ PartLds<32> L[2];
    __shared__ float Ut[2][kHeads][16][17];
    __shared__ int pre[kPkMaxJets + 1];  // tiles of jets 0 .. b-1
    __shared__ int wsum[kPkWaves];
    __shared__ int redo;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    {
        typename MlpLds<kMode>::template Staging<kPkThreads> st;
        st.load(w32, w16, wx2, bias);
        st.store(M);
    }
    // prefix sums of the tile counts, kPkThreads jets at a time
    if (tid == 0) pre[0] = 0;
    for (int b0 = 0; b0 < B; b0 += kPkThreads) {
        const int b = b0 + tid;
        int v = 0;
        if (b < B) {  // (b differs from lane to lane: no PackedJet here)
            int n;
            const bool ok = packed_jet_ok(cu, uoff, b, N, max_n, u_elems, kHeads, n);
            const int T = ok ? (n + kTile - 1) / kTile : 0;
            v = T * (T + 1) / 2;
        }
        for (int o = 1; o < 64; o <<= 1) {
            const int t = __shfl_up(v, o);
            if (lane >= o) v += t;
        }
        if (lane == 63) wsum[wave] = v;
        __syncthreads();
        int before = pre[b0];
        for (int w = 0; w < wave; ++w) before += wsum[w];
        if (b < B) pre[b + 1] = before + v;
        __syncthreads();
    }
    const int S = pre[B];

    if (tid == 0) redo = 0;
    __syncthreads();
    const bool failed = packed_tiles_sweep<kMode, false, OutT>(M, L, Ut, pre, p4, cu, uoff, B, S,
                                                               w32, U);
    if constexpr (kMode == kMlpF16x2) {
        // an activation left the fp16 range somewhere: this workgroup's tiles
        // again, all in exact float32 (rare; kept out of the main sweep)
        if (failed && lane == 0) redo = 1;
        __syncthreads();
        if (redo) packed_tiles_sweep<kMode, true, OutT>(M, L, Ut, pre, p4, cu, uoff, B, S, w32, U);
    }
}

// u_off[0] = 0, u_off[b+1] = u_off[b] + n_b ld_b (0 for a jet whose n_b is
// negative or beyond 256): one workgroup scans the batch in chunks.
__global__ __launch_bounds__(1024) void packed_offsets_kernel(const int *__restrict__ cu, int B,
                                                              int64_t *__restrict__ uoff) {
    __shared__ int64_t wsum[16];
    __shared__ int64_t carry;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid == 0) {
        carry = 0;
        uoff[0] = 0;
    }
    __syncthreads();
    for (int c0 = 0; c0 < B; c0 += 1024) {
        const int b = c0 + tid;
        int64_t v = 0;
        if (b < B) {
            const int n = cu[b + 1] - cu[b];
            v = (n >= 0 && n <= kMaxP) ? (int64_t)n * packed_ld(n) : 0;
        }
        // inclusive scan inside the wave, then across the 16 waves
        for (int o = 1; o < 64; o <<= 1) {
            const int64_t t = __shfl_up(v, o);
            if (lane >= o) v += t;
        }
        if (lane == 63) wsum[wave] = v;
        __syncthreads();
        int64_t before = carry;
        for (int w = 0; w < wave; ++w) before += wsum[w];
        if (b < B) uoff[b + 1] = before + v;
        __syncthreads();
        if (tid == 1023) carry = before + v;
        __syncthreads();
    }
}

hipError_t launch_packed_offsets(const int *cu, int B, int64_t *uoff, hipStream_t s) {
    hipLaunchKernelGGL(packed_offsets_kernel, dim3(1), dim3(1024), 0, s, cu, B, uoff);
    return hipGetLastError();
}

template <int kMode, typename OutT>
static hipError_t launch_packed(const float *p4, const int *cu, const int64_t *uoff, int B,
                                int N, int max_n, const pip_pair_mlp *m, OutT *U,
                                int64_t u_elems, hipStream_t s) {
    const int Tmax = (max_n + kTile - 1) / kTile;
    if (Tmax == 0) return hipSuccess;
    if (B <= kPkMaxJets) {
        // enough workgroups for two per CU, fewer when the batch has fewer tiles
        const long most = (long)B * Tmax * (Tmax + 1) / 2;
        const int grid = (int)std::max<long>(1, std::min<long>(2L * cu_count(), most));
        hipLaunchKernelGGL((pair_embed_packed_tiles_kernel<kMode, OutT>), dim3((unsigned)grid),
                           dim3(kPkThreads), 0, s, (const float4 *)p4, cu, uoff, B, N, max_n,
                           u_elems, (const float4 *)m->w32, (const v8bf *)m->w16,
                           (const v8h *)m->wx2, m->bias, U);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((pair_embed_packed_kernel<kMode, OutT>), dim3((unsigned)(B * Tmax)),
                       dim3(kPkThreads), 0, s, (const float4 *)p4, cu, uoff, B, N, Tmax, max_n,
                       u_elems, (const float4 *)m->w32, (const v8bf *)m->w16,
                       (const v8h *)m->wx2, m->bias, U);
    return hipGetLastError();
}

hipError_t launch_pair_embed_packed_f32(const float *p4, const int *cu, const int64_t *uoff,
                                        int B, int N, int max_n, const pip_pair_mlp *m,
                                        float *U, int64_t u_elems, hipStream_t s) {
    return m->f16ok ? launch_packed<kMlpF16x2, float>(p4, cu, uoff, B, N, max_n, m, U, u_elems, s)
                    : launch_packed<kMlpF32, float>(p4, cu, uoff, B, N, max_n, m, U, u_elems, s);
}

hipError_t launch_pair_embed_packed_bf16(const float *p4, const int *cu, const int64_t *uoff,
                                         int B, int N, int max_n, const pip_pair_mlp *m,
                                         uint16_t *U, int64_t u_elems, hipStream_t s) {
    return launch_packed<kMlpBf16, uint16_t>(p4, cu, uoff, B, N, max_n, m, U, u_elems, s);
}

}  // namespace pip

// packed_embed.hip -- the offsets of the U blocks of jets packed back to back.
//
// Packed layout (variable length, no padding): jet b owns rows cu[b] ..
// cu[b+1]-1 of the particle arrays (cu_seqlens, the `ptr` of the lloca
// transformer_v2.Transformer.forward documentation), n_b = cu[b+1] - cu[b],
// and its bias is one (8, n_b, ld_b) block, ld_b = n_b rounded up to a
// multiple of 8 (rows start 16-byte aligned for the attention's vector loads;
// the <= 7 columns past n_b in each row are written as 0), starting at
// element 8 u_off[b] with u_off[b] = sum_{j<b} n_j ld_j.  The pair embedding
// of a packed batch is the padded kernel's packed form (pair_embed.hip); the
// attention reads the same blocks (attention.hip).
#include "pip_internal.h"
#include "pip_packed.h"

namespace pip {

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

}  // namespace pip

// pip_packed.h -- jets packed back to back (variable length, no padding).
//
// Jet b owns rows cu[b] .. cu[b+1]-1 of the particle arrays (cu_seqlens, the
// `ptr` of the lloca transformer_v2.Transformer.forward documentation) and the
// (8, n_b, ld_b) bias block at element 8 u_off[b], ld_b = n_b rounded up to 8.
#pragma once

#include "pip_device.h"

namespace pip {

__device__ __forceinline__ int packed_ld(int n) { return (n + 7) & ~7; }

// Is jet b of a packed batch consistent (its rows inside the N particle
// rows, 0 <= n <= min(max_n, 256), its U block of n ld elements per head
// inside u_elems), and its size n.  b may differ from lane to lane.
__device__ __forceinline__ bool packed_jet_ok(const int *__restrict__ cu,
                                              const int64_t *__restrict__ uoff, int b, int N,
                                              int max_n, int64_t u_elems, int heads, int &n) {
    const int start = cu[b], end = cu[b + 1];
    const int64_t a0 = uoff[b], a1 = uoff[b + 1];
    n = end - start;
    return start >= 0 && n >= 0 && n <= max_n && n <= kMaxP && end <= N && a0 >= 0 &&
           a1 - a0 == (int64_t)n * packed_ld(n) && a1 <= u_elems / heads;
}

}  // namespace pip

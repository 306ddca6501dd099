// noalloc.hip -- pip_block_stack_noalloc: the block stack (pip_block_stack)
// with its workspace in a fixed device array of the library instead of a
// caller buffer, for callers that cannot allocate device memory (code under
// stream capture, tight serving loops, harnesses that forbid allocation).
//
// `scratch` below is a file-scope device array: each GPU the library runs on
// holds its own copy, at its own address, until the process ends.  In host
// code its name is only a host-side handle, so the device address is looked
// up once per device with hipGetSymbolAddress (with that device current) and
// kept in a per-device table; kernels get that address, never the name.
// Every call on a GPU shares that GPU's array: calls that overlap on one GPU
// (two streams, two host threads) race on it.  The stack's kernels write
// every byte they later read within one call (packed weights, column scales,
// the per-layer attention output), so nothing has to start at zero and the
// previous call's contents never leak into a result.
#include <mutex>

#include "pip_internal.h"

namespace {

__device__ __align__(256) unsigned char scratch[PIP_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];  // device address of `scratch`; null until looked up

// The current device's address of `scratch` (looked up on its first call).
pip_status device_scratch(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return PIP_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return PIP_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return PIP_ERR_HIP;
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return PIP_OK;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

extern "C" pip_status pip_block_stack_noalloc(float *X, const float *Wq, const float *Wk,
                                              const float *Wv, const float *Wo, const float *U,
                                              const uint8_t *mask, int64_t B, int64_t P,
                                              int64_t C, int64_t H, int64_t L, void *stream) {
    // the same checks, in the same order, as pip_block_stack
    if (C < 0 || H < 0 || L < 0 || B < 0 || P < 0) return PIP_ERR_SHAPE;
    if (B == 0 || P == 0) return PIP_OK;
    if (P % 16 != 0 || P > PIP_MAX_P || B > (int64_t)1 << 24) return PIP_ERR_UNSUPPORTED;
    if (L == 0) return PIP_OK;
    if (!X || !Wq || !Wk || !Wv || !Wo || !U || !mask) return PIP_ERR_NULL;
    if (H == 0 || C != (int64_t)PIP_HEAD_DIM * H) return PIP_ERR_SHAPE;
    if (H > 16 || L > (1 << 20)) return PIP_ERR_UNSUPPORTED;
    if (!aligned16(X) || !aligned16(Wq) || !aligned16(Wk) || !aligned16(Wv) ||
        !aligned16(Wo) || !aligned16(U))
        return PIP_ERR_ALIGN;
    const size_t need = pip_block_stack_workspace_bytes(B, P, C, L);
    if (need == 0) return PIP_ERR_UNSUPPORTED;
    if (need > (size_t)PIP_NOALLOC_SCRATCH_BYTES) return PIP_ERR_TOO_LARGE;
    void *ws = nullptr;
    pip_status st = device_scratch(&ws);
    if (st != PIP_OK) return st;
    const hipError_t e = pip::launch_block_stack(X, Wq, Wk, Wv, Wo, U, mask, (int)B, (int)P,
                                                 (int)C, (int)H, (int)L, ws,
                                                 (hipStream_t)stream);
    return e == hipSuccess ? PIP_OK : PIP_ERR_HIP;
}

// pip_internal.h -- host-side declarations shared by the libpip sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pip.h"

// Device-resident folded pair MLP.  Packed operand layouts (each operand is 64
// lane values, one per lane of a wave):
//  float32 (w32), operands in this order:
//   L1  c = 0..3:                 lane l -> W1'[16c + l%16][l/16]
//   L2  (co, ci, r) 4x4x4:        lane l -> W2'[16co + l%16][16ci + 4(l/16) + r]
//   L3  (co, ci, r) 4x4x4:        same with W3'
//   L4  (ci, r) 4x4:              lane l -> W4[l%16][16ci + 4(l/16) + r] (rows >= 8: 0)
//  bfloat16 (w16), 8 values per lane per operand:
//   L2, L3  (co, s) 4x2:  slot j<4 -> W'[16co + l%16][32s + 4(l/16) + j]
//                         slot j>=4 -> W'[16co + l%16][32s + 16 + 4(l/16) + j-4]
//   L4      s = 0..1:     same with W4 (rows >= 8: 0)
//  bias: b1' (64) | b2' (64) | b3' (64) | b4 (8), plain.
struct pip_pair_mlp {
    int device;
    float *w32;
    uint16_t *w16;
    float *bias;
};

namespace pip {
constexpr int kW32Ops = 4 + 64 + 64 + 16;  // 148
constexpr int kW32L1 = 0, kW32L2 = 4 * 64, kW32L3 = 68 * 64, kW32L4 = 132 * 64;
constexpr int kW16Ops = 8 + 8 + 2;         // 18, each 64 lanes x 8 bf16
constexpr int kW16L2 = 0, kW16L3 = 8 * 512, kW16L4 = 16 * 512;
constexpr int kBiasL1 = 0, kBiasL2 = 64, kBiasL3 = 128, kBiasL4 = 192;

hipError_t launch_pair_features(const float *p4, const uint8_t *mask, int B, int P, float *F,
                                hipStream_t s);
hipError_t launch_pair_embed_f32(const float *p4, const uint8_t *mask, int B, int P,
                                 const pip_pair_mlp *m, float *U, hipStream_t s);
hipError_t launch_pair_embed_bf16(const float *p4, const uint8_t *mask, int B, int P,
                                  const pip_pair_mlp *m, uint16_t *U, hipStream_t s);
hipError_t launch_attention_f32(const float *Q, const float *K, const float *V,
                                const float *U, const uint8_t *mask, int B, int H, int P,
                                float *O, hipStream_t s);
hipError_t launch_attention_bf16(const uint16_t *Q, const uint16_t *K, const uint16_t *V,
                                 const uint16_t *U, const uint8_t *mask, int B, int H, int P,
                                 uint16_t *O, hipStream_t s);
hipError_t launch_embed_attention_f32(const float *p4, const uint8_t *mask, int B, int P,
                                      const pip_pair_mlp *m, const float *Q, const float *K,
                                      const float *V, float *O, hipStream_t s);
hipError_t launch_embed_attention_bf16(const float *p4, const uint8_t *mask, int B, int P,
                                       const pip_pair_mlp *m, const uint16_t *Q,
                                       const uint16_t *K, const uint16_t *V, uint16_t *O,
                                       hipStream_t s);
hipError_t launch_block_stack(float *X, const float *Wq, const float *Wk, const float *Wv,
                              const float *Wo, const float *U, const uint8_t *mask, int B,
                              int P, int C, int H, int L, float *ws, hipStream_t s);
}  // namespace pip

// pip_internal.h -- host-side declarations shared by the libpip sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pip.h"

// Device-resident folded pair MLP: w32 holds the float32 MFMA operands of all
// four layers, w16 the bfloat16 operands of layers 2..4, bias the folded
// biases b1' | b2' | b3' | b4.  Operand layouts are documented in pip_mlp.h;
// the bf16 operand (layer 2 or 3, co, s) of lane l holds, in slot j,
// W'[16co + l%16][32s + (j < 4 ? 0 : 16) + 4(l/16) + (j & 3)], stored at
// ((layer * 8 + co * 2 + s) * 64 + l) * 8 + j; layer 4 uses operands 16 + s.
// wx2 holds the fp16 hi operands of layers 2..4 followed by the fp16 lo
// operands (same layout as w16); wtx2 the same for W'^T of layers 2 and 3
// (operand (layer, it, s) of lane l holds in slot j W'[32s + (j < 4 ? 0 :
// 16) + 4(l/16) + (j & 3)][16it + l%16], 16 hi operands then 16 lo ones),
// the operands of the backward chain; f16ok is set when every folded weight
// of layers 2..4 lies inside the fp16 range, which the fp16 x 2 chain needs.
struct pip_pair_mlp {
    int device;
    int f16ok;
    float *w32;
    uint16_t *w16;
    uint16_t *wx2;
    uint16_t *wtx2;
    float *bias;
    float *wplain;  // the folded weights in pip_pair_mlp_fold's plain layout (backward)
    int8_t *w8;     // int8 operands of layers 2..4 (int8 mode, layout in abi.hip)
    float *q8;      // their per-channel scales and sums (int8 mode)
};

namespace pip {
// compute units of the current device (cached per device)
int cu_count();
constexpr int kW16L2 = 0, kW16L3 = 8 * 512, kW16L4 = 16 * 512;  // bf16 element offsets

hipError_t launch_pair_features(const float *p4, const uint8_t *mask, int B, int P, float *F,
                                hipStream_t s);
hipError_t launch_pair_embed_f32(const float *p4, const uint8_t *mask, int B, int P,
                                 const pip_pair_mlp *m, float *U, hipStream_t s);
hipError_t launch_pair_embed_bf16(const float *p4, const uint8_t *mask, int B, int P,
                                  const pip_pair_mlp *m, uint16_t *U, hipStream_t s);
// act_scale / act_zero: quantisation of the inputs of layers 2, 3, 4 (host)
hipError_t launch_pair_embed_int8(const float *p4, const uint8_t *mask, int B, int P,
                                  const pip_pair_mlp *m, const float *act_scale,
                                  const int *act_zero, uint16_t *U, hipStream_t s);
// workgroups per (jet, head) of the attention kernel, and the jets its grid
// covers (B rounded up to a multiple of 8)
int attention_chunks(int P);
int64_t attention_jet_slots(int64_t B);
hipError_t launch_attention_f32(const float *Q, const float *K, const float *V,
                                const float *U, const uint8_t *mask, int B, int H, int P,
                                float scale, float *O, hipStream_t s);
hipError_t launch_attention_bf16(const uint16_t *Q, const uint16_t *K, const uint16_t *V,
                                 const uint16_t *U, const uint8_t *mask, int B, int H, int P,
                                 float scale, uint16_t *O, hipStream_t s);
hipError_t launch_embed_attention_f32(const float *p4, const uint8_t *mask, int B, int P,
                                      const pip_pair_mlp *m, const float *Q, const float *K,
                                      const float *V, float scale, float *O, hipStream_t s);
hipError_t launch_embed_attention_bf16(const float *p4, const uint8_t *mask, int B, int P,
                                       const pip_pair_mlp *m, const uint16_t *Q,
                                       const uint16_t *K, const uint16_t *V, float scale,
                                       uint16_t *O, hipStream_t s);
// packed (variable-length) layout
hipError_t launch_packed_offsets(const int *cu, int B, int64_t *uoff, hipStream_t s);
hipError_t launch_pair_embed_packed_f32(const float *p4, const int *cu, const int64_t *uoff,
                                        int B, int N, int max_n, const pip_pair_mlp *m,
                                        float *U, int64_t u_elems, hipStream_t s);
hipError_t launch_pair_embed_packed_bf16(const float *p4, const int *cu, const int64_t *uoff,
                                         int B, int N, int max_n, const pip_pair_mlp *m,
                                         uint16_t *U, int64_t u_elems, hipStream_t s);
hipError_t launch_attention_packed_f32(const float *Q, const float *K, const float *V,
                                       const float *U, const int *cu, const int64_t *uoff, int B,
                                       int H, int N, int max_n, int64_t u_elems, float scale,
                                       float *O, hipStream_t s);
hipError_t launch_attention_packed_bf16(const uint16_t *Q, const uint16_t *K,
                                        const uint16_t *V, const uint16_t *U, const int *cu,
                                        const int64_t *uoff, int B, int H, int N, int max_n,
                                        int64_t u_elems, float scale, uint16_t *O,
                                        hipStream_t s);
// backward pass
hipError_t launch_attention_bwd_f32(const float *Q, const float *K, const float *V,
                                    const float *U, const uint8_t *mask, const float *dO, int B,
                                    int H, int P, float scale, float *dQ, float *dK, float *dV,
                                    float *dU, hipStream_t s);
size_t mlp_bwd_workspace(int B, int P);
hipError_t launch_mlp_bwd_f32(const float *p4, const uint8_t *mask, int B, int P,
                              const pip_pair_mlp *m, const float *dU, float *grad, void *ws,
                              hipStream_t s);
// bytes of workspace the block stack needs
size_t block_stack_workspace(int B, int P, int C, int L);
hipError_t launch_block_stack(float *X, const float *Wq, const float *Wk, const float *Wv,
                              const float *Wo, const float *U, const uint8_t *mask, int B,
                              int P, int C, int H, int L, void *ws, hipStream_t s);
}  // namespace pip

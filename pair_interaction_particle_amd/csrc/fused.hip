// fused.hip -- placeholder until the fused kernel lands.
#include "pip_internal.h"
namespace pip {
hipError_t launch_embed_attention_f32(const float *, const uint8_t *, int, int, const pip_pair_mlp *,
                                      const float *, const float *, const float *, float *, hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t launch_embed_attention_bf16(const float *, const uint8_t *, int, int, const pip_pair_mlp *,
                                       const uint16_t *, const uint16_t *, const uint16_t *, uint16_t *,
                                       hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t launch_block_stack(float *, const float *, const float *, const float *, const float *,
                              const float *, const uint8_t *, int, int, int, int, int, float *, hipStream_t) {
    return hipErrorNotSupported;
}
}  // namespace pip

/*
 * pip.h -- C ABI of the MI355X pair-interaction library (libpip.so).
 *
 * The path: for every particle pair of a jet, four Lorentz-invariant features
 * (ln kT, ln z, ln dR, ln m2) go through a pointwise pair MLP
 * 4 -> 64 -> 64 -> 64 -> 8 (eval-mode BatchNorm folded into the weights, GELU
 * between layers), which gives one additive attention-bias plane U_h per head;
 * masked multi-head attention softmax(Q K^T / sqrt(D) + U_h) V then consumes
 * it.  Source: "Event Classification with Masked Transformer Autoencoders"
 * (ml4sci_cms_e2e26 README), section "How the Kernel Fusion Works",
 * paragraphs "Fusion 2" (features + Conv1d MLP with BatchNorm + GELU, BN
 * folded at eval time, bias written as (B, H, P, P)) and "Fusion 3"
 * (softmax(Q K^T / sqrt(d) + bias) V, flash-style online softmax).  The four
 * features are those of the Particle Transformer paper (Qu et al., ICML 2022)
 * that the README lists under References.
 *
 * Conventions shared by every entry point:
 *  - All arrays are dense, row-major (C order), and 16-byte aligned.
 *  - Arrays passed to the compute entries are DEVICE pointers owned by the
 *    caller; the library never allocates, frees or synchronises inside them.
 *    Each call only enqueues kernels on `stream` (a hipStream_t; NULL = the
 *    null stream) and returns.
 *  - 4-momenta are energy-first (E, px, py, pz), float32, shaped (B, P, 4),
 *    as in the lloca transformer_v2.Transformer.forward documentation
 *    (p_ref parameter).
 *  - mask is uint8 (B, P); nonzero marks a real particle.  Masks need not be
 *    prefixes.  Values stored in padded slots (p4, Q, K, V, U) are never
 *    read into a result: every output that involves a padded slot is exactly
 *    +0.0 (bit pattern 0), padded query rows included.
 *  - Pair features clamp each logarithm's argument below at PIP_FEATURE_EPS.
 *  - dtype codes: PIP_F32 (float32) or PIP_BF16 (bfloat16 bit patterns stored
 *    as uint16).
 *  - Errors are returned, never thrown; nothing is launched when a call
 *    returns an error other than PIP_ERR_HIP.  PIP_ERR_HIP means a HIP
 *    runtime call failed; hipGetLastError() was consumed.
 *  - An empty problem (B == 0 or P == 0; also H == 0 for attention, L == 0
 *    for the block stack) is a no-op that returns PIP_OK once the sizes and
 *    dtype are valid; its array pointers are not checked and may be NULL.
 */
#ifndef PIP_H
#define PIP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PIP_VERSION 1
#define PIP_FEATURE_EPS 1e-8 /* clamp of every feature's log argument */
#define PIP_HIDDEN 64        /* pair-MLP hidden width */
#define PIP_HEADS 8          /* pair-MLP outputs = attention heads */
#define PIP_HEAD_DIM 16      /* the only head dimension the kernels take */
#define PIP_MAX_P 256        /* largest particle count per jet */

typedef enum {
    PIP_OK = 0,
    PIP_ERR_NULL = 1,        /* a required pointer is NULL */
    PIP_ERR_SHAPE = 2,       /* a size is negative, zero where it cannot be, or inconsistent */
    PIP_ERR_ALIGN = 3,       /* a pointer is not 16-byte aligned */
    PIP_ERR_DTYPE = 4,       /* unknown dtype code */
    PIP_ERR_UNSUPPORTED = 5, /* well-formed but outside what the kernels take
                                (P % 16 != 0, P > 256, D != 16, H != 8 where fixed, ...) */
    PIP_ERR_HIP = 6          /* a HIP runtime call (launch, alloc, copy) failed */
} pip_status;

typedef enum { PIP_F32 = 0, PIP_BF16 = 1 } pip_dtype;

/* Raw (unfolded) pair-MLP parameters, HOST float32 pointers, exactly as a
 * PyTorch ParT pair embedding stores them: Conv1d(k=1) weights (out, in) and
 * biases, then eval-mode BatchNorm1d (gamma, beta, running mean, running var)
 * after each of the three hidden linears, before its GELU.
 *   w1 (64, 4)  w2 (64, 64)  w3 (64, 64)  w4 (8, 64);  b1..b3 (64), b4 (8)
 *   bn_*[k] (64) for hidden layer k = 0, 1, 2
 *   in_* (4): optional BatchNorm on the 4 input features (all NULL = none)
 * Any bias pointer may be NULL (= zeros).  bn_eps is BatchNorm's epsilon. */
typedef struct {
    const float *w1, *b1, *w2, *b2, *w3, *b3, *w4, *b4;
    const float *bn_gamma[3], *bn_beta[3], *bn_mean[3], *bn_var[3];
    const float *in_gamma, *in_beta, *in_mean, *in_var;
    float bn_eps;
} pip_pair_mlp_params;

/* Opaque folded + MFMA-packed pair MLP resident on one device. */
typedef struct pip_pair_mlp pip_pair_mlp;

/* Human-readable name of a status code (static string). */
const char *pip_status_string(int status);
int pip_version(void);

/* Fold eval-mode BatchNorm into the linear layers on the host, in float64
 * ("Fusion 2": BatchNorm folded into the linear weights at eval time):
 *   s = gamma / sqrt(var + eps);  W' = diag(s) W;  b' = s (b - mean) + beta,
 * and the optional input BatchNorm into layer 1 from the right.
 * Outputs (HOST, float32, plain (out, in) layout):
 *   w_out: w1' (64*4) | w2' (64*64) | w3' (64*64) | w4 (8*64)  = 8,960 floats
 *   b_out: b1' (64) | b2' (64) | b3' (64) | b4 (8)             = 200 floats
 * Touches no GPU.  Errors: PIP_ERR_NULL, PIP_ERR_SHAPE (var + eps <= 0). */
pip_status pip_pair_mlp_fold(const pip_pair_mlp_params *raw, float *w_out, float *b_out);

/* Fold (as pip_pair_mlp_fold), repack into MFMA operand order (float32 and
 * bfloat16 copies) and upload to the CURRENT device.  *out receives a handle
 * the caller frees with pip_pair_mlp_destroy.  Allocates device memory once
 * (about 60 KB); not meant for the hot loop.
 * Errors: PIP_ERR_NULL, PIP_ERR_SHAPE, PIP_ERR_HIP. */
pip_status pip_pair_mlp_create(const pip_pair_mlp_params *raw, pip_pair_mlp **out);
pip_status pip_pair_mlp_destroy(pip_pair_mlp *mlp);

/* Pair features F (B, 4, P, P) float32 (device), channel order
 * [ln kT, ln z, ln dR, ln m2], of every ordered pair of real particles, the
 * diagonal included; 0 where a or b is padded.  Diagnostic/parity entry
 * ("Fusion 2" names the four features).
 * Requires P % 16 == 0, 16 <= P <= 256.  Errors: NULL, SHAPE, ALIGN,
 * UNSUPPORTED, HIP. */
pip_status pip_pair_features(const float *p4, const uint8_t *mask, int64_t B, int64_t P,
                             float *F, void *stream);

/* Pair embedding: U (B, 8, P, P) in u_dtype (device) = the pair MLP applied
 * to the features of every ordered pair ("Fusion 2": features and the whole
 * MLP in one launch, hidden states kept on chip, only the (B, H, P, P) bias
 * written).  U[b, h, a, c] is the bias of head h for query a and key c; U is
 * symmetric in (a, c).  Pairs touching a padded slot are exactly 0.
 * u_dtype PIP_F32: float32 MLP.  PIP_BF16: layer 1 float32, hidden layers
 * 2..4 bfloat16 operands with float32 accumulation, U stored as bfloat16.
 * `mask` must be 16-byte aligned too (its rows are read as 16-byte vectors).
 * Requires P % 16 == 0, 16 <= P <= 256.  Errors: NULL, SHAPE, ALIGN, DTYPE,
 * UNSUPPORTED, HIP. */
pip_status pip_pair_embed(const float *p4, const uint8_t *mask, int64_t B, int64_t P,
                          const pip_pair_mlp *mlp, void *U, int u_dtype, void *stream);

/* Masked biased attention ("Fusion 3"): for every head h and real query a,
 *   O[b,h,a,:] = sum_c softmax_c(Q[b,h,a,:] . K[b,h,c,:] / sqrt(D) + U[b,h,a,c]) V[b,h,c,:]
 * over real keys c only; padded query rows are 0.  Q, K, V, O are (B, H, P, D),
 * U is (B, H, P, P), all in `dtype` (PIP_BF16: bf16 storage, MFMA in bf16
 * with float32 accumulation, softmax in float32).
 * Requires D == 16, P % 16 == 0, 16 <= P <= 256, H >= 1.  Errors: NULL,
 * SHAPE, ALIGN, DTYPE, UNSUPPORTED, HIP. */
pip_status pip_pair_bias_attention(const void *Q, const void *K, const void *V, const void *U,
                                   const uint8_t *mask, int64_t B, int64_t H, int64_t P,
                                   int64_t D, void *O, int dtype, void *stream);

/* Fused pair embedding + attention with H = 8: the same O as pip_pair_embed
 * followed by pip_pair_bias_attention, but U only ever lives on chip.
 * Q, K, V, O are (B, 8, P, D) in `dtype` (PIP_BF16: the MLP as in
 * pip_pair_embed's bf16 mode, U kept in float32 on chip, attention as in
 * pip_pair_bias_attention's bf16 mode).  Unlike the other entries it also
 * requires `mask` to be 16-byte aligned (rows are read as 16-byte vectors).
 * Requires D == 16, P % 16 == 0, 16 <= P <= 256.  Errors: NULL, SHAPE,
 * ALIGN, DTYPE, UNSUPPORTED, HIP. */
pip_status pip_pair_embed_attention(const float *p4, const uint8_t *mask,
                                    const pip_pair_mlp *mlp, const void *Q, const void *K,
                                    const void *V, int64_t B, int64_t P, int64_t D, void *O,
                                    int dtype, void *stream);

/* Bytes of device workspace pip_block_stack needs for L layers: the attention
 * output of a layer (B * P * C floats) plus every layer's weights packed as
 * split fp16 matrix-core operands (L * 4 * C^2 * 2 * 2 bytes for C a multiple
 * of 32) and their column scales.  0 for sizes the stack does not take. */
size_t pip_block_stack_workspace_bytes(int64_t B, int64_t P, int64_t C, int64_t L);

/* L attention layers reusing one bias U (the ParT encoder's attention
 * sublayer with embed C and H heads, "Architecture Comparison"), float32:
 * for l = 0..L-1:
 *   Q = X Wq[l], K = X Wk[l], V = X Wv[l]   (head h owns columns h*16 .. h*16+15)
 *   O = masked biased attention per head with U (B, H, P, P)
 *   X <- X + O Wo[l]
 * X (B, P, C) is updated in place; Wq, Wk, Wv, Wo are (L, C, C) applied as
 * X @ W.  Padded rows of X are left unchanged (their O is 0).  workspace
 * must hold pip_block_stack_workspace_bytes(B, P, C, L) bytes; its contents
 * are scratch (overwritten by every call; calls that share a workspace on
 * different streams race).  The products run on the fp16 matrix cores with
 * split operands (hi + lo per float32 value, each row and weight column
 * scaled by an exact power of two first), float32-faithful to ~1e-6.
 * Requires C == 16 * H, 1 <= H <= 16, P % 16 == 0, 16 <= P <= 256.
 * Errors: NULL, SHAPE, ALIGN, UNSUPPORTED, HIP. */
pip_status pip_block_stack(float *X, const float *Wq, const float *Wk, const float *Wv,
                           const float *Wo, const float *U, const uint8_t *mask, int64_t B,
                           int64_t P, int64_t C, int64_t H, int64_t L, void *workspace,
                           size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* PIP_H */

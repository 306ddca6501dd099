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
/* bytes of the fixed per-device scratch array behind pip_block_stack_noalloc */
#define PIP_NOALLOC_SCRATCH_BYTES (16u << 20)
/* gradient arrays of the pair MLP (pip_pair_mlp_backward, pip_pair_mlp_unfold_grads) */
#define PIP_PAIR_MLP_FOLDED_GRADS 9160
#define PIP_PAIR_MLP_RAW_GRADS 9552
/* L-GATr: components of one multivector; largest scalar channel count */
#define PIP_LGATR_MV 16
#define PIP_LGATR_MAX_S 256

typedef enum {
    PIP_OK = 0,
    PIP_ERR_NULL = 1,        /* a required pointer is NULL */
    PIP_ERR_SHAPE = 2,       /* a size is negative, zero where it cannot be, or inconsistent */
    PIP_ERR_ALIGN = 3,       /* a pointer is not 16-byte aligned */
    PIP_ERR_DTYPE = 4,       /* unknown dtype code */
    PIP_ERR_UNSUPPORTED = 5, /* well-formed but outside what the kernels take
                                (P % 16 != 0, P > 256, D != 16, H != 8 where fixed, ...) */
    PIP_ERR_HIP = 6,         /* a HIP runtime call (launch, alloc, copy) failed */
    PIP_ERR_VALUE = 7,       /* a scalar argument is outside its domain (a scale that is
                                not finite) */
    PIP_ERR_TOO_LARGE = 8    /* the problem needs more scratch than the library's fixed
                                device buffer holds (pip_block_stack_noalloc) */
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

/* Fold (as pip_pair_mlp_fold), repack into MFMA operand order and upload to
 * the CURRENT device.  The handle holds every operand form the kernels take
 * (float32, fp16 hi / lo and bfloat16), so it has no dtype of its own: the
 * compute entries choose the precision per call.  *out receives a handle
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

/* Pair embedding with int8 inputs to the hidden linears: the "Economical Jet
 * Taggers" summary (gist.science, Technische Samenvatting, Methodologie,
 * "Datatype Kwantisering") quantises the inputs of linear layers to int8
 * with a zero point and keeps bfloat16 for the rest.  Here: features and
 * layer 1 float32, GELU float32; the inputs h of layers 2, 3, 4 quantised
 * per tensor, q = clamp(rint(h / S) + Z, -128, 127) with the caller's
 * act_scale[l] = S > 0 and act_zero[l] = Z in [-128, 127] (HOST arrays of 3,
 * a calibration of the model); the folded weights of layers 2, 3, 4
 * quantised per output channel when the handle is created, sw = max |W'| /
 * 127, Wq = clamp(rint(W' / sw), -127, 127); each product on the int8 matrix
 * cores with exact int32 sums, y = S sw (sum Wq q - Z sum Wq) + b'.  U
 * (B, 8, P, P) is stored as bfloat16; pairs touching a padded slot are +0.0.
 * Requires P % 16 == 0, 16 <= P <= 256.  Errors: NULL, SHAPE, ALIGN,
 * UNSUPPORTED, VALUE (a scale not finite and positive, a zero point out of
 * range), HIP. */
pip_status pip_pair_embed_int8(const float *p4, const uint8_t *mask, int64_t B, int64_t P,
                               const pip_pair_mlp *mlp, const float *act_scale,
                               const int32_t *act_zero, void *U, void *stream);

/* Masked biased attention ("Fusion 3"): for every head h and real query a,
 *   O[b,h,a,:] = sum_c softmax_c(scale * Q[b,h,a,:] . K[b,h,c,:] + U[b,h,a,c]) V[b,h,c,:]
 * over real keys c only; padded query rows are 0.  "Fusion 3" writes the
 * score scale as 1/sqrt(d); `scale` is that factor, passed by the caller
 * (0.25 for D = 16), and must be finite (PIP_ERR_VALUE otherwise).  U is
 * added after the scaling, unscaled.  Q, K, V, O are (B, H, P, D), U is
 * (B, H, P, P), all in `dtype`.
 * PIP_F32: float32-faithful; the products run on the fp16 matrix cores with
 * split operands (hi + lo), K and V scaled per head and Q per row by exact
 * powers of two first, so any finite magnitudes keep ~2^-22 relative product
 * error.  Real Q, K or V entries that are not finite give non-finite outputs
 * in the rows they reach.
 * PIP_BF16: bf16 storage, MFMA in bf16 with float32 accumulation, softmax in
 * float32.
 * Requires D == 16, P % 16 == 0, 16 <= P <= 256, H >= 1.  Errors: NULL,
 * SHAPE, ALIGN, DTYPE, UNSUPPORTED, VALUE, HIP. */
pip_status pip_pair_bias_attention(const void *Q, const void *K, const void *V, const void *U,
                                   const uint8_t *mask, int64_t B, int64_t H, int64_t P,
                                   int64_t D, float scale, void *O, int dtype, void *stream);

/* Fused pair embedding + attention with H = 8: the same O as pip_pair_embed
 * followed by pip_pair_bias_attention (same `scale`), but U only ever lives
 * on chip.  Q, K, V, O are (B, 8, P, D) in `dtype` (PIP_BF16: the MLP as in
 * pip_pair_embed's bf16 mode, U kept in float32 on chip, attention as in
 * pip_pair_bias_attention's bf16 mode).  Unlike the other entries it also
 * requires `mask` to be 16-byte aligned (rows are read as 16-byte vectors).
 * Requires D == 16, P % 16 == 0, 16 <= P <= 256.  Errors: NULL, SHAPE,
 * ALIGN, DTYPE, UNSUPPORTED, VALUE, HIP. */
pip_status pip_pair_embed_attention(const float *p4, const uint8_t *mask,
                                    const pip_pair_mlp *mlp, const void *Q, const void *K,
                                    const void *V, int64_t B, int64_t P, int64_t D, float scale,
                                    void *O, int dtype, void *stream);

/* ---- Backward pass (float32).  Fusion 3 of the ml4sci_cms_e2e26 README names
 * a forward and a backward kernel for the biased attention; the README's
 * end-to-end benchmarks have a "Train" column.  A training step runs
 * pip_pair_bias_attention_backward (dL/dO -> dQ, dK, dV and dU = dL/dU) and
 * then pip_pair_mlp_backward (dU -> the gradient of the pair MLP's
 * parameters; the features have none).  BatchNorm is in eval mode (running
 * statistics fixed), as in the forward. */

/* Gradients of pip_pair_bias_attention for dL/dO = dO (B, H, P, D): with
 * p = softmax over real keys of s_c = scale q.k_c + U[a, c],
 *   dS = p o (dO v^T - dO . O),  dU = dS,  dQ = scale dS K,  dK = scale dS^T Q,
 *   dV = P^T dO.
 * dQ, dK, dV are (B, H, P, D) and dU (B, H, P, P), all written in full:
 * every entry that involves a padded slot is +0.0 (values in padded slots of
 * the inputs, dO included, are never read into a result).  The forward is
 * recomputed from Q, K, V, U (no saved statistics).  Only PIP_F32 (float32
 * matrix cores, float32 results); PIP_BF16 returns PIP_ERR_UNSUPPORTED.
 * The query blocks' contributions to dK and dV are added in a fixed order:
 * every output is the same bit for bit on every run.
 * Requires D == 16, P % 16 == 0, P <= 256.  Errors: NULL, SHAPE, ALIGN,
 * DTYPE, UNSUPPORTED, VALUE, HIP. */
pip_status pip_pair_bias_attention_backward(const void *Q, const void *K, const void *V,
                                            const void *U, const uint8_t *mask,
                                            const void *dO, int64_t B, int64_t H, int64_t P,
                                            int64_t D, float scale, void *dQ, void *dK,
                                            void *dV, void *dU, int dtype, void *stream);

/* Bytes of workspace pip_pair_mlp_backward needs: PIP_PAIR_MLP_FOLDED_GRADS
 * floats per (jet, row tile of 16) slot (S = B * P/16 slots) and per
 * workgroup of the fp16 x 2 kernel (Gx = 16 S for S < 16, else 256), one per
 * 32 of max(S, Gx) for the fixed-order reduction; then 3 Gx + S + 2 ints
 * (the workgroups' overflow flags and the plan of their shares). */
size_t pip_pair_mlp_backward_workspace_bytes(int64_t B, int64_t P);

/* Gradient of L with respect to the folded pair-MLP parameters, for dL/dU =
 * dU (B, 8, P, P) float32 and U = pip_pair_embed(p4, mask, mlp): every
 * unique real pair contributes the backward of its MLP evaluation with
 * g = dU[a, c] + dU[c, a] (dU[a, a] on the diagonal; U is symmetric), so
 * dU's padded entries are never read into the result.  grad (device,
 * PIP_PAIR_MLP_FOLDED_GRADS floats) has pip_pair_mlp_fold's layout:
 *   dW1' (64*4) dW2' (64*64) dW3' (64*64) dW4 (8*64) | db1' db2' db3' (64) db4 (8)
 * GELU in its erf form, Phi evaluated to 7.5e-8.  When the handle's weights
 * fit fp16 (as for the fp16 x 2 forward), the products run on the fp16
 * matrix cores with every float32 factor split into two fp16 halves
 * (relative error ~2^-22 per product) and g scaled by a power of two per
 * round of 128 pairs; if a sum leaves the fp16 range, the whole gradient is
 * recomputed with float32 products, as it is for other weights.
 * workspace: pip_pair_mlp_backward_workspace_bytes(B, P) bytes, scratch
 * (overwritten; calls sharing one on different streams race).  Every sum
 * is taken in a fixed order: the result is the same bit for bit on every
 * run.  Requires P % 16 == 0, P <= 256.  Errors: NULL, SHAPE, ALIGN,
 * UNSUPPORTED, HIP. */
pip_status pip_pair_mlp_backward(const float *p4, const uint8_t *mask, int64_t B, int64_t P,
                                 const pip_pair_mlp *mlp, const float *dU, float *grad,
                                 void *workspace, size_t workspace_bytes, void *stream);

/* Chain rule from the folded gradient (HOST, PIP_PAIR_MLP_FOLDED_GRADS) to
 * the raw parameters of `raw` (HOST, PIP_PAIR_MLP_RAW_GRADS floats), in
 * float64, through W' = diag(s) W diag(si), b' = s (W ti + b - mean) + beta,
 * s = gamma / sqrt(var + eps) (si, ti: the optional input BatchNorm):
 *   w1 (64*4) b1 g1 be1 (64 each) | w2 (64*64) b2 g2 be2 | w3 (64*64) b3 g3 be3 |
 *   w4 (8*64) b4 (8) | in_gamma (4) in_beta (4)   (0 without input BatchNorm)
 * (g = BatchNorm gamma, be = beta; running statistics are not trained).
 * Touches no GPU.  Errors: NULL, SHAPE (var + eps <= 0). */
pip_status pip_pair_mlp_unfold_grads(const pip_pair_mlp_params *raw, const float *grad_folded,
                                     float *grad_raw);

/* ---- Packed variable-length layout.  Jets are stored back to back instead
 * of zero-padded to P slots: jet b owns particle rows cu_seqlens[b] ..
 * cu_seqlens[b+1]-1, n_b = cu_seqlens[b+1] - cu_seqlens[b] (the `ptr` of the
 * lloca transformer_v2.Transformer.forward documentation; the gist.science
 * summary of "Virtues and Vices of Equivariant Transformers", Methodologie,
 * names sparse representations as the way to skip padding).  Every row is a
 * real particle; there is no mask.
 *   p4      (N, 4) float32, energy-first
 *   Q, K, V, O  (H, N, D), head-major: head h of jet b is rows
 *           h*N + cu_seqlens[b] .. h*N + cu_seqlens[b+1]-1
 *   U       jet b: (H, n_b, ld_b) with ld_b = n_b rounded up to a multiple of 8
 *           (rows start 16-byte aligned; pip_pair_embed_packed writes the <= 7
 *           columns past n_b as 0 and attention never reads them into a
 *           result), starting at element H * u_offsets[b], where
 *           u_offsets[0] = 0 and u_offsets[b+1] = u_offsets[b] + n_b * ld_b.
 *           u_elems is the U buffer's length in elements (>= H * u_offsets[B]).
 * cu_seqlens is int32 (B + 1), u_offsets int64 (B + 1), both DEVICE arrays
 * (4- and 8-byte aligned).  max_n (<= 256) bounds every n_b; the kernels read
 * cu_seqlens / u_offsets on the device and skip any jet whose entries are
 * inconsistent (n_b < 0 or > max_n, rows past N, a U block of the wrong size
 * or past u_elems): nothing of such a jet is written.
 * Results equal those of the padded entries on the same jets (mask = the
 * first n_b slots), row for row. */

/* u_offsets (B + 1, device int64) from cu_seqlens (B + 1, device int32), on
 * the stream (one workgroup scans the batch).  Errors: NULL, SHAPE, ALIGN,
 * UNSUPPORTED (B > 2^24), HIP. */
pip_status pip_packed_u_offsets(const int32_t *cu_seqlens, int64_t B, int64_t *u_offsets,
                                void *stream);

/* pip_pair_embed on the packed layout ("Fusion 2"): U blocks as above, in
 * u_dtype (PIP_F32 or PIP_BF16, the same arithmetic as pip_pair_embed).  No
 * padded tile is computed or written.  Errors: NULL, SHAPE, ALIGN, DTYPE,
 * UNSUPPORTED (max_n > 256, N > 2^30, B > 2^24), HIP. */
pip_status pip_pair_embed_packed(const float *p4, const int32_t *cu_seqlens,
                                 const int64_t *u_offsets, int64_t B, int64_t N, int64_t max_n,
                                 const pip_pair_mlp *mlp, void *U, int64_t u_elems, int u_dtype,
                                 void *stream);

/* pip_pair_bias_attention on the packed layout ("Fusion 3"): for every jet b,
 * head h and row a < n_b,
 *   O[h, cu[b]+a, :] = sum_{c < n_b} softmax_c(scale Q[h,cu[b]+a,:] . K[h,cu[b]+c,:]
 *                                              + U_b[h, a, c]) V[h, cu[b]+c, :].
 * Rows of skipped jets are not written.  dtype as in pip_pair_bias_attention.
 * Requires D == 16.  Errors: NULL, SHAPE, ALIGN, DTYPE, UNSUPPORTED, VALUE,
 * HIP. */
pip_status pip_pair_bias_attention_packed(const void *Q, const void *K, const void *V,
                                          const void *U, const int32_t *cu_seqlens,
                                          const int64_t *u_offsets, int64_t B, int64_t H,
                                          int64_t N, int64_t max_n, int64_t D, float scale,
                                          int64_t u_elems, void *O, int dtype, void *stream);

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

/* pip_block_stack without a workspace argument and without any allocation,
 * for callers that cannot allocate device memory: code under HIP stream or
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments (minus the workspace), result and errors as pip_block_stack.
 * The workspace lives in a fixed array of PIP_NOALLOC_SCRATCH_BYTES (16 MiB)
 * inside the library, one per GPU, held until the process ends; problems
 * whose pip_block_stack_workspace_bytes exceed it return PIP_ERR_TOO_LARGE
 * before any launch (B=128, P=128, C=128, L=8 needs about 10 MiB).  All calls
 * on one GPU share that GPU's array: calls that overlap on one GPU (other
 * streams, other host threads) race and must be serialised by the caller.
 * The first call on a device looks the array's address up (no allocation);
 * nothing in the array needs to start at zero.
 * Errors: NULL, SHAPE, ALIGN, UNSUPPORTED, TOO_LARGE, HIP. */
pip_status pip_block_stack_noalloc(float *X, const float *Wq, const float *Wk, const float *Wv,
                                   const float *Wo, const float *U, const uint8_t *mask,
                                   int64_t B, int64_t P, int64_t C, int64_t H, int64_t L,
                                   void *stream);

/* ---- L-GATr: spacetime-algebra multivectors ----------------------------
 * Source: README "How the Kernel Fusion Works", "Fusion 1" (the equivariant
 * linear layer of L-GATr: its weights span the 10 linear maps of a
 * multivector that commute with Lorentz transformations; the fused form
 * expands them once into W_eff over the concatenated [multivector
 * components, scalars] and applies one contraction) and "Results", table
 * "L-GATr Kernels" (the equivariant linear layer and the geometric product
 * at B=128, items=128, 8 multivector and 16 scalar channels).
 * A multivector of Cl(1,3) (generators e0..e3, e0^2 = +1, e1^2 = e2^2 =
 * e3^2 = -1) is PIP_LGATR_MV = 16 float32 components in blade order
 *   1, e0, e1, e2, e3, e01, e02, e03, e12, e13, e23, e012, e013, e023, e123, e0123
 * (generator indices ascending within a blade). */

/* z = x y, the geometric product of n multivector pairs; x, y, z are
 * (n, 16) float32 device arrays.  z may be x or y (each thread reads its
 * pair before it writes).  n == 0 is a no-op.
 * Errors: NULL, SHAPE (n < 0), ALIGN, UNSUPPORTED (n > 2^38), HIP. */
pip_status pip_lgatr_geometric_product(const float *x, const float *y, int64_t n, float *z,
                                       void *stream);

/* Host only: the expanded weight W_eff of the equivariant linear layer,
 * rows out_mv*16 + out_s, columns in_mv*16 + in_s (row-major float32, caller's
 * HOST buffer), row/column (c*16 + k) = channel c component k, then the
 * scalar channels.  Basis weights w (out_mv, in_mv, 10): w[o][i][q] for
 * q = 0..4 multiplies the grade-q part of input channel i, q = 5..9 the
 * pseudoscalar e0123 times its grade-(q-5) part (left product).  s2mv
 * (out_mv, in_s) feeds the scalars into the scalar component of the
 * multivector outputs, mv2s (out_s, in_mv) the scalar component of the
 * multivector inputs into the scalar outputs, ss (out_s, in_s) scalars to
 * scalars; a NULL matrix is zero.  Any sizes >= 0.
 * Errors: NULL (w_eff, or w with in_mv, out_mv > 0), SHAPE. */
pip_status pip_lgatr_equilinear_expand(const float *w, const float *s2mv, const float *mv2s,
                                       const float *ss, int in_mv, int out_mv, int in_s,
                                       int out_s, float *w_eff);

/* Device-resident equivariant linear layer: W_eff (pip_lgatr_equilinear_expand)
 * and the biases b_mv (out_mv; added to the scalar component of each
 * multivector output) and b_s (out_s), packed once as the layer's MFMA
 * operands on the current device.  Arguments are HOST arrays (NULL = zero,
 * except w).  Requires in_mv, out_mv in {8, 16}; in_s, out_s multiples of
 * 16 in [0, PIP_LGATR_MAX_S].  Errors: NULL, SHAPE, UNSUPPORTED, HIP. */
typedef struct pip_equilinear pip_equilinear;
pip_status pip_lgatr_equilinear_create(const float *w, const float *s2mv, const float *mv2s,
                                       const float *ss, const float *b_mv, const float *b_s,
                                       int in_mv, int out_mv, int in_s, int out_s,
                                       pip_equilinear **out);
pip_status pip_lgatr_equilinear_destroy(pip_equilinear *layer);

/* y = the equivariant linear layer on n items: x_mv (n, in_mv, 16), x_s
 * (n, in_s) -> y_mv (n, out_mv, 16), y_s (n, out_s), float32 device arrays
 * (x_s / y_s unused and may be NULL when in_s / out_s is 0).  Equal to
 * [y_mv_flat, y_s] = W_eff [x_mv_flat, x_s] + bias, computed in float32 on
 * the matrix cores.  Outputs must not overlap inputs.  The current device
 * must be the layer's.  n == 0 is a no-op.
 * Errors: NULL, SHAPE, ALIGN, UNSUPPORTED (other device, n > 2^34), HIP. */
pip_status pip_lgatr_equilinear(const pip_equilinear *layer, const float *x_mv, const float *x_s,
                                int64_t n, float *y_mv, float *y_s, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* PIP_H */

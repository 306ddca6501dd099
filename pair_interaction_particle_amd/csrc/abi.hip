// abi.hip -- the extern "C" entry points of libpip: argument validation, the
// host-side BatchNorm fold and MFMA operand packing, and kernel dispatch.
// Every check happens before the first HIP call, so an invalid call costs no
// GPU work and can be exercised without a GPU.
#include <math.h>
#include <string.h>

#include <cmath>
#include <vector>

#include "pip_internal.h"
#include "pip_mlp.h"

namespace {

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

pip_status hip_status(hipError_t e) { return e == hipSuccess ? PIP_OK : PIP_ERR_HIP; }

// Sizes the kernels take for the pair grid: 16 <= P <= 256, P % 16 == 0.
pip_status check_pair_grid(int64_t B, int64_t P) {
    if (B < 0 || P < 0) return PIP_ERR_SHAPE;
    if (B == 0 || P == 0) return PIP_OK;
    if (P % 16 != 0 || P > PIP_MAX_P) return PIP_ERR_UNSUPPORTED;
    if (B > (int64_t)1 << 24) return PIP_ERR_UNSUPPORTED;  // keeps the grid in range
    return PIP_OK;
}

// The handle's weights live on the device it was created on.
pip_status check_device(const pip_pair_mlp *m) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return PIP_ERR_HIP;
    return dev == m->device ? PIP_OK : PIP_ERR_UNSUPPORTED;
}

uint16_t host_bf16(float x) {  // round to nearest even; NaN stays NaN
    uint32_t u;
    memcpy(&u, &x, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

}  // namespace

extern "C" {

const char *pip_status_string(int s) {
    switch (s) {
        case PIP_OK: return "ok";
        case PIP_ERR_NULL: return "null pointer";
        case PIP_ERR_SHAPE: return "bad shape";
        case PIP_ERR_ALIGN: return "pointer not 16-byte aligned";
        case PIP_ERR_DTYPE: return "unknown dtype";
        case PIP_ERR_UNSUPPORTED: return "unsupported size or configuration";
        case PIP_ERR_HIP: return "HIP runtime error";
        case PIP_ERR_VALUE: return "invalid argument value";
        case PIP_ERR_TOO_LARGE: return "problem exceeds the fixed scratch buffer";
        default: return "unknown status";
    }
}

int pip_version(void) { return PIP_VERSION; }

}  // extern "C"

// The BatchNorm fold in float64 (pip_pair_mlp_fold rounds it to float32; the
// int8 weights are quantised from it directly).
static pip_status fold_double(const pip_pair_mlp_params *raw, double *w_out, double *b_out) {
    if (!raw || !w_out || !b_out) return PIP_ERR_NULL;
    if (!raw->w1 || !raw->w2 || !raw->w3 || !raw->w4) return PIP_ERR_NULL;
    for (int k = 0; k < 3; ++k)
        if (!raw->bn_gamma[k] || !raw->bn_beta[k] || !raw->bn_mean[k] || !raw->bn_var[k])
            return PIP_ERR_NULL;
    const int nin = (raw->in_gamma != 0) + (raw->in_beta != 0) + (raw->in_mean != 0) +
                    (raw->in_var != 0);
    if (nin != 0 && nin != 4) return PIP_ERR_NULL;
    const double eps = raw->bn_eps;

    // input BatchNorm as x' = si * x + ti (identity when absent)
    double si[4], ti[4];
    for (int k = 0; k < 4; ++k) {
        if (nin) {
            const double v = (double)raw->in_var[k] + eps;
            if (!(v > 0.0)) return PIP_ERR_SHAPE;
            si[k] = (double)raw->in_gamma[k] / sqrt(v);
            ti[k] = (double)raw->in_beta[k] - si[k] * (double)raw->in_mean[k];
        } else {
            si[k] = 1.0;
            ti[k] = 0.0;
        }
    }
    const float *W[3] = {raw->w1, raw->w2, raw->w3};
    const float *bias[3] = {raw->b1, raw->b2, raw->b3};
    const int nins[3] = {4, 64, 64};
    double *wo = w_out;
    for (int l = 0; l < 3; ++l) {
        const int ni = nins[l];
        for (int o = 0; o < 64; ++o) {
            const double v = (double)raw->bn_var[l][o] + eps;
            if (!(v > 0.0)) return PIP_ERR_SHAPE;
            const double s = (double)raw->bn_gamma[l][o] / sqrt(v);
            double z = bias[l] ? (double)bias[l][o] : 0.0;
            for (int i = 0; i < ni; ++i) {
                const double w = (double)W[l][o * ni + i];
                if (l == 0) {
                    wo[o * ni + i] = s * w * si[i];
                    z += w * ti[i];
                } else {
                    wo[o * ni + i] = s * w;
                }
            }
            b_out[64 * l + o] = s * (z - (double)raw->bn_mean[l][o]) + (double)raw->bn_beta[l][o];
        }
        wo += 64 * ni;
    }
    for (int i = 0; i < 8 * 64; ++i) wo[i] = raw->w4[i];
    for (int o = 0; o < 8; ++o) b_out[192 + o] = raw->b4 ? raw->b4[o] : 0.0;
    return PIP_OK;
}

extern "C" {

pip_status pip_pair_mlp_fold(const pip_pair_mlp_params *raw, float *w_out, float *b_out) {
    if (!raw || !w_out || !b_out) return PIP_ERR_NULL;
    double w[8960], b[200];
    const pip_status st = fold_double(raw, w, b);
    if (st != PIP_OK) return st;
    for (int i = 0; i < 8960; ++i) w_out[i] = (float)w[i];
    for (int i = 0; i < 200; ++i) b_out[i] = (float)b[i];
    return PIP_OK;
}


pip_status pip_pair_mlp_create(const pip_pair_mlp_params *raw, pip_pair_mlp **out) {
    if (!out) return PIP_ERR_NULL;
    *out = nullptr;
    std::vector<float> w(64 * 4 + 2 * 64 * 64 + 8 * 64), b(200);
    pip_status st = pip_pair_mlp_fold(raw, w.data(), b.data());
    if (st != PIP_OK) return st;
    const float *W1 = w.data(), *W2 = W1 + 256, *W3 = W2 + 4096, *W4 = W3 + 4096;

    // float32 operands, grouped by four per lane (layouts in pip_mlp.h):
    // operand op of lane l lives at ((op / 4) * 64 + l) * 4 + op % 4.
    std::vector<float> p32(pip::kW32Floats);
    auto at32 = [&](int op, int l) -> float & { return p32[((op / 4) * 64 + l) * 4 + op % 4]; };
    for (int c = 0; c < 4; ++c)
        for (int l = 0; l < 64; ++l) at32(c, l) = W1[(16 * c + l % 16) * 4 + l / 16];
    const float *Wh[2] = {W2, W3};
    for (int t = 0; t < 2; ++t)
        for (int co = 0; co < 4; ++co)
            for (int ci = 0; ci < 4; ++ci)
                for (int r = 0; r < 4; ++r)
                    for (int l = 0; l < 64; ++l)
                        at32(4 + 64 * t + (co * 4 + ci) * 4 + r, l) =
                            Wh[t][(16 * co + l % 16) * 64 + 16 * ci + 4 * (l / 16) + r];
    for (int ci = 0; ci < 4; ++ci)
        for (int r = 0; r < 4; ++r)
            for (int l = 0; l < 64; ++l)
                at32(132 + ci * 4 + r, l) =
                    (l % 16 < 8) ? W4[(l % 16) * 64 + 16 * ci + 4 * (l / 16) + r] : 0.0f;

    // bfloat16 operands: 8 values per lane; slot j < 4 -> channel 32s + 4g + j,
    // slot j >= 4 -> channel 32s + 16 + 4g + (j - 4)
    std::vector<uint16_t> p16(pip::kW16Elems);
    auto chan = [](int s, int g, int j) { return 32 * s + (j < 4 ? 0 : 16) + 4 * g + (j & 3); };
    const int offs16[2] = {pip::kW16L2, pip::kW16L3};
    for (int t = 0; t < 2; ++t)
        for (int co = 0; co < 4; ++co)
            for (int s = 0; s < 2; ++s)
                for (int l = 0; l < 64; ++l)
                    for (int j = 0; j < 8; ++j)
                        p16[offs16[t] + ((co * 2 + s) * 64 + l) * 8 + j] =
                            host_bf16(Wh[t][(16 * co + l % 16) * 64 + chan(s, l / 16, j)]);
    for (int s = 0; s < 2; ++s)
        for (int l = 0; l < 64; ++l)
            for (int j = 0; j < 8; ++j)
                p16[pip::kW16L4 + (s * 64 + l) * 8 + j] =
                    (l % 16 < 8) ? host_bf16(W4[(l % 16) * 64 + chan(s, l / 16, j)]) : 0;

    // fp16 hi / lo operands (same slot layout as the bf16 ones): hi = fp16(w),
    // lo = fp16(w - hi), both round to nearest even.  The fp16 x 2 chain is
    // used only when every layer's folded weights are well scaled for fp16:
    // 2^-8 <= max |W'| <= 2^14 per layer (finite), so products carry at most
    // ~2^-22 relative error plus ~2^-25 absolute per factor in fp16's
    // subnormal range; otherwise the exact float32 chain runs.
    std::vector<uint16_t> px2(2 * pip::kW16Elems);
    bool f16ok = true;
    for (const float *Wl : {W2, W3, W4}) {
        const int n = (Wl == W4) ? 8 * 64 : 64 * 64;
        float mx = 0.0f;
        for (int i = 0; i < n; ++i) {
            if (!std::isfinite(Wl[i])) f16ok = false;
            mx = fmaxf(mx, fabsf(Wl[i]));
        }
        if (!(mx >= 0.00390625f && mx <= 16384.0f)) f16ok = false;
    }
    auto put_x2 = [&](size_t at, float wv) {
        const _Float16 hi = (_Float16)wv;
        const _Float16 lo = (_Float16)(wv - (float)hi);
        px2[at] = __builtin_bit_cast(uint16_t, hi);
        px2[pip::kW16Elems + at] = __builtin_bit_cast(uint16_t, lo);
    };
    for (int t = 0; t < 2; ++t)
        for (int co = 0; co < 4; ++co)
            for (int s = 0; s < 2; ++s)
                for (int l = 0; l < 64; ++l)
                    for (int j = 0; j < 8; ++j)
                        put_x2(offs16[t] + ((co * 2 + s) * 64 + l) * 8 + j,
                               Wh[t][(16 * co + l % 16) * 64 + chan(s, l / 16, j)]);
    for (int s = 0; s < 2; ++s)
        for (int l = 0; l < 64; ++l)
            for (int j = 0; j < 8; ++j)
                put_x2(pip::kW16L4 + (s * 64 + l) * 8 + j,
                       (l % 16 < 8) ? W4[(l % 16) * 64 + chan(s, l / 16, j)] : 0.0f);
    // the transposed operands of layers 2 and 3 for the backward chain:
    // operand (t, it, s) of lane l, slot j: W'[chan(s, l/16, j)][16 it + l%16]
    constexpr size_t kWt = 16 * 64 * 8;
    std::vector<uint16_t> ptx2(2 * kWt);
    for (int t = 0; t < 2; ++t)
        for (int it = 0; it < 4; ++it)
            for (int s = 0; s < 2; ++s)
                for (int l = 0; l < 64; ++l)
                    for (int j = 0; j < 8; ++j) {
                        const float wv = Wh[t][chan(s, l / 16, j) * 64 + 16 * it + l % 16];
                        const _Float16 hi = (_Float16)wv;
                        const _Float16 lo = (_Float16)(wv - (float)hi);
                        const size_t at = (((size_t)t * 8 + it * 2 + s) * 64 + l) * 8 + j;
                        ptx2[at] = __builtin_bit_cast(uint16_t, hi);
                        ptx2[kWt + at] = __builtin_bit_cast(uint16_t, lo);
                    }

    // int8 weights of layers 2, 3, 4 from the float64 fold: per output channel
    // sw = max |W'| / 127 (1 for an all-zero row), Wq = clamp(rint(W' / sw),
    // -127, 127).  Operand (layer, co) of lane l holds, in byte 4c + r of
    // dword c, Wq[16co + l%16][16c + 4(l/16) + r] (the order the int8 chain
    // keeps its inputs in); layer 4 rows >= 8 are 0.  q8: sw (channels 0..63
    // layer 2, 64..127 layer 3, 128..135 layer 4, padded to 144) then the
    // per-channel sums of Wq, as floats.
    std::vector<int8_t> p8(pip::kW8Ops * 64 * 16, 0);
    std::vector<float> q8(pip::kQ8Floats, 0.0f);
    {
        double wd[8960], bd[200];
        fold_double(raw, wd, bd);  // cannot fail: pip_pair_mlp_fold above succeeded
        const double *Wq3[3] = {wd + 256, wd + 4352, wd + 8448};
        const int nout[3] = {64, 64, 8};
        for (int l = 0; l < 3; ++l)
            for (int o = 0; o < nout[l]; ++o) {
                double mx = 0.0;
                for (int i = 0; i < 64; ++i) mx = fmax(mx, fabs(Wq3[l][o * 64 + i]));
                const double sw = mx > 0.0 ? mx / 127.0 : 1.0;
                int sum = 0;
                for (int i = 0; i < 64; ++i) {
                    double q = rint(Wq3[l][o * 64 + i] / sw);
                    q = q < -127.0 ? -127.0 : (q > 127.0 ? 127.0 : q);
                    const int qi = (int)q;
                    sum += qi;
                    const int co = o / 16, row = o % 16, c = i / 16, g = (i % 16) / 4, r = i % 4;
                    const int lane = 16 * g + row;
                    p8[(((l * 4 + co) * 64 + lane) * 4 + c) * 4 + r] = (int8_t)qi;
                }
                q8[64 * l + o] = (float)sw;
                q8[pip::kQ8Floats / 2 + 64 * l + o] = (float)sum;
            }
    }

    pip_pair_mlp *m = new pip_pair_mlp();
    m->f16ok = f16ok ? 1 : 0;
    m->w8 = nullptr;
    m->q8 = nullptr;
    m->w32 = nullptr;
    m->w16 = nullptr;
    m->wx2 = nullptr;
    m->wtx2 = nullptr;
    m->bias = nullptr;
    m->wplain = nullptr;
    hipError_t e = hipGetDevice(&m->device);
    if (e == hipSuccess) e = hipMalloc((void **)&m->w32, p32.size() * sizeof(float));
    if (e == hipSuccess) e = hipMalloc((void **)&m->w16, p16.size() * sizeof(uint16_t));
    if (e == hipSuccess) e = hipMalloc((void **)&m->wx2, px2.size() * sizeof(uint16_t));
    if (e == hipSuccess) e = hipMalloc((void **)&m->wtx2, ptx2.size() * sizeof(uint16_t));
    if (e == hipSuccess) e = hipMalloc((void **)&m->bias, b.size() * sizeof(float));
    if (e == hipSuccess) e = hipMalloc((void **)&m->wplain, w.size() * sizeof(float));
    if (e == hipSuccess) e = hipMalloc((void **)&m->w8, p8.size());
    if (e == hipSuccess) e = hipMalloc((void **)&m->q8, q8.size() * sizeof(float));
    if (e == hipSuccess) e = hipMemcpy(m->w8, p8.data(), p8.size(), hipMemcpyHostToDevice);
    if (e == hipSuccess)
        e = hipMemcpy(m->q8, q8.data(), q8.size() * sizeof(float), hipMemcpyHostToDevice);
    if (e == hipSuccess)
        e = hipMemcpy(m->wplain, w.data(), w.size() * sizeof(float), hipMemcpyHostToDevice);
    if (e == hipSuccess)
        e = hipMemcpy(m->w32, p32.data(), p32.size() * sizeof(float), hipMemcpyHostToDevice);
    if (e == hipSuccess)
        e = hipMemcpy(m->w16, p16.data(), p16.size() * sizeof(uint16_t), hipMemcpyHostToDevice);
    if (e == hipSuccess)
        e = hipMemcpy(m->wx2, px2.data(), px2.size() * sizeof(uint16_t), hipMemcpyHostToDevice);
    if (e == hipSuccess)
        e = hipMemcpy(m->wtx2, ptx2.data(), ptx2.size() * sizeof(uint16_t),
                      hipMemcpyHostToDevice);
    if (e == hipSuccess)
        e = hipMemcpy(m->bias, b.data(), b.size() * sizeof(float), hipMemcpyHostToDevice);
    if (e != hipSuccess) {
        pip_pair_mlp_destroy(m);
        return PIP_ERR_HIP;
    }
    *out = m;
    return PIP_OK;
}

pip_status pip_pair_mlp_destroy(pip_pair_mlp *m) {
    if (!m) return PIP_ERR_NULL;
    hipError_t e = hipSuccess, e2;
    if (m->w32 && (e2 = hipFree(m->w32)) != hipSuccess) e = e2;
    if (m->w16 && (e2 = hipFree(m->w16)) != hipSuccess) e = e2;
    if (m->wx2 && (e2 = hipFree(m->wx2)) != hipSuccess) e = e2;
    if (m->wtx2 && (e2 = hipFree(m->wtx2)) != hipSuccess) e = e2;
    if (m->bias && (e2 = hipFree(m->bias)) != hipSuccess) e = e2;
    if (m->wplain && (e2 = hipFree(m->wplain)) != hipSuccess) e = e2;
    if (m->w8 && (e2 = hipFree(m->w8)) != hipSuccess) e = e2;
    if (m->q8 && (e2 = hipFree(m->q8)) != hipSuccess) e = e2;
    delete m;
    return hip_status(e);
}

pip_status pip_pair_features(const float *p4, const uint8_t *mask, int64_t B, int64_t P,
                             float *F, void *stream) {
    pip_status st = check_pair_grid(B, P);
    if (st != PIP_OK || B == 0 || P == 0) return st;
    if (!p4 || !mask || !F) return PIP_ERR_NULL;
    if (!aligned16(p4) || !aligned16(F)) return PIP_ERR_ALIGN;
    return hip_status(pip::launch_pair_features(p4, mask, (int)B, (int)P, F, (hipStream_t)stream));
}

pip_status pip_pair_embed(const float *p4, const uint8_t *mask, int64_t B, int64_t P,
                          const pip_pair_mlp *mlp, void *U, int u_dtype, void *stream) {
    if (u_dtype != PIP_F32 && u_dtype != PIP_BF16) return PIP_ERR_DTYPE;
    pip_status st = check_pair_grid(B, P);
    if (st != PIP_OK || B == 0 || P == 0) return st;
    if (!p4 || !mask || !mlp || !U) return PIP_ERR_NULL;
    if (!aligned16(p4) || !aligned16(mask) || !aligned16(U)) return PIP_ERR_ALIGN;
    if ((st = check_device(mlp)) != PIP_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    if (u_dtype == PIP_F32)
        return hip_status(pip::launch_pair_embed_f32(p4, mask, (int)B, (int)P, mlp, (float *)U, s));
    return hip_status(pip::launch_pair_embed_bf16(p4, mask, (int)B, (int)P, mlp, (uint16_t *)U, s));
}

pip_status pip_pair_embed_int8(const float *p4, const uint8_t *mask, int64_t B, int64_t P,
                               const pip_pair_mlp *mlp, const float *act_scale,
                               const int32_t *act_zero, void *U, void *stream) {
    pip_status st = check_pair_grid(B, P);
    if (st != PIP_OK) return st;
    if (!act_scale || !act_zero) return PIP_ERR_NULL;
    for (int l = 0; l < 3; ++l) {
        if (!std::isfinite(act_scale[l]) || !(act_scale[l] > 0.0f) ||
            !std::isfinite(1.0f / act_scale[l]))
            return PIP_ERR_VALUE;
        if (act_zero[l] < -128 || act_zero[l] > 127) return PIP_ERR_VALUE;
    }
    if (B == 0 || P == 0) return PIP_OK;
    if (!p4 || !mask || !mlp || !U) return PIP_ERR_NULL;
    if (!aligned16(p4) || !aligned16(mask) || !aligned16(U)) return PIP_ERR_ALIGN;
    if ((st = check_device(mlp)) != PIP_OK) return st;
    return hip_status(pip::launch_pair_embed_int8(p4, mask, (int)B, (int)P, mlp, act_scale,
                                                  act_zero, (uint16_t *)U,
                                                  (hipStream_t)stream));
}

pip_status pip_pair_bias_attention(const void *Q, const void *K, const void *V, const void *U,
                                   const uint8_t *mask, int64_t B, int64_t H, int64_t P,
                                   int64_t D, float scale, void *O, int dtype, void *stream) {
    if (dtype != PIP_F32 && dtype != PIP_BF16) return PIP_ERR_DTYPE;
    if (H < 0 || D < 0) return PIP_ERR_SHAPE;
    pip_status st = check_pair_grid(B, P);
    if (st != PIP_OK) return st;
    if (!std::isfinite(scale)) return PIP_ERR_VALUE;
    if (B == 0 || P == 0 || H == 0) return PIP_OK;
    if (!Q || !K || !V || !U || !mask || !O) return PIP_ERR_NULL;
    if (D != PIP_HEAD_DIM) return PIP_ERR_UNSUPPORTED;
    if (pip::attention_jet_slots(B) * H * pip::attention_chunks((int)P) > ((int64_t)1 << 31) - 1)
        return PIP_ERR_UNSUPPORTED;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(U) || !aligned16(O))
        return PIP_ERR_ALIGN;
    hipStream_t s = (hipStream_t)stream;
    if (dtype == PIP_F32)
        return hip_status(pip::launch_attention_f32((const float *)Q, (const float *)K,
                                                    (const float *)V, (const float *)U, mask,
                                                    (int)B, (int)H, (int)P, scale, (float *)O,
                                                    s));
    return hip_status(pip::launch_attention_bf16((const uint16_t *)Q, (const uint16_t *)K,
                                                 (const uint16_t *)V, (const uint16_t *)U, mask,
                                                 (int)B, (int)H, (int)P, scale, (uint16_t *)O,
                                                 s));
}

pip_status pip_pair_embed_attention(const float *p4, const uint8_t *mask,
                                    const pip_pair_mlp *mlp, const void *Q, const void *K,
                                    const void *V, int64_t B, int64_t P, int64_t D, float scale,
                                    void *O, int dtype, void *stream) {
    if (dtype != PIP_F32 && dtype != PIP_BF16) return PIP_ERR_DTYPE;
    if (D < 0) return PIP_ERR_SHAPE;
    pip_status st = check_pair_grid(B, P);
    if (st != PIP_OK) return st;
    if (!std::isfinite(scale)) return PIP_ERR_VALUE;
    if (B == 0 || P == 0) return PIP_OK;
    if (!p4 || !mask || !mlp || !Q || !K || !V || !O) return PIP_ERR_NULL;
    if (D != PIP_HEAD_DIM) return PIP_ERR_UNSUPPORTED;
    if (!aligned16(p4) || !aligned16(mask) || !aligned16(Q) || !aligned16(K) ||
        !aligned16(V) || !aligned16(O))
        return PIP_ERR_ALIGN;
    if ((st = check_device(mlp)) != PIP_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    if (dtype == PIP_F32)
        return hip_status(pip::launch_embed_attention_f32(p4, mask, (int)B, (int)P, mlp,
                                                          (const float *)Q, (const float *)K,
                                                          (const float *)V, scale, (float *)O,
                                                          s));
    return hip_status(pip::launch_embed_attention_bf16(
        p4, mask, (int)B, (int)P, mlp, (const uint16_t *)Q, (const uint16_t *)K,
        (const uint16_t *)V, scale, (uint16_t *)O, s));
}

pip_status pip_packed_u_offsets(const int32_t *cu_seqlens, int64_t B, int64_t *u_offsets,
                                void *stream) {
    if (B < 0) return PIP_ERR_SHAPE;
    if (B > ((int64_t)1 << 24)) return PIP_ERR_UNSUPPORTED;
    if (!cu_seqlens || !u_offsets) return PIP_ERR_NULL;
    if (((uintptr_t)cu_seqlens & 3u) || ((uintptr_t)u_offsets & 7u)) return PIP_ERR_ALIGN;
    return hip_status(pip::launch_packed_offsets(cu_seqlens, (int)B, u_offsets,
                                                 (hipStream_t)stream));
}

// Sizes the packed kernels take: B jets, N particles, max_n <= 256.
static pip_status check_packed(int64_t B, int64_t N, int64_t max_n, int64_t u_elems) {
    if (B < 0 || N < 0 || max_n < 0 || u_elems < 0) return PIP_ERR_SHAPE;
    if (max_n > PIP_MAX_P || B > ((int64_t)1 << 24) || N > ((int64_t)1 << 30))
        return PIP_ERR_UNSUPPORTED;
    return PIP_OK;
}

pip_status pip_pair_embed_packed(const float *p4, const int32_t *cu_seqlens,
                                 const int64_t *u_offsets, int64_t B, int64_t N, int64_t max_n,
                                 const pip_pair_mlp *mlp, void *U, int64_t u_elems, int u_dtype,
                                 void *stream) {
    if (u_dtype != PIP_F32 && u_dtype != PIP_BF16) return PIP_ERR_DTYPE;
    pip_status st = check_packed(B, N, max_n, u_elems);
    if (st != PIP_OK) return st;
    if (B == 0 || max_n == 0) return PIP_OK;
    if (!p4 || !cu_seqlens || !u_offsets || !mlp || !U) return PIP_ERR_NULL;
    if (!aligned16(p4) || !aligned16(U) || ((uintptr_t)cu_seqlens & 3u) ||
        ((uintptr_t)u_offsets & 7u))
        return PIP_ERR_ALIGN;
    if ((st = check_device(mlp)) != PIP_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    if (u_dtype == PIP_F32)
        return hip_status(pip::launch_pair_embed_packed_f32(p4, cu_seqlens, u_offsets, (int)B,
                                                            (int)N, (int)max_n, mlp, (float *)U,
                                                            u_elems, s));
    return hip_status(pip::launch_pair_embed_packed_bf16(p4, cu_seqlens, u_offsets, (int)B,
                                                         (int)N, (int)max_n, mlp, (uint16_t *)U,
                                                         u_elems, s));
}

pip_status pip_pair_bias_attention_packed(const void *Q, const void *K, const void *V,
                                          const void *U, const int32_t *cu_seqlens,
                                          const int64_t *u_offsets, int64_t B, int64_t H,
                                          int64_t N, int64_t max_n, int64_t D, float scale,
                                          int64_t u_elems, void *O, int dtype, void *stream) {
    if (dtype != PIP_F32 && dtype != PIP_BF16) return PIP_ERR_DTYPE;
    if (H < 0 || D < 0) return PIP_ERR_SHAPE;
    pip_status st = check_packed(B, N, max_n, u_elems);
    if (st != PIP_OK) return st;
    if (!std::isfinite(scale)) return PIP_ERR_VALUE;
    if (B == 0 || H == 0 || max_n == 0) return PIP_OK;
    if (!Q || !K || !V || !U || !cu_seqlens || !u_offsets || !O) return PIP_ERR_NULL;
    if (D != PIP_HEAD_DIM) return PIP_ERR_UNSUPPORTED;
    if (pip::attention_jet_slots(B) * H * pip::attention_chunks((int)((max_n + 15) & ~15)) >
            ((int64_t)1 << 31) - 1 ||
        H * N > ((int64_t)1 << 31))
        return PIP_ERR_UNSUPPORTED;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(U) || !aligned16(O) ||
        ((uintptr_t)cu_seqlens & 3u) || ((uintptr_t)u_offsets & 7u))
        return PIP_ERR_ALIGN;
    hipStream_t s = (hipStream_t)stream;
    if (dtype == PIP_F32)
        return hip_status(pip::launch_attention_packed_f32(
            (const float *)Q, (const float *)K, (const float *)V, (const float *)U, cu_seqlens,
            u_offsets, (int)B, (int)H, (int)N, (int)max_n, u_elems, scale, (float *)O, s));
    return hip_status(pip::launch_attention_packed_bf16(
        (const uint16_t *)Q, (const uint16_t *)K, (const uint16_t *)V, (const uint16_t *)U,
        cu_seqlens, u_offsets, (int)B, (int)H, (int)N, (int)max_n, u_elems, scale,
        (uint16_t *)O, s));
}

pip_status pip_pair_bias_attention_backward(const void *Q, const void *K, const void *V,
                                            const void *U, const uint8_t *mask,
                                            const void *dO, int64_t B, int64_t H, int64_t P,
                                            int64_t D, float scale, void *dQ, void *dK,
                                            void *dV, void *dU, int dtype, void *stream) {
    if (dtype != PIP_F32 && dtype != PIP_BF16) return PIP_ERR_DTYPE;
    if (H < 0 || D < 0) return PIP_ERR_SHAPE;
    pip_status st = check_pair_grid(B, P);
    if (st != PIP_OK) return st;
    if (!std::isfinite(scale)) return PIP_ERR_VALUE;
    if (B == 0 || P == 0 || H == 0) return PIP_OK;
    if (!Q || !K || !V || !U || !mask || !dO || !dQ || !dK || !dV || !dU) return PIP_ERR_NULL;
    if (D != PIP_HEAD_DIM || dtype != PIP_F32) return PIP_ERR_UNSUPPORTED;
    if (pip::attention_jet_slots(B) * H > ((int64_t)1 << 31) - 1) return PIP_ERR_UNSUPPORTED;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(U) || !aligned16(dO) ||
        !aligned16(dQ) || !aligned16(dK) || !aligned16(dV) || !aligned16(dU))
        return PIP_ERR_ALIGN;
    return hip_status(pip::launch_attention_bwd_f32(
        (const float *)Q, (const float *)K, (const float *)V, (const float *)U, mask,
        (const float *)dO, (int)B, (int)H, (int)P, scale, (float *)dQ, (float *)dK,
        (float *)dV, (float *)dU, (hipStream_t)stream));
}

size_t pip_pair_mlp_backward_workspace_bytes(int64_t B, int64_t P) {
    if (B <= 0 || P <= 0 || check_pair_grid(B, P) != PIP_OK) return 0;
    return pip::mlp_bwd_workspace((int)B, (int)P);
}

pip_status pip_pair_mlp_backward(const float *p4, const uint8_t *mask, int64_t B, int64_t P,
                                 const pip_pair_mlp *mlp, const float *dU, float *grad,
                                 void *workspace, size_t workspace_bytes, void *stream) {
    pip_status st = check_pair_grid(B, P);
    if (st != PIP_OK) return st;
    if (!grad || !mlp) return PIP_ERR_NULL;
    if (((uintptr_t)grad & 3u)) return PIP_ERR_ALIGN;
    if ((st = check_device(mlp)) != PIP_OK) return st;
    if (B == 0 || P == 0)  // no pair: the gradient is 0 (a fill kernel, no memset node)
        return hip_status(pip::launch_mlp_bwd_f32(nullptr, nullptr, 0, 16, mlp, nullptr, grad,
                                                  nullptr, (hipStream_t)stream));
    if (!p4 || !mask || !dU || !workspace) return PIP_ERR_NULL;
    if (workspace_bytes < pip_pair_mlp_backward_workspace_bytes(B, P)) return PIP_ERR_SHAPE;
    if (!aligned16(p4) || !aligned16(dU) || !aligned16(workspace)) return PIP_ERR_ALIGN;
    return hip_status(pip::launch_mlp_bwd_f32(p4, mask, (int)B, (int)P, mlp, dU, grad,
                                              workspace, (hipStream_t)stream));
}

pip_status pip_pair_mlp_unfold_grads(const pip_pair_mlp_params *raw, const float *gf,
                                     float *gr) {
    if (!raw || !gf || !gr) return PIP_ERR_NULL;
    if (!raw->w1 || !raw->w2 || !raw->w3 || !raw->w4) return PIP_ERR_NULL;
    for (int k = 0; k < 3; ++k)
        if (!raw->bn_gamma[k] || !raw->bn_beta[k] || !raw->bn_mean[k] || !raw->bn_var[k])
            return PIP_ERR_NULL;
    const int nin = (raw->in_gamma != 0) + (raw->in_beta != 0) + (raw->in_mean != 0) +
                    (raw->in_var != 0);
    if (nin != 0 && nin != 4) return PIP_ERR_NULL;
    const double eps = raw->bn_eps;
    // input BatchNorm as x' = si x + ti (identity when absent)
    double si[4], ti[4], sdin[4];
    for (int i = 0; i < 4; ++i) {
        if (nin) {
            const double v = (double)raw->in_var[i] + eps;
            if (!(v > 0.0)) return PIP_ERR_SHAPE;
            sdin[i] = sqrt(v);
            si[i] = (double)raw->in_gamma[i] / sdin[i];
            ti[i] = (double)raw->in_beta[i] - si[i] * (double)raw->in_mean[i];
        } else {
            sdin[i] = si[i] = 1.0;
            ti[i] = 0.0;
        }
    }
    // folded (gf): W1' (64x4) W2' W3' (64x64) W4 (8x64) | b1' b2' b3' (64) b4 (8)
    // raw (gr): w1 b1 g1 be1 | w2 b2 g2 be2 | w3 b3 g3 be3 | w4 b4 | in_g in_be
    const int nins[3] = {4, 64, 64}, wof[3] = {0, 256, 4352}, bof[3] = {8960, 9024, 9088};
    const float *W[3] = {raw->w1, raw->w2, raw->w3};
    const float *bias[3] = {raw->b1, raw->b2, raw->b3};
    int ro = 0;
    double dsi[4] = {0, 0, 0, 0}, dti[4] = {0, 0, 0, 0};
    for (int l = 0; l < 3; ++l) {
        const int ni = nins[l];
        float *gw = gr + ro, *gb = gw + 64 * ni, *gg = gb + 64, *gbe = gg + 64;
        for (int o = 0; o < 64; ++o) {
            const double v = (double)raw->bn_var[l][o] + eps;
            if (!(v > 0.0)) return PIP_ERR_SHAPE;
            const double sd = sqrt(v), s = (double)raw->bn_gamma[l][o] / sd;
            const double db = gf[bof[l] + o];
            double z = bias[l] ? (double)bias[l][o] : 0.0, dg = 0.0;
            for (int i = 0; i < ni; ++i) {
                const double w = W[l][o * ni + i], dw = gf[wof[l] + o * ni + i];
                if (l == 0) {
                    gw[o * ni + i] = (float)(s * (dw * si[i] + db * ti[i]));
                    dg += dw * w * si[i];
                    z += w * ti[i];
                    dsi[i] += s * w * dw;
                    dti[i] += s * w * db;
                } else {
                    gw[o * ni + i] = (float)(s * dw);
                    dg += dw * w;
                }
            }
            gb[o] = (float)(s * db);
            gg[o] = (float)((dg + db * (z - (double)raw->bn_mean[l][o])) / sd);
            gbe[o] = (float)db;
        }
        ro += 64 * ni + 3 * 64;
    }
    for (int e = 0; e < 8 * 64 + 8; ++e) gr[ro + e] = gf[8448 + (e < 512 ? e : 704 + e - 512)];
    ro += 8 * 64 + 8;
    for (int i = 0; i < 4; ++i) {
        gr[ro + i] = nin ? (float)(dsi[i] / sdin[i] - dti[i] * (double)raw->in_mean[i] / sdin[i])
                         : 0.0f;
        gr[ro + 4 + i] = nin ? (float)dti[i] : 0.0f;
    }
    return PIP_OK;
}

size_t pip_block_stack_workspace_bytes(int64_t B, int64_t P, int64_t C, int64_t L) {
    if (B <= 0 || P <= 0 || C <= 0 || L <= 0) return 0;
    if (check_pair_grid(B, P) != PIP_OK || C % 16 != 0 || C > 16 * 16 || L > (1 << 20))
        return 0;
    return pip::block_stack_workspace((int)B, (int)P, (int)C, (int)L);
}

pip_status pip_block_stack(float *X, const float *Wq, const float *Wk, const float *Wv,
                           const float *Wo, const float *U, const uint8_t *mask, int64_t B,
                           int64_t P, int64_t C, int64_t H, int64_t L, void *workspace,
                           size_t workspace_bytes, void *stream) {
    if (C < 0 || H < 0 || L < 0) return PIP_ERR_SHAPE;
    pip_status st = check_pair_grid(B, P);
    if (st != PIP_OK) return st;
    if (B == 0 || P == 0 || L == 0) return PIP_OK;
    if (!X || !Wq || !Wk || !Wv || !Wo || !U || !mask) return PIP_ERR_NULL;
    if (H == 0 || C != (int64_t)PIP_HEAD_DIM * H) return PIP_ERR_SHAPE;
    if (H > 16) return PIP_ERR_UNSUPPORTED;
    if (!workspace) return PIP_ERR_NULL;
    if (L > (1 << 20)) return PIP_ERR_UNSUPPORTED;
    if (workspace_bytes < pip_block_stack_workspace_bytes(B, P, C, L)) return PIP_ERR_SHAPE;
    if (!aligned16(X) || !aligned16(Wq) || !aligned16(Wk) || !aligned16(Wv) ||
        !aligned16(Wo) || !aligned16(U) || !aligned16(workspace))
        return PIP_ERR_ALIGN;
    return hip_status(pip::launch_block_stack(X, Wq, Wk, Wv, Wo, U, mask, (int)B, (int)P,
                                              (int)C, (int)H, (int)L, workspace,
                                              (hipStream_t)stream));
}

}  // extern "C"

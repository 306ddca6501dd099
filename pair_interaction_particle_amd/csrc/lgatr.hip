// lgatr.hip -- the two L-GATr kernels: the geometric product of the spacetime
// algebra Cl(1,3) and the equivariant linear layer as one block-sparse MFMA
// contraction, with their extern "C" entry points.
//
// [R] README "How the Kernel Fusion Works", Fusion 1: the layer's weights
// span the 10 linear maps of a multivector that commute with Lorentz
// transformations; the fused form expands them once into one weight matrix
// W_eff over the concatenated [multivector components, scalars] and applies
// it as a single contraction.  "Results", table "L-GATr Kernels": the
// geometric product of two multivector tensors.
//
// Algebra: generators e0..e3 with e0^2 = +1, e1^2 = e2^2 = e3^2 = -1; a blade
// is a set of generators (a 4-bit mask), stored in grade order
//   1, e0, e1, e2, e3, e01, e02, e03, e12, e13, e23, e012, e013, e023, e123, e0123.
// The 10 equivariant maps are the 5 grade projections and e0123 times each.
//
// Structure exploited on gfx950: e0123 e_k = +-e_(15-k) in this order, so an
// output component k of the layer depends only on input components k and
// 15-k.  W_eff is therefore block diagonal over the 8 component pairs
// (k, 15-k): 7 dense blocks of (2 out_mv) x (2 in_mv) and one for the pair
// (1, e0123) that also carries the scalar channels.  Each block is a dense
// contraction over items, done with v_mfma_f32_16x16x4_f32 in float32: the
// weights are the A operand (packed per lane on the host), the items the
// columns, and every lane keeps its items' inputs and outputs in registers,
// so no LDS is used and nothing is read twice.
#include <string.h>

#include <type_traits>
#include <vector>

#include "pip_device.h"
#include "pip_internal.h"

namespace {

using pip::v4f;

// ---- blade algebra ---------------------------------------------------------
constexpr int kBladeMask[16] = {0, 1, 2, 4, 8, 3, 5, 9, 6, 10, 12, 7, 11, 13, 14, 15};

__host__ __device__ constexpr int blade_of_mask(int mask) {
    int k = 0;
    while (kBladeMask[k] != mask) ++k;
    return k;
}

__host__ __device__ constexpr int bit_count(int v) {
    int c = 0;
    for (; v; v &= v - 1) ++c;
    return c;
}

// e_A e_B = blade_sign(A, B) e_(A xor B), for blade indices a, b: the parity
// of the transpositions that sort the generators, times the square of every
// repeated spatial generator (-1 each).
__host__ __device__ constexpr int blade_sign(int a, int b) {
    const int A = kBladeMask[a], B = kBladeMask[b];
    int swaps = 0;
    for (int s = A >> 1; s; s >>= 1) swaps += bit_count(s & B);
    swaps += bit_count(A & B & 14);
    return (swaps & 1) ? -1 : 1;
}

__host__ __device__ constexpr int blade_prod(int a, int b) {
    return blade_of_mask(kBladeMask[a] ^ kBladeMask[b]);
}

// ---- geometric product -------------------------------------------------------
// One thread per multivector pair: 4 dwordx4 loads per operand, the 256 signed
// products of the Cayley table (indices and signs fold to constants), 4
// dwordx4 stores.
__global__ __launch_bounds__(256) void geometric_product_kernel(const float4 *__restrict__ x,
                                                                const float4 *__restrict__ y,
                                                                int64_t n,
                                                                float4 *__restrict__ z) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= n) return;
    float a[16], b[16], c[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float4 u = x[4 * t + q], v = y[4 * t + q];
        a[4 * q] = u.x, a[4 * q + 1] = u.y, a[4 * q + 2] = u.z, a[4 * q + 3] = u.w;
        b[4 * q] = v.x, b[4 * q + 1] = v.y, b[4 * q + 2] = v.z, b[4 * q + 3] = v.w;
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) c[k] = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int k = blade_prod(i, j);
            c[k] = __builtin_fmaf(blade_sign(i, j) > 0 ? a[i] : -a[i], b[j], c[k]);
        }
#pragma unroll
    for (int q = 0; q < 4; ++q)
        z[4 * t + q] = make_float4(c[4 * q], c[4 * q + 1], c[4 * q + 2], c[4 * q + 3]);
}

// ---- equivariant linear layer ------------------------------------------------
// Operand order (host packing and kernel agree).  Lane l, column m = l % 16,
// k-group kq = l / 16; a 16-item tile per workgroup.
//  * multivector features of pair block p (components c = p, d = 15 - p):
//    k-step s in [0, in_mv/2): h = s / (in_mv/4), g = s % (in_mv/4); lane
//    group kq supplies channel i = (in_mv/4) kq + g, component (h ? d : c).
//  * scalar features, chunk u of 16: step s' in [0, 4): lane group kq
//    supplies scalar 16u + 4kq + s'.
//  * multivector output rows of block p, row tile t: D row rho = 4kq + r is
//    channel o = 2(4t + kq) + (r & 1), component ((r >> 1) ? d : c).
//  * scalar output rows, tile t: D row rho is scalar 16t + rho.
// Packed float4 groups of 64 lanes (4 consecutive k-steps each):
//   section A  mv -> mv:      ((p * TI + t) * QI + q)             p < 8, t < TI, q < QI
//   section B  s -> mv (p=0): nA + t * US + u
//   section C  -> scalars:    nA + nB + t * (QI + US) + (q | QI + u)
// with TI = out_mv / 8, QI = in_mv / 8, US = in_s / 16.  Bias: TI float4
// per lane (rows of block 0), then out_s / 16 (scalar rows).
struct EquiShape {
    int im, om, is, os;
    int ti() const { return om / 8; }
    int qi() const { return im / 8; }
    int us() const { return is / 16; }
    int ts() const { return os / 16; }
    int nA() const { return 8 * ti() * qi(); }
    int nB() const { return ti() * us(); }
    int nC() const { return ts() * (qi() + us()); }
    int groups() const { return nA() + nB() + nC(); }
    int bias_groups() const { return ti() + ts(); }
};

// One workgroup of 4 waves per 16-item tile (the MFMA column count): the
// tile is read with coalesced 16-byte loads into LDS (rows padded by 4
// floats), the 8 pair blocks and the scalar rows are split over the 4 waves
// (about 12 MFMAs each at 8 -> 8 channels, so a wave's dependent chain is a
// quarter of the whole), the multivector outputs meet in a second LDS tile
// and leave with coalesced stores.
template <int IM, int OM>
__global__ __launch_bounds__(256) void equilinear_kernel(
    const float4 *__restrict__ xmv, const float4 *__restrict__ xs, int64_t n, int IS, int OS,
    const float4 *__restrict__ wpk, const float4 *__restrict__ bias, float4 *__restrict__ ymv,
    float4 *__restrict__ ys) {
    constexpr int CI = IM / 4, TI = OM / 8, QI = IM / 8;
    constexpr int XROW = IM * 16 + 4, YROW = OM * 16 + 4;
    __shared__ float4 xt4[16 * XROW / 4], yt4[16 * YROW / 4];
    float *xt = (float *)xt4, *yt = (float *)yt4;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, m = lane & 15, kq = lane >> 4;
    const int64_t item0 = (int64_t)blockIdx.x * 16, item = item0 + m;
    const bool live = item < n;
    const int US = IS >> 4, TS = OS >> 4;
    constexpr int nA = 8 * TI * QI;
    const int nB = TI * US;

#pragma unroll
    for (int j = 0; j < IM / 4; ++j) {
        const int e = threadIdx.x + 256 * j, it = e / (4 * IM), c4 = e % (4 * IM);
        const float4 v = item0 + it < n ? xmv[(item0 + it) * (4 * IM) + c4]
                                        : make_float4(0.f, 0.f, 0.f, 0.f);
        *(float4 *)(xt + it * XROW + 4 * c4) = v;
    }
    __syncthreads();

    auto xs_chunk = [&](int u) -> float4 {
        return live ? xs[(item * IS + 16 * u + 4 * kq) >> 2] : make_float4(0.f, 0.f, 0.f, 0.f);
    };
    auto step4 = [&](v4f acc, const float4 w, float b0, float b1, float b2, float b3) {
        acc = pip::mfma4(w.x, b0, acc);
        acc = pip::mfma4(w.y, b1, acc);
        acc = pip::mfma4(w.z, b2, acc);
        return pip::mfma4(w.w, b3, acc);
    };
    // this lane's inputs of pair block (c, d): channel CI kq + g, component c / d
    auto inputs = [&](float (&xb)[CI][2], int c, int d) {
#pragma unroll
        for (int g = 0; g < CI; ++g) {
            xb[g][0] = xt[m * XROW + (CI * kq + g) * 16 + c];
            xb[g][1] = xt[m * XROW + (CI * kq + g) * 16 + d];
        }
    };
    auto mv_steps = [&](v4f acc, const float4 w, int q, const float (&xb)[CI][2]) {
        float b[4];
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
            const int s = 4 * q + s4;
            b[s4] = xb[s % CI][s / CI];
        }
        return step4(acc, w, b[0], b[1], b[2], b[3]);
    };
    auto block = [&](auto P_) {
        constexpr int p = decltype(P_)::value, c = p, d = 15 - p;
        float xb[CI][2];
        inputs(xb, c, d);
#pragma unroll
        for (int t = 0; t < TI; ++t) {
            v4f acc = {0.f, 0.f, 0.f, 0.f};
            if (p == 0) {
                const float4 bv = bias[t * 64 + lane];
                acc = v4f{bv.x, bv.y, bv.z, bv.w};
            }
#pragma unroll
            for (int q = 0; q < QI; ++q)
                acc = mv_steps(acc, wpk[((p * TI + t) * QI + q) * 64 + lane], q, xb);
            if (p == 0)
                for (int u = 0; u < US; ++u) {
                    const float4 sv = xs_chunk(u);
                    acc = step4(acc, wpk[(nA + t * US + u) * 64 + lane], sv.x, sv.y, sv.z, sv.w);
                }
#pragma unroll
            for (int r = 0; r < 4; ++r)
                yt[m * YROW + (2 * (4 * t + kq) + (r & 1)) * 16 + ((r >> 1) ? d : c)] = acc[r];
        }
    };
    auto scalar_rows = [&]() {
        float xb[CI][2];
        inputs(xb, 0, 15);
        for (int t = 0; t < TS; ++t) {
            const float4 bv = bias[(TI + t) * 64 + lane];
            v4f acc = {bv.x, bv.y, bv.z, bv.w};
            const int g0 = nA + nB + t * (QI + US);
#pragma unroll
            for (int q = 0; q < QI; ++q) acc = mv_steps(acc, wpk[(g0 + q) * 64 + lane], q, xb);
            for (int u = 0; u < US; ++u) {
                const float4 sv = xs_chunk(u);
                acc = step4(acc, wpk[(g0 + QI + u) * 64 + lane], sv.x, sv.y, sv.z, sv.w);
            }
            if (live)
                ys[(item * OS + 16 * t + 4 * kq) >> 2] = make_float4(acc[0], acc[1], acc[2], acc[3]);
        }
    };
    using I = int;
    if (wv == 0) {
        block(std::integral_constant<I, 0>{});
        block(std::integral_constant<I, 4>{});
    } else if (wv == 1) {
        block(std::integral_constant<I, 1>{});
        block(std::integral_constant<I, 5>{});
        block(std::integral_constant<I, 7>{});
    } else if (wv == 2) {
        block(std::integral_constant<I, 2>{});
        block(std::integral_constant<I, 6>{});
    } else {
        block(std::integral_constant<I, 3>{});
        scalar_rows();
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < OM / 4; ++j) {
        const int e = threadIdx.x + 256 * j, it = e / (4 * OM), c4 = e % (4 * OM);
        if (item0 + it < n)
            ymv[(item0 + it) * (4 * OM) + c4] = *(const float4 *)(yt + it * YROW + 4 * c4);
    }
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// W_eff (rows out_mv*16 + out_s, columns in_mv*16 + in_s; row-major) from the
// basis weights: grade projection q puts w[o][i][q] on (o, k) <- (i, k) for
// every component k of grade q; e0123 times grade q puts sign * w[o][i][5+q]
// on (o, 15-k) <- (i, k), where e0123 e_k = sign e_(15-k).
void expand(const float *w, const float *s2mv, const float *mv2s, const float *ss, int im,
            int om, int is, int os, float *weff) {
    const int64_t cols = (int64_t)im * 16 + is, rows = (int64_t)om * 16 + os;
    for (int64_t e = 0; e < rows * cols; ++e) weff[e] = 0.0f;
    for (int o = 0; o < om; ++o)
        for (int i = 0; i < im; ++i)
            for (int k = 0; k < 16; ++k) {
                const float *wb = w + ((int64_t)o * im + i) * 10;
                const int grade = bit_count(kBladeMask[k]);
                const int dk = blade_prod(15, k);
                weff[((int64_t)o * 16 + k) * cols + i * 16 + k] = wb[grade];
                weff[((int64_t)o * 16 + dk) * cols + i * 16 + k] =
                    blade_sign(15, k) > 0 ? wb[5 + grade] : -wb[5 + grade];
            }
    for (int o = 0; o < om; ++o)
        for (int j = 0; j < is; ++j)
            weff[((int64_t)o * 16) * cols + im * 16 + j] = s2mv ? s2mv[(int64_t)o * is + j] : 0.f;
    for (int o = 0; o < os; ++o) {
        float *row = weff + ((int64_t)om * 16 + o) * cols;
        for (int i = 0; i < im; ++i) row[i * 16] = mv2s ? mv2s[(int64_t)o * im + i] : 0.f;
        for (int j = 0; j < is; ++j) row[im * 16 + j] = ss ? ss[(int64_t)o * is + j] : 0.f;
    }
}

pip_status check_equi_sizes(int im, int om, int is, int os, bool device) {
    if (im < 0 || om < 0 || is < 0 || os < 0) return PIP_ERR_SHAPE;
    if (!device) return PIP_OK;
    if ((im != 8 && im != 16) || (om != 8 && om != 16)) return PIP_ERR_UNSUPPORTED;
    if (is % 16 || os % 16 || is > PIP_LGATR_MAX_S || os > PIP_LGATR_MAX_S)
        return PIP_ERR_UNSUPPORTED;
    return PIP_OK;
}

}  // namespace

struct pip_equilinear {
    int device;
    EquiShape sh;
    float4 *wpk;   // packed operand groups
    float4 *bias;  // packed bias groups
};

extern "C" {

pip_status pip_lgatr_geometric_product(const float *x, const float *y, int64_t n, float *z,
                                       void *stream_) {
    hipStream_t stream = (hipStream_t)stream_;
    if (n < 0) return PIP_ERR_SHAPE;
    if (n == 0) return PIP_OK;
    if (!x || !y || !z) return PIP_ERR_NULL;
    if (!aligned16(x) || !aligned16(y) || !aligned16(z)) return PIP_ERR_ALIGN;
    if (n > ((int64_t)1 << 38)) return PIP_ERR_UNSUPPORTED;  // grid of n / 256 workgroups
    const int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(geometric_product_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const float4 *)x, (const float4 *)y, n, (float4 *)z);
    return hipGetLastError() == hipSuccess ? PIP_OK : PIP_ERR_HIP;
}

pip_status pip_lgatr_equilinear_expand(const float *w, const float *s2mv, const float *mv2s,
                                       const float *ss, int in_mv, int out_mv, int in_s,
                                       int out_s, float *w_eff) {
    const pip_status st = check_equi_sizes(in_mv, out_mv, in_s, out_s, false);
    if (st != PIP_OK) return st;
    if (!w_eff || (!w && in_mv > 0 && out_mv > 0)) return PIP_ERR_NULL;
    expand(w, s2mv, mv2s, ss, in_mv, out_mv, in_s, out_s, w_eff);
    return PIP_OK;
}

pip_status pip_lgatr_equilinear_create(const float *w, const float *s2mv, const float *mv2s,
                                       const float *ss, const float *b_mv, const float *b_s,
                                       int in_mv, int out_mv, int in_s, int out_s,
                                       pip_equilinear **out) {
    if (!out) return PIP_ERR_NULL;
    *out = nullptr;
    const pip_status st = check_equi_sizes(in_mv, out_mv, in_s, out_s, true);
    if (st != PIP_OK) return st;
    if (!w) return PIP_ERR_NULL;
    const EquiShape sh{in_mv, out_mv, in_s, out_s};
    const int cols = in_mv * 16 + in_s;
    std::vector<float> weff((size_t)(out_mv * 16 + out_s) * cols);
    expand(w, s2mv, mv2s, ss, in_mv, out_mv, in_s, out_s, weff.data());
    auto W = [&](int row, int col) { return weff[(size_t)row * cols + col]; };

    const int CI = in_mv / 4;
    // row rho of mv row tile t of block p -> (output row of W_eff)
    auto mv_row = [&](int p, int t, int rho) {
        const int o = 2 * (4 * t + rho / 4) + (rho & 1);
        return o * 16 + (((rho >> 1) & 1) ? 15 - p : p);
    };
    // k-step s of the mv features of block p, lane group kq -> column
    auto mv_col = [&](int p, int s, int kq) {
        const int h = s / CI, g = s % CI;
        return (CI * kq + g) * 16 + (h ? 15 - p : p);
    };
    std::vector<float> pk((size_t)sh.groups() * 256, 0.0f);
    auto put = [&](int grp, int lane, int s4, float v) { pk[((size_t)grp * 64 + lane) * 4 + s4] = v; };
    for (int lane = 0; lane < 64; ++lane) {
        const int rho = lane & 15, kq = lane >> 4;
        for (int s4 = 0; s4 < 4; ++s4) {
            for (int p = 0; p < 8; ++p)
                for (int t = 0; t < sh.ti(); ++t)
                    for (int q = 0; q < sh.qi(); ++q)
                        put((p * sh.ti() + t) * sh.qi() + q, lane, s4,
                            W(mv_row(p, t, rho), mv_col(p, 4 * q + s4, kq)));
            for (int t = 0; t < sh.ti(); ++t)
                for (int u = 0; u < sh.us(); ++u)
                    put(sh.nA() + t * sh.us() + u, lane, s4,
                        W(mv_row(0, t, rho), in_mv * 16 + 16 * u + 4 * kq + s4));
            for (int t = 0; t < sh.ts(); ++t) {
                const int row = out_mv * 16 + 16 * t + rho;
                const int g0 = sh.nA() + sh.nB() + t * (sh.qi() + sh.us());
                for (int q = 0; q < sh.qi(); ++q)
                    put(g0 + q, lane, s4, W(row, mv_col(0, 4 * q + s4, kq)));
                for (int u = 0; u < sh.us(); ++u)
                    put(g0 + sh.qi() + u, lane, s4, W(row, in_mv * 16 + 16 * u + 4 * kq + s4));
            }
        }
    }
    // bias: lane l, slot r carries D row 4(l/16) + r
    std::vector<float> bk((size_t)sh.bias_groups() * 256, 0.0f);
    for (int lane = 0; lane < 64; ++lane)
        for (int r = 0; r < 4; ++r) {
            const int rho = 4 * (lane >> 4) + r;
            for (int t = 0; t < sh.ti(); ++t) {
                const int row = mv_row(0, t, rho);
                bk[((size_t)t * 64 + lane) * 4 + r] = (row % 16 == 0 && b_mv) ? b_mv[row / 16] : 0.f;
            }
            for (int t = 0; t < sh.ts(); ++t)
                bk[((size_t)(sh.ti() + t) * 64 + lane) * 4 + r] = b_s ? b_s[16 * t + rho] : 0.f;
        }

    pip_equilinear *h = new pip_equilinear();
    h->sh = sh;
    h->wpk = nullptr;
    h->bias = nullptr;
    hipError_t e = hipGetDevice(&h->device);
    if (e == hipSuccess) e = hipMalloc(&h->wpk, pk.size() * sizeof(float));
    if (e == hipSuccess) e = hipMalloc(&h->bias, bk.size() * sizeof(float));
    if (e == hipSuccess)
        e = hipMemcpy(h->wpk, pk.data(), pk.size() * sizeof(float), hipMemcpyHostToDevice);
    if (e == hipSuccess)
        e = hipMemcpy(h->bias, bk.data(), bk.size() * sizeof(float), hipMemcpyHostToDevice);
    if (e != hipSuccess) {  // (the first error is the one reported)
        if (h->wpk) (void)hipFree(h->wpk);
        if (h->bias) (void)hipFree(h->bias);
        delete h;
        return PIP_ERR_HIP;
    }
    *out = h;
    return PIP_OK;
}

pip_status pip_lgatr_equilinear_destroy(pip_equilinear *h) {
    if (!h) return PIP_OK;
    const hipError_t a = hipFree(h->wpk), b = hipFree(h->bias);
    delete h;
    return a == hipSuccess && b == hipSuccess ? PIP_OK : PIP_ERR_HIP;
}

pip_status pip_lgatr_equilinear(const pip_equilinear *h, const float *x_mv, const float *x_s,
                                int64_t n, float *y_mv, float *y_s, void *stream_) {
    hipStream_t stream = (hipStream_t)stream_;
    if (!h) return PIP_ERR_NULL;
    if (n < 0) return PIP_ERR_SHAPE;
    if (n == 0) return PIP_OK;
    const EquiShape &sh = h->sh;
    if (!x_mv || !y_mv || (sh.is > 0 && !x_s) || (sh.os > 0 && !y_s)) return PIP_ERR_NULL;
    if (!aligned16(x_mv) || !aligned16(y_mv) || (sh.is > 0 && !aligned16(x_s)) ||
        (sh.os > 0 && !aligned16(y_s)))
        return PIP_ERR_ALIGN;
    if (n > ((int64_t)1 << 34)) return PIP_ERR_UNSUPPORTED;  // grid of n / 16 workgroups
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return PIP_ERR_HIP;
    if (dev != h->device) return PIP_ERR_UNSUPPORTED;
    const int64_t blocks = (n + 15) / 16;
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), 0, stream,
                           (const float4 *)x_mv, (const float4 *)x_s, n, sh.is, sh.os,
                           (const float4 *)h->wpk, (const float4 *)h->bias, (float4 *)y_mv,
                           (float4 *)y_s);
    };
    if (sh.im == 8 && sh.om == 8) go(equilinear_kernel<8, 8>);
    else if (sh.im == 8) go(equilinear_kernel<8, 16>);
    else if (sh.om == 8) go(equilinear_kernel<16, 8>);
    else go(equilinear_kernel<16, 16>);
    return hipGetLastError() == hipSuccess ? PIP_OK : PIP_ERR_HIP;
}

}  // extern "C"

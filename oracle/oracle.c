/*
 * oracle.c -- plain, slow, float64 CPU reference of the pair-interaction path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark load this library.  The product (the HIP
 * library) never calls it, and the two share no source, header, table or
 * constant.  Build: gcc -O2 -fopenmp -ffp-contract=off -fPIC -shared.
 * (-ffp-contract=off keeps every product and sum a separately rounded IEEE
 * operation, so the arithmetic below is exactly what is written.)
 *
 * What it computes, and where the pages say so:
 *
 *  [R] "Event Classification with Masked Transformer Autoencoders"
 *      (ml4sci_cms_e2e26 README), section "How the Kernel Fusion Works":
 *      - "Fusion 2": for every particle pair the four Lorentz-invariant
 *        features ln kT, ln z, ln dR, ln m2 go through a 4-layer pointwise
 *        (Conv1d, k=1) MLP 4 -> 64 -> 64 -> 64 -> 8 with BatchNorm + GELU;
 *        the result is the attention bias of shape (B, H, P, P).  The four
 *        features are those of the Particle Transformer paper listed in the
 *        README's References (Qu et al., ICML 2022).
 *      - "Fusion 3": attention is softmax(Q K^T / sqrt(d) + bias) V.
 *      - "Architecture Comparison": ParT uses 8 heads and PairEmbed
 *        4->64->64->64->8, i.e. one bias plane per head.
 *      - "Fusion 1" and "Results" table "L-GATr Kernels": the L-GATr
 *        equivariant linear layer on [multivectors, scalars] (its weights
 *        span the 10 Lorentz-equivariant maps of a 16-component multivector)
 *        and the geometric product of two multivector tensors.
 *  [S] gist.science summary of "Virtues and Vices of Equivariant
 *      Transformers", "Methodologie": ParT pair features are invariant under
 *      SO(2) x SO+(1,1) (azimuthal rotation x longitudinal boost).
 *  [L] lloca transformer_v2.Transformer.forward: 4-momenta energy-first.
 *
 * Readings taken where the pages are silent:
 *  - eps is a parameter (1e-8 in every workload); each feature is the log of
 *    its argument clamped below at eps.
 *  - y is the true rapidity 0.5 ln((E+pz)/(E-pz)), both arguments floored at
 *    1e-300 so that E <= |pz| stays finite.
 *  - dphi is wrapped into (-pi, pi].
 *  - the pair set is every ordered pair (a, b) of real particles, a == b
 *    included; pairs touching a padded slot give exactly 0.
 *  - BatchNorm (eval mode, running statistics) follows each hidden linear and
 *    precedes its GELU; an optional BatchNorm on the 4 input features; none
 *    after the last linear.  GELU is the exact erf form.
 *  - output channel h of the MLP is the bias of head h.
 *  - a padded query row gives O = 0; padded keys get weight exactly 0.
 *  - L-GATr: the spacetime algebra Cl(1,3), metric (+,-,-,-), blades of
 *    sorted generator indices in grade order; the 10 equivariant maps are the
 *    5 grade projections and the pseudoscalar (left) times each of them;
 *    scalar channels enter only the scalar component of the multivector
 *    outputs, and the scalar outputs read only the scalar component of the
 *    multivector inputs.
 *
 * Parity pins live in tests/test_oracle_*.py; parity is pinned for every
 * function here (closed forms, symmetries, brute force, library routines).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define HID 64   /* hidden width of the pair MLP ([R] Fusion 2) */
#define NIN 4    /* four pair features */
#define NOUT 8   /* one output channel per head */
#define RAP_FLOOR 1e-300

typedef struct {
    const double *w1, *b1, *w2, *b2, *w3, *b3, *w4, *b4; /* conv1d(k=1) (out,in) */
    const double *bn_gamma[3], *bn_beta[3], *bn_mean[3], *bn_var[3];
    const double *in_gamma, *in_beta, *in_mean, *in_var; /* all NULL: no input BN */
    double bn_eps;
} oracle_mlp;

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ------------------------------------------------------------ kinematics */
/* Transverse momentum, rapidity and azimuth of one energy-first 4-vector. */
void oracle_particle(const double *p, double *out3) {
    double E = p[0], px = p[1], py = p[2], pz = p[3];
    double num = E + pz, den = E - pz;
    if (!(num > RAP_FLOOR)) num = RAP_FLOOR;
    if (!(den > RAP_FLOOR)) den = RAP_FLOOR;
    out3[0] = hypot(px, py);
    out3[1] = 0.5 * log(num / den);
    out3[2] = atan2(py, px);
}

static double clamp_eps(double x, double eps) { return (x > eps) ? x : eps; }

/* The four pair features of particles a and b ([R] Fusion 2, ParT paper). */
void oracle_pair_feature(const double *pa, const double *pb, double eps, double *f4) {
    double ka[3], kb[3];
    oracle_particle(pa, ka);
    oracle_particle(pb, kb);
    double ptmin = (ka[0] < kb[0]) ? ka[0] : kb[0];
    double dy = ka[1] - kb[1];
    double dphi = ka[2] - kb[2];
    if (dphi > M_PI) dphi -= 2.0 * M_PI;
    else if (dphi <= -M_PI) dphi += 2.0 * M_PI;
    double dr = sqrt(dy * dy + dphi * dphi);
    /* invariant mass squared of the pair, (E_a+E_b)^2 - |p_a+p_b|^2 */
    double es = pa[0] + pb[0], xs = pa[1] + pb[1];
    double ys = pa[2] + pb[2], zs = pa[3] + pb[3];
    double m2 = es * es - xs * xs - ys * ys - zs * zs;
    double ptsum = ka[0] + kb[0];
    f4[0] = log(clamp_eps(ptmin * dr, eps));                   /* ln kT */
    f4[1] = log(clamp_eps(ptmin / clamp_eps(ptsum, eps), eps)); /* ln z  */
    f4[2] = log(clamp_eps(dr, eps));                           /* ln dR */
    f4[3] = log(clamp_eps(m2, eps));                           /* ln m2 */
}

/* F (B, 4, P, P): features of every ordered real pair, 0 where a or b is
 * padded.  p4 is (B, P, 4) energy-first, mask (B, P), nonzero = real. */
int oracle_pair_features(const double *p4, const uint8_t *mask, int64_t B, int64_t P,
                         double eps, double *F) {
    if (!p4 || !mask || !F || B < 0 || P < 0) return 1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t b = 0; b < B; ++b) {
        const double *pj = p4 + b * P * 4;
        const uint8_t *mj = mask + b * P;
        double *Fj = F + b * 4 * P * P;
        for (int64_t a = 0; a < P; ++a)
            for (int64_t c = 0; c < P; ++c) {
                double f[4] = {0.0, 0.0, 0.0, 0.0};
                if (mj[a] && mj[c]) oracle_pair_feature(pj + 4 * a, pj + 4 * c, eps, f);
                for (int k = 0; k < 4; ++k) Fj[(k * P + a) * P + c] = f[k];
            }
    }
    return 0;
}

/* ------------------------------------------------------------ pair MLP */
/* GELU(x) = x * Phi(x) with Phi the standard normal CDF, written through
 * erfc (Phi(x) = erfc(-x / sqrt 2) / 2) so the negative tail does not cancel. */
double oracle_gelu(double x) { return x * 0.5 * erfc(-x / sqrt(2.0)); }

/* eval-mode BatchNorm of one channel with running statistics */
static double batchnorm(double x, double gamma, double beta, double mean, double var,
                        double eps) {
    return gamma * (x - mean) / sqrt(var + eps) + beta;
}

/* y = W x + b for W (nout, nin) row-major */
static void linear(const double *W, const double *bias, const double *x, int nin, int nout,
                   double *y) {
    for (int o = 0; o < nout; ++o) {
        double s = bias ? bias[o] : 0.0;
        for (int i = 0; i < nin; ++i) s += W[o * nin + i] * x[i];
        y[o] = s;
    }
}

/* BN of layer l then GELU, channel by channel: h = GELU(BN_l(a)) */
static void bn_gelu(const oracle_mlp *m, int l, const double *a, double *h) {
    for (int o = 0; o < HID; ++o)
        h[o] = oracle_gelu(batchnorm(a[o], m->bn_gamma[l][o], m->bn_beta[l][o],
                                     m->bn_mean[l][o], m->bn_var[l][o], m->bn_eps));
}

/* The pointwise pair MLP on one feature vector ([R] Fusion 2): optional input
 * BN, then three (linear -> BN -> GELU) layers of width 64, then a linear to 8
 * head channels. */
void oracle_mlp_pair(const oracle_mlp *m, const double *f_in, double *u_out) {
    double x[NIN], a[HID], h[HID];
    for (int k = 0; k < NIN; ++k)
        x[k] = m->in_gamma ? batchnorm(f_in[k], m->in_gamma[k], m->in_beta[k],
                                       m->in_mean[k], m->in_var[k], m->bn_eps)
                           : f_in[k];
    linear(m->w1, m->b1, x, NIN, HID, a);
    bn_gelu(m, 0, a, h);
    linear(m->w2, m->b2, h, HID, HID, a);
    bn_gelu(m, 1, a, h);
    linear(m->w3, m->b3, h, HID, HID, a);
    bn_gelu(m, 2, a, h);
    linear(m->w4, m->b4, h, HID, NOUT, u_out);
}

/* U (B, 8, P, P) from features F (B, 4, P, P); 0 where a or b is padded. */
int oracle_pair_mlp(const double *F, const uint8_t *mask, int64_t B, int64_t P,
                    const oracle_mlp *m, double *U) {
    if (!F || !mask || !m || !U || B < 0 || P < 0) return 1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t b = 0; b < B; ++b) {
        const uint8_t *mj = mask + b * P;
        for (int64_t a = 0; a < P; ++a)
            for (int64_t c = 0; c < P; ++c) {
                double f[NIN], u[NOUT] = {0};
                if (mj[a] && mj[c]) {
                    for (int k = 0; k < NIN; ++k) f[k] = F[((b * NIN + k) * P + a) * P + c];
                    oracle_mlp_pair(m, f, u);
                }
                for (int h = 0; h < NOUT; ++h) U[((b * NOUT + h) * P + a) * P + c] = u[h];
            }
    }
    return 0;
}

/* Features then MLP, pair by pair: U (B, 8, P, P) from p4 (B, P, 4). */
int oracle_pair_embed(const double *p4, const uint8_t *mask, int64_t B, int64_t P, double eps,
                      const oracle_mlp *m, double *U) {
    if (!p4 || !mask || !m || !U || B < 0 || P < 0) return 1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t b = 0; b < B; ++b) {
        const double *pj = p4 + b * P * 4;
        const uint8_t *mj = mask + b * P;
        for (int64_t a = 0; a < P; ++a)
            for (int64_t c = 0; c < P; ++c) {
                double f[NIN], u[NOUT] = {0};
                if (mj[a] && mj[c]) {
                    oracle_pair_feature(pj + 4 * a, pj + 4 * c, eps, f);
                    oracle_mlp_pair(m, f, u);
                }
                for (int h = 0; h < NOUT; ++h) U[((b * NOUT + h) * P + a) * P + c] = u[h];
            }
    }
    return 0;
}

/* ------------------------------------------------------------ attention */
/* One head of masked biased attention for one jet ([R] Fusion 3):
 * for each real query a, s_c = scale (q_a . k_c) + Ub[a, c] over real keys c
 * (Fusion 3 writes the scale as 1/sqrt(d)), p = softmax(s) (two passes: max,
 * then exp and sum), O_a = sum_c p_c v_c.
 * q, k, v, o are (P, ld) with the head's D columns starting at column 0. */
static void attention_head(const double *q, const double *k, const double *v, int64_t ld,
                           const double *Ub, const uint8_t *mj, int64_t P, int64_t D,
                           double scale, double *o, double *s) {
    for (int64_t a = 0; a < P; ++a) {
        double *oa = o + a * ld;
        for (int64_t d = 0; d < D; ++d) oa[d] = 0.0;
        if (!mj[a]) continue;
        double mx = -INFINITY;
        int any = 0;
        for (int64_t c = 0; c < P; ++c) {
            if (!mj[c]) continue;
            double dot = 0.0;
            for (int64_t d = 0; d < D; ++d) dot += q[a * ld + d] * k[c * ld + d];
            s[c] = dot * scale + Ub[a * P + c];
            if (!any || s[c] > mx) mx = s[c];
            any = 1;
        }
        if (!any) continue;
        double Z = 0.0;
        for (int64_t c = 0; c < P; ++c) {
            if (!mj[c]) continue;
            s[c] = exp(s[c] - mx);
            Z += s[c];
        }
        for (int64_t c = 0; c < P; ++c) {
            if (!mj[c]) continue;
            double p = s[c] / Z;
            for (int64_t d = 0; d < D; ++d) oa[d] += p * v[c * ld + d];
        }
    }
}

/* O (B, H, P, D) = masked biased attention of Q, K, V (B, H, P, D) with bias
 * U (B, H, P, P) and score scale `scale` (1/sqrt(D) in the pages' formula). */
int oracle_attention(const double *Q, const double *K, const double *V, const double *U,
                     const uint8_t *mask, int64_t B, int64_t H, int64_t P, int64_t D,
                     double scale, double *O) {
    if (!Q || !K || !V || !U || !mask || !O || B < 0 || H < 1 || P < 0 || D < 1) return 1;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(P > 0 ? P : 1));
#pragma omp for schedule(dynamic, 1)
        for (int64_t bh = 0; bh < B * H; ++bh) {
            int64_t b = bh / H;
            size_t off = (size_t)bh * P * D;
            attention_head(Q + off, K + off, V + off, D, U + (size_t)bh * P * P, mask + b * P,
                           P, D, scale, O + off, s);
        }
        free(s);
    }
    return 0;
}

/* Features, MLP and attention in sequence (the result the fused entry must
 * reproduce): O (B, 8, P, D). */
int oracle_pair_embed_attention(const double *p4, const uint8_t *mask, int64_t B, int64_t P,
                                double eps, const oracle_mlp *m, const double *Q,
                                const double *K, const double *V, int64_t D, double scale,
                                double *O) {
    if (!p4 || !mask || !m || !Q || !K || !V || !O) return 1;
    double *U = (double *)malloc(sizeof(double) * (size_t)B * NOUT * P * P);
    if (!U) return 2;
    int rc = oracle_pair_embed(p4, mask, B, P, eps, m, U);
    if (!rc) rc = oracle_attention(Q, K, V, U, mask, B, NOUT, P, D, scale, O);
    free(U);
    return rc;
}

/* ------------------------------------------------------------ block stack */
/* Y (P, C) = X (P, C) @ W (C, C) */
static void matmul(const double *X, const double *W, int64_t P, int64_t C, double *Y) {
    for (int64_t r = 0; r < P; ++r)
        for (int64_t j = 0; j < C; ++j) {
            double s = 0.0;
            for (int64_t i = 0; i < C; ++i) s += X[r * C + i] * W[i * C + j];
            Y[r * C + j] = s;
        }
}

/* L attention layers reusing one bias U (B, H, P, P): per layer
 * Q = X Wq, K = X Wk, V = X Wv (head h owns columns h*D .. h*D+D-1, D = C/H),
 * O = masked biased attention per head, X <- X + O Wo.
 * X0 (B, P, C), W* (L, C, C) applied as X @ W; result Xout (B, P, C). */
int oracle_block_stack(const double *X0, const double *Wq, const double *Wk, const double *Wv,
                       const double *Wo, const double *U, const uint8_t *mask, int64_t B,
                       int64_t P, int64_t C, int64_t H, int64_t L, double *Xout) {
    if (!X0 || !Wq || !Wk || !Wv || !Wo || !U || !mask || !Xout) return 1;
    if (H < 1 || C % H != 0) return 1;
    int64_t D = C / H;
    int err = 0;
#pragma omp parallel
    {
        double *q = (double *)malloc(sizeof(double) * (size_t)P * C * 5 + sizeof(double) * P);
        if (!q) {
#pragma omp atomic write
            err = 2;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t b = 0; b < B; ++b) {
            if (!q) continue;
            double *k = q + P * C, *v = k + P * C, *o = v + P * C, *t = o + P * C,
                   *s = t + P * C;
            double *X = Xout + b * P * C;
            memcpy(X, X0 + b * P * C, sizeof(double) * (size_t)P * C);
            for (int64_t l = 0; l < L; ++l) {
                matmul(X, Wq + l * C * C, P, C, q);
                matmul(X, Wk + l * C * C, P, C, k);
                matmul(X, Wv + l * C * C, P, C, v);
                for (int64_t h = 0; h < H; ++h)
                    attention_head(q + h * D, k + h * D, v + h * D, C,
                                   U + ((size_t)b * H + h) * P * P, mask + b * P, P, D,
                                   1.0 / sqrt((double)D), o + h * D, s);
                matmul(o, Wo + l * C * C, P, C, t);
                for (int64_t i = 0; i < P * C; ++i) X[i] += t[i];
            }
        }
        free(q);
    }
    return err;
}

/* ------------------------------------------------------------ backward */
/* Gradients of the masked biased attention ([R] Fusion 3 names forward and
 * backward kernels) for a loss L with dL/dO = dO, by the chain rule through
 * s_c = scale (q_a . k_c) + U[a, c], p = softmax over real c, O_a = sum p_c v_c:
 *   dp_c = dO_a . v_c,   dS_c = p_c (dp_c - dO_a . O_a),   dU[a, c] = dS_c,
 *   dQ_a = scale sum_c dS_c k_c,  dK_c += scale dS_c q_a,  dV_c += p_c dO_a.
 * Everything that involves a padded slot is 0.  All arrays (B, H, P, D) or
 * (B, H, P, P) like the forward's. */
int oracle_attention_backward(const double *Q, const double *K, const double *V,
                              const double *U, const uint8_t *mask, int64_t B, int64_t H,
                              int64_t P, int64_t D, double scale, const double *dO, double *dQ,
                              double *dK, double *dV, double *dU) {
    if (!Q || !K || !V || !U || !mask || !dO || !dQ || !dK || !dV || !dU) return 1;
    if (B < 0 || H < 1 || P < 0 || D < 1) return 1;
#pragma omp parallel
    {
        double *p = (double *)malloc(sizeof(double) * (size_t)(P > 0 ? P : 1));
        double *o = (double *)malloc(sizeof(double) * (size_t)D);
#pragma omp for schedule(dynamic, 1)
        for (int64_t bh = 0; bh < B * H; ++bh) {
            const int64_t b = bh / H;
            const size_t off = (size_t)bh * P * D;
            const double *q = Q + off, *k = K + off, *v = V + off, *g = dO + off;
            const double *Ub = U + (size_t)bh * P * P;
            double *dq = dQ + off, *dk = dK + off, *dv = dV + off, *du = dU + (size_t)bh * P * P;
            const uint8_t *mj = mask + b * P;
            for (int64_t i = 0; i < P * D; ++i) dq[i] = dk[i] = dv[i] = 0.0;
            for (int64_t i = 0; i < P * P; ++i) du[i] = 0.0;
            for (int64_t a = 0; a < P; ++a) {
                if (!mj[a]) continue;
                /* forward of row a: two-pass softmax, then O_a */
                double mx = -INFINITY;
                int any = 0;
                for (int64_t c = 0; c < P; ++c) {
                    if (!mj[c]) continue;
                    double dot = 0.0;
                    for (int64_t d = 0; d < D; ++d) dot += q[a * D + d] * k[c * D + d];
                    p[c] = dot * scale + Ub[a * P + c];
                    if (!any || p[c] > mx) mx = p[c];
                    any = 1;
                }
                if (!any) continue;
                double Z = 0.0;
                for (int64_t c = 0; c < P; ++c)
                    if (mj[c]) {
                        p[c] = exp(p[c] - mx);
                        Z += p[c];
                    }
                for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
                for (int64_t c = 0; c < P; ++c)
                    if (mj[c]) {
                        p[c] /= Z;
                        for (int64_t d = 0; d < D; ++d) o[d] += p[c] * v[c * D + d];
                    }
                double Da = 0.0; /* dO_a . O_a */
                for (int64_t d = 0; d < D; ++d) Da += g[a * D + d] * o[d];
                for (int64_t c = 0; c < P; ++c) {
                    if (!mj[c]) continue;
                    double dp = 0.0;
                    for (int64_t d = 0; d < D; ++d) dp += g[a * D + d] * v[c * D + d];
                    const double ds = p[c] * (dp - Da);
                    du[a * P + c] = ds;
                    for (int64_t d = 0; d < D; ++d) {
                        dq[a * D + d] += scale * ds * k[c * D + d];
                        dk[c * D + d] += scale * ds * q[a * D + d];
                        dv[c * D + d] += p[c] * g[a * D + d];
                    }
                }
            }
        }
        free(p);
        free(o);
    }
    return 0;
}

/* d GELU(x) / dx = Phi(x) + x phi(x) (exact erf form) */
static double gelu_grad(double x) {
    return 0.5 * erfc(-x / sqrt(2.0)) + x * exp(-0.5 * x * x) / sqrt(2.0 * M_PI);
}

/* Layout of the raw-parameter gradient array of the pair MLP (the
 * parameters of pip_pair_mlp_params that a training step updates; BatchNorm
 * running statistics are not trained):
 *   w1 (64*4) b1 (64) g1 (64) be1 (64) | w2 (64*64) b2 g2 be2 | w3 (64*64) b3 g3 be3 |
 *   w4 (8*64) b4 (8) | in_g (4) in_be (4)      (input BN entries 0 when absent) */
#define GR_W1 0
#define GR_L1 (GR_W1 + HID * NIN)
#define GR_W2 (GR_L1 + 3 * HID)
#define GR_L2 (GR_W2 + HID * HID)
#define GR_W3 (GR_L2 + 3 * HID)
#define GR_L3 (GR_W3 + HID * HID)
#define GR_W4 (GR_L3 + 3 * HID)
#define GR_B4 (GR_W4 + NOUT * HID)
#define GR_IN (GR_B4 + NOUT)
#define GR_TOTAL (GR_IN + 2 * NIN)

int oracle_pair_mlp_grad_count(void) { return GR_TOTAL; }

/* Adds to grad (GR_TOTAL) the gradient of u . gu for one feature vector f,
 * where u = MLP(f) as in oracle_mlp_pair: forward keeping every
 * intermediate, then the chain rule layer by layer. */
static void mlp_pair_backward(const oracle_mlp *m, const double *f_in, const double *gu,
                              double *grad) {
    double x[NIN], xh[NIN]; /* BN'd input, normalised input (input BN) */
    double z[3][HID], y[3][HID], h[3][HID], zn[3][HID];
    for (int k = 0; k < NIN; ++k) {
        if (m->in_gamma) {
            xh[k] = (f_in[k] - m->in_mean[k]) / sqrt(m->in_var[k] + m->bn_eps);
            x[k] = m->in_gamma[k] * xh[k] + m->in_beta[k];
        } else {
            xh[k] = 0.0;
            x[k] = f_in[k];
        }
    }
    const double *W[3] = {m->w1, m->w2, m->w3}, *bb[3] = {m->b1, m->b2, m->b3};
    for (int l = 0; l < 3; ++l) {
        const double *in = l == 0 ? x : h[l - 1];
        linear(W[l], bb[l], in, l == 0 ? NIN : HID, HID, z[l]);
        for (int o = 0; o < HID; ++o) {
            zn[l][o] = (z[l][o] - m->bn_mean[l][o]) / sqrt(m->bn_var[l][o] + m->bn_eps);
            y[l][o] = m->bn_gamma[l][o] * zn[l][o] + m->bn_beta[l][o];
            h[l][o] = oracle_gelu(y[l][o]);
        }
    }
    /* output layer */
    double dh[HID], dz[HID];
    for (int o = 0; o < NOUT; ++o) {
        grad[GR_B4 + o] += gu[o];
        for (int i = 0; i < HID; ++i) grad[GR_W4 + o * HID + i] += gu[o] * h[2][i];
    }
    for (int i = 0; i < HID; ++i) {
        double s = 0.0;
        for (int o = 0; o < NOUT; ++o) s += m->w4[o * HID + i] * gu[o];
        dh[i] = s;
    }
    const int wbase[3] = {GR_W1, GR_W2, GR_W3}, lbase[3] = {GR_L1, GR_L2, GR_L3};
    for (int l = 2; l >= 0; --l) {
        const int nin = l == 0 ? NIN : HID;
        const double *in = l == 0 ? x : h[l - 1];
        for (int o = 0; o < HID; ++o) {
            const double dy = dh[o] * gelu_grad(y[l][o]);
            grad[lbase[l] + 2 * HID + o] += dy;               /* beta */
            grad[lbase[l] + HID + o] += dy * zn[l][o];        /* gamma */
            dz[o] = dy * m->bn_gamma[l][o] / sqrt(m->bn_var[l][o] + m->bn_eps);
            grad[lbase[l] + o] += dz[o];                      /* conv bias */
            for (int i = 0; i < nin; ++i) grad[wbase[l] + o * nin + i] += dz[o] * in[i];
        }
        if (l > 0) {
            for (int i = 0; i < HID; ++i) {
                double s = 0.0;
                for (int o = 0; o < HID; ++o) s += W[l][o * HID + i] * dz[o];
                dh[i] = s;
            }
        } else if (m->in_gamma) {
            for (int i = 0; i < NIN; ++i) {
                double dx = 0.0;
                for (int o = 0; o < HID; ++o) dx += m->w1[o * NIN + i] * dz[o];
                grad[GR_IN + i] += dx * xh[i];       /* input BN gamma */
                grad[GR_IN + NIN + i] += dx;         /* input BN beta */
            }
        }
    }
}

/* Gradient of L = sum_{b,h,a,c} U[b,h,a,c] dU[b,h,a,c] with respect to the
 * raw MLP parameters, U = oracle_pair_mlp(F, mask): every ordered real pair
 * contributes the backward of its own MLP evaluation.  grad: GR_TOTAL. */
int oracle_pair_mlp_backward(const double *F, const uint8_t *mask, int64_t B, int64_t P,
                             const oracle_mlp *m, const double *dU, double *grad) {
    if (!F || !mask || !m || !dU || !grad || B < 0 || P < 0) return 1;
    for (int i = 0; i < GR_TOTAL; ++i) grad[i] = 0.0;
#pragma omp parallel
    {
        double *gl = (double *)calloc(GR_TOTAL, sizeof(double));
#pragma omp for schedule(dynamic, 1)
        for (int64_t b = 0; b < B; ++b) {
            const uint8_t *mj = mask + b * P;
            for (int64_t a = 0; a < P; ++a)
                for (int64_t c = 0; c < P; ++c) {
                    if (!(mj[a] && mj[c])) continue;
                    double f[NIN], gu[NOUT];
                    for (int k = 0; k < NIN; ++k) f[k] = F[((b * NIN + k) * P + a) * P + c];
                    for (int h = 0; h < NOUT; ++h) gu[h] = dU[((b * NOUT + h) * P + a) * P + c];
                    mlp_pair_backward(m, f, gu, gl);
                }
        }
#pragma omp critical
        for (int i = 0; i < GR_TOTAL; ++i) grad[i] += gl[i];
        free(gl);
    }
    return 0;
}

/* ------------------------------------------------------------ int8 variant */
/* The pair MLP with int8 inputs to its hidden linears, after the "Economical
 * Jet Taggers" summary (gist.science, Technische Samenvatting, Methodologie,
 * "Datatype Kwantisering": inputs of linear layers quantised to int8 with a
 * zero point).  Readings: BatchNorm is folded first (the deployed linear is
 * W' = diag(s) W, b' = s (b - mean) + beta, input BatchNorm folded into layer
 * 1); layer 1 and every GELU stay in high precision; the inputs h of layers
 * 2, 3, 4 are quantised per tensor with a given scale S and zero point Z,
 *     q = clamp(rint(h / S) + Z, -128, 127),   h^ = S (q - Z);
 * the weights of layers 2, 3, 4 per output channel o, symmetrically,
 *     sw_o = max_i |W'[o][i]| / 127,  Wq = clamp(rint(W' / sw_o), -127, 127),
 * and the layer output is sum_i sw_o Wq[o][i] h^_i + b'_o.  rint rounds half
 * to even.  Everything here is float64.
 * tie (B, P, P) flags the pairs where some h / S + Z lies within tie_delta of
 * a rounding boundary (a half-integer): there a float32 implementation may
 * legitimately take the other code. */
static void fold_layers(const oracle_mlp *m, double *W1, double *b1, double *W2, double *b2,
                        double *W3, double *b3) {
    double si[NIN], ti[NIN];
    for (int k = 0; k < NIN; ++k) {
        if (m->in_gamma) {
            si[k] = m->in_gamma[k] / sqrt(m->in_var[k] + m->bn_eps);
            ti[k] = m->in_beta[k] - si[k] * m->in_mean[k];
        } else {
            si[k] = 1.0;
            ti[k] = 0.0;
        }
    }
    const double *W[3] = {m->w1, m->w2, m->w3}, *bb[3] = {m->b1, m->b2, m->b3};
    double *Wo[3] = {W1, W2, W3}, *bo[3] = {b1, b2, b3};
    for (int l = 0; l < 3; ++l) {
        const int nin = l == 0 ? NIN : HID;
        for (int o = 0; o < HID; ++o) {
            const double s = m->bn_gamma[l][o] / sqrt(m->bn_var[l][o] + m->bn_eps);
            double z = bb[l] ? bb[l][o] : 0.0;
            for (int i = 0; i < nin; ++i) {
                const double w = W[l][o * nin + i];
                if (l == 0) {
                    Wo[l][o * nin + i] = s * w * si[i];
                    z += w * ti[i];
                } else {
                    Wo[l][o * nin + i] = s * w;
                }
            }
            bo[l][o] = s * (z - m->bn_mean[l][o]) + m->bn_beta[l][o];
        }
    }
}

/* per-channel symmetric int8 weights: Wq (as doubles) and sw */
static void quant_weights(const double *W, int nout, int nin, double *Wq, double *sw) {
    for (int o = 0; o < nout; ++o) {
        double mx = 0.0;
        for (int i = 0; i < nin; ++i) mx = fmax(mx, fabs(W[o * nin + i]));
        sw[o] = mx > 0.0 ? mx / 127.0 : 1.0;
        for (int i = 0; i < nin; ++i) {
            double q = rint(W[o * nin + i] / sw[o]);
            Wq[o * nin + i] = q < -127.0 ? -127.0 : (q > 127.0 ? 127.0 : q);
        }
    }
}

/* fake-quantise h (n values) with scale S and zero point Z; returns whether
 * some value was within delta of a rounding boundary */
static int quant_act(double *h, int n, double S, double Z, double delta) {
    int tie = 0;
    for (int i = 0; i < n; ++i) {
        const double d = h[i] / S + Z;
        if (fabs(d - floor(d) - 0.5) < delta) tie = 1;
        double q = rint(h[i] / S) + Z;
        q = q < -128.0 ? -128.0 : (q > 127.0 ? 127.0 : q);
        h[i] = S * (q - Z);
    }
    return tie;
}

int oracle_pair_embed_int8(const double *p4, const uint8_t *mask, int64_t B, int64_t P,
                           double eps, const oracle_mlp *m, const double *act_scale,
                           const double *act_zero, double tie_delta, double *U, uint8_t *tie) {
    if (!p4 || !mask || !m || !act_scale || !act_zero || !U || !tie || B < 0 || P < 0) return 1;
    static const int kW = HID * NIN + 2 * HID * HID;
    double *W = (double *)malloc(sizeof(double) * (kW + 3 * HID + 2 * HID * HID + NOUT * HID +
                                                   2 * HID + NOUT));
    if (!W) return 2;
    double *W1 = W, *W2 = W1 + HID * NIN, *W3 = W2 + HID * HID;
    double *b1 = W3 + HID * HID, *b2 = b1 + HID, *b3 = b2 + HID;
    double *Q2 = b3 + HID, *Q3 = Q2 + HID * HID, *Q4 = Q3 + HID * HID;
    double *s2 = Q4 + NOUT * HID, *s3 = s2 + HID, *s4 = s3 + HID;
    fold_layers(m, W1, b1, W2, b2, W3, b3);
    quant_weights(W2, HID, HID, Q2, s2);
    quant_weights(W3, HID, HID, Q3, s3);
    quant_weights(m->w4, NOUT, HID, Q4, s4);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t b = 0; b < B; ++b) {
        const double *pj = p4 + b * P * 4;
        const uint8_t *mj = mask + b * P;
        for (int64_t a = 0; a < P; ++a)
            for (int64_t c = 0; c < P; ++c) {
                double f[NIN], h[HID], y[HID], u[NOUT] = {0};
                int t = 0;
                if (mj[a] && mj[c]) {
                    oracle_pair_feature(pj + 4 * a, pj + 4 * c, eps, f);
                    linear(W1, b1, f, NIN, HID, y);
                    for (int o = 0; o < HID; ++o) h[o] = oracle_gelu(y[o]);
                    const double *Qs[2] = {Q2, Q3}, *ss[2] = {s2, s3}, *bs[2] = {b2, b3};
                    for (int l = 0; l < 2; ++l) {
                        t |= quant_act(h, HID, act_scale[l], act_zero[l], tie_delta);
                        for (int o = 0; o < HID; ++o) {
                            double acc = 0.0;
                            for (int i = 0; i < HID; ++i) acc += Qs[l][o * HID + i] * h[i];
                            y[o] = ss[l][o] * acc + bs[l][o];
                        }
                        for (int o = 0; o < HID; ++o) h[o] = oracle_gelu(y[o]);
                    }
                    t |= quant_act(h, HID, act_scale[2], act_zero[2], tie_delta);
                    for (int o = 0; o < NOUT; ++o) {
                        double acc = 0.0;
                        for (int i = 0; i < HID; ++i) acc += Q4[o * HID + i] * h[i];
                        u[o] = s4[o] * acc + (m->b4 ? m->b4[o] : 0.0);
                    }
                }
                for (int hh = 0; hh < NOUT; ++hh) U[((b * NOUT + hh) * P + a) * P + c] = u[hh];
                tie[(b * P + a) * P + c] = (uint8_t)t;
            }
    }
    free(W);
    return 0;
}

/* Smallest and largest input of each hidden linear (h1, h2, h3) of the
 * float pair MLP over the real pairs: a calibration of the int8 variant's
 * activation ranges.  out6 = {min1, max1, min2, max2, min3, max3}. */
int oracle_pair_mlp_ranges(const double *p4, const uint8_t *mask, int64_t B, int64_t P,
                           double eps, const oracle_mlp *m, double *out6) {
    if (!p4 || !mask || !m || !out6) return 1;
    double W1[HID * NIN], W2[HID * HID], W3[HID * HID], b1[HID], b2[HID], b3[HID];
    fold_layers(m, W1, b1, W2, b2, W3, b3);
    for (int l = 0; l < 3; ++l) {
        out6[2 * l] = INFINITY;
        out6[2 * l + 1] = -INFINITY;
    }
    for (int64_t b = 0; b < B; ++b)
        for (int64_t a = 0; a < P; ++a)
            for (int64_t c = 0; c <= a; ++c) {
                if (!(mask[b * P + a] && mask[b * P + c])) continue;
                double f[NIN], y[HID], h[HID];
                oracle_pair_feature(p4 + (b * P + a) * 4, p4 + (b * P + c) * 4, eps, f);
                const double *Ws[3] = {W1, W2, W3}, *bs[3] = {b1, b2, b3};
                const double *in = f;
                for (int l = 0; l < 3; ++l) {
                    linear(Ws[l], bs[l], in, l == 0 ? NIN : HID, HID, y);
                    for (int o = 0; o < HID; ++o) {
                        h[o] = oracle_gelu(y[o]);
                        out6[2 * l] = fmin(out6[2 * l], h[o]);
                        out6[2 * l + 1] = fmax(out6[2 * l + 1], h[o]);
                    }
                    in = h;
                }
            }
    return 0;
}

/* ------------------------------------------------------------ L-GATr */
/* The spacetime algebra Cl(1,3) of L-GATr ([R] "How the Kernel Fusion Works",
 * Fusion 1; "Results", table "L-GATr Kernels"): metric diag(+1, -1, -1, -1)
 * on e0..e3, 16 basis blades in grade order
 *   1, e0, e1, e2, e3, e01, e02, e03, e12, e13, e23, e012, e013, e023, e123, e0123.
 * A blade is a set of generators (bit g = e_g); the product of two blades is
 * the symmetric difference, with sign (-1)^(number of generator pairs that
 * must be swapped to sort) times the metric of every repeated generator. */
static const int BLADE_BITS[16] = {0, 1, 2, 4, 8, 3, 5, 9, 6, 10, 12, 7, 11, 13, 14, 15};

static int blade_index(int bits) {
    for (int i = 0; i < 16; ++i)
        if (BLADE_BITS[i] == bits) return i;
    return -1;
}

static int popcount4(int x) { return (x & 1) + ((x >> 1) & 1) + ((x >> 2) & 1) + ((x >> 3) & 1); }

/* e_A e_B = sign * e_{A xor B} for blade index a, b */
static int blade_product(int a, int b, int *sign) {
    const int A = BLADE_BITS[a], B = BLADE_BITS[b];
    int swaps = 0;
    for (int i = 0; i < 4; ++i)        /* generator i of A ... */
        if (A >> i & 1)
            for (int j = 0; j < i; ++j) /* ... passes every smaller generator j of B */
                if (B >> j & 1) ++swaps;
    int s = (swaps & 1) ? -1 : 1;
    const int common = A & B;
    for (int g = 1; g < 4; ++g)
        if (common >> g & 1) s = -s; /* e1^2 = e2^2 = e3^2 = -1; e0^2 = +1 */
    *sign = s;
    return blade_index(A ^ B);
}

int oracle_blade_grade(int i) { return popcount4(BLADE_BITS[i]); }

/* z = x y for n multivectors (n, 16) */
void oracle_geometric_product(const double *x, const double *y, int64_t n, double *z) {
    for (int64_t m = 0; m < n; ++m) {
        const double *a = x + 16 * m, *b = y + 16 * m;
        double *c = z + 16 * m;
        for (int k = 0; k < 16; ++k) c[k] = 0.0;
        for (int i = 0; i < 16; ++i)
            for (int j = 0; j < 16; ++j) {
                int s;
                const int k = blade_product(i, j, &s);
                c[k] += s * a[i] * b[j];
            }
    }
}

/* The Lorentz-equivariant linear maps of one multivector, basis map q:
 * q = 0..4: the grade-q part of x; q = 5..9: e0123 times the grade-(q-5)
 * part (left multiplication by the pseudoscalar, which every proper
 * orthochronous Lorentz transformation leaves invariant). */
static void equi_basis(const double *x, int q, double *y) {
    double part[16];
    const int grade = q < 5 ? q : q - 5;
    for (int i = 0; i < 16; ++i) part[i] = popcount4(BLADE_BITS[i]) == grade ? x[i] : 0.0;
    if (q < 5) {
        for (int i = 0; i < 16; ++i) y[i] = part[i];
        return;
    }
    double ps[16] = {0};
    ps[15] = 1.0;
    oracle_geometric_product(ps, part, 1, y);
}

/* EquiLinear on n items (the structure of L-GATr's equivariant linear layer):
 *   y_mv[o] = sum_i sum_q w[o][i][q] basis_q(x_mv[i])
 *             + (sum_j s2mv[o][j] x_s[j] + b_mv[o]) e_scalar
 *   y_s[o]  = sum_j ss[o][j] x_s[j] + sum_i mv2s[o][i] x_mv[i][scalar] + b_s[o]
 * x_mv (n, in_mv, 16), x_s (n, in_s), w (out_mv, in_mv, 10), s2mv (out_mv,
 * in_s), mv2s (out_s, in_mv), ss (out_s, in_s); NULL matrices and biases are
 * zero.  y_mv (n, out_mv, 16), y_s (n, out_s). */
int oracle_equilinear(const double *x_mv, const double *x_s, int64_t n, int64_t in_mv,
                      int64_t in_s, int64_t out_mv, int64_t out_s, const double *w,
                      const double *s2mv, const double *mv2s, const double *ss,
                      const double *b_mv, const double *b_s, double *y_mv, double *y_s) {
    if (!x_mv || !w || !y_mv || n < 0 || in_mv < 0 || out_mv < 0 || in_s < 0 || out_s < 0)
        return 1;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < n; ++m) {
        double t[16];
        for (int64_t o = 0; o < out_mv; ++o) {
            double *y = y_mv + (m * out_mv + o) * 16;
            for (int k = 0; k < 16; ++k) y[k] = 0.0;
            for (int64_t i = 0; i < in_mv; ++i)
                for (int q = 0; q < 10; ++q) {
                    const double wq = w[(o * in_mv + i) * 10 + q];
                    equi_basis(x_mv + (m * in_mv + i) * 16, q, t);
                    for (int k = 0; k < 16; ++k) y[k] += wq * t[k];
                }
            double sc = b_mv ? b_mv[o] : 0.0;
            if (s2mv)
                for (int64_t j = 0; j < in_s; ++j) sc += s2mv[o * in_s + j] * x_s[m * in_s + j];
            y[0] += sc;
        }
        for (int64_t o = 0; o < out_s; ++o) {
            double v = b_s ? b_s[o] : 0.0;
            if (ss)
                for (int64_t j = 0; j < in_s; ++j) v += ss[o * in_s + j] * x_s[m * in_s + j];
            if (mv2s)
                for (int64_t i = 0; i < in_mv; ++i)
                    v += mv2s[o * in_mv + i] * x_mv[(m * in_mv + i) * 16];
            y_s[m * out_s + o] = v;
        }
    }
    return 0;
}

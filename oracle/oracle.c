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
 *  [S] gist.science summary of "Virtues and Vices of Equivariant
 *      Transformers", "Methodologie": ParT pair features are invariant under
 *      SO(2) x SO+(1,1) (azimuthal rotation x longitudinal boost).
 *  [L] lloca transformer_v2.Transformer.forward: 4-momenta energy-first.
 *
 * Readings taken where the pages are silent (each also listed in the design doc):
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

"""Fit the polynomial of the device GELU and print it as C++ constants.

GELU(x) = x Phi(x) = max(x, 0) - |x| Phi(-|x|), and for a >= 0
Phi(-a) = 2^(-Q(a)) with Q(a) = -log2 Phi(-a), a smooth function that grows
like a^2 / (2 ln 2).  Q is fitted on [0, A] by a polynomial of degree n with
iteratively reweighted least squares towards the minimax of the GELU error
|x| ln2 Phi(-a) |dQ| (Chebyshev nodes).  For odd n the fitted polynomial has
a positive leading coefficient and keeps growing beyond A, so 2^-Q underflows
to 0 for large |x| and no clamp is needed (checked below on [-40, 40]).  The
device then needs n FMAs, one v_exp_f32, one integer max (for max(x, 0), on
the bit pattern) and one FMA per element, with no branch.

The backward of the MLP also needs Phi itself (GELU'(x) = Phi(x) + x phi(x)),
so a third table fits Phi(-a) = 2^(-R(a)) towards the minimax of the absolute
error of Phi (degree 8, the lowest degree whose fit keeps growing beyond A
with an error below 1e-7).

Run:  python gen_gelu_coeffs.py   (prints the tables pasted into pip_mlp.h
                                    and mlp_bwd.hip)
"""
import numpy as np
from scipy.special import log_ndtr, ndtr

A = 7.0


def fit(deg, A=A, nodes=6000, iters=40, phi=False):
    k = np.arange(nodes)
    a = (A / 2) * (1 - np.cos(np.pi * (k + 0.5) / nodes))
    Q = -log_ndtr(-a) / np.log(2)
    # GELU error |x| ln2 Phi(-a) dQ, or (phi) the error of Phi, ln2 Phi(-a) dQ
    w = (1.0 if phi else np.maximum(a, 0.02)) * ndtr(-a) * np.log(2)
    V = np.vander(a, deg + 1, increasing=True)
    ww = w.copy()
    for _ in range(iters):
        c, *_ = np.linalg.lstsq(V * ww[:, None], Q * ww, rcond=None)
        err = np.abs((V @ c - Q) * w)
        ww = w * (err / err.max()) ** 0.6 + 1e-30
    return c


def max_error(c):
    """Largest |GELU error| on [-40, 40] of the unclamped float32 evaluation,
    beyond the float32 spacing of x itself."""
    xs = np.linspace(-40, 40, 800001)
    x32 = xs.astype(np.float32)
    ax = np.abs(x32)
    c32 = c.astype(np.float32)
    p = np.full_like(ax, c32[-1])
    for cc in c32[-2::-1]:
        p = (p * ax + cc).astype(np.float32)
    assert np.all(np.diff(p[x32 > A]) >= 0), "Q must keep growing beyond the fit range"
    with np.errstate(over="ignore", under="ignore"):
        h = np.exp2(-p.astype(np.float64)).astype(np.float32)
    g = (np.maximum(x32, 0) - (ax * h).astype(np.float32)).astype(np.float32)
    xx = x32.astype(np.float64)
    err = np.abs(g.astype(np.float64) - xx * ndtr(xx))
    return float(err.max())


def max_phi_error(c):
    """Largest |Phi error| on [-40, 40] of the float32 evaluation
    Phi(x) = x > 0 ? 1 - t : t, t = 2^-R(|x|)."""
    xs = np.linspace(-40, 40, 800001).astype(np.float32)
    ax = np.abs(xs)
    c32 = c.astype(np.float32)
    p = np.full_like(ax, c32[-1])
    for cc in c32[-2::-1]:
        p = (p * ax + cc).astype(np.float32)
    assert np.all(np.diff(p[xs > A]) >= 0), "R must keep growing beyond the fit range"
    with np.errstate(over="ignore", under="ignore"):
        t = np.exp2(-p.astype(np.float64)).astype(np.float32)
    ph = np.where(xs > 0, (1 - t).astype(np.float32), t)
    return float(np.abs(ph.astype(np.float64) - ndtr(xs.astype(np.float64))).max())


if __name__ == "__main__":
    for deg, name in ((5, "kGeluQ"), (3, "kGeluQ3")):
        c = fit(deg)
        print("// degree %d fitted on [0, %.1f]: max |GELU error| on [-40, 40] %.2e "
              "(float32 evaluation, no clamp)" % (deg, A, max_error(c)))
        print("constexpr float %s[%d] = {%s};" % (
            name, deg + 1, ", ".join("%.9ef" % v for v in c.astype(np.float32))))
    c = fit(8, phi=True)
    print("// degree 8 fitted on [0, %.1f]: max |Phi error| on [-40, 40] %.2e "
          "(float32 evaluation, no clamp)" % (A, max_phi_error(c)))
    print("constexpr float kPhiR[9] = {%s};" % ", ".join("%.9ef" % v for v in c.astype(np.float32)))

"""CPU oracle of the pair-interaction path (float64, plain C, OpenMP over jets).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the smoke check and by
the CPU-baseline leg of ``bench.py``; never by the product package.  The C
source (``oracle.c``) is independent of the HIP library: no shared code,
headers or constants.  Every function here takes numpy arrays, upcasts them
exactly to float64 and returns float64 results.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

EPS = 1e-8  # feature clamp used by every workload


class _Mlp(C.Structure):
    _fields_ = [
        ("w1", C.c_void_p), ("b1", C.c_void_p), ("w2", C.c_void_p), ("b2", C.c_void_p),
        ("w3", C.c_void_p), ("b3", C.c_void_p), ("w4", C.c_void_p), ("b4", C.c_void_p),
        ("bn_gamma", C.c_void_p * 3), ("bn_beta", C.c_void_p * 3),
        ("bn_mean", C.c_void_p * 3), ("bn_var", C.c_void_p * 3),
        ("in_gamma", C.c_void_p), ("in_beta", C.c_void_p),
        ("in_mean", C.c_void_p), ("in_var", C.c_void_p),
        ("bn_eps", C.c_double),
    ]


def build(force: bool = True) -> str:
    from . import build as _b
    return _b.build(force=force)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        L = C.CDLL(_LIB_PATH)
        i64, dp, u8p = C.c_int64, C.c_void_p, C.c_void_p
        L.oracle_num_threads.restype = C.c_int
        L.oracle_set_num_threads.argtypes = [C.c_int]
        L.oracle_particle.argtypes = [dp, dp]
        L.oracle_pair_feature.argtypes = [dp, dp, C.c_double, dp]
        L.oracle_gelu.argtypes = [C.c_double]
        L.oracle_gelu.restype = C.c_double
        L.oracle_mlp_pair.argtypes = [C.POINTER(_Mlp), dp, dp]
        L.oracle_pair_features.argtypes = [dp, u8p, i64, i64, C.c_double, dp]
        L.oracle_pair_mlp.argtypes = [dp, u8p, i64, i64, C.POINTER(_Mlp), dp]
        L.oracle_pair_embed.argtypes = [dp, u8p, i64, i64, C.c_double, C.POINTER(_Mlp), dp]
        L.oracle_attention.argtypes = [dp, dp, dp, dp, u8p, i64, i64, i64, i64, C.c_double, dp]
        L.oracle_pair_embed_attention.argtypes = [dp, u8p, i64, i64, C.c_double,
                                                  C.POINTER(_Mlp), dp, dp, dp, i64, C.c_double,
                                                  dp]
        L.oracle_block_stack.argtypes = [dp, dp, dp, dp, dp, dp, u8p, i64, i64, i64, i64,
                                         i64, dp]
        L.oracle_attention_backward.argtypes = [dp, dp, dp, dp, u8p, i64, i64, i64, i64,
                                                C.c_double, dp, dp, dp, dp, dp]
        L.oracle_pair_mlp_backward.argtypes = [dp, u8p, i64, i64, C.POINTER(_Mlp), dp, dp]
        L.oracle_pair_mlp_grad_count.restype = C.c_int
        L.oracle_pair_embed_int8.argtypes = [dp, u8p, i64, i64, C.c_double, C.POINTER(_Mlp), dp,
                                             dp, C.c_double, dp, u8p]
        L.oracle_pair_mlp_ranges.argtypes = [dp, u8p, i64, i64, C.c_double, C.POINTER(_Mlp), dp]
        L.oracle_geometric_product.argtypes = [dp, dp, i64, dp]
        L.oracle_blade_grade.argtypes = [C.c_int]
        L.oracle_blade_grade.restype = C.c_int
        L.oracle_equilinear.argtypes = [dp, dp, i64, i64, i64, i64, i64, dp, dp, dp, dp, dp, dp,
                                         dp, dp]
        for f in ("oracle_attention_backward", "oracle_pair_mlp_backward",
                  "oracle_pair_embed_int8", "oracle_pair_mlp_ranges", "oracle_equilinear",
                  "oracle_pair_features", "oracle_pair_mlp", "oracle_pair_embed",
                  "oracle_attention", "oracle_pair_embed_attention", "oracle_block_stack"):
            getattr(L, f).restype = C.c_int
        _lib = L
    return _lib


def _f64(x):
    return np.ascontiguousarray(x, dtype=np.float64)


def _u8(m):
    return np.ascontiguousarray(np.asarray(m) != 0, dtype=np.uint8)


def _ptr(a):
    return a.ctypes.data_as(C.c_void_p) if a is not None else None


class _MlpArgs:
    """Keeps the float64 copies alive while the C struct points at them."""

    def __init__(self, p: dict):
        self.arrs = {}
        for k, v in p.items():
            if isinstance(v, np.ndarray):
                self.arrs[k] = _f64(v)
        a = self.arrs
        s = _Mlp()
        for i in range(1, 5):
            setattr(s, f"w{i}", _ptr(a[f"w{i}"]))
            b = a.get(f"b{i}")
            setattr(s, f"b{i}", _ptr(b) if b is not None else None)
        for i in range(3):
            s.bn_gamma[i] = _ptr(a[f"bn{i + 1}_gamma"])
            s.bn_beta[i] = _ptr(a[f"bn{i + 1}_beta"])
            s.bn_mean[i] = _ptr(a[f"bn{i + 1}_mean"])
            s.bn_var[i] = _ptr(a[f"bn{i + 1}_var"])
        if "in_gamma" in a:
            s.in_gamma, s.in_beta = _ptr(a["in_gamma"]), _ptr(a["in_beta"])
            s.in_mean, s.in_var = _ptr(a["in_mean"]), _ptr(a["in_var"])
        s.bn_eps = float(p.get("bn_eps", 1e-5))
        self.struct = s


def num_threads() -> int:
    return lib().oracle_num_threads()


def set_num_threads(n: int) -> None:
    lib().oracle_set_num_threads(int(n))


def particle(p4) -> np.ndarray:
    """(pT, y, phi) of one energy-first 4-vector."""
    p = _f64(p4).reshape(4)
    out = np.zeros(3)
    lib().oracle_particle(_ptr(p), _ptr(out))
    return out


def pair_feature(pa, pb, eps: float = EPS) -> np.ndarray:
    """[ln kT, ln z, ln dR, ln m2] of one pair of 4-vectors."""
    a, b = _f64(pa).reshape(4), _f64(pb).reshape(4)
    out = np.zeros(4)
    lib().oracle_pair_feature(_ptr(a), _ptr(b), float(eps), _ptr(out))
    return out


def gelu(x: float) -> float:
    return lib().oracle_gelu(float(x))


def mlp_pair(params: dict, f4) -> np.ndarray:
    m = _MlpArgs(params)
    f = _f64(f4).reshape(4)
    out = np.zeros(8)
    lib().oracle_mlp_pair(C.byref(m.struct), _ptr(f), _ptr(out))
    return out


def pair_features(p4, mask, eps: float = EPS) -> np.ndarray:
    """F (B, 4, P, P) from p4 (B, P, 4) and mask (B, P)."""
    p = _f64(p4)
    B, P = p.shape[:2]
    m = _u8(mask)
    F = np.zeros((B, 4, P, P))
    rc = lib().oracle_pair_features(_ptr(p), _ptr(m), B, P, float(eps), _ptr(F))
    assert rc == 0
    return F


def pair_mlp(F, mask, params: dict) -> np.ndarray:
    """U (B, 8, P, P) from features F (B, 4, P, P)."""
    f = _f64(F)
    B, _, P, _ = f.shape
    m = _u8(mask)
    a = _MlpArgs(params)
    U = np.zeros((B, 8, P, P))
    rc = lib().oracle_pair_mlp(_ptr(f), _ptr(m), B, P, C.byref(a.struct), _ptr(U))
    assert rc == 0
    return U


def pair_embed(p4, mask, params: dict, eps: float = EPS) -> np.ndarray:
    """U (B, 8, P, P) from p4 (B, P, 4): features then MLP, pair by pair."""
    p = _f64(p4)
    B, P = p.shape[:2]
    m = _u8(mask)
    a = _MlpArgs(params)
    U = np.zeros((B, 8, P, P))
    rc = lib().oracle_pair_embed(_ptr(p), _ptr(m), B, P, float(eps), C.byref(a.struct),
                                 _ptr(U))
    assert rc == 0
    return U


def attention(Q, K, V, U, mask, scale=None) -> np.ndarray:
    """O (B, H, P, D): masked softmax(scale Q K^T + U) V per head; scale
    defaults to 1 / sqrt(D)."""
    q, k, v, u = _f64(Q), _f64(K), _f64(V), _f64(U)
    B, H, P, D = q.shape
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    assert k.shape == q.shape and v.shape == q.shape and u.shape == (B, H, P, P)
    m = _u8(mask)
    O = np.zeros((B, H, P, D))
    rc = lib().oracle_attention(_ptr(q), _ptr(k), _ptr(v), _ptr(u), _ptr(m), B, H, P, D,
                                scale, _ptr(O))
    assert rc == 0
    return O


def pair_embed_attention(p4, mask, params: dict, Q, K, V, eps: float = EPS,
                         scale=None) -> np.ndarray:
    p = _f64(p4)
    q, k, v = _f64(Q), _f64(K), _f64(V)
    B, H, P, D = q.shape
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    assert H == 8 and p.shape == (B, P, 4)
    m = _u8(mask)
    a = _MlpArgs(params)
    O = np.zeros((B, H, P, D))
    rc = lib().oracle_pair_embed_attention(_ptr(p), _ptr(m), B, P, float(eps),
                                           C.byref(a.struct), _ptr(q), _ptr(k), _ptr(v), D,
                                           scale, _ptr(O))
    assert rc == 0
    return O


def block_stack(X0, Wq, Wk, Wv, Wo, U, mask) -> np.ndarray:
    """X after L layers of X <- X + Attn(X Wq, X Wk, X Wv; U) Wo."""
    x0 = _f64(X0)
    B, P, Cw = x0.shape
    wq, wk, wv, wo = _f64(Wq), _f64(Wk), _f64(Wv), _f64(Wo)
    L = wq.shape[0]
    u = _f64(U)
    H = u.shape[1]
    m = _u8(mask)
    X = np.zeros_like(x0)
    rc = lib().oracle_block_stack(_ptr(x0), _ptr(wq), _ptr(wk), _ptr(wv), _ptr(wo), _ptr(u),
                                  _ptr(m), B, P, Cw, H, L, _ptr(X))
    assert rc == 0
    return X


# ---------------------------------------------------------------- backward
GRAD_LAYOUT = (("w1", (64, 4)), ("b1", (64,)), ("bn1_gamma", (64,)), ("bn1_beta", (64,)),
               ("w2", (64, 64)), ("b2", (64,)), ("bn2_gamma", (64,)), ("bn2_beta", (64,)),
               ("w3", (64, 64)), ("b3", (64,)), ("bn3_gamma", (64,)), ("bn3_beta", (64,)),
               ("w4", (8, 64)), ("b4", (8,)), ("in_gamma", (4,)), ("in_beta", (4,)))


def attention_backward(Q, K, V, U, mask, dO, scale=None):
    """(dQ, dK, dV, dU) of the masked biased attention for dL/dO = dO."""
    q, k, v, u, g = _f64(Q), _f64(K), _f64(V), _f64(U), _f64(dO)
    B, H, P, D = q.shape
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    m = _u8(mask)
    dQ, dK, dV = np.zeros_like(q), np.zeros_like(q), np.zeros_like(q)
    dU = np.zeros_like(u)
    rc = lib().oracle_attention_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(u), _ptr(m), B, H, P,
                                         D, scale, _ptr(g), _ptr(dQ), _ptr(dK), _ptr(dV),
                                         _ptr(dU))
    assert rc == 0
    return dQ, dK, dV, dU


def pair_mlp_backward(F, mask, params: dict, dU) -> dict:
    """Gradients of sum(U * dU) with respect to the raw MLP parameters (conv
    weights and biases, BatchNorm gamma and beta, input BatchNorm gamma and
    beta), U = pair_mlp(F, mask, params).  Returns {name: float64 array}."""
    f, g = _f64(F), _f64(dU)
    B, _, P, _ = f.shape
    m = _u8(mask)
    a = _MlpArgs(params)
    n = lib().oracle_pair_mlp_grad_count()
    out = np.zeros(n)
    rc = lib().oracle_pair_mlp_backward(_ptr(f), _ptr(m), B, P, C.byref(a.struct), _ptr(g),
                                        _ptr(out))
    assert rc == 0
    res, o = {}, 0
    for name, shape in GRAD_LAYOUT:
        size = int(np.prod(shape))
        res[name] = out[o:o + size].reshape(shape)
        o += size
    assert o == n
    return res


def pair_embed_backward(p4, mask, params: dict, dU, eps: float = EPS) -> dict:
    """pair_mlp_backward on the features of p4 (the features have no
    parameters)."""
    return pair_mlp_backward(pair_features(p4, mask, eps), mask, params, dU)


# ---------------------------------------------------------------- int8 variant
def pair_embed_int8(p4, mask, params: dict, act_scale, act_zero, tie_delta=3e-4,
                    eps: float = EPS):
    """(U, tie): the pair MLP with int8 inputs to layers 2, 3, 4 (per-tensor
    scale / zero point) and per-channel int8 weights, float64 otherwise;
    tie (B, P, P) marks pairs with a quantisation decision within tie_delta
    of a rounding boundary."""
    p = _f64(p4)
    B, P = p.shape[:2]
    m = _u8(mask)
    a = _MlpArgs(params)
    s = np.ascontiguousarray(act_scale, dtype=np.float64)
    z = np.ascontiguousarray(act_zero, dtype=np.float64)
    assert s.shape == (3,) and z.shape == (3,)
    U = np.zeros((B, 8, P, P))
    tie = np.zeros((B, P, P), np.uint8)
    rc = lib().oracle_pair_embed_int8(_ptr(p), _ptr(m), B, P, float(eps), C.byref(a.struct),
                                      _ptr(s), _ptr(z), float(tie_delta), _ptr(U), _ptr(tie))
    assert rc == 0
    return U, tie.astype(bool)


def pair_mlp_ranges(p4, mask, params: dict, eps: float = EPS) -> np.ndarray:
    """[[min, max] of h1], [.. h2], [.. h3] of the float MLP over real pairs."""
    p = _f64(p4)
    B, P = p.shape[:2]
    m = _u8(mask)
    a = _MlpArgs(params)
    out = np.zeros(6)
    rc = lib().oracle_pair_mlp_ranges(_ptr(p), _ptr(m), B, P, float(eps), C.byref(a.struct),
                                      _ptr(out))
    assert rc == 0
    return out.reshape(3, 2)


def int8_calibration(ranges) -> tuple:
    """Per-tensor (scale, zero point) of each hidden input from its range:
    S = (max - min) / 255, Z = -128 - rint(min / S), so that [min, max]
    maps onto [-128, 127]."""
    r = np.asarray(ranges, np.float64)
    S = (r[:, 1] - r[:, 0]) / 255.0
    Z = -128.0 - np.rint(r[:, 0] / S)
    return S, Z


# ---------------------------------------------------------------- L-GATr
def geometric_product(x, y) -> np.ndarray:
    """z = x y in Cl(1,3) for multivectors (..., 16) in grade order."""
    a, b = _f64(x), _f64(y)
    shape = np.broadcast_shapes(a.shape, b.shape)
    a = np.ascontiguousarray(np.broadcast_to(a, shape)).reshape(-1, 16)
    b = np.ascontiguousarray(np.broadcast_to(b, shape)).reshape(-1, 16)
    z = np.zeros_like(a)
    lib().oracle_geometric_product(_ptr(a), _ptr(b), a.shape[0], _ptr(z))
    return z.reshape(shape)


def blade_grades() -> np.ndarray:
    return np.array([lib().oracle_blade_grade(i) for i in range(16)])


def equilinear(x_mv, x_s, w, s2mv=None, mv2s=None, ss=None, b_mv=None, b_s=None):
    """(y_mv, y_s) of the equivariant linear layer: x_mv (n, in_mv, 16),
    x_s (n, in_s), w (out_mv, in_mv, 10), s2mv (out_mv, in_s), mv2s
    (out_s, in_mv), ss (out_s, in_s), b_mv (out_mv), b_s (out_s)."""
    xm = _f64(x_mv)
    n, in_mv, _ = xm.shape
    xs = _f64(x_s) if x_s is not None else np.zeros((n, 0))
    in_s = xs.shape[1]
    wm = _f64(w)
    out_mv = wm.shape[0]
    out_s = 0
    for a, ax in ((mv2s, 0), (ss, 0), (b_s, 0)):
        if a is not None:
            out_s = np.asarray(a).shape[ax]
    arrs = [None if a is None else _f64(a) for a in (s2mv, mv2s, ss, b_mv, b_s)]
    y_mv = np.zeros((n, out_mv, 16))
    y_s = np.zeros((n, out_s))
    rc = lib().oracle_equilinear(_ptr(xm), _ptr(xs), n, in_mv, in_s, out_mv, out_s, _ptr(wm),
                                 *[_ptr(a) for a in arrs], _ptr(y_mv), _ptr(y_s))
    assert rc == 0
    return y_mv, y_s

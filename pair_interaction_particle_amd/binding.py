"""ctypes binding of libpip (include/pip.h): argument marshalling only.

Every function takes torch tensors that already live on the GPU, checks
dtype / device / contiguity, passes raw device pointers plus sizes to the C
ABI and enqueues on torch's current HIP stream.  All arithmetic happens in the
HIP kernels of libpip.so; if the library is missing this module raises -- it
has no fallback.
"""
from __future__ import annotations

import ctypes as C
import os
import re

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpip.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "pip.h")

PIP_F32, PIP_BF16 = 0, 1
STATUS = {0: "PIP_OK", 1: "PIP_ERR_NULL", 2: "PIP_ERR_SHAPE", 3: "PIP_ERR_ALIGN",
          4: "PIP_ERR_DTYPE", 5: "PIP_ERR_UNSUPPORTED", 6: "PIP_ERR_HIP"}
W_FOLDED = 64 * 4 + 2 * 64 * 64 + 8 * 64
B_FOLDED = 3 * 64 + 8

_lib = None


class PipError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__("%s failed: %s (%s)" % (fn, STATUS.get(status, status),
                                                 lib().pip_status_string(status).decode()))


class _Params(C.Structure):
    _fields_ = [
        ("w1", C.c_void_p), ("b1", C.c_void_p), ("w2", C.c_void_p), ("b2", C.c_void_p),
        ("w3", C.c_void_p), ("b3", C.c_void_p), ("w4", C.c_void_p), ("b4", C.c_void_p),
        ("bn_gamma", C.c_void_p * 3), ("bn_beta", C.c_void_p * 3),
        ("bn_mean", C.c_void_p * 3), ("bn_var", C.c_void_p * 3),
        ("in_gamma", C.c_void_p), ("in_beta", C.c_void_p),
        ("in_mean", C.c_void_p), ("in_var", C.c_void_p),
        ("bn_eps", C.c_float),
    ]


def header_functions() -> list:
    """Names of the functions include/pip.h declares."""
    src = open(HEADER_PATH).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(pip_[a-z0-9_]+)\s*\(", src)))


def lib():
    """Load libpip.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libpip.so is not built (%s); run __graft_entry__.build()"
                               % LIB_PATH)
        L = C.CDLL(LIB_PATH)
        vp, i64, i = C.c_void_p, C.c_int64, C.c_int
        L.pip_status_string.argtypes = [i]
        L.pip_status_string.restype = C.c_char_p
        L.pip_version.restype = i
        L.pip_pair_mlp_fold.argtypes = [C.POINTER(_Params), vp, vp]
        L.pip_pair_mlp_create.argtypes = [C.POINTER(_Params), C.POINTER(vp)]
        L.pip_pair_mlp_destroy.argtypes = [vp]
        L.pip_pair_features.argtypes = [vp, vp, i64, i64, vp, vp]
        L.pip_pair_embed.argtypes = [vp, vp, i64, i64, vp, vp, i, vp]
        L.pip_pair_bias_attention.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, vp, i, vp]
        L.pip_pair_embed_attention.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, vp, i, vp]
        L.pip_block_stack_workspace_bytes.argtypes = [i64, i64, i64, i64]
        L.pip_block_stack_workspace_bytes.restype = C.c_size_t
        L.pip_block_stack.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, vp,
                                      C.c_size_t, vp]
        for f in ("pip_pair_mlp_fold", "pip_pair_mlp_create", "pip_pair_mlp_destroy",
                  "pip_pair_features", "pip_pair_embed", "pip_pair_bias_attention",
                  "pip_pair_embed_attention", "pip_block_stack"):
            getattr(L, f).restype = i
        _lib = L
    return _lib


def _check(fn, st):
    if st != 0:
        raise PipError(fn, st)


# ---------------------------------------------------------------- parameters
class _HostParams:
    """float32 host copies of the raw MLP parameters and the C struct over them."""

    def __init__(self, p: dict):
        self.keep = {}

        def ptr(name):
            if name not in p or p[name] is None:
                return None
            a = np.ascontiguousarray(np.asarray(p[name], dtype=np.float32))
            self.keep[name] = a
            return a.ctypes.data

        s = _Params()
        for k in range(1, 5):
            setattr(s, "w%d" % k, ptr("w%d" % k))
            setattr(s, "b%d" % k, ptr("b%d" % k))
        for k in range(3):
            s.bn_gamma[k] = ptr("bn%d_gamma" % (k + 1))
            s.bn_beta[k] = ptr("bn%d_beta" % (k + 1))
            s.bn_mean[k] = ptr("bn%d_mean" % (k + 1))
            s.bn_var[k] = ptr("bn%d_var" % (k + 1))
        s.in_gamma, s.in_beta = ptr("in_gamma"), ptr("in_beta")
        s.in_mean, s.in_var = ptr("in_mean"), ptr("in_var")
        s.bn_eps = float(p.get("bn_eps", 1e-5))
        self.struct = s


def fold(params: dict):
    """Host-side BatchNorm fold (pip_pair_mlp_fold): returns float32 arrays
    (w1' (64,4), w2' (64,64), w3' (64,64), w4 (8,64)) and (b1', b2', b3', b4)."""
    hp = _HostParams(params)
    w = np.zeros(W_FOLDED, np.float32)
    b = np.zeros(B_FOLDED, np.float32)
    _check("pip_pair_mlp_fold", lib().pip_pair_mlp_fold(C.byref(hp.struct), w.ctypes.data,
                                                        b.ctypes.data))
    ws = (w[:256].reshape(64, 4), w[256:4352].reshape(64, 64), w[4352:8448].reshape(64, 64),
          w[8448:].reshape(8, 64))
    bs = (b[:64], b[64:128], b[128:192], b[192:])
    return ws, bs


class PairMLP:
    """Folded, MFMA-packed pair MLP resident on the current GPU."""

    def __init__(self, params: dict):
        hp = _HostParams(params)
        h = C.c_void_p()
        _check("pip_pair_mlp_create", lib().pip_pair_mlp_create(C.byref(hp.struct), C.byref(h)))
        self._h = h

    @property
    def handle(self):
        return self._h

    def close(self):
        if self._h is not None and self._h.value:
            _check("pip_pair_mlp_destroy", lib().pip_pair_mlp_destroy(self._h))
        self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ---------------------------------------------------------------- tensors
def _torch():
    import torch
    return torch


def _stream():
    return _torch().cuda.current_stream().cuda_stream


def _dev(t, name, dtype=None, shape=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    return t.data_ptr()


def _code(dtype):
    torch = _torch()
    if dtype in (torch.float32, "f32", "float32"):
        return PIP_F32, torch.float32
    if dtype in (torch.bfloat16, "bf16", "bfloat16"):
        return PIP_BF16, torch.bfloat16
    raise TypeError("dtype must be float32 or bfloat16")


def pair_features(p4, mask, out=None):
    """F (B, 4, P, P) float32: [ln kT, ln z, ln dR, ln m2] of every real pair."""
    torch = _torch()
    B, P = p4.shape[:2]
    if out is None:
        out = torch.empty((B, 4, P, P), device=p4.device, dtype=torch.float32)
    st = lib().pip_pair_features(_dev(p4, "p4", torch.float32, (B, P, 4)),
                                 _dev(mask, "mask", torch.uint8, (B, P)), B, P,
                                 _dev(out, "F", torch.float32, (B, 4, P, P)), _stream())
    _check("pip_pair_features", st)
    return out


def pair_embed(p4, mask, mlp: PairMLP, dtype="f32", out=None):
    """U (B, 8, P, P) in float32 or bfloat16 from p4 (B, P, 4) and mask (B, P)."""
    torch = _torch()
    code, tdt = _code(dtype)
    B, P = p4.shape[:2]
    if out is None:
        out = torch.empty((B, 8, P, P), device=p4.device, dtype=tdt)
    st = lib().pip_pair_embed(_dev(p4, "p4", torch.float32, (B, P, 4)),
                              _dev(mask, "mask", torch.uint8, (B, P)), B, P, mlp.handle,
                              _dev(out, "U", tdt, (B, 8, P, P)), code, _stream())
    _check("pip_pair_embed", st)
    return out


def pair_bias_attention(q, k, v, u, mask, out=None):
    """O (B, H, P, D) = masked softmax(Q K^T / sqrt(D) + U) V, dtype of q."""
    torch = _torch()
    code, tdt = _code(q.dtype)
    B, H, P, D = q.shape
    if out is None:
        out = torch.empty_like(q)
    st = lib().pip_pair_bias_attention(
        _dev(q, "Q", tdt), _dev(k, "K", tdt, q.shape), _dev(v, "V", tdt, q.shape),
        _dev(u, "U", tdt, (B, H, P, P)), _dev(mask, "mask", torch.uint8, (B, P)), B, H, P, D,
        _dev(out, "O", tdt, q.shape), code, _stream())
    _check("pip_pair_bias_attention", st)
    return out


def pair_embed_attention(p4, mask, mlp: PairMLP, q, k, v, out=None):
    """Fused pair embedding + attention (H = 8): O (B, 8, P, D), dtype of q."""
    torch = _torch()
    code, tdt = _code(q.dtype)
    B, H, P, D = q.shape
    if out is None:
        out = torch.empty_like(q)
    st = lib().pip_pair_embed_attention(
        _dev(p4, "p4", torch.float32, (B, P, 4)), _dev(mask, "mask", torch.uint8, (B, P)),
        mlp.handle, _dev(q, "Q", tdt, (B, 8, P, D)), _dev(k, "K", tdt, q.shape),
        _dev(v, "V", tdt, q.shape), B, P, D, _dev(out, "O", tdt, q.shape), code, _stream())
    _check("pip_pair_embed_attention", st)
    return out


def block_stack_workspace_bytes(B, P, C_, L_):
    return int(lib().pip_block_stack_workspace_bytes(B, P, C_, L_))


def block_stack(x, wq, wk, wv, wo, u, mask, workspace=None):
    """In place: L layers of X <- X + Attn(X Wq, X Wk, X Wv; U) Wo.  Returns x."""
    torch = _torch()
    B, P, Cw = x.shape
    L = wq.shape[0]
    H = u.shape[1]
    nbytes = block_stack_workspace_bytes(B, P, Cw, L)
    if workspace is None:
        workspace = torch.empty(max(nbytes // 4, 1), device=x.device, dtype=torch.float32)
    st = lib().pip_block_stack(
        _dev(x, "X", torch.float32, (B, P, Cw)), _dev(wq, "Wq", torch.float32, (L, Cw, Cw)),
        _dev(wk, "Wk", torch.float32, (L, Cw, Cw)), _dev(wv, "Wv", torch.float32, (L, Cw, Cw)),
        _dev(wo, "Wo", torch.float32, (L, Cw, Cw)), _dev(u, "U", torch.float32, (B, H, P, P)),
        _dev(mask, "mask", torch.uint8, (B, P)), B, P, Cw, H, L,
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream())
    _check("pip_block_stack", st)
    return x

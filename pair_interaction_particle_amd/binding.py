"""ctypes binding of libpip (include/pip.h): argument marshalling only.

Every function takes torch tensors that already live on the GPU, checks
dtype / device / contiguity, passes raw device pointers plus sizes to the C
ABI and enqueues on torch's current HIP stream.  All arithmetic happens in the
HIP kernels of libpip.so; if the library is missing this module raises -- it
has no fallback.
"""
from __future__ import annotations

import ctypes as C
import math
import os
import re

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpip.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "pip.h")

PIP_F32, PIP_BF16 = 0, 1
STATUS = {0: "PIP_OK", 1: "PIP_ERR_NULL", 2: "PIP_ERR_SHAPE", 3: "PIP_ERR_ALIGN",
          4: "PIP_ERR_DTYPE", 5: "PIP_ERR_UNSUPPORTED", 6: "PIP_ERR_HIP", 7: "PIP_ERR_VALUE",
          8: "PIP_ERR_TOO_LARGE"}
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
            raise RuntimeError("libpip.so is not built (%s); build it with "
                               "python -m pair_interaction_particle_amd.build" % LIB_PATH)
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
        f32 = C.c_float
        L.pip_pair_bias_attention.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, f32, vp,
                                              i, vp]
        L.pip_pair_embed_attention.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, f32, vp,
                                               i, vp]
        L.pip_packed_u_offsets.argtypes = [vp, i64, vp, vp]
        L.pip_pair_embed_packed.argtypes = [vp, vp, vp, i64, i64, i64, vp, vp, i64, i, vp]
        L.pip_pair_bias_attention_packed.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64,
                                                     i64, f32, i64, vp, i, vp]
        L.pip_pair_embed_int8.argtypes = [vp, vp, i64, i64, vp, vp, vp, vp, vp]
        L.pip_pair_bias_attention_backward.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64,
                                                       i64, f32, vp, vp, vp, vp, i, vp]
        L.pip_pair_mlp_backward_workspace_bytes.argtypes = [i64, i64]
        L.pip_pair_mlp_backward_workspace_bytes.restype = C.c_size_t
        L.pip_pair_mlp_backward.argtypes = [vp, vp, i64, i64, vp, vp, vp, vp, C.c_size_t, vp]
        L.pip_pair_mlp_unfold_grads.argtypes = [C.POINTER(_Params), vp, vp]
        L.pip_block_stack_workspace_bytes.argtypes = [i64, i64, i64, i64]
        L.pip_block_stack_workspace_bytes.restype = C.c_size_t
        L.pip_block_stack.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, vp,
                                      C.c_size_t, vp]
        L.pip_block_stack_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64,
                                              i64, vp]
        L.pip_lgatr_geometric_product.argtypes = [vp, vp, i64, vp, vp]
        L.pip_lgatr_equilinear_expand.argtypes = [vp, vp, vp, vp, i, i, i, i, vp]
        L.pip_lgatr_equilinear_create.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i,
                                                  C.POINTER(vp)]
        L.pip_lgatr_equilinear_destroy.argtypes = [vp]
        L.pip_lgatr_equilinear.argtypes = [vp, vp, vp, i64, vp, vp, vp]
        for f in ("pip_lgatr_geometric_product", "pip_lgatr_equilinear_expand",
                  "pip_lgatr_equilinear_create", "pip_lgatr_equilinear_destroy",
                  "pip_lgatr_equilinear",
                  "pip_pair_mlp_fold", "pip_pair_mlp_create", "pip_pair_mlp_destroy",
                  "pip_pair_features", "pip_pair_embed", "pip_pair_bias_attention",
                  "pip_pair_embed_attention", "pip_block_stack", "pip_block_stack_noalloc",
                  "pip_packed_u_offsets", "pip_pair_embed_packed",
                  "pip_pair_bias_attention_packed", "pip_pair_bias_attention_backward",
                  "pip_pair_mlp_backward", "pip_pair_mlp_unfold_grads", "pip_pair_embed_int8"):
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


def pair_bias_attention(q, k, v, u, mask, out=None, scale=None):
    """O (B, H, P, D) = masked softmax(scale Q K^T + U) V, dtype of q;
    scale defaults to 1 / sqrt(D)."""
    torch = _torch()
    code, tdt = _code(q.dtype)
    B, H, P, D = q.shape
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    st = lib().pip_pair_bias_attention(
        _dev(q, "Q", tdt), _dev(k, "K", tdt, q.shape), _dev(v, "V", tdt, q.shape),
        _dev(u, "U", tdt, (B, H, P, P)), _dev(mask, "mask", torch.uint8, (B, P)), B, H, P, D,
        scale, _dev(out, "O", tdt, q.shape), code, _stream())
    _check("pip_pair_bias_attention", st)
    return out


def pair_embed_attention(p4, mask, mlp: PairMLP, q, k, v, out=None, scale=None):
    """Fused pair embedding + attention (H = 8): O (B, 8, P, D), dtype of q;
    scale defaults to 1 / sqrt(D)."""
    torch = _torch()
    code, tdt = _code(q.dtype)
    B, H, P, D = q.shape
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    st = lib().pip_pair_embed_attention(
        _dev(p4, "p4", torch.float32, (B, P, 4)), _dev(mask, "mask", torch.uint8, (B, P)),
        mlp.handle, _dev(q, "Q", tdt, (B, 8, P, D)), _dev(k, "K", tdt, q.shape),
        _dev(v, "V", tdt, q.shape), B, P, D, scale, _dev(out, "O", tdt, q.shape), code,
        _stream())
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


def block_stack_noalloc(x, wq, wk, wv, wo, u, mask):
    """pip_block_stack_noalloc: as block_stack, with the workspace in the
    library's fixed per-GPU scratch array (no allocation).  Returns x."""
    torch = _torch()
    B, P, Cw = x.shape
    L = wq.shape[0]
    H = u.shape[1]
    st = lib().pip_block_stack_noalloc(
        _dev(x, "X", torch.float32, (B, P, Cw)), _dev(wq, "Wq", torch.float32, (L, Cw, Cw)),
        _dev(wk, "Wk", torch.float32, (L, Cw, Cw)), _dev(wv, "Wv", torch.float32, (L, Cw, Cw)),
        _dev(wo, "Wo", torch.float32, (L, Cw, Cw)), _dev(u, "U", torch.float32, (B, H, P, P)),
        _dev(mask, "mask", torch.uint8, (B, P)), B, P, Cw, H, L, _stream())
    _check("pip_block_stack_noalloc", st)
    return x


# ---------------------------------------------------------------- packed layout
def packed_ld(n):
    """Row stride of a packed jet's U block: n rounded up to a multiple of 8."""
    return (int(n) + 7) // 8 * 8


def packed_u_offsets(cu):
    """u_offsets (B + 1, int64, device) of the packed U blocks, computed on the
    GPU from cu_seqlens (B + 1, int32, device)."""
    torch = _torch()
    B = cu.numel() - 1
    out = torch.empty(B + 1, device=cu.device, dtype=torch.int64)
    _check("pip_packed_u_offsets",
           lib().pip_packed_u_offsets(_dev(cu, "cu_seqlens", torch.int32), B,
                                      _dev(out, "u_offsets", torch.int64), _stream()))
    return out


def _packed_sizes(cu):
    """(B, max_n, total U pairs) from a host copy of cu_seqlens, for sizing
    outputs (the kernels read cu_seqlens on the device)."""
    c = cu.cpu().numpy().astype(np.int64)
    n = np.diff(c)
    ld = (n + 7) // 8 * 8
    return len(n), int(n.max()) if len(n) else 0, int((n * ld).sum())


def pair_embed_packed(p4, cu, mlp: PairMLP, dtype="f32", u_offsets=None, max_n=None,
                      out=None):
    """Packed U (one (8, n_b, ld_b) block per jet, concatenated) from p4 (N, 4)
    and cu_seqlens (B + 1).  Returns (U, u_offsets)."""
    torch = _torch()
    code, tdt = _code(dtype)
    N = p4.shape[0]
    B = cu.numel() - 1
    if max_n is None or out is None:
        _, mx, pairs = _packed_sizes(cu)  # host copy of cu: only to size outputs
        max_n = mx if max_n is None else int(max_n)
        if out is None:
            out = torch.empty(8 * pairs, device=p4.device, dtype=tdt)
    if u_offsets is None:
        u_offsets = packed_u_offsets(cu)
    st = lib().pip_pair_embed_packed(
        _dev(p4, "p4", torch.float32, (N, 4)), _dev(cu, "cu_seqlens", torch.int32, (B + 1,)),
        _dev(u_offsets, "u_offsets", torch.int64, (B + 1,)), B, N, max_n, mlp.handle,
        _dev(out, "U", tdt), out.numel(), code, _stream())
    _check("pip_pair_embed_packed", st)
    return out, u_offsets


def pair_bias_attention_packed(q, k, v, u, cu, u_offsets, max_n=None, out=None, scale=None):
    """O (H, N, D) on the packed layout: per jet and head, masked-free
    softmax(scale Q K^T + U_b) V over the jet's rows; dtype of q."""
    torch = _torch()
    code, tdt = _code(q.dtype)
    H, N, D = q.shape
    B = cu.numel() - 1
    if max_n is None:
        max_n = _packed_sizes(cu)[1]
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    st = lib().pip_pair_bias_attention_packed(
        _dev(q, "Q", tdt), _dev(k, "K", tdt, q.shape), _dev(v, "V", tdt, q.shape),
        _dev(u, "U", tdt), _dev(cu, "cu_seqlens", torch.int32, (B + 1,)),
        _dev(u_offsets, "u_offsets", torch.int64, (B + 1,)), B, H, N, int(max_n), D, scale,
        u.numel(), _dev(out, "O", tdt, q.shape), code, _stream())
    _check("pip_pair_bias_attention_packed", st)
    return out


# ---------------------------------------------------------------- backward
FOLDED_GRADS, RAW_GRADS = 9160, 9552
RAW_GRAD_LAYOUT = (("w1", (64, 4)), ("b1", (64,)), ("bn1_gamma", (64,)), ("bn1_beta", (64,)),
                   ("w2", (64, 64)), ("b2", (64,)), ("bn2_gamma", (64,)), ("bn2_beta", (64,)),
                   ("w3", (64, 64)), ("b3", (64,)), ("bn3_gamma", (64,)), ("bn3_beta", (64,)),
                   ("w4", (8, 64)), ("b4", (8,)), ("in_gamma", (4,)), ("in_beta", (4,)))


def pair_bias_attention_backward(q, k, v, u, mask, dO, scale=None):
    """(dQ, dK, dV, dU) of pair_bias_attention for dL/dO = dO (float32)."""
    torch = _torch()
    code, tdt = _code(q.dtype)
    B, H, P, D = q.shape
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    dQ, dK, dV = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    dU = torch.empty_like(u)
    st = lib().pip_pair_bias_attention_backward(
        _dev(q, "Q", tdt), _dev(k, "K", tdt, q.shape), _dev(v, "V", tdt, q.shape),
        _dev(u, "U", tdt, (B, H, P, P)), _dev(mask, "mask", torch.uint8, (B, P)),
        _dev(dO, "dO", tdt, q.shape), B, H, P, D, scale, _dev(dQ, "dQ", tdt),
        _dev(dK, "dK", tdt), _dev(dV, "dV", tdt), _dev(dU, "dU", tdt), code, _stream())
    _check("pip_pair_bias_attention_backward", st)
    return dQ, dK, dV, dU


def pair_mlp_backward(p4, mask, mlp: PairMLP, dU, workspace=None):
    """Folded-parameter gradient (device, FOLDED_GRADS floats) of sum(U * dU)."""
    torch = _torch()
    B, P = p4.shape[:2]
    nbytes = int(lib().pip_pair_mlp_backward_workspace_bytes(B, P))
    if workspace is None:
        workspace = torch.empty(max(nbytes // 4, 1), device=p4.device, dtype=torch.float32)
    grad = torch.empty(FOLDED_GRADS, device=p4.device, dtype=torch.float32)
    st = lib().pip_pair_mlp_backward(
        _dev(p4, "p4", torch.float32, (B, P, 4)), _dev(mask, "mask", torch.uint8, (B, P)), B, P,
        mlp.handle, _dev(dU, "dU", torch.float32, (B, 8, P, P)), _dev(grad, "grad"),
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream())
    _check("pip_pair_mlp_backward", st)
    return grad


def unfold_grads(params: dict, grad_folded) -> dict:
    """pip_pair_mlp_unfold_grads: raw-parameter gradients {name: float32
    array} from the folded gradient (host array or tensor)."""
    hp = _HostParams(params)
    gf = np.ascontiguousarray(np.asarray(grad_folded, dtype=np.float32)).reshape(-1)
    assert gf.size == FOLDED_GRADS
    gr = np.zeros(RAW_GRADS, np.float32)
    _check("pip_pair_mlp_unfold_grads",
           lib().pip_pair_mlp_unfold_grads(C.byref(hp.struct), gf.ctypes.data, gr.ctypes.data))
    out, o = {}, 0
    for name, shape in RAW_GRAD_LAYOUT:
        size = int(np.prod(shape))
        out[name] = gr[o:o + size].reshape(shape)
        o += size
    return out


# ---------------------------------------------------------------- int8 variant
def pair_embed_int8(p4, mask, mlp: PairMLP, act_scale, act_zero, out=None):
    """U (B, 8, P, P) bfloat16 with int8 inputs to the hidden linears:
    act_scale / act_zero (3 each) quantise the inputs of layers 2, 3, 4."""
    torch = _torch()
    B, P = p4.shape[:2]
    s = np.ascontiguousarray(np.asarray(act_scale, dtype=np.float32).reshape(3))
    z = np.ascontiguousarray(np.asarray(act_zero, dtype=np.int32).reshape(3))
    if out is None:
        out = torch.empty((B, 8, P, P), device=p4.device, dtype=torch.bfloat16)
    st = lib().pip_pair_embed_int8(_dev(p4, "p4", torch.float32, (B, P, 4)),
                                   _dev(mask, "mask", torch.uint8, (B, P)), B, P, mlp.handle,
                                   s.ctypes.data, z.ctypes.data,
                                   _dev(out, "U", torch.bfloat16, (B, 8, P, P)), _stream())
    _check("pip_pair_embed_int8", st)
    return out


# ---------------------------------------------------------------- L-GATr
LGATR_MV = 16


def _host_f32(a, shape=None, name="array"):
    if a is None:
        return None
    arr = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    if shape is not None and arr.shape != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), arr.shape))
    return arr


def _equi_weights(w, s2mv, mv2s, ss, in_s, out_s):
    w = _host_f32(w)
    if w is None or w.ndim != 3 or w.shape[2] != 10:
        raise ValueError("w must have shape (out_mv, in_mv, 10)")
    out_mv, in_mv = w.shape[:2]
    return (w, _host_f32(s2mv, (out_mv, in_s), "s2mv"), _host_f32(mv2s, (out_s, in_mv), "mv2s"),
            _host_f32(ss, (out_s, in_s), "ss"), in_mv, out_mv)


def _p(a):
    return None if a is None else a.ctypes.data


def equilinear_expand(w, s2mv=None, mv2s=None, ss=None, in_s=0, out_s=0):
    """W_eff (out_mv*16 + out_s, in_mv*16 + in_s) float32 of the equivariant
    linear layer (host only; pip_lgatr_equilinear_expand)."""
    w, s2mv, mv2s, ss, in_mv, out_mv = _equi_weights(w, s2mv, mv2s, ss, in_s, out_s)
    out = np.zeros((out_mv * 16 + out_s, in_mv * 16 + in_s), np.float32)
    _check("pip_lgatr_equilinear_expand",
           lib().pip_lgatr_equilinear_expand(_p(w), _p(s2mv), _p(mv2s), _p(ss), in_mv, out_mv,
                                             in_s, out_s, out.ctypes.data))
    return out


class EquiLinear:
    """L-GATr equivariant linear layer, W_eff packed on the current GPU."""

    def __init__(self, w, s2mv=None, mv2s=None, ss=None, b_mv=None, b_s=None, in_s=0, out_s=0):
        w, s2mv, mv2s, ss, in_mv, out_mv = _equi_weights(w, s2mv, mv2s, ss, in_s, out_s)
        self._keep = (w, s2mv, mv2s, ss, _host_f32(b_mv, (out_mv,), "b_mv"),
                      _host_f32(b_s, (out_s,), "b_s"))
        self.in_mv, self.out_mv, self.in_s, self.out_s = in_mv, out_mv, in_s, out_s
        h = C.c_void_p()
        _check("pip_lgatr_equilinear_create",
               lib().pip_lgatr_equilinear_create(*[_p(a) for a in self._keep], in_mv, out_mv,
                                                 in_s, out_s, C.byref(h)))
        self._h = h

    def __call__(self, x_mv, x_s=None, y_mv=None, y_s=None):
        torch = _torch()
        n = x_mv.shape[0]
        px = _dev(x_mv, "x_mv", torch.float32, (n, self.in_mv, 16))
        ps = _dev(x_s, "x_s", torch.float32, (n, self.in_s)) if self.in_s else None
        if y_mv is None:
            y_mv = torch.empty((n, self.out_mv, 16), device=x_mv.device, dtype=torch.float32)
        if y_s is None and self.out_s:
            y_s = torch.empty((n, self.out_s), device=x_mv.device, dtype=torch.float32)
        py = _dev(y_mv, "y_mv", torch.float32, (n, self.out_mv, 16))
        pys = _dev(y_s, "y_s", torch.float32, (n, self.out_s)) if self.out_s else None
        _check("pip_lgatr_equilinear",
               lib().pip_lgatr_equilinear(self._h, px, ps, n, py, pys, _stream()))
        return y_mv, y_s

    def close(self):
        if self._h is not None and self._h.value:
            _check("pip_lgatr_equilinear_destroy", lib().pip_lgatr_equilinear_destroy(self._h))
        self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def geometric_product(x, y, out=None):
    """z = x y (Cl(1,3) geometric product) of float32 multivectors (..., 16)."""
    torch = _torch()
    if x.shape != y.shape or x.shape[-1] != 16:
        raise ValueError("x and y must have the same shape (..., 16)")
    px = _dev(x, "x", torch.float32)
    py = _dev(y, "y", torch.float32)
    if out is None:
        out = torch.empty_like(x)
    pz = _dev(out, "out", torch.float32, x.shape)
    _check("pip_lgatr_geometric_product",
           lib().pip_lgatr_geometric_product(px, py, x.numel() // 16, pz, _stream()))
    return out

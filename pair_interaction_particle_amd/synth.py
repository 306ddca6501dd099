"""Seeded synthetic inputs for the pair-interaction path.

This module only *draws* inputs: jets of 4-momenta with padding masks, pair-MLP
parameters (raw, unfolded BatchNorm), per-head Q/K/V, and the residual stream
and projection weights of the block stack.  It holds none of the path's
arithmetic (no invariants, no MLP, no attention), so the CPU oracle and the HIP
path can both be fed from it without sharing any of the method.

Workload shapes follow the kernel-level benchmark of the ml4sci_cms_e2e26
README ("Results", table "ParT Kernels": N=128 jets, P=128 slots, H=8 heads,
D=16) and the batch-512 shape named in its "Fusion 2" paragraph.  The data the
pages measured on (QuarkGluon) is not available, so jets are synthetic:

* multiplicity n ~ integer-uniform (inclusive), slots >= n are padding (mask 0,
  all values 0);
* per jet: jet_y ~ U(-2, 2), jet_phi ~ U(-pi, pi);
* per particle: pT log-uniform on [0.5, 500] GeV, y = jet_y + N(0, sigma),
  phi = wrap(jet_phi + N(0, sigma)); massless, E = |p| (a fraction of massive
  particles with m ~ U(0, 1) GeV and E = sqrt(|p|^2 + m^2) where asked);
* 4-vectors are energy-first (E, px, py, pz), the convention of the lloca
  ``transformer_v2.Transformer.forward`` documentation (``p_ref`` parameter).

Everything is generated in float64 with ``numpy.random.default_rng`` streams
spawned from one ``SeedSequence`` (kinematics, MLP parameters, Q/K/V, block
stack each get their own stream), then stored as float32 (and bf16 with
round-to-nearest-even where a workload asks for bf16).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = [
    "WORKLOADS",
    "Workload",
    "make_jets",
    "make_mlp_params",
    "make_qkv",
    "make_block_stack",
    "make_workload",
    "bf16_round",
    "bf16_bits",
    "bf16_bits_to_f32",
    "pack_rows",
    "pack_heads",
    "cu_seqlens",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and distribution recipe of one synthetic workload."""

    name: str
    B: int
    P: int
    n_min: int
    n_max: int
    H: int = 8
    D: int = 16
    sigma: float = 0.4
    massive_frac: float = 0.0
    dtype: str = "f32"          # "f32" or "bf16" for Q/K/V/U/O and the hidden MLP
    fixed_n: tuple | None = None
    C: int = 0                  # block stack: embedding width (0 = no block stack)
    L: int = 0                  # block stack: number of layers
    entry: str = "pair_embed+pair_bias_attention"


WORKLOADS = {
    # Tiny case the oracle finishes instantly: 2 jets, 16 slots, 11 and 16 real.
    "tiny": Workload("tiny", B=2, P=16, n_min=11, n_max=16, fixed_n=(11, 16)),
    # The README's kernel-benchmark shape: N=128, P=128, H=8, D=16.
    "kernel": Workload("kernel", B=128, P=128, n_min=20, n_max=128),
    # Training-batch scale for the fused entry (batch 512, P=128), 5% massive.
    "fused512": Workload("fused512", B=512, P=128, n_min=20, n_max=128,
                         massive_frac=0.05, entry="pair_embed_attention"),
    # Large jets, bf16 variant, wider spread.
    "large_bf16": Workload("large_bf16", B=64, P=256, n_min=60, n_max=256,
                           sigma=0.8, dtype="bf16"),
    # Eight attention layers reusing one bias, embed 128.
    "stack8": Workload("stack8", B=128, P=128, n_min=20, n_max=128, C=128, L=8,
                       entry="block_stack"),
}


def _streams(seed: int):
    ss = np.random.SeedSequence(seed)
    kin, mlp, qkv, stack = ss.spawn(4)
    return (np.random.default_rng(kin), np.random.default_rng(mlp),
            np.random.default_rng(qkv), np.random.default_rng(stack))


# ---------------------------------------------------------------- bf16 storage
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    rounding = ((u >> 16) & 1) + 0x7FFF
    out = ((u + rounding) >> 16).astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> the float32 values they encode (exact)."""
    u = np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 and return them as float32."""
    return bf16_bits_to_f32(bf16_bits(x))


# ---------------------------------------------------------------- generators
def make_jets(B: int, P: int, n_min: int, n_max: int, *, sigma: float = 0.4,
              massive_frac: float = 0.0, fixed_n=None, rng=None, seed: int = 0):
    """Synthetic padded jets.

    Returns ``(p4, mask, n)``: p4 float32 (B, P, 4) energy-first, mask uint8
    (B, P) with 1 on the first n[b] slots, n int64 (B,).  Padded slots are 0.
    """
    if rng is None:
        rng = _streams(seed)[0]
    if fixed_n is not None:
        n = np.asarray(fixed_n, dtype=np.int64)
        assert n.shape == (B,)
    else:
        n = rng.integers(n_min, n_max + 1, size=B).astype(np.int64)
    jet_y = rng.uniform(-2.0, 2.0, size=B)
    jet_phi = rng.uniform(-math.pi, math.pi, size=B)
    pt = np.exp(rng.uniform(math.log(0.5), math.log(500.0), size=(B, P)))
    y = jet_y[:, None] + rng.normal(0.0, sigma, size=(B, P))
    phi = jet_phi[:, None] + rng.normal(0.0, sigma, size=(B, P))
    phi = np.mod(phi + math.pi, 2.0 * math.pi) - math.pi
    if massive_frac > 0.0:
        is_massive = rng.random(size=(B, P)) < massive_frac
        m = rng.uniform(0.0, 1.0, size=(B, P)) * is_massive
    else:
        m = np.zeros((B, P))
    px = pt * np.cos(phi)
    py = pt * np.sin(phi)
    pz = pt * np.sinh(y)
    E = np.sqrt(px * px + py * py + pz * pz + m * m)
    p4 = np.stack([E, px, py, pz], axis=-1)
    mask = (np.arange(P)[None, :] < n[:, None]).astype(np.uint8)
    p4 = np.where(mask[..., None] != 0, p4, 0.0).astype(np.float32)
    return p4, mask, n


def make_mlp_params(*, rng=None, seed: int = 0, biases: bool = False,
                    input_bn: bool = False, widths=(4, 64, 64, 64, 8)):
    """Raw (unfolded) pair-MLP parameters as float32 arrays.

    Conv1d(k=1) weights are Xavier-normal, std = sqrt(2 / (fan_in + fan_out)),
    shaped (out, in).  Conv biases are zero unless ``biases``.  BatchNorm after
    each hidden linear: gamma ~ U(0.5, 1.5), beta ~ N(0, 0.1), running mean ~
    N(0, 0.1), running var ~ U(0.5, 2), eps 1e-5.  ``input_bn`` adds a
    BatchNorm on the 4 input features (mean ~ N(0, 3), var ~ U(1, 30), so that
    it actually rescales the log-features).
    """
    if rng is None:
        rng = _streams(seed)[1]
    p = {}
    nl = len(widths) - 1
    for k in range(nl):
        fi, fo = widths[k], widths[k + 1]
        std = math.sqrt(2.0 / (fi + fo))
        p[f"w{k + 1}"] = rng.normal(0.0, std, size=(fo, fi)).astype(np.float32)
        if biases:
            p[f"b{k + 1}"] = rng.normal(0.0, 0.1, size=fo).astype(np.float32)
        else:
            p[f"b{k + 1}"] = np.zeros(fo, dtype=np.float32)
    for k in range(nl - 1):
        c = widths[k + 1]
        p[f"bn{k + 1}_gamma"] = rng.uniform(0.5, 1.5, size=c).astype(np.float32)
        p[f"bn{k + 1}_beta"] = rng.normal(0.0, 0.1, size=c).astype(np.float32)
        p[f"bn{k + 1}_mean"] = rng.normal(0.0, 0.1, size=c).astype(np.float32)
        p[f"bn{k + 1}_var"] = rng.uniform(0.5, 2.0, size=c).astype(np.float32)
    if input_bn:
        c = widths[0]
        p["in_gamma"] = rng.uniform(0.5, 1.5, size=c).astype(np.float32)
        p["in_beta"] = rng.normal(0.0, 0.1, size=c).astype(np.float32)
        p["in_mean"] = rng.normal(0.0, 3.0, size=c).astype(np.float32)
        p["in_var"] = rng.uniform(1.0, 30.0, size=c).astype(np.float32)
    p["bn_eps"] = 1e-5
    return p


def make_qkv(B: int, H: int, P: int, D: int, mask, *, rng=None, seed: int = 0,
             dtype: str = "f32"):
    """Per-head Q, K, V ~ N(0, 1), shaped (B, H, P, D); padded slots are 0.

    For ``dtype == "bf16"`` the values are rounded to bf16 (RNE) and returned
    as float32 holding bf16-exact values; use :func:`bf16_bits` for storage.
    """
    if rng is None:
        rng = _streams(seed)[2]
    out = []
    keep = (np.asarray(mask) != 0)[:, None, :, None]
    for _ in range(3):
        x = rng.normal(0.0, 1.0, size=(B, H, P, D))
        x = np.where(keep, x, 0.0).astype(np.float32)
        if dtype == "bf16":
            x = bf16_round(x)
        out.append(x)
    return tuple(out)


def make_block_stack(B: int, P: int, C: int, L: int, mask, *, rng=None,
                     seed: int = 0):
    """Residual stream X0 ~ N(0, 1) on real rows (0 on padded rows), shape
    (B, P, C), and per-layer projections Wq, Wk, Wv, Wo ~ N(0, 1/C) (variance
    1/C), each shaped (L, C, C) and applied as ``X @ W``."""
    if rng is None:
        rng = _streams(seed)[3]
    keep = (np.asarray(mask) != 0)[:, :, None]
    x0 = np.where(keep, rng.normal(0.0, 1.0, size=(B, P, C)), 0.0).astype(np.float32)
    std = 1.0 / math.sqrt(C)
    ws = [rng.normal(0.0, std, size=(L, C, C)).astype(np.float32) for _ in range(4)]
    return x0, ws[0], ws[1], ws[2], ws[3]


def make_workload(name: str, seed: int = 0) -> dict:
    """All inputs of a named workload (see ``WORKLOADS``), deterministic in
    ``seed``.  Keys: p4, mask, n, mlp, q, k, v (float32; bf16-exact values for
    bf16 workloads) and, for the block stack, x0, wq, wk, wv, wo."""
    w = WORKLOADS[name]
    kin, mlp_rng, qkv_rng, stack_rng = _streams(seed)
    p4, mask, n = make_jets(w.B, w.P, w.n_min, w.n_max, sigma=w.sigma,
                            massive_frac=w.massive_frac, fixed_n=w.fixed_n,
                            rng=kin)
    out = {"workload": w, "p4": p4, "mask": mask, "n": n,
           "mlp": make_mlp_params(rng=mlp_rng)}
    q, k, v = make_qkv(w.B, w.H, w.P, w.D, mask, rng=qkv_rng, dtype=w.dtype)
    out.update(q=q, k=k, v=v)
    if w.C:
        x0, wq, wk, wv, wo = make_block_stack(w.B, w.P, w.C, w.L, mask, rng=stack_rng)
        out.update(x0=x0, wq=wq, wk=wk, wv=wv, wo=wo)
    return out


# ---------------------------------------------------------------- packed layout
def cu_seqlens(mask) -> np.ndarray:
    """int32 (B + 1) offsets of jets packed back to back, from a mask whose
    real slots are a prefix of each row."""
    n = (np.asarray(mask) != 0).sum(axis=1).astype(np.int64)
    return np.concatenate([[0], np.cumsum(n)]).astype(np.int32)


def pack_rows(x, mask) -> np.ndarray:
    """(B, P, ...) -> (N, ...): the real rows of every jet, back to back
    (prefix masks)."""
    m = np.asarray(mask) != 0
    return np.ascontiguousarray(np.asarray(x)[m])


def pack_heads(x, mask) -> np.ndarray:
    """(B, H, P, D) -> (H, N, D): per head, the real rows of every jet back to
    back (prefix masks)."""
    x = np.asarray(x)
    m = np.asarray(mask) != 0
    return np.ascontiguousarray(np.stack([x[:, h][m] for h in range(x.shape[1])]))


# ---------------------------------------------------------------- L-GATr
def multivectors(shape, rng, scale=1.0) -> np.ndarray:
    """float32 multivectors (*shape, 16), every component N(0, scale^2)
    (hidden-layer activations: all grades populated)."""
    return (rng.normal(0.0, scale, size=tuple(shape) + (16,))).astype(np.float32)


def equilinear_params(in_mv, out_mv, in_s, out_s, rng, biases=True) -> dict:
    """Random float32 weights of an equivariant linear layer, each block
    N(0, 1/fan_in) (fan_in = in_mv + in_s), as keyword arguments of the
    layer's constructors."""
    sd = 1.0 / np.sqrt(max(in_mv + in_s, 1))
    f = lambda *s: rng.normal(0.0, sd, size=s).astype(np.float32)  # noqa: E731
    p = dict(w=f(out_mv, in_mv, 10), s2mv=f(out_mv, in_s), mv2s=f(out_s, in_mv),
             ss=f(out_s, in_s))
    if biases:
        p["b_mv"] = rng.normal(0.0, 0.1, size=out_mv).astype(np.float32)
        p["b_s"] = rng.normal(0.0, 0.1, size=out_s).astype(np.float32)
    return p

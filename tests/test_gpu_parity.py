"""GPU parity: the HIP path (through the C ABI) against the float64 oracle on
the same seeded inputs, element by element.

Bars: float32 |err| <= 1e-4 (1 + |ref|); bfloat16 attention outputs
|err| <= 2e-2 (1 + |ref|); bfloat16 U |err| <= 2e-2 (1 + |ref|) off the
diagonal and <= 3e-2 (1 + |ref|) on diagonal pairs (a == c); every output
that involves a padded slot is +0.0 bit for bit.

The diagonal bf16 U bar follows from the bf16 arithmetic itself: layers 2-4
take bf16 operands (unit roundoff 2^-9), and on diagonal pairs three of the
four features sit at the ln(eps) clamp (-18.4), which drives large
first-layer activations.  tests/test_bf16_bar.py emulates exactly those
roundings in float64 on two of the cases below and reaches 2.4e-2 to
2.7e-2 (1 + |ref|) on the diagonal, below 1.2e-2 elsewhere.  The oracle's
inputs are always the synthetic inputs themselves (bf16 workloads: the
bf16-rounded values), never anything the GPU produced.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from pair_interaction_particle_amd import binding as pip
from pair_interaction_particle_amd import synth

pytestmark = pytest.mark.gpu

TOL32, TOLBF, TOLBF_U = 1e-4, 2e-2, 3e-2


def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda", 0)


def g(x, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x)).to(dev())
    return t if dtype is None else t.to(dtype)


def host(t):
    torch.cuda.synchronize()
    return t.float().cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


def assert_close(got, ref, tol, what):
    got = np.asarray(got, np.float64)
    err = np.abs(got - ref)
    bound = tol * (1.0 + np.abs(ref))
    bad = ~(err <= bound)
    if bad.any():
        idx = np.unravel_index(np.argmax(np.where(bad, err / bound, 0)), ref.shape)
        raise AssertionError("%s: %d of %d beyond tolerance; worst at %s got %r ref %r"
                             % (what, bad.sum(), bad.size, idx, got[idx], ref[idx]))


def assert_close_u_bf16(got, ref, what):
    """bf16 U (B, 8, P, P): the attention bar off the diagonal, the wider
    diagonal bar on pairs a == c."""
    P = ref.shape[-1]
    diag = np.broadcast_to(np.eye(P, dtype=bool), ref.shape)
    assert_close(np.where(diag, 0.0, got), np.where(diag, 0.0, ref), TOLBF,
                 what + " (off the diagonal)")
    assert_close(np.where(diag, got, 0.0), np.where(diag, ref, 0.0), TOLBF_U,
                 what + " (diagonal)")


def assert_zero_bits(t_np, sel, what):
    a = np.ascontiguousarray(t_np)
    bits = a.view(np.uint32) if a.dtype == np.float32 else a.view(np.uint16)
    nz = bits[sel] != 0
    assert not nz.any(), "%s: %d padded entries are not +0.0" % (what, nz.sum())


def pair_mask(mask):
    m = mask.astype(bool)
    return m[:, :, None] & m[:, None, :]


def ragged_jets(B, P, ns, seed, hole=True, sigma=0.4):
    p4, mask, _ = synth.make_jets(B, P, 1, P, fixed_n=tuple(ns), seed=seed, sigma=sigma)
    if hole and B > 0 and ns[0] > 3:
        mask = mask.copy()
        mask[0, 2] = 0  # a non-prefix hole
    return p4, mask


def mlp_for(seed, **kw):
    return synth.make_mlp_params(rng=np.random.default_rng(seed), **kw)


# ---------------------------------------------------------------- features
@pytest.mark.parametrize("B,P,ns", [(2, 16, (11, 16)), (5, 48, (48, 33, 1, 0, 17)),
                                    (2, 256, (256, 131))])
def test_pair_features(B, P, ns):
    p4, mask = ragged_jets(B, P, ns, seed=B * 100 + P)
    F = host(pip.pair_features(g(p4), g(mask)))
    ref = oracle.pair_features(p4, mask)
    real = pair_mask(mask)
    assert_close(F, ref, TOL32, "features")
    assert_zero_bits(F.transpose(0, 2, 3, 1), ~real, "features padding")


# ---------------------------------------------------------------- pair embed
@pytest.mark.parametrize("B,P,ns,kw", [
    (2, 16, (11, 16), {}),
    (6, 64, (64, 50, 17, 16, 1, 0), {"biases": True, "input_bn": True}),
    (3, 256, (256, 200, 33), {"biases": True}),
])
def test_pair_embed_f32_ragged(B, P, ns, kw):
    p4, mask = ragged_jets(B, P, ns, seed=7 + P)
    params = mlp_for(P, **kw)
    mlp = pip.PairMLP(params)
    U = host(pip.pair_embed(g(p4), g(mask), mlp))
    ref = oracle.pair_embed(p4, mask, params)
    assert_close(U, ref, TOL32, "U f32")
    real = pair_mask(mask)
    assert_zero_bits(U.transpose(0, 2, 3, 1), ~real, "U padding")
    np.testing.assert_array_equal(U, U.transpose(0, 1, 3, 2))  # exactly symmetric


def test_pair_embed_f32_kernel_workload():
    d = synth.make_workload("kernel")
    mlp = pip.PairMLP(d["mlp"])
    U = host(pip.pair_embed(g(d["p4"]), g(d["mask"]), mlp))
    ref = oracle.pair_embed(d["p4"], d["mask"], d["mlp"])
    assert_close(U, ref, TOL32, "U f32 (B=128, P=128)")
    assert_zero_bits(U.transpose(0, 2, 3, 1), ~pair_mask(d["mask"]), "U padding")


def test_pair_embed_bf16_large_workload():
    d = synth.make_workload("large_bf16")
    mlp = pip.PairMLP(d["mlp"])
    U = host(pip.pair_embed(g(d["p4"]), g(d["mask"]), mlp, dtype="bf16"))
    ref = oracle.pair_embed(d["p4"], d["mask"], d["mlp"])
    assert_close_u_bf16(U, ref, "U bf16 (B=64, P=256)")
    assert_zero_bits(U.transpose(0, 2, 3, 1), ~pair_mask(d["mask"]), "U bf16 padding")


def test_pair_embed_fp16_overflow_redoes_exactly():
    # One hidden channel of layer 1 is driven to ~8e4 (beyond fp16) through a
    # large bias but read out through tiny layer-2 weights, so the problem
    # stays well conditioned while the fp16 x 2 chain overflows; the folded
    # weights are well scaled, so that chain is the one chosen.  The affected
    # waves must redo their share with the exact float32 chain.
    p4, mask = ragged_jets(3, 48, (48, 30, 17), seed=21)
    params = mlp_for(21, biases=True)
    params["b1"] = params["b1"].copy()
    params["b1"][5] = 8.0e4
    params["w2"] = params["w2"].copy()
    params["w2"][:, 5] = 1.0e-5
    ws = pip.fold(params)[0]
    assert all(2 ** -8 <= np.abs(w).max() <= 2 ** 14 for w in ws[1:])
    assert np.abs(ws[0][5]).max() < 1.0 and pip.fold(params)[1][0][5] > 65504.0 / 3
    mlp = pip.PairMLP(params)
    U = host(pip.pair_embed(g(p4), g(mask), mlp))
    ref = oracle.pair_embed(p4, mask, params)
    assert_close(U, ref, TOL32, "U f32 with an fp16-overflowing hidden channel")


def test_pair_embed_badly_scaled_weights_use_exact_chain():
    # layer 3 x 1e5 and layer 4 x 1e-5: far outside the well-scaled range, so
    # the exact float32 chain runs; U stays O(1) and well conditioned.
    p4, mask = ragged_jets(2, 32, (32, 19), seed=22)
    params = mlp_for(22)
    params["w3"] = (params["w3"] * 1e5).astype(np.float32)
    params["w4"] = (params["w4"] * 1e-5).astype(np.float32)
    mlp = pip.PairMLP(params)
    U = host(pip.pair_embed(g(p4), g(mask), mlp))
    ref = oracle.pair_embed(p4, mask, params)
    assert_close(U, ref, TOL32, "U f32 with badly scaled weights")


def test_pair_embed_ignores_padding_values():
    p4, mask = ragged_jets(3, 32, (20, 32, 9), seed=3)
    params = mlp_for(3, biases=True)
    mlp = pip.PairMLP(params)
    U0 = host(pip.pair_embed(g(p4), g(mask), mlp))
    bad = p4.copy()
    bad[mask == 0] = np.nan
    bad[2, 30] = [1e30, -1e30, 3e29, -7e29]
    U1 = host(pip.pair_embed(g(bad), g(mask), mlp))
    np.testing.assert_array_equal(U1.view(np.uint32), U0.view(np.uint32))


# ---------------------------------------------------------------- attention
def rand_qkv(B, H, P, mask, seed, dtype="f32"):
    return synth.make_qkv(B, H, P, 16, mask, rng=np.random.default_rng(seed), dtype=dtype)


@pytest.mark.parametrize("B,H,P,ns", [(2, 8, 16, (11, 16)), (5, 3, 48, (48, 33, 1, 0, 17)),
                                      (2, 8, 256, (256, 77))])
def test_attention_f32_ragged(B, H, P, ns):
    _, mask = ragged_jets(B, P, ns, seed=P)
    q, k, v = rand_qkv(B, H, P, mask, seed=P)
    u = np.random.default_rng(P + 1).normal(0, 1.5, size=(B, H, P, P)).astype(np.float32)
    O = host(pip.pair_bias_attention(g(q), g(k), g(v), g(u), g(mask)))
    ref = oracle.attention(q, k, v, u, mask)
    assert_close(O, ref, TOL32, "O f32")
    assert_zero_bits(O.transpose(0, 2, 1, 3), mask == 0, "O padded rows")


def test_attention_f32_kernel_workload_with_oracle_bias():
    d = synth.make_workload("kernel")
    U = oracle.pair_embed(d["p4"], d["mask"], d["mlp"]).astype(np.float32)
    O = host(pip.pair_bias_attention(g(d["q"]), g(d["k"]), g(d["v"]), g(U), g(d["mask"])))
    ref = oracle.attention(d["q"], d["k"], d["v"], U, d["mask"])
    assert_close(O, ref, TOL32, "O f32 (B=128, P=128)")
    assert_zero_bits(O.transpose(0, 2, 1, 3), d["mask"] == 0, "O padded rows")


def test_attention_bf16_large_workload():
    d = synth.make_workload("large_bf16")
    U = synth.bf16_round(oracle.pair_embed(d["p4"], d["mask"], d["mlp"]).astype(np.float32))
    bf = torch.bfloat16
    O = host(pip.pair_bias_attention(g(d["q"], bf), g(d["k"], bf), g(d["v"], bf), g(U, bf),
                                     g(d["mask"])))
    ref = oracle.attention(d["q"], d["k"], d["v"], U, d["mask"])
    assert_close(O, ref, TOLBF, "O bf16 (B=64, P=256)")
    assert_zero_bits(O.transpose(0, 2, 1, 3), d["mask"] == 0, "O bf16 padded rows")


def assert_close_v_scaled(O, ref, lam, tol, what):
    """Attention is linear in V: O(Q, K, lam V, U) = lam O(Q, K, V, U).  For V
    scaled by lam per jet the bar is applied to the problem with V unscaled,
    i.e. to O / lam (a cancellation inside a sum of values of size lam is
    not an O(1) problem)."""
    lam = np.asarray(lam, np.float64)[:, None, None, None]
    assert_close(np.asarray(O, np.float64) / lam, ref / lam, tol, what)


def test_attention_f32_values_beyond_fp16_range():
    # jet 0: K x 1e5 and Q x 1e-5 (scores unchanged); jet 1: V x 1e5; jet 2:
    # Q x 1e5 and K x 1e-5.  Each puts real Q, K or V values beyond the fp16
    # range; the per-head (K, V) and per-row (Q) powers of two bring them
    # back before the fp16 split.
    B, H, P = 3, 2, 48
    _, mask = ragged_jets(B, P, (48, 30, 17), seed=31)
    q, k, v = rand_qkv(B, H, P, mask, seed=31)
    k[0] *= 1e5
    q[0] *= 1e-5
    v[1] *= 1e5
    q[2] *= 1e5
    k[2] *= 1e-5
    u = np.random.default_rng(32).normal(0, 1.5, size=(B, H, P, P)).astype(np.float32)
    O = host(pip.pair_bias_attention(g(q), g(k), g(v), g(u), g(mask)))
    ref = oracle.attention(q, k, v, u, mask)
    assert_close_v_scaled(O, ref, [1.0, 1e5, 1.0], TOL32, "O f32 with values beyond fp16")
    assert_zero_bits(O.transpose(0, 2, 1, 3), mask == 0, "O padded rows")


@pytest.mark.parametrize("P", [128, 256])
def test_attention_f32_imbalanced_magnitudes_inside_fp16_range(P):
    # Every value stays inside the fp16 range, but a plain hi + lo split of the
    # small operand would fall into fp16 subnormals (absolute quantum 2^-24):
    # jet 0: Q x 2^-13, K x 2^13; jet 1: Q x 2^13, K x 2^-13 (scores
    # unchanged); jet 2: every Q row and K row of head 0 scaled by its own
    # power of two in [2^-12, 2^12] (the scores then span many magnitudes) and
    # V x 2^-14; jet 3: V x 2^13.
    B, H = 4, 8
    _, mask = ragged_jets(B, P, (P, P - 37, P // 2 + 3, 70), seed=33 + P)
    q0, k0, v0 = rand_qkv(B, H, P, mask, seed=33 + P)
    q, k, v = q0.copy(), k0.copy(), v0.copy()
    q[0] *= 2.0 ** -13
    k[0] *= 2.0 ** 13
    q[1] *= 2.0 ** 13
    k[1] *= 2.0 ** -13
    rng = np.random.default_rng(34 + P)
    q[2, 0] *= (2.0 ** rng.integers(-12, 13, size=P))[:, None]
    k[2, 0] *= (2.0 ** rng.integers(-12, 13, size=P))[:, None]
    v[2] *= 2.0 ** -14
    v[3] *= 2.0 ** 13
    assert max(np.abs(x).max() for x in (q, k, v)) < 65504.0
    u = np.random.default_rng(35 + P).normal(0, 1.5, size=(B, H, P, P)).astype(np.float32)
    O = host(pip.pair_bias_attention(g(q), g(k), g(v), g(u), g(mask)))
    ref = oracle.attention(q, k, v, u, mask)
    assert_close_v_scaled(O, ref, [1.0, 1.0, 2.0 ** -14, 2.0 ** 13], TOL32,
                          "O f32 imbalanced magnitudes P=%d" % P)
    assert_zero_bits(O.transpose(0, 2, 1, 3), mask == 0, "O padded rows")
    # Powers of two are normalised away exactly (Q per row, K and V per head):
    # jets 0 and 1 give the unscaled inputs' result bit for bit, jet 3 that
    # result times 2^13.
    O0 = host(pip.pair_bias_attention(g(q0), g(k0), g(v0), g(u), g(mask)))
    np.testing.assert_array_equal(O[:2].view(np.uint32), O0[:2].view(np.uint32))
    np.testing.assert_array_equal(O[3], O0[3] * np.float32(2.0 ** 13))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_attention_and_fused_with_a_non_default_scale(dtype):
    # the score scale is an argument of the boundary; 0.1 and -0.37 through
    # the ABI against the oracle with the same scale
    B, P = 3, 64
    p4, mask = ragged_jets(B, P, (64, 41, 9), seed=36)
    params = mlp_for(36, biases=True)
    mlp = pip.PairMLP(params)
    q, k, v = rand_qkv(B, 8, P, mask, seed=36, dtype=dtype)
    tt = torch.bfloat16 if dtype == "bf16" else None
    tol = TOLBF if dtype == "bf16" else TOL32
    Uref = oracle.pair_embed(p4, mask, params).astype(np.float32)
    if dtype == "bf16":
        Uref = synth.bf16_round(Uref)
    for sc in (0.1, -0.37):
        O = host(pip.pair_bias_attention(g(q, tt), g(k, tt), g(v, tt), g(Uref, tt), g(mask),
                                         scale=sc))
        assert_close(O, oracle.attention(q, k, v, Uref, mask, scale=sc), tol,
                     "O %s scale %g" % (dtype, sc))
        O2 = host(pip.pair_embed_attention(g(p4), g(mask), mlp, g(q, tt), g(k, tt), g(v, tt),
                                           scale=sc))
        assert_close(O2, oracle.pair_embed_attention(p4, mask, params, q, k, v, scale=sc), tol,
                     "fused O %s scale %g" % (dtype, sc))
        assert_zero_bits(O2.transpose(0, 2, 1, 3), mask == 0, "fused padded rows")


def test_attention_ignores_padding_values_and_empty_jets():
    B, H, P = 3, 8, 32
    _, mask = ragged_jets(B, P, (20, 0, 9), seed=5)
    q, k, v = rand_qkv(B, H, P, mask, seed=5)
    u = np.random.default_rng(6).normal(0, 1, size=(B, H, P, P)).astype(np.float32)
    O0 = host(pip.pair_bias_attention(g(q), g(k), g(v), g(u), g(mask)))
    q2, k2, v2, u2 = (x.copy() for x in (q, k, v, u))
    pad = mask == 0
    for x in (q2, k2, v2):
        x[pad[:, None, :, None].repeat(H, 1).repeat(16, 3)] = np.nan
    u2[np.broadcast_to(pad[:, None, None, :], u2.shape)] = 1e30
    u2[np.broadcast_to(pad[:, None, :, None], u2.shape)] = np.nan
    O1 = host(pip.pair_bias_attention(g(q2), g(k2), g(v2), g(u2), g(mask)))
    np.testing.assert_array_equal(O1.view(np.uint32), O0.view(np.uint32))
    assert np.all(O0.view(np.uint32)[1] == 0)  # the all-padded jet


def test_embed_then_attention_chain_f32():
    d = synth.make_workload("tiny")
    mlp = pip.PairMLP(d["mlp"])
    U = pip.pair_embed(g(d["p4"]), g(d["mask"]), mlp)
    O = host(pip.pair_bias_attention(g(d["q"]), g(d["k"]), g(d["v"]), U, g(d["mask"])))
    ref = oracle.pair_embed_attention(d["p4"], d["mask"], d["mlp"], d["q"], d["k"], d["v"])
    assert_close(O, ref, TOL32, "embed -> attention (tiny)")


def test_empty_batch_is_a_noop():
    mlp = pip.PairMLP(mlp_for(1))
    p4 = torch.zeros((0, 16, 4), device=dev())
    mask = torch.zeros((0, 16), device=dev(), dtype=torch.uint8)
    U = pip.pair_embed(p4, mask, mlp)
    assert U.shape == (0, 8, 16, 16)


# ---------------------------------------------------------------- edge shapes
@pytest.mark.parametrize("H", [1, 5, 16])
def test_attention_f32_head_counts(H):
    B, P = 3, 32
    _, mask = ragged_jets(B, P, (32, 17, 3), seed=40 + H)
    q, k, v = rand_qkv(B, H, P, mask, seed=40 + H)
    u = np.random.default_rng(41 + H).normal(0, 1, size=(B, H, P, P)).astype(np.float32)
    O = host(pip.pair_bias_attention(g(q), g(k), g(v), g(u), g(mask)))
    ref = oracle.attention(q, k, v, u, mask)
    assert_close(O, ref, TOL32, "O f32 H=%d" % H)
    assert_zero_bits(O.transpose(0, 2, 1, 3), mask == 0, "O padded rows")


@pytest.mark.parametrize("B,P,ns", [(3, 48, (48, 20, 1)), (1, 256, (256,)), (2, 144, (144, 0))])
def test_pair_embed_bf16_ragged(B, P, ns):
    p4, mask = ragged_jets(B, P, ns, seed=50 + P)
    params = mlp_for(50 + P, biases=True)
    mlp = pip.PairMLP(params)
    U = host(pip.pair_embed(g(p4), g(mask), mlp, dtype="bf16"))
    ref = oracle.pair_embed(p4, mask, params)
    assert_close_u_bf16(U, ref, "U bf16 P=%d" % P)
    assert_zero_bits(U.transpose(0, 2, 3, 1), ~pair_mask(mask), "U bf16 padding")


def test_pair_embed_across_launch_segments():
    # more than 65,536 jets: the launcher cuts the batch into segments (p4,
    # mask and U offset per segment); the jets on both sides of the cut and a
    # few early ones are compared with the oracle (each jet is independent)
    B, P = 65536 + 40, 16
    rng = np.random.default_rng(91)
    ns = tuple(int(x) for x in rng.integers(0, 5, size=B))
    p4, mask = ragged_jets(B, P, ns, seed=91, hole=False)
    params = mlp_for(91, biases=True)
    mlp = pip.PairMLP(params)
    Ud = pip.pair_embed(g(p4), g(mask), mlp)
    sel = np.r_[0:24, 65536 - 24:B]
    U = host(Ud[torch.from_numpy(sel).cuda()])
    ref = oracle.pair_embed(p4[sel], mask[sel], params)
    assert_close(U, ref, TOL32, "U across the 65,536-jet segment boundary")
    assert_zero_bits(U, np.broadcast_to(~pair_mask(mask[sel])[:, None], U.shape), "U padded pairs")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_pair_embed_more_jets_than_threads(dtype):
    # B > 512: each entry of the in-kernel cost scan covers a range of jets, the
    # split points are walked from the range start, and the zero tiles read
    # jet activity from the mask (empty jets and holes included)
    B, P = 1300, 32
    rng = np.random.default_rng(81)
    ns = tuple(int(x) for x in rng.integers(0, P + 1, size=B))
    p4, mask = ragged_jets(B, P, ns, seed=81)
    params = mlp_for(81, biases=True)
    mlp = pip.PairMLP(params)
    U = host(pip.pair_embed(g(p4), g(mask), mlp, dtype=dtype))
    ref = oracle.pair_embed(p4, mask, params)
    if dtype == "f32":
        assert_close(U, ref, TOL32, "U f32 B=1300")
    else:
        assert_close_u_bf16(U, ref, "U bf16 B=1300")
    assert_zero_bits(U.transpose(0, 2, 3, 1), ~pair_mask(mask), "U %s B=1300 padding" % dtype)


def test_single_full_jet_at_max_p_every_entry():
    B, P = 1, 256
    p4, mask = ragged_jets(B, P, (256,), seed=60, hole=False)
    params = mlp_for(60)
    mlp = pip.PairMLP(params)
    q, k, v = rand_qkv(B, 8, P, mask, seed=60)
    U = host(pip.pair_embed(g(p4), g(mask), mlp))
    assert_close(U, oracle.pair_embed(p4, mask, params), TOL32, "U P=256")
    O = host(pip.pair_bias_attention(g(q), g(k), g(v), g(U), g(mask)))
    ref = oracle.pair_embed_attention(p4, mask, params, q, k, v)
    assert_close(O, ref, TOL32, "O P=256")
    O2 = host(pip.pair_embed_attention(g(p4), g(mask), mlp, g(q), g(k), g(v)))
    assert_close(O2, ref, TOL32, "fused O P=256")


# ---------------------------------------------------------------- masks that are not prefixes
def scattered_mask(B, P, seed):
    """Jet 0: a random half of the slots; jet 1: odd slots only; jet 2: the
    last 40 slots; jet 3: two slots far apart (the rest of a jet is padding)."""
    assert B == 4
    m = np.zeros((B, P), dtype=np.uint8)
    m[0, np.random.default_rng(seed).random(P) < 0.5] = 1
    m[1, 1::2] = 1
    m[2, P - 40:] = 1
    m[3, [5, P - 8]] = 1
    return m


@pytest.mark.parametrize("P", [128, 160])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_scattered_masks_every_entry(dtype, P):
    # Work estimates and fast paths assume real slots first; any other layout
    # may only move split points, never change a result.  Padded particles keep
    # non-zero values, which every entry must ignore.
    B = 4
    mask = scattered_mask(B, P, seed=P)
    p4, _ = ragged_jets(B, P, (P,) * B, seed=90 + P, hole=False)
    params = mlp_for(90 + P, biases=True)
    mlp = pip.PairMLP(params)
    bf = dtype == "bf16"
    tt = torch.bfloat16 if bf else None
    real = pair_mask(mask)
    what = "%s P=%d scattered" % (dtype, P)

    U = host(pip.pair_embed(g(p4), g(mask), mlp, dtype=dtype))
    Uref = oracle.pair_embed(p4, mask, params)
    if bf:
        assert_close_u_bf16(U, Uref, "U " + what)
    else:
        assert_close(U, Uref, TOL32, "U " + what)
    assert_zero_bits(U.transpose(0, 2, 3, 1), ~real, "U padding " + what)

    q, k, v = rand_qkv(B, 8, P, mask, seed=91 + P, dtype=dtype)
    Uin = Uref.astype(np.float32)
    if bf:
        Uin = synth.bf16_round(Uin)
    O = host(pip.pair_bias_attention(g(q, tt), g(k, tt), g(v, tt), g(Uin, tt), g(mask)))
    assert_close(O, oracle.attention(q, k, v, Uin, mask), TOLBF if bf else TOL32, "O " + what)
    assert_zero_bits(O.transpose(0, 2, 1, 3), mask == 0, "O padded rows " + what)

    O2 = host(pip.pair_embed_attention(g(p4), g(mask), mlp, g(q, tt), g(k, tt), g(v, tt)))
    ref2 = oracle.pair_embed_attention(p4, mask, params, q, k, v)
    assert_close(O2, ref2, TOLBF if bf else TOL32, "fused O " + what)
    assert_zero_bits(O2.transpose(0, 2, 1, 3), mask == 0, "fused O padded rows " + what)

    if not bf:
        F = host(pip.pair_features(g(p4), g(mask)))
        assert_close(F, oracle.pair_features(p4, mask), TOL32, "features " + what)
        assert_zero_bits(F.transpose(0, 2, 3, 1), ~real, "features padding " + what)
        x0, wq, wk, wv, wo = synth.make_block_stack(B, P, 128, 2, mask,
                                                    rng=np.random.default_rng(92 + P))
        X = g(x0)
        pip.block_stack(X, g(wq), g(wk), g(wv), g(wo), g(Uin), g(mask))
        got = host(X)
        ref = oracle.block_stack(x0, wq, wk, wv, wo, Uin, mask)
        sel = mask != 0
        assert_close(got[sel], ref[sel], TOL32, "block stack X " + what)
        np.testing.assert_array_equal(got[~sel].view(np.uint32), x0[~sel].view(np.uint32))


# ---------------------------------------------------------------- beam-axis particles
def beam_axis_jets(P, seed):
    """Three jets with particles on the beam axis (pT = 0): massless forward
    and backward (E = |pz|, the rapidity floor), massive ones (finite y),
    one with E < |pz|, and a jet whose only real particles all have pT = 0
    (the pT sum in ln z clamped at eps)."""
    p4, mask = ragged_jets(3, P, (P, P - 20, 5), seed=seed, hole=False)
    p4 = p4.copy()
    p4[0, 3] = [7.0, 0.0, 0.0, 7.0]
    p4[0, 10] = [2.5, 0.0, 0.0, -2.5]
    p4[0, P - 1] = [5.0, 0.0, 0.0, 3.0]
    p4[1, 0] = [1.0, 0.0, 0.0, 2.0]
    p4[1, 7] = [40.0, 0.0, 0.0, -40.0]
    p4[2, :5] = [[5.0, 0.0, 0.0, 3.0], [5.0, 0.0, 0.0, -4.0], [9.0, 0.0, 0.0, 9.0],
                 [3.0, 0.0, 0.0, -3.0], [2.0, 0.0, 0.0, 1.0]]
    return p4, mask


@pytest.mark.parametrize("P", [32, 144])
def test_beam_axis_particles_every_entry(P):
    p4, mask = beam_axis_jets(P, seed=70 + P)
    params = mlp_for(70 + P, biases=True)
    mlp = pip.PairMLP(params)
    real = pair_mask(mask)
    F = host(pip.pair_features(g(p4), g(mask)))
    Fref = oracle.pair_features(p4, mask)
    assert np.all(np.isfinite(Fref))
    assert_close(F, Fref, TOL32, "features beam axis P=%d" % P)
    assert_zero_bits(F.transpose(0, 2, 3, 1), ~real, "features padding")
    Uref = oracle.pair_embed(p4, mask, params)
    for dtype in ("f32", "bf16"):
        U = host(pip.pair_embed(g(p4), g(mask), mlp, dtype=dtype))
        if dtype == "f32":
            assert_close(U, Uref, TOL32, "U f32 beam axis P=%d" % P)
        else:
            assert_close_u_bf16(U, Uref, "U bf16 beam axis P=%d" % P)
        assert_zero_bits(U.transpose(0, 2, 3, 1), ~real, "U padding")
    q, k, v = rand_qkv(3, 8, P, mask, seed=71 + P)
    O = host(pip.pair_embed_attention(g(p4), g(mask), mlp, g(q), g(k), g(v)))
    assert_close(O, oracle.pair_embed_attention(p4, mask, params, q, k, v), TOL32,
                 "fused O beam axis P=%d" % P)

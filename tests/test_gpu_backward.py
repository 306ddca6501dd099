"""GPU parity of the backward pass (through the C ABI) against the float64
oracle: the biased attention's dQ, dK, dV, dU, and the pair MLP's parameter
gradients (folded on the GPU, unfolded to the raw parameters on the host).

Bars: float32 |err| <= 1e-4 (1 + |ref|) for the attention gradients (each a
sum over at most 256 keys or queries); every entry that involves a padded
slot is +0.0 bit for bit, and padded inputs (dO and dU included) never reach
a result.  The MLP gradients are sums over up to ~10^6 ordered pairs of
terms of both signs; float32 summation of N terms carries an error of order
N u max|term| in the worst case, so their bar is stated relative to the
tensor's scale: |err| <= 1e-4 (1 + |ref|) + 1e-5 max|ref|.  Every sum is
taken in a fixed order, so repeated runs agree bit for bit (checked)."""
import numpy as np
import pytest
import torch

import oracle
from pair_interaction_particle_amd import binding as pip
from pair_interaction_particle_amd import synth
from test_gpu_parity import (TOL32, assert_close, assert_zero_bits, g, host, mlp_for,
                             pair_mask, ragged_jets, rand_qkv)

pytestmark = pytest.mark.gpu


def check_grads(got, ref, what):
    for name in got:
        r = ref[name]
        bound = 1e-4 * (1.0 + np.abs(r)) + 1e-5 * np.abs(r).max()
        err = np.abs(got[name].astype(np.float64) - r)
        bad = ~(err <= bound)
        assert not bad.any(), "%s %s: %d beyond, worst err %g (bound %g, ref %g)" % (
            what, name, bad.sum(), err.max(), bound[np.unravel_index(err.argmax(), err.shape)],
            r.reshape(-1)[err.argmax()])


def attn_inputs(B, H, P, ns, seed):
    _, mask = ragged_jets(B, P, ns, seed=seed)
    q, k, v = rand_qkv(B, H, P, mask, seed=seed)
    rng = np.random.default_rng(seed + 1)
    u = rng.normal(0, 1.5, size=(B, H, P, P)).astype(np.float32)
    dO = rng.normal(0, 1, size=(B, H, P, 16)).astype(np.float32)
    dO[np.broadcast_to((mask == 0)[:, None, :, None], dO.shape)] = 0.0
    return q, k, v, u, dO, mask


@pytest.mark.parametrize("B,H,P,ns", [(2, 8, 16, (11, 16)), (5, 3, 48, (48, 33, 1, 0, 17)),
                                      (2, 8, 256, (256, 77)), (3, 1, 144, (144, 130, 5))])
def test_attention_backward_ragged(B, H, P, ns):
    q, k, v, u, dO, mask = attn_inputs(B, H, P, ns, seed=200 + P)
    got = [host(x) for x in pip.pair_bias_attention_backward(g(q), g(k), g(v), g(u), g(mask),
                                                             g(dO))]
    ref = oracle.attention_backward(q, k, v, u, mask, dO)
    for name, a, r in zip(("dQ", "dK", "dV", "dU"), got, ref):
        assert_close(a, r, TOL32, "%s P=%d" % (name, P))
    for name, a in zip(("dQ", "dK", "dV"), got[:3]):
        assert_zero_bits(a.transpose(0, 2, 1, 3), mask == 0, name + " padded rows")
    assert_zero_bits(got[3].transpose(0, 2, 3, 1), ~pair_mask(mask), "dU padded pairs")


def test_attention_backward_ignores_padding_and_takes_the_scale():
    B, H, P = 3, 4, 32
    q, k, v, u, dO, mask = attn_inputs(B, H, P, (20, 0, 32), seed=211)
    base = [host(x) for x in pip.pair_bias_attention_backward(
        g(q), g(k), g(v), g(u), g(mask), g(dO), scale=0.3)]
    ref = oracle.attention_backward(q, k, v, u, mask, dO, scale=0.3)
    for name, a, r in zip(("dQ", "dK", "dV", "dU"), base, ref):
        assert_close(a, r, TOL32, name + " scale 0.3")
    pad = mask == 0
    q2, k2, v2, u2, d2 = (x.copy() for x in (q, k, v, u, dO))
    for x in (q2, k2, v2, d2):
        x[np.broadcast_to(pad[:, None, :, None], x.shape)] = np.nan
    u2[np.broadcast_to(pad[:, None, None, :], u2.shape)] = 1e30
    u2[np.broadcast_to(pad[:, None, :, None], u2.shape)] = np.nan
    again = [host(x) for x in pip.pair_bias_attention_backward(
        g(q2), g(k2), g(v2), g(u2), g(mask), g(d2), scale=0.3)]
    for a, b in zip(base, again):
        np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))


def test_attention_backward_kernel_workload():
    d = synth.make_workload("kernel")
    mask = d["mask"]
    U = oracle.pair_embed(d["p4"], mask, d["mlp"]).astype(np.float32)
    rng = np.random.default_rng(212)
    dO = rng.normal(0, 1, size=d["q"].shape).astype(np.float32)
    got = [host(x) for x in pip.pair_bias_attention_backward(
        g(d["q"]), g(d["k"]), g(d["v"]), g(U), g(mask), g(dO))]
    ref = oracle.attention_backward(d["q"], d["k"], d["v"], U, mask, dO)
    for name, a, r in zip(("dQ", "dK", "dV", "dU"), got, ref):
        assert_close(a, r, TOL32, name + " (B=128, P=128)")
    assert_zero_bits(got[3].transpose(0, 2, 3, 1), ~pair_mask(mask), "dU padded pairs")
    # every sum is taken in a fixed order: a second run is the same bit for bit
    again = [host(x) for x in pip.pair_bias_attention_backward(
        g(d["q"]), g(d["k"]), g(d["v"]), g(U), g(mask), g(dO))]
    for a, b in zip(got, again):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("B,P,ns,kw", [(3, 32, (32, 19, 0), {"biases": True}),
                                       (2, 48, (48, 37), {"biases": True, "input_bn": True}),
                                       (1, 256, (200,), {})])
def test_pair_mlp_backward_ragged(B, P, ns, kw):
    p4, mask = ragged_jets(B, P, ns, seed=220 + P)
    params = mlp_for(220 + P, **kw)
    mlp = pip.PairMLP(params)
    rng = np.random.default_rng(221 + P)
    dU = rng.normal(0, 1, size=(B, 8, P, P)).astype(np.float32)
    gf = host(pip.pair_mlp_backward(g(p4), g(mask), mlp, g(dU)))
    got = pip.unfold_grads(params, gf)
    ref = oracle.pair_embed_backward(p4, mask, params, dU)
    if "input_bn" not in kw:
        got = {k: v for k, v in got.items() if not k.startswith("in_")}
    check_grads(got, ref, "MLP grads P=%d" % P)
    # padded entries of dU are never read: NaN there changes nothing, bit for
    # bit (every sum is taken in a fixed order)
    dU2 = dU.copy()
    dU2[~np.broadcast_to(pair_mask(mask)[:, None], dU2.shape)] = np.nan
    gf2 = host(pip.pair_mlp_backward(g(p4), g(mask), mlp, g(dU2)))
    assert np.array_equal(gf2.view(np.uint32), gf.view(np.uint32))


def test_pair_mlp_backward_kernel_workload():
    d = synth.make_workload("kernel")
    mask = d["mask"]
    mlp = pip.PairMLP(d["mlp"])
    rng = np.random.default_rng(230)
    dU = rng.normal(0, 1, size=(128, 8, 128, 128)).astype(np.float32)
    gf = host(pip.pair_mlp_backward(g(d["p4"]), g(mask), mlp, g(dU)))
    got = {k: v for k, v in pip.unfold_grads(d["mlp"], gf).items() if not k.startswith("in_")}
    ref = oracle.pair_embed_backward(d["p4"], mask, d["mlp"], dU)
    check_grads(got, ref, "MLP grads (B=128, P=128)")
    gf2 = host(pip.pair_mlp_backward(g(d["p4"]), g(mask), mlp, g(dU)))
    assert np.array_equal(gf2.view(np.uint32), gf.view(np.uint32))


def _redo_flags(ws, B, P):
    # after the partial sums (one per slot, one per fp16 x 2 workgroup, the
    # chunk sums) the workspace holds one int per fp16 x 2 workgroup: 1 where
    # its sums left the fp16 range (then float32 recomputes the gradient)
    slots = B * (P // 16)
    gx = 16 * slots if slots < 16 else 256
    G = min(gx, torch.cuda.get_device_properties(0).multi_processor_count)
    chunks = (max(slots, gx) + 31) // 32
    flat = host(ws).view(np.int32)
    off = (slots + gx + chunks) * 9160
    return flat[off:off + G]


def _ws(B, P):
    n = int(pip.lib().pip_pair_mlp_backward_workspace_bytes(B, P))
    return torch.empty(n // 4, device="cuda", dtype=torch.float32)


def test_pair_mlp_backward_fp16_path_is_taken_and_scale_equivariant():
    # Well-scaled weights take the fp16 x 2 kernel, and no slot of this input
    # needs the float32 redo.  g is scaled per round by a power of two, so
    # scaling dU by 2^40 or 2^-40 scales the gradient by exactly that factor,
    # bit for bit.
    B, P = 3, 48
    p4, mask = ragged_jets(B, P, (48, 37, 9), seed=240)
    params = mlp_for(240, biases=True)
    mlp = pip.PairMLP(params)
    rng = np.random.default_rng(241)
    dU = rng.normal(0, 1, size=(B, 8, P, P)).astype(np.float32)
    ws = _ws(B, P)
    gf = host(pip.pair_mlp_backward(g(p4), g(mask), mlp, g(dU), workspace=ws))
    assert not _redo_flags(ws, B, P).any()
    got = {k: v for k, v in pip.unfold_grads(params, gf).items() if not k.startswith("in_")}
    check_grads(got, oracle.pair_embed_backward(p4, mask, params, dU), "MLP grads fp16 x 2")
    for k in (40, -40):
        s = np.float32(2.0 ** k)
        gk = host(pip.pair_mlp_backward(g(p4), g(mask), mlp, g(dU * s), workspace=ws))
        assert not _redo_flags(ws, B, P).any()
        np.testing.assert_array_equal((gf * s).view(np.uint32), gk.view(np.uint32))


def test_pair_mlp_backward_fp16_overflow_redoes_exactly():
    # One hidden channel of layer 1 at ~8e4 (beyond fp16), read out through
    # tiny layer-2 weights: the folded weights are well scaled, so the fp16 x 2
    # kernel runs, its sums for the real slots come out non-finite, and those
    # slots are recomputed with float32 products.
    B, P = 3, 48
    p4, mask = ragged_jets(B, P, (48, 30, 17), seed=242)
    params = mlp_for(242, biases=True)
    params["b1"] = params["b1"].copy()
    params["b1"][5] = 8.0e4
    params["w2"] = params["w2"].copy()
    params["w2"][:, 5] = 1.0e-5
    ws_f = pip.fold(params)[0]
    assert all(2 ** -8 <= np.abs(w).max() <= 2 ** 14 for w in ws_f[1:])
    mlp = pip.PairMLP(params)
    rng = np.random.default_rng(243)
    dU = rng.normal(0, 1, size=(B, 8, P, P)).astype(np.float32)
    ws = _ws(B, P)
    gf = host(pip.pair_mlp_backward(g(p4), g(mask), mlp, g(dU), workspace=ws))
    assert _redo_flags(ws, B, P).any()
    got = {k: v for k, v in pip.unfold_grads(params, gf).items() if not k.startswith("in_")}
    check_grads(got, oracle.pair_embed_backward(p4, mask, params, dU), "MLP grads, redo")


def test_pair_mlp_backward_badly_scaled_weights():
    # weights outside the fp16 range: every slot takes float32 products
    B, P = 2, 32
    p4, mask = ragged_jets(B, P, (32, 19), seed=244)
    params = mlp_for(244)
    params["w3"] = (params["w3"] * 1e5).astype(np.float32)
    params["w4"] = (params["w4"] * 1e-5).astype(np.float32)
    mlp = pip.PairMLP(params)
    rng = np.random.default_rng(245)
    dU = rng.normal(0, 1, size=(B, 8, P, P)).astype(np.float32)
    gf = host(pip.pair_mlp_backward(g(p4), g(mask), mlp, g(dU)))
    got = {k: v for k, v in pip.unfold_grads(params, gf).items() if not k.startswith("in_")}
    check_grads(got, oracle.pair_embed_backward(p4, mask, params, dU), "MLP grads, f32 weights")

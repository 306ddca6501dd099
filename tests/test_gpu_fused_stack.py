"""GPU parity of the fused pair_embed_attention entry and of the block stack
against the float64 oracle (through the C ABI).  Bars as in
test_gpu_parity.py: float32 |err| <= 1e-4 (1 + |ref|), bfloat16
<= 2e-2 (1 + |ref|), padded outputs exactly +0.0."""
import numpy as np
import pytest
import torch

import oracle
from pair_interaction_particle_amd import binding as pip
from pair_interaction_particle_amd import synth
from test_gpu_parity import (TOL32, TOLBF, assert_close, assert_zero_bits, g, host, mlp_for,
                             ragged_jets, rand_qkv)

pytestmark = pytest.mark.gpu


def with_empty_jets(B, ns):
    """Append empty jets until the batch is more than half the CU count: the
    fused entry then takes the jet kernel at P <= 128 (smaller batches take
    the row kernel)."""
    extra = max(0, torch.cuda.get_device_properties(0).multi_processor_count // 2 + 1 - B)
    return B + extra, tuple(ns) + (0,) * extra


@pytest.mark.parametrize("fill", [False, True])  # True: padded to the jet kernel's batch sizes
@pytest.mark.parametrize("B,P,ns", [
    (2, 16, (11, 16)),
    (6, 64, (64, 50, 17, 16, 1, 0)),   # ragged, empty jet, hole
    (3, 128, (128, 20, 77)),           # the jet kernel's largest P
    (3, 256, (256, 131, 0)),           # row kernel only (P > 128)
    (2, 144, (144, 40)),               # row kernel only, odd block count
])
def test_fused_f32(B, P, ns, fill):
    seed = P + B
    if fill:
        B, ns = with_empty_jets(B, ns)
    p4, mask = ragged_jets(B, P, ns, seed=seed)
    params = mlp_for(P, biases=True, input_bn=(P == 64))
    q, k, v = rand_qkv(B, 8, P, mask, seed=P)
    mlp = pip.PairMLP(params)
    O = host(pip.pair_embed_attention(g(p4), g(mask), mlp, g(q), g(k), g(v)))
    ref = oracle.pair_embed_attention(p4, mask, params, q, k, v)
    assert_close(O, ref, TOL32, "fused O f32 P=%d" % P)
    assert_zero_bits(O.transpose(0, 2, 1, 3), mask == 0, "fused O padded rows")


@pytest.mark.parametrize("fill", [False, True])
@pytest.mark.parametrize("B,P,ns", [(4, 128, (128, 60, 9, 100)), (2, 256, (256, 90))])
def test_fused_bf16(B, P, ns, fill):
    if fill:
        B, ns = with_empty_jets(B, ns)
    p4, mask = ragged_jets(B, P, ns, seed=P + 7, sigma=0.8)
    params = mlp_for(P + 1)
    q, k, v = rand_qkv(B, 8, P, mask, seed=P + 1, dtype="bf16")
    mlp = pip.PairMLP(params)
    bf = torch.bfloat16
    O = host(pip.pair_embed_attention(g(p4), g(mask), mlp, g(q, bf), g(k, bf), g(v, bf)))
    ref = oracle.pair_embed_attention(p4, mask, params, q, k, v)
    assert_close(O, ref, TOLBF, "fused O bf16 P=%d" % P)
    assert_zero_bits(O.transpose(0, 2, 1, 3), mask == 0, "fused bf16 padded rows")


@pytest.mark.parametrize("fill", [False, True])
@pytest.mark.parametrize("P,ns", [(48, (48, 30, 17)), (160, (160, 70, 17))])
def test_fused_f32_mlp_modes(P, ns, fill):
    # The fp16 x 2 chain with a hidden channel beyond fp16 (redone exactly),
    # then the exact chain chosen for badly scaled weights; jet and row kernel.
    B = 3
    if fill:
        B, ns = with_empty_jets(B, ns)
    p4, mask = ragged_jets(B, P, ns, seed=P + 21)
    q, k, v = rand_qkv(B, 8, P, mask, seed=P + 21)
    over = mlp_for(21, biases=True)
    over["b1"] = over["b1"].copy()
    over["b1"][5] = 8.0e4
    over["w2"] = over["w2"].copy()
    over["w2"][:, 5] = 1.0e-5
    scaled = mlp_for(22)
    scaled["w3"] = (scaled["w3"] * 1e5).astype(np.float32)
    scaled["w4"] = (scaled["w4"] * 1e-5).astype(np.float32)
    for name, params in (("overflow", over), ("badly scaled", scaled)):
        mlp = pip.PairMLP(params)
        O = host(pip.pair_embed_attention(g(p4), g(mask), mlp, g(q), g(k), g(v)))
        ref = oracle.pair_embed_attention(p4, mask, params, q, k, v)
        assert_close(O, ref, TOL32, "fused O f32, %s weights, P=%d" % (name, P))


def test_fused_batch512_workload():
    d = synth.make_workload("fused512")
    mlp = pip.PairMLP(d["mlp"])
    O = host(pip.pair_embed_attention(g(d["p4"]), g(d["mask"]), mlp, g(d["q"]), g(d["k"]),
                                      g(d["v"])))
    ref = oracle.pair_embed_attention(d["p4"], d["mask"], d["mlp"], d["q"], d["k"], d["v"])
    assert_close(O, ref, TOL32, "fused O (B=512, P=128)")
    assert_zero_bits(O.transpose(0, 2, 1, 3), d["mask"] == 0, "fused O padded rows")


def test_fused_matches_unfused_and_ignores_padding():
    B, P = 3, 64
    p4, mask = ragged_jets(B, P, (64, 33, 5), seed=11)
    params = mlp_for(11, biases=True)
    q, k, v = rand_qkv(B, 8, P, mask, seed=11)
    mlp = pip.PairMLP(params)
    O0 = host(pip.pair_embed_attention(g(p4), g(mask), mlp, g(q), g(k), g(v)))
    pad = mask == 0
    p4b = p4.copy()
    p4b[pad] = np.nan
    qb, kb, vb = (x.copy() for x in (q, k, v))
    for x in (qb, kb, vb):
        x[np.broadcast_to(pad[:, None, :, None], x.shape)] = np.nan
    O1 = host(pip.pair_embed_attention(g(p4b), g(mask), mlp, g(qb), g(kb), g(vb)))
    np.testing.assert_array_equal(O1.view(np.uint32), O0.view(np.uint32))
    U = pip.pair_embed(g(p4), g(mask), mlp)
    O2 = host(pip.pair_bias_attention(g(q), g(k), g(v), U, g(mask)))
    np.testing.assert_allclose(O0, O2, rtol=0, atol=2e-5)


def test_block_stack_workload():
    d = synth.make_workload("stack8")
    U = oracle.pair_embed(d["p4"], d["mask"], d["mlp"]).astype(np.float32)
    X = g(d["x0"])
    pip.block_stack(X, g(d["wq"]), g(d["wk"]), g(d["wv"]), g(d["wo"]), g(U), g(d["mask"]))
    got = host(X)
    ref = oracle.block_stack(d["x0"], d["wq"], d["wk"], d["wv"], d["wo"], U, d["mask"])
    assert_close(got, ref, TOL32, "block stack X (B=128, P=128, C=128, L=8)")
    assert_zero_bits(got, d["mask"] == 0, "padded rows of X")


@pytest.mark.parametrize("B,P,C,L,ns", [(3, 48, 32, 3, (48, 17, 0)), (2, 32, 256, 2, (30, 32))])
def test_block_stack_ragged_padded_rows_untouched(B, P, C, L, ns):
    rng = np.random.default_rng(C + L)
    _, mask = ragged_jets(B, P, ns, seed=C)
    x0, wq, wk, wv, wo = synth.make_block_stack(B, P, C, L, mask, rng=rng)
    x0 = x0.copy()
    x0[mask == 0] = rng.normal(0, 5, size=(int((mask == 0).sum()), C))  # junk padding
    H = C // 16
    U = rng.normal(0, 1, size=(B, H, P, P)).astype(np.float32)
    X = g(x0)
    pip.block_stack(X, g(wq), g(wk), g(wv), g(wo), g(U), g(mask))
    got = host(X)
    ref = oracle.block_stack(x0, wq, wk, wv, wo, U, mask)
    real = mask != 0
    assert_close(got[real], ref[real], TOL32, "block stack X C=%d" % C)
    np.testing.assert_array_equal(got[~real].view(np.uint32), x0[~real].view(np.uint32))


@pytest.mark.parametrize("B,P,C,L,ns", [
    (5, 128, 80, 2, (128, 100, 33, 1, 0)),  # H = 5: the last head pair has one head
    (2, 16, 16, 3, (16, 5)),                # H = 1, one row block
    (3, 112, 128, 1, (112, 97, 64)),        # P = 112: seven row blocks (odd)
])
def test_block_stack_shapes(B, P, C, L, ns):
    # odd head counts, a single head, odd block counts, empty and
    # one-particle jets, a non-prefix hole, junk padding
    rng = np.random.default_rng(B * 1000 + C)
    _, mask = ragged_jets(B, P, ns, seed=C + 1)
    x0, wq, wk, wv, wo = synth.make_block_stack(B, P, C, L, mask, rng=rng)
    x0 = x0.copy()
    x0[mask == 0] = rng.normal(0, 5, size=(int((mask == 0).sum()), C))
    H = C // 16
    U = rng.normal(0, 1, size=(B, H, P, P)).astype(np.float32)
    X = g(x0)
    pip.block_stack(X, g(wq), g(wk), g(wv), g(wo), g(U), g(mask))
    got = host(X)
    ref = oracle.block_stack(x0, wq, wk, wv, wo, U, mask)
    real = mask != 0
    assert_close(got[real], ref[real], TOL32, "block stack X B=%d P=%d C=%d" % (B, P, C))
    np.testing.assert_array_equal(got[~real].view(np.uint32), x0[~real].view(np.uint32))


def test_block_stack_more_jets_than_compute_units_scattered_masks():
    # 300 jets (more workgroups than CUs), masks with holes anywhere
    B, P, C, L = 300, 64, 128, 1
    rng = np.random.default_rng(300)
    mask = (rng.random((B, P)) < rng.uniform(0.1, 1.0, size=(B, 1))).astype(np.uint8)
    x0, wq, wk, wv, wo = synth.make_block_stack(B, P, C, L, mask, rng=rng)
    U = rng.normal(0, 1, size=(B, 8, P, P)).astype(np.float32)
    X = g(x0)
    pip.block_stack(X, g(wq), g(wk), g(wv), g(wo), g(U), g(mask))
    got = host(X)
    ref = oracle.block_stack(x0, wq, wk, wv, wo, U, mask)
    real = mask != 0
    assert_close(got[real], ref[real], TOL32, "block stack X B=300 scattered masks")
    np.testing.assert_array_equal(got[~real].view(np.uint32), x0[~real].view(np.uint32))


def test_block_stack_badly_scaled_rows_and_weights():
    # X rows over nine decades (up to ~3e5, beyond the fp16 range) and
    # weights scaled per matrix: every product runs on split fp16 operands
    # after exact powers of two, so large rows must not overflow and tiny
    # ones keep their relative accuracy.  Q and K are scaled down so that the
    # scores stay O(10) (a softmax over scores of size S amplifies float32
    # rounding by S, in any implementation).
    B, P, C, L = 3, 64, 64, 2
    rng = np.random.default_rng(77)
    _, mask = ragged_jets(B, P, (64, 40, 9), seed=77)
    x0, wq, wk, wv, wo = synth.make_block_stack(B, P, C, L, mask, rng=rng)
    x0 = (x0 * 10.0 ** rng.uniform(-4, 5.5, size=(B, P, 1))).astype(np.float32)
    wq = (wq * 1e-5).astype(np.float32)
    wk = (wk * 1e-5).astype(np.float32)
    wo = (wo * 1e-2).astype(np.float32)
    U = rng.normal(0, 1, size=(B, 4, P, P)).astype(np.float32)
    X = g(x0)
    pip.block_stack(X, g(wq), g(wk), g(wv), g(wo), g(U), g(mask))
    got = host(X)
    ref = oracle.block_stack(x0, wq, wk, wv, wo, U, mask)
    real = mask != 0
    # the bar relative to each row's own largest entry (attention mixes rows
    # of very different magnitude into each row)
    scale = np.abs(ref).max(axis=-1, keepdims=True) + 1e-30
    assert_close((got / scale)[real], (ref / scale)[real], TOL32, "block stack, scaled rows")


def test_fused_many_jets_unsorted_path():
    # more jets than the in-kernel ranking takes: workgroups take jets in index order
    B, P = 2100, 16
    rng = np.random.default_rng(70)
    ns = tuple(int(x) for x in rng.integers(0, 17, size=B))
    p4, mask = ragged_jets(B, P, ns, seed=70, hole=False)
    params = mlp_for(70)
    q, k, v = rand_qkv(B, 8, P, mask, seed=70)
    mlp = pip.PairMLP(params)
    O = host(pip.pair_embed_attention(g(p4), g(mask), mlp, g(q), g(k), g(v)))
    ref = oracle.pair_embed_attention(p4, mask, params, q, k, v)
    assert_close(O, ref, TOL32, "fused O B=2100")
    assert_zero_bits(O.transpose(0, 2, 1, 3), mask == 0, "fused O padded rows")

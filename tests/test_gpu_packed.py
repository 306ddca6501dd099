"""GPU parity of the packed variable-length layout (jets back to back,
cu_seqlens offsets, no padding) against the float64 oracle, through the C ABI.

The packed entries compute the same definition as the padded ones on the real
particles, so the expected values are the oracle's padded results on the same
jets (mask = the first n_b slots), gathered into the packed layout.  Bars as
in test_gpu_parity.py; the <= 7 columns past n_b of each U row are +0.0 bit
for bit; offsets are integers and match exactly."""
import numpy as np
import pytest
import torch

import oracle
from pair_interaction_particle_amd import binding as pip
from pair_interaction_particle_amd import synth
from test_gpu_parity import TOL32, TOLBF, TOLBF_U, assert_close, g, host, mlp_for

pytestmark = pytest.mark.gpu


def jets(ns, P, seed, sigma=0.4):
    p4, mask, _ = synth.make_jets(len(ns), P, 1, P, fixed_n=tuple(ns), seed=seed, sigma=sigma)
    return p4, mask


def u_blocks(U, ns, heads=8):
    """Split a packed U (flat) into per-jet (heads, n, ld) arrays."""
    out, off = [], 0
    for n in ns:
        ld = pip.packed_ld(n)
        out.append(U[off:off + heads * n * ld].reshape(heads, n, ld))
        off += heads * n * ld
    return out, off


def check_u(Ug, Uref, ns, tol_off, tol_diag, what):
    blocks, total = u_blocks(Ug, ns)
    assert total == Ug.size
    for b, (blk, n) in enumerate(zip(blocks, ns)):
        ref = Uref[b, :, :n, :n]
        got = blk[:, :, :n].astype(np.float64)
        diag = np.broadcast_to(np.eye(n, dtype=bool), ref.shape)
        assert_close(np.where(diag, 0.0, got), np.where(diag, 0.0, ref), tol_off,
                     "%s jet %d (off the diagonal)" % (what, b))
        assert_close(np.where(diag, got, 0.0), np.where(diag, ref, 0.0), tol_diag,
                     "%s jet %d (diagonal)" % (what, b))
        pad = np.ascontiguousarray(blk[:, :, n:])
        bits = pad.view(np.uint32) if pad.dtype == np.float32 else pad.view(np.uint16)
        assert not bits.any(), "%s jet %d: row padding not +0.0" % (what, b)


NS = (17, 0, 1, 128, 33, 7, 200, 16, 256, 64, 0, 95)


def test_u_offsets_match_the_exact_prefix_sum():
    ns = np.array(NS + (3, 250, 41) * 700, dtype=np.int64)  # B > one scan chunk
    cu = np.concatenate([[0], np.cumsum(ns)]).astype(np.int32)
    ld = (ns + 7) // 8 * 8
    ref = np.concatenate([[0], np.cumsum(ns * ld)])
    got = pip.packed_u_offsets(g(cu)).cpu().numpy()
    np.testing.assert_array_equal(got, ref)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_packed_embed_and_attention_ragged(dtype):
    P = 256
    p4, mask = jets(NS, P, seed=101)
    params = mlp_for(101, biases=True, input_bn=True)
    mlp = pip.PairMLP(params)
    cu = synth.cu_seqlens(mask)
    U, uoff = pip.pair_embed_packed(g(synth.pack_rows(p4, mask)), g(cu), mlp, dtype=dtype)
    Uref = oracle.pair_embed(p4, mask, params)
    bf = dtype == "bf16"
    check_u(host(U), Uref, NS, TOLBF if bf else TOL32, TOLBF_U if bf else TOL32,
            "packed U " + dtype)
    # attention on the packed layout, fed the oracle's U (packed the same way)
    q, k, v = synth.make_qkv(len(NS), 8, P, 16, mask, rng=np.random.default_rng(102),
                             dtype=dtype)
    Uin = Uref.astype(np.float32)
    if bf:
        Uin = synth.bf16_round(Uin)
    flat = np.concatenate([np.pad(Uin[b, :, :n, :n], ((0, 0), (0, 0), (0, pip.packed_ld(n) - n)))
                           .reshape(-1) for b, n in enumerate(NS)]).astype(np.float32)
    tt = torch.bfloat16 if bf else None
    qp, kp, vp = (g(synth.pack_heads(x, mask), tt) for x in (q, k, v))
    O = host(pip.pair_bias_attention_packed(qp, kp, vp, g(flat, tt), g(cu), uoff))
    ref = synth.pack_heads(oracle.attention(q, k, v, Uin, mask), mask)
    assert_close(O, ref, TOLBF if bf else TOL32, "packed O " + dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_packed_embed_writes_every_element(dtype):
    # an output buffer full of NaN: every element of every jet's block (rows
    # < n, the columns up to ld included) must be written, and nothing else
    ns = NS + (8, 24, 40, 15, 31, 2)
    P = 256
    p4, mask = jets(ns, P, seed=141)
    params = mlp_for(141, biases=True)
    mlp = pip.PairMLP(params)
    cu = synth.cu_seqlens(mask)
    n = np.asarray(ns, dtype=np.int64)
    total = int(8 * (n * ((n + 7) // 8 * 8)).sum())
    bf = dtype == "bf16"
    tdt = torch.bfloat16 if bf else torch.float32
    out = torch.full((total + 64,), float("nan"), device="cuda", dtype=tdt)
    U, _ = pip.pair_embed_packed(g(synth.pack_rows(p4, mask)), g(cu), mlp, dtype=dtype,
                                 out=out[:total])
    tail = host(out[total:]).astype(np.float64)
    assert np.isnan(tail).all(), "packed U: written past the last jet's block"
    Uref = oracle.pair_embed(p4, mask, params)
    check_u(host(U), Uref, ns, TOLBF if bf else TOL32, TOLBF_U if bf else TOL32,
            "packed U %s (NaN-filled output)" % dtype)


def test_packed_embed_across_launch_segments():
    # more than 65,536 jets: the launcher passes each segment its part of
    # cu / u_off (rows and U offsets stay absolute); jets on both sides of the
    # cut and a few early ones are compared with the oracle
    B, P = 65536 + 40, 16
    rng = np.random.default_rng(92)
    ns = tuple(int(x) for x in rng.integers(0, 5, size=B))
    p4, mask = jets(ns, P, seed=92)
    params = mlp_for(92, biases=True)
    mlp = pip.PairMLP(params)
    cu = synth.cu_seqlens(mask)
    U, uoff = pip.pair_embed_packed(g(synth.pack_rows(p4, mask)), g(cu), mlp)
    Ug, uo = host(U), uoff.cpu().numpy()
    sel = np.r_[0:24, 65536 - 24:B]
    ref = oracle.pair_embed(p4[sel], mask[sel], params)
    for i, b in enumerate(sel):
        n = ns[b]
        ld = pip.packed_ld(n)
        blk = Ug[8 * uo[b]:8 * uo[b + 1]].reshape(8, n, ld)
        assert_close(blk[:, :, :n], ref[i, :, :n, :n], TOL32, "packed U jet %d" % b)
        pad = np.ascontiguousarray(blk[:, :, n:])
        assert not pad.view(np.uint32).any(), "packed U jet %d: row padding not +0.0" % b


def test_packed_kernel_workload_f32():
    d = synth.make_workload("kernel")
    mask, ns = d["mask"], d["n"]
    cu = synth.cu_seqlens(mask)
    mlp = pip.PairMLP(d["mlp"])
    U, uoff = pip.pair_embed_packed(g(synth.pack_rows(d["p4"], mask)), g(cu), mlp)
    Uref = oracle.pair_embed(d["p4"], mask, d["mlp"])
    check_u(host(U), Uref, ns, TOL32, TOL32, "packed U (B=128, n~U{20..128})")
    qp, kp, vp = (g(synth.pack_heads(d[x], mask)) for x in ("q", "k", "v"))
    O = host(pip.pair_bias_attention_packed(qp, kp, vp, U, g(cu), uoff))
    ref = synth.pack_heads(oracle.attention(d["q"], d["k"], d["v"], Uref, mask), mask)
    # the attention was fed the GPU's own U: compare with the oracle's
    # attention on the oracle's U at the float32 bar (U error ~1e-6)
    assert_close(O, ref, TOL32, "packed O (B=128)")


def test_packed_large_bf16_workload():
    d = synth.make_workload("large_bf16")
    mask, ns = d["mask"], d["n"]
    cu = synth.cu_seqlens(mask)
    mlp = pip.PairMLP(d["mlp"])
    U, uoff = pip.pair_embed_packed(g(synth.pack_rows(d["p4"], mask)), g(cu), mlp, dtype="bf16")
    Uref = oracle.pair_embed(d["p4"], mask, d["mlp"])
    check_u(host(U), Uref, ns, TOLBF, TOLBF_U, "packed U bf16 (B=64, P=256)")


def test_inconsistent_jets_are_skipped():
    # jet 2's end offset is corrupted (so jets 2 and 3 are inconsistent), and
    # jet 5 is longer than max_n: nothing of them is written, the rest is
    # computed as usual
    ns = (20, 9, 33, 40, 12, 70, 5)
    P = 80
    p4, mask = jets(ns, P, seed=111)
    params = mlp_for(111)
    mlp = pip.PairMLP(params)
    cu = synth.cu_seqlens(mask)
    uoff = pip.packed_u_offsets(g(cu))
    bad = uoff.clone()
    bad[3] += 8
    total = 8 * int(uoff[-1])
    U = torch.full((total,), float("nan"), device="cuda")
    pip.pair_embed_packed(g(synth.pack_rows(p4, mask)), g(cu), mlp, u_offsets=bad,
                          max_n=64, out=U)
    Ug = host(U)
    Uref = oracle.pair_embed(p4, mask, params)
    blocks, _ = u_blocks(Ug, ns)
    for b, n in enumerate(ns):
        if b in (2, 3, 5):
            assert np.isnan(blocks[b]).all(), "skipped jet %d was written" % b
        else:
            assert_close(blocks[b][:, :, :n], Uref[b, :, :n, :n], TOL32, "jet %d" % b)
    # attention: the same jets skipped, their O rows untouched
    q, k, v = synth.make_qkv(len(ns), 8, P, 16, mask, rng=np.random.default_rng(112))
    qp, kp, vp = (g(synth.pack_heads(x, mask)) for x in (q, k, v))
    O = torch.full_like(qp, float("nan"))
    Uok = torch.from_numpy(np.nan_to_num(Ug)).cuda()
    pip.pair_bias_attention_packed(qp, kp, vp, Uok, g(cu), bad, max_n=64, out=O)
    Og = host(O)
    c = np.asarray(cu)
    for b in range(len(ns)):
        rows = Og[:, c[b]:c[b + 1]]
        if b in (2, 3, 5):
            assert np.isnan(rows).all(), "skipped jet %d: O written" % b
        else:
            assert np.isfinite(rows).all()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_packed_embed_more_jets_than_threads(dtype):
    # far more jets than a workgroup has threads (512): each thread sums the
    # work of a range of jets, and the split walks the packed entries
    rng = np.random.default_rng(131)
    ns = tuple(int(x) for x in rng.integers(0, 41, size=4100))
    P = 48
    p4, mask = jets(ns, P, seed=131)
    params = mlp_for(131, biases=True)
    mlp = pip.PairMLP(params)
    cu = synth.cu_seqlens(mask)
    U, _ = pip.pair_embed_packed(g(synth.pack_rows(p4, mask)), g(cu), mlp, dtype=dtype)
    Uref = oracle.pair_embed(p4, mask, params)
    bf = dtype == "bf16"
    check_u(host(U), Uref, ns, TOLBF if bf else TOL32, TOLBF_U if bf else TOL32,
            "packed U %s (B=4100)" % dtype)

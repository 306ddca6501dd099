"""Host-side checks of the L-GATr entry points (no GPU): the host expansion
of the equivariant linear layer's basis weights into W_eff against the
oracle's layer, and argument validation before any HIP call."""
import ctypes as C

import numpy as np
import pytest

import oracle
from pair_interaction_particle_amd import binding

OK, NULL, SHAPE, ALIGN, UNSUP = 0, 1, 2, 3, 5
A16, A17 = 0x10000, 0x10001


def oracle_weff(w, s2mv, mv2s, ss, in_s, out_s):
    """W_eff of the oracle's layer, one column per unit input."""
    out_mv, in_mv, _ = w.shape
    k = in_mv * 16 + in_s
    eye = np.eye(k)
    args = dict(w=w, s2mv=s2mv, mv2s=mv2s, ss=ss)
    y_mv, y_s = oracle.equilinear(eye[:, :in_mv * 16].reshape(k, in_mv, 16), eye[:, in_mv * 16:],
                                  **args)
    if y_s.shape[1] == 0 and out_s:
        y_s = np.zeros((k, out_s))
    return np.concatenate([y_mv.reshape(k, -1), y_s], axis=1).T


@pytest.mark.parametrize("shape", [(1, 1, 0, 0), (3, 5, 4, 2), (8, 8, 16, 16), (16, 8, 32, 48)])
def test_expand_matches_the_oracle_layer(shape):
    in_mv, out_mv, in_s, out_s = shape
    rng = np.random.default_rng(sum(shape))
    w = rng.normal(size=(out_mv, in_mv, 10)).astype(np.float32)
    s2mv = rng.normal(size=(out_mv, in_s)).astype(np.float32)
    mv2s = rng.normal(size=(out_s, in_mv)).astype(np.float32)
    ss = rng.normal(size=(out_s, in_s)).astype(np.float32)
    got = binding.equilinear_expand(w, s2mv, mv2s, ss, in_s, out_s)
    want = oracle_weff(w, s2mv, mv2s, ss, in_s, out_s)
    assert got.shape == want.shape
    # every entry is one weight, possibly negated: exact
    assert np.array_equal(got.astype(np.float64), want)


def test_expand_null_matrices_are_zero():
    rng = np.random.default_rng(3)
    w = rng.normal(size=(2, 3, 10)).astype(np.float32)
    got = binding.equilinear_expand(w, None, None, None, 4, 5)
    assert np.all(got[:, 48:] == 0) and np.all(got[32:] == 0)
    assert np.array_equal(got[:32, :48], binding.equilinear_expand(w)[:, :])


def test_lgatr_validation():
    L = binding.lib()
    gp = L.pip_lgatr_geometric_product
    assert gp(A16, A16, -1, A16, None) == SHAPE
    assert gp(None, None, 0, None, None) == OK
    assert gp(None, A16, 4, A16, None) == NULL
    assert gp(A16, A17, 4, A16, None) == ALIGN
    ex = L.pip_lgatr_equilinear_expand
    assert ex(A16, None, None, None, 8, 8, 16, 16, None) == NULL
    assert ex(A16, None, None, None, -1, 8, 16, 16, A16) == SHAPE
    cr = L.pip_lgatr_equilinear_create
    h = C.c_void_p()
    w = np.zeros((8, 8, 10), np.float32)
    for bad in ((4, 8, 16, 16), (8, 12, 16, 16), (8, 8, 8, 16), (8, 8, 16, 272)):
        assert cr(w.ctypes.data, None, None, None, None, None, *bad, C.byref(h)) == UNSUP
    assert cr(w.ctypes.data, None, None, None, None, None, 8, 8, -16, 16, C.byref(h)) == SHAPE
    assert cr(None, None, None, None, None, None, 8, 8, 16, 16, C.byref(h)) == NULL
    assert cr(w.ctypes.data, None, None, None, None, None, 8, 8, 16, 16, None) == NULL
    assert L.pip_lgatr_equilinear(None, A16, A16, 4, A16, A16, None) == NULL
    assert L.pip_lgatr_equilinear_destroy(None) == OK


def test_bench_cpu_sample_of_the_lgatr_workload():
    # the oracle leg of the benchmark's L-GATr workload runs on host arrays only
    import bench
    from pair_interaction_particle_amd import synth
    rng = np.random.default_rng(9)
    n = 2 * bench.LGATR_ITEMS
    d = {"params": synth.equilinear_params(8, 8, 16, 16, rng),
         "x_mv": synth.multivectors((n, 8), rng),
         "x_s": rng.normal(size=(n, 16)).astype(np.float32),
         "y": synth.multivectors((n, 8), rng)}
    r = bench.cpu_sample("lgatr", d, 1)
    assert r["value"] > 0 and r["kind"] == "oracle" and "128 items" in r["sample"]

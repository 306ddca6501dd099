"""GPU parity of the int8 pair embedding (pip_pair_embed_int8) against the
oracle's float64 int8 MLP on the same seeded inputs and quantisation
parameters (scales rounded to float32 first: the kernel takes them so).

The oracle models the quantisation exactly, so the GPU differs from it by
float32 arithmetic before each rounding decision and by the bfloat16
storage of U (relative 2^-9).  Bar: |err| <= 3e-3 (1 + |ref|) on every pair
whose quantisation decisions all lie farther than 3e-4 code units from a
rounding boundary (a float32 error of order 1e-5 code units cannot flip
them).  A pair with a decision within 3e-4 of a boundary may legitimately
take the neighbouring code: there the bar is 5e-2 (1 + |ref|).  Pairs
touching padding are +0.0 bit for bit."""
import json
import os

import numpy as np
import pytest

import oracle
from pair_interaction_particle_amd import binding as pip
from pair_interaction_particle_amd import synth
from test_gpu_parity import assert_zero_bits, g, host, mlp_for, pair_mask, ragged_jets

pytestmark = pytest.mark.gpu

TIE_DELTA, TOL_CLEAR, TOL_TIE = 3e-4, 3e-3, 5e-2
CALIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                     "int8_calibration.json")


def check(U, ref, tie, mask, what):
    real = pair_mask(mask)
    err = np.abs(U.astype(np.float64) - ref)
    bound = np.where(np.broadcast_to(tie[:, None], ref.shape), TOL_TIE, TOL_CLEAR) * (
        1.0 + np.abs(ref))
    bad = ~(err <= bound)
    assert not bad.any(), "%s: %d beyond (%d tie pairs of %d real); worst err %g at %s" % (
        what, bad.sum(), int(tie[real].sum()), int(real.sum()), err.max(),
        np.unravel_index(np.argmax(np.where(bad, err / bound, 0)), ref.shape))
    assert_zero_bits(U.transpose(0, 2, 3, 1), ~real, what + " padding")
    return int(tie[real].sum()), int(real.sum())


def run(p4, mask, params, S, Z):
    S32 = np.asarray(S, np.float32)
    mlp = pip.PairMLP(params)
    U = host(pip.pair_embed_int8(g(p4), g(mask), mlp, S32, np.asarray(Z, np.int32)))
    ref, tie = oracle.pair_embed_int8(p4, mask, params, S32.astype(np.float64),
                                      np.asarray(Z, np.float64), tie_delta=TIE_DELTA)
    return U, ref, tie


@pytest.mark.parametrize("B,P,ns,kw", [(2, 16, (11, 16), {}),
                                       (4, 64, (64, 50, 17, 0), {"biases": True}),
                                       (2, 256, (256, 131), {"biases": True, "input_bn": True})])
def test_int8_embed_ragged(B, P, ns, kw):
    p4, mask = ragged_jets(B, P, ns, seed=300 + P)
    params = mlp_for(300 + P, **kw)
    S, Z = oracle.int8_calibration(oracle.pair_mlp_ranges(p4, mask, params))
    U, ref, tie = run(p4, mask, params, S, Z)
    check(U, ref, tie, mask, "int8 U P=%d" % P)


def test_int8_embed_clamping_zero_points():
    # zero points at the ends of the range clamp part of every layer's inputs
    p4, mask = ragged_jets(3, 48, (48, 30, 7), seed=310)
    params = mlp_for(310, biases=True)
    U, ref, tie = run(p4, mask, params, [0.03, 0.05, 0.02], [100, -128, 127])
    check(U, ref, tie, mask, "int8 U clamping")


def test_int8_embed_kernel_workload():
    d = synth.make_workload("kernel")
    c = json.load(open(CALIB))["kernel"]
    U, ref, tie = run(d["p4"], d["mask"], d["mlp"], c["act_scale"], c["act_zero"])
    ntie, nreal = check(U, ref, tie, d["mask"], "int8 U (B=128, P=128)")
    assert ntie < 0.2 * nreal

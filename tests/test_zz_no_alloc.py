"""pip_block_stack_noalloc (the block stack with its workspace in the
library's fixed per-GPU scratch array) against pip_block_stack with a caller
workspace, through the C ABI: two calls in a row, the second on a smaller
problem, each held to the float32 bar and, since both run the same kernels on
the same inputs, to the same bits."""
import numpy as np
import pytest
import torch

from pair_interaction_particle_amd import binding as pip
from pair_interaction_particle_amd import synth

pytestmark = pytest.mark.gpu

TOL32 = 1e-4


def _case(B, P, C, L, ns, seed):
    p4, mask, _ = synth.make_jets(B, P, 1, P, fixed_n=ns, seed=seed)
    mask = mask.copy()
    mask[0, 1] = 0  # a hole
    H = C // 16
    rng = np.random.default_rng(seed)
    u = rng.normal(0, 1.0, size=(B, H, P, P)).astype(np.float32)
    x0, wq, wk, wv, wo = synth.make_block_stack(B, P, C, L, mask, rng=rng)
    return mask, u, x0, (wq, wk, wv, wo)


def _run_both(mask, u, x0, ws):
    dev = torch.device("cuda", 0)
    g = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    m, U, W = g(mask), g(u), [g(w) for w in ws]
    X1 = g(x0)
    pip.block_stack(X1, *W, U, m)
    X2 = g(x0)
    pip.block_stack_noalloc(X2, *W, U, m)
    torch.cuda.synchronize()
    return X1.cpu().numpy(), X2.cpu().numpy()


def test_noalloc_matches_the_workspace_entry_twice_second_smaller():
    for (B, P, C, L, ns, seed) in ((6, 64, 128, 3, (64, 50, 17, 16, 1, 0), 5),
                                  (2, 32, 64, 2, (32, 9), 6)):
        mask, u, x0, ws = _case(B, P, C, L, ns, seed)
        ref, got = _run_both(mask, u, x0, ws)
        err = np.abs(got.astype(np.float64) - ref) / (1.0 + np.abs(ref))
        assert err.max() <= TOL32, (B, P, C, L, err.max())
        np.testing.assert_array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_noalloc_rejects_problems_beyond_its_scratch():
    B, P, C, L = 512, 128, 128, 8  # ~34 MiB of workspace > 16 MiB
    assert pip.block_stack_workspace_bytes(B, P, C, L) > 16 << 20
    dev = torch.device("cuda", 0)
    x = torch.zeros((B, P, C), device=dev)
    w = torch.zeros((L, C, C), device=dev)
    u = torch.zeros((B, 8, P, P), device=dev)
    m = torch.ones((B, P), device=dev, dtype=torch.uint8)
    with pytest.raises(pip.PipError) as e:
        pip.block_stack_noalloc(x, w, w, w, w, u, m)
    assert e.value.status == 8  # PIP_ERR_TOO_LARGE

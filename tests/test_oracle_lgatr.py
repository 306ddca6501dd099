"""Pins of the oracle's L-GATr functions: the geometric product of the
spacetime algebra Cl(1,3) and the equivariant linear layer.

Source: [R] README "How the Kernel Fusion Works" (Fusion 1: the equivariant
linear layer is a 10-dimensional subspace of the 16x16 maps that commute with
Lorentz transformations) and "Results", table "L-GATr Kernels".

Nothing here reuses the oracle's blade algebra.  The independent route is the
Dirac matrix representation: four complex 4x4 matrices with
g_mu g_nu + g_nu g_mu = 2 eta_mu_nu, eta = diag(+1, -1, -1, -1), represent
Cl(1,3) faithfully, so the geometric product is a matrix product, and a
Lorentz transformation acts on a blade by replacing each generator e_a with
the vector Lambda e_a (the vectors stay orthogonal, so their geometric
product is their wedge product).
"""
import itertools

import numpy as np
import pytest
import scipy.linalg as sl

import oracle

# Blade order: sorted generator indices, grade by grade.
BLADES = [()] + [(a,) for a in range(4)] + list(itertools.combinations(range(4), 2)) \
    + list(itertools.combinations(range(4), 3)) + [(0, 1, 2, 3)]
GRADES = np.array([len(b) for b in BLADES])
ETA = np.diag([1.0, -1.0, -1.0, -1.0])

_S = [np.array([[0, 1], [1, 0]], complex), np.array([[0, -1j], [1j, 0]]),
      np.array([[1, 0], [0, -1]], complex)]
_Z2 = np.zeros((2, 2), complex)
_I2 = np.eye(2, dtype=complex)
GAMMA = [np.block([[_I2, _Z2], [_Z2, -_I2]])] + [np.block([[_Z2, s], [-s, _Z2]]) for s in _S]


def _blade_matrix(vectors):
    m = np.eye(4, dtype=complex)
    for v in vectors:
        m = m @ v
    return m


GB = [_blade_matrix([GAMMA[a] for a in b]) for b in BLADES]
GB_INV = [np.linalg.inv(g) for g in GB]


def to_matrix(x):
    return sum(c * g for c, g in zip(x, GB))


def from_matrix(m):
    out = np.array([np.trace(gi @ m) / 4 for gi in GB_INV])
    assert np.abs(out.imag).max() < 1e-9
    return out.real


def lorentz(rng, boost=1.0):
    """A random proper orthochronous Lorentz transformation (rotation and boost)."""
    gen = np.zeros((4, 4))
    th = rng.normal(0, 1.0, 3)
    be = rng.normal(0, boost, 3)
    for k, (i, j) in enumerate(((1, 2), (1, 3), (2, 3))):
        gen[i, j] -= th[k]
        gen[j, i] += th[k]
    for k in range(3):
        gen[0, k + 1] = gen[k + 1, 0] = be[k]
    lam = sl.expm(gen)
    np.testing.assert_allclose(lam.T @ ETA @ lam, ETA, atol=1e-9 * np.abs(lam).max() ** 2)
    assert lam[0, 0] >= 1 and np.linalg.det(lam) > 0
    return lam


def action(lam):
    """16x16 matrix of the Lorentz transformation on multivector components."""
    rows = []
    for b in BLADES:
        vecs = [sum(lam[mu, a] * GAMMA[mu] for mu in range(4)) for a in b]
        rows.append(from_matrix(_blade_matrix(vecs)))
    return np.array(rows).T


def test_dirac_representation_is_faithful():
    for i, j in itertools.product(range(4), repeat=2):
        np.testing.assert_allclose(GAMMA[i] @ GAMMA[j] + GAMMA[j] @ GAMMA[i],
                                   2 * ETA[i, j] * np.eye(4), atol=1e-15)
    gram = np.array([[np.trace(GB_INV[a] @ GB[b]) / 4 for b in range(16)] for a in range(16)])
    np.testing.assert_allclose(gram, np.eye(16), atol=1e-12)


def test_grades_follow_blade_order():
    assert oracle.blade_grades().tolist() == GRADES.tolist()


def test_geometric_product_matches_matrix_product():
    rng = np.random.default_rng(0)
    x, y = rng.normal(size=(40, 16)), rng.normal(size=(40, 16))
    z = oracle.geometric_product(x, y)
    for a, b, c in zip(x, y, z):
        np.testing.assert_allclose(c, from_matrix(to_matrix(a) @ to_matrix(b)), atol=1e-12)


def test_geometric_product_textbook_values():
    e = np.eye(16)
    gp = oracle.geometric_product
    # e0^2 = +1, e1^2 = e2^2 = e3^2 = -1 for the metric (+,-,-,-)
    assert gp(e[1], e[1])[0] == 1.0
    for k in (2, 3, 4):
        assert gp(e[k], e[k])[0] == -1.0
    # e0 e1 = e01 = -e1 e0; the pseudoscalar squares to -1
    assert gp(e[1], e[2]).tolist() == e[5].tolist()
    assert gp(e[2], e[1]).tolist() == (-e[5]).tolist()
    assert gp(e[15], e[15]).tolist() == (-e[0]).tolist()
    # a vector squares to its Minkowski norm
    v = np.zeros(16)
    v[1:5] = [3.0, 1.0, 2.0, 0.5]
    sq = gp(v, v)
    assert sq[0] == 9 - 1 - 4 - 0.25 and np.all(sq[1:] == 0)


def test_geometric_product_is_associative_and_lorentz_covariant():
    rng = np.random.default_rng(1)
    x, y, w = (rng.normal(size=(30, 16)) for _ in range(3))
    gp = oracle.geometric_product
    np.testing.assert_allclose(gp(gp(x, y), w), gp(x, gp(y, w)), atol=1e-12)
    for _ in range(3):
        rho = action(lorentz(rng))
        lhs = gp(x @ rho.T, y @ rho.T)
        rhs = gp(x, y) @ rho.T
        np.testing.assert_allclose(lhs, rhs, atol=1e-9 * np.abs(rhs).max())


def _basis_map(q):
    """16x16 matrix of equivariant basis map q, read off the oracle."""
    w = np.zeros((1, 1, 10))
    w[0, 0, q] = 1.0
    y, _ = oracle.equilinear(np.eye(16).reshape(16, 1, 16), None, w)
    return y[:, 0, :].T


def test_equilinear_basis_maps():
    rng = np.random.default_rng(2)
    x = rng.normal(size=16)
    for q in range(10):
        part = np.where(GRADES == q % 5, x, 0.0)
        want = part if q < 5 else from_matrix(GB[15] @ to_matrix(part))
        np.testing.assert_allclose(_basis_map(q) @ x, want, atol=1e-12)


def test_equilinear_basis_spans_the_commutant():
    # every 16x16 map commuting with the Lorentz action, solved from scratch
    rng = np.random.default_rng(3)
    rows = []
    for _ in range(3):
        r = action(lorentz(rng))
        rows.append(np.kron(np.eye(16), r) - np.kron(r.T, np.eye(16)))  # vec(M R - R M)
    ns = sl.null_space(np.vstack(rows), rcond=1e-9)
    assert ns.shape[1] == 10
    basis = np.array([_basis_map(q).reshape(-1, order="F") for q in range(10)]).T
    assert np.linalg.matrix_rank(basis, tol=1e-9) == 10
    resid = basis - ns @ (ns.T @ basis)
    assert np.abs(resid).max() < 1e-9


def _layer(rng, in_mv, out_mv, in_s, out_s):
    return dict(w=rng.normal(size=(out_mv, in_mv, 10)) / np.sqrt(in_mv),
                s2mv=rng.normal(size=(out_mv, in_s)), mv2s=rng.normal(size=(out_s, in_mv)),
                ss=rng.normal(size=(out_s, in_s)), b_mv=rng.normal(size=out_mv),
                b_s=rng.normal(size=out_s))


def test_equilinear_is_lorentz_equivariant():
    rng = np.random.default_rng(4)
    p = _layer(rng, 3, 5, 4, 2)
    x_mv, x_s = rng.normal(size=(7, 3, 16)), rng.normal(size=(7, 4))
    y_mv, y_s = oracle.equilinear(x_mv, x_s, **p)
    for _ in range(3):
        rho = action(lorentz(rng))
        t_mv, t_s = oracle.equilinear(x_mv @ rho.T, x_s, **p)
        np.testing.assert_allclose(t_mv, y_mv @ rho.T, atol=1e-9 * np.abs(y_mv).max())
        np.testing.assert_allclose(t_s, y_s, atol=1e-9 * np.abs(y_s).max())


def test_equilinear_scalar_channels():
    rng = np.random.default_rng(5)
    p = _layer(rng, 3, 5, 4, 2)
    x_s = rng.normal(size=(6, 4))
    y_mv, y_s = oracle.equilinear(np.zeros((6, 3, 16)), x_s, **p)
    np.testing.assert_allclose(y_mv[:, :, 0], x_s @ p["s2mv"].T + p["b_mv"], atol=1e-12)
    assert np.all(y_mv[:, :, 1:] == 0)
    np.testing.assert_allclose(y_s, x_s @ p["ss"].T + p["b_s"], atol=1e-12)
    # the scalar outputs see only the scalar component of the multivector inputs
    x_mv = rng.normal(size=(6, 3, 16))
    _, t_s = oracle.equilinear(x_mv, x_s, **p)
    np.testing.assert_allclose(t_s - y_s, x_mv[:, :, 0] @ p["mv2s"].T, atol=1e-12)


@pytest.mark.parametrize("shape", [(2, 3, 0, 0), (8, 8, 16, 16)])
def test_equilinear_is_one_linear_map(shape):
    # the layer is affine in the concatenated [mv_flat, scalars]: W_eff built
    # from unit inputs reproduces it on random inputs (the single-GEMM form)
    in_mv, out_mv, in_s, out_s = shape
    rng = np.random.default_rng(6)
    p = _layer(rng, *shape)
    k = in_mv * 16 + in_s
    eye = np.eye(k)
    zero_mv, zero_s = oracle.equilinear(np.zeros((1, in_mv, 16)), np.zeros((1, in_s)), **p)
    cols_mv, cols_s = oracle.equilinear(eye[:, :in_mv * 16].reshape(k, in_mv, 16),
                                        eye[:, in_mv * 16:], **p)
    bias = np.concatenate([zero_mv.reshape(-1), zero_s.reshape(-1)])
    w_eff = np.concatenate([cols_mv.reshape(k, -1), cols_s], axis=1).T - bias[:, None]
    x_mv, x_s = rng.normal(size=(9, in_mv, 16)), rng.normal(size=(9, in_s))
    y_mv, y_s = oracle.equilinear(x_mv, x_s, **p)
    flat = np.concatenate([x_mv.reshape(9, -1), x_s], axis=1) @ w_eff.T + bias
    np.testing.assert_allclose(flat[:, :out_mv * 16].reshape(9, out_mv, 16), y_mv, atol=1e-12)
    np.testing.assert_allclose(flat[:, out_mv * 16:], y_s, atol=1e-12)
    # at most two nonzero input components per output component and channel
    blk = np.abs(w_eff[:out_mv * 16, :in_mv * 16]).reshape(out_mv, 16, in_mv, 16) > 0
    assert blk.sum(axis=3).max() <= 2

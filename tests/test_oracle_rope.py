"""Oracle pins for axial RoPE at grid coordinates (and its sequence control).

The rotation is checked against the matrix exponential of its generator (an
independent construction), against R(0) = I, norm preservation and the
displacement identity <R(a)q, R(b)k> = <q, R(b-a)k> (paper summary §B.2).
The sequence-index control (paper summary §B.4) is checked the same way,
against the matrix exponential of its 1-D generator at the packed index.
"""
import numpy as np
import pytest

import oracle
import pack3d_inputs as pi
from refs import rotation, rotate_all, sequence_rotate_all


def _desc(grid, D, H=2, B=1):
    return oracle.make_desc(B, int(np.prod(grid)), H, D, grid, (2, 2, 2))


@pytest.mark.parametrize("D", [6, 24, 48, 96])
def test_rope_matches_matrix_exponential(D):
    grid = (3, 4, 5)
    c = pi.packing_coords(grid, "random", seed=11)
    rng = np.random.default_rng(D)
    x = rng.standard_normal((2, c.shape[0], 2, D))
    d = _desc(grid, D, H=2, B=2)
    y = oracle.rope_axial(d, c, x)
    assert np.allclose(y, rotate_all(c, x), rtol=0, atol=1e-12)


def test_rope_large_coordinates_match_matrix_exponential():
    grid = (64, 64, 64)
    c = np.array([[63, 0, 17], [0, 63, 63], [31, 32, 33]], dtype=np.int32)
    rng = np.random.default_rng(5)
    x = rng.standard_normal((1, 3, 1, 48))
    d = oracle.make_desc(1, 3, 1, 48, grid, (4, 4, 4))
    y = oracle.rope_axial(d, c, x)
    assert np.allclose(y, rotate_all(c, x), rtol=0, atol=1e-11)


def test_rope_identity_at_origin_and_norm():
    grid = (2, 2, 2)
    c = pi.raster_coords(grid)
    rng = np.random.default_rng(0)
    x = rng.standard_normal((1, 8, 3, 24))
    d = _desc(grid, 24, H=3)
    zero = np.zeros_like(c)
    d1 = oracle.make_desc(1, 8, 3, 24, grid, (2, 2, 2))
    # every coordinate zero: rotation is exactly the identity
    y0 = oracle.rope_axial(d1, zero, x)
    assert np.array_equal(y0, x)
    y = oracle.rope_axial(d, c, x)
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)


def test_displacement_identity():
    rng = np.random.default_rng(1)
    D = 48
    for _ in range(20):
        a = rng.integers(0, 64, 3)
        b = rng.integers(0, 64, 3)
        q = rng.standard_normal(D)
        k = rng.standard_normal(D)
        d = oracle.make_desc(1, 2, 1, D, (64, 64, 64), (4, 4, 4))
        rot = oracle.rope_axial(d, np.stack([a, b]).astype(np.int32),
                                np.stack([q, k])[None, :, None, :])[0, :, 0]
        lhs = rot[0] @ rot[1]
        rhs = q @ (rotation(b - a, D) @ k)
        assert abs(lhs - rhs) < 1e-10 * (1 + abs(lhs))


def test_sequence_control_is_an_actual_rotation():
    # the corrected experiments note that an earlier packed control had no
    # active rotary pairs (project page, Ch. 10); this control must turn
    grid = (8, 8, 8)
    c = pi.raster_coords(grid)
    d = oracle.make_desc(1, 512, 1, 24, grid, (2, 2, 2))
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 512, 1, 24))
    k = rng.standard_normal((1, 512, 1, 24))
    qs, ks = oracle.rope_sequence(d, q), oracle.rope_sequence(d, k)
    raw = np.einsum("nd,md->nm", q[0, :, 0], k[0, :, 0])
    seq = np.einsum("nd,md->nm", qs[0, :, 0], ks[0, :, 0])
    assert np.abs(seq - raw).max() > 1e-3
    # and it is a rotation at the packed index: position 0 is the identity
    assert np.array_equal(qs[0, 0], q[0, 0])
    assert np.allclose(np.linalg.norm(qs, axis=-1), np.linalg.norm(q, axis=-1))


@pytest.mark.parametrize("D", [6, 24, 48])
def test_sequence_control_matches_matrix_exponential(D):
    # 1-D RoPE at the packed index i over all D channels, theta_p = base^(-2p/D):
    # the rotation of a generator that carries the index, built independently
    N, H, B = 40, 2, 2
    rng = np.random.default_rng(30 + D)
    x = rng.standard_normal((B, N, H, D))
    d = oracle.make_desc(B, N, H, D, (2, 4, 5), (2, 2, 2))
    # expm of angles up to N rad carries ~1e-12 of its own error
    assert np.allclose(oracle.rope_sequence(d, x), sequence_rotate_all(x), rtol=0, atol=1e-10)


def test_sequence_control_relative_offset():
    # the 1-D rotation is relative in the packed index: <R(i)q, R(j)k> depends
    # on j - i only, so two pairs with the same index gap give the same logit
    D, N = 24, 64
    rng = np.random.default_rng(31)
    q, k = rng.standard_normal(D), rng.standard_normal(D)
    x = np.zeros((1, N, 2, D))
    x[0, :, 0] = q
    x[0, :, 1] = k
    d = oracle.make_desc(1, N, 2, D, (4, 4, 4), (2, 2, 2))
    y = oracle.rope_sequence(d, x)[0]
    for i, j in [(0, 5), (17, 22), (58, 63)]:
        assert abs(y[i, 0] @ y[j, 1] - y[0, 0] @ y[5, 1]) < 1e-10

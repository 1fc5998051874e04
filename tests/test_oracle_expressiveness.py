"""The two-block construction of paper summary §B.6 (coordinate-aware
compression is strictly more expressive), run through the oracle's global
branch: two blocks whose members carry one and the same key, so that their
coordinate-blind pooled keys coincide, and opposite values (+u, -u, |u| = 1).
A query that should read block 0 gets squared error exactly 1 from
coordinate-blind pooling (equal logits: the output is the mean, 0) for every
query norm, while with rotate-then-pool the two summaries differ and a query
along their difference drives the error to 0 as its norm grows (there is no
fixed norm bound)."""
import numpy as np

import oracle
from refs import rotation


def _global_output(rope, lam, D=6):
    grid, block = (1, 1, 4), (1, 1, 2)          # two blocks of two tokens along x
    c = np.array([[0, 0, x] for x in range(4)], dtype=np.int32)
    rng = np.random.default_rng(2)
    kvec = rng.standard_normal(D)
    u = rng.standard_normal(D)
    u /= np.linalg.norm(u)
    k = np.tile(kvec, (1, 4, 1, 1))
    v = np.stack([u, u, -u, -u])[None, :, None, :]
    d = oracle.make_desc(1, 4, 1, D, grid, block)
    slot, _, _ = oracle.index(d, c)
    kr = oracle.rope_axial(d, c, k) if rope else k
    ks, vs = oracle.summaries(d, slot, kr, v)
    direction = ks[0, 0, 0] - ks[0, 0, 1]
    q = np.zeros((1, 4, 1, D))
    if rope:  # choose q so that the rotated query points along the difference
        q[0, 0, 0] = rotation(c[0], D).T @ (lam * direction)
    else:
        q[0, 0, 0] = lam * kvec
    qr = oracle.rope_axial(d, c, q) if rope else q
    og = oracle.global_(d, c, qr, ks, vs)
    return og[0, 0, 0], u, direction


def test_blind_pooling_cannot_separate_the_blocks():
    for lam in (1.0, 10.0, 1000.0):
        o, u, direction = _global_output(False, lam)
        assert np.abs(direction).max() == 0.0            # identical pooled keys
        assert abs(np.sum((o - u) ** 2) - 1.0) < 1e-12   # squared error exactly 1


def test_rotate_then_pool_approximates_the_target():
    errs = []
    for lam in (0.02, 0.1, 0.3, 1.0, 10.0):
        o, u, direction = _global_output(True, lam)
        assert np.linalg.norm(direction) > 1e-3          # the summaries differ
        errs.append(float(np.sum((o - u) ** 2)))
    # falls with the query norm (strictly until the softmax saturates in fp64)
    assert all(b < a or b == 0.0 for a, b in zip(errs, errs[1:]))
    assert 1e-3 < errs[0] < 1.0 and errs[-1] <= 1e-8

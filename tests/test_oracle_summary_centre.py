"""Oracle pins for the summary-centre variant of the compressed branch: pool
the unrotated keys, then rotate the mean once at the block centre (paper
summary §B.7, §B.8; project page Ch. 3, "One block, two ways to summarize
it").

centre value  <- R(c_m) applied to the block mean, R built as the matrix
                 exponential of its generator at the half-integer centre
1x1x1 blocks  <- identical to rotate-then-pool
swap          <- blind to exchanging two members inside a block, while
                 rotate-then-pool is not
drift bound   <- |<q~, ks_centre> - <q~, ks_rtp>| is at most
                 sum over planes of |q~_plane| * mean_j 2|sin(theta (c_m - c_j)/2)| |k_j,plane|
                 (|R(a)x - R(b)x| = 2|sin((a-b)/2)| |x|), and it grows with
                 block size and with rotary frequency (paper summary §B.8)
"""
import numpy as np
import pytest

import oracle
import pack3d_inputs as pi
from refs import block_ids, rotation


def _setup(grid, block, B=1, H=1, D=12, kind="random", seed=0, base=10000.0):
    c = pi.packing_coords(grid, kind, block=block, seed=seed + 100)
    rng = np.random.default_rng(seed)
    N = c.shape[0]
    q, k, v = (rng.standard_normal((B, N, H, D)) for _ in range(3))
    d = oracle.make_desc(B, N, H, D, grid, block, rope_base=base)
    return d, c, q, k, v


def _centre(grid, block, m):
    My = -(-grid[1] // block[1])
    Mx = -(-grid[2] // block[2])
    o = np.array([(m // (My * Mx)) * block[0], ((m // Mx) % My) * block[1], (m % Mx) * block[2]])
    ext = np.minimum(np.array(block), np.array(grid) - o)
    return o + 0.5 * (ext - 1)


@pytest.mark.parametrize("grid,block", [((4, 4, 4), (2, 2, 2)), ((5, 6, 7), (2, 3, 4)),
                                        ((3, 8, 5), (3, 2, 2))])
def test_centre_summary_is_block_mean_rotated_at_centre(grid, block):
    D = 12
    d, c, q, k, v = _setup(grid, block, D=D)
    slot, _, _ = oracle.index(d, c)
    ks, vs = oracle.summaries_centre(d, slot, k, v)
    bid = block_ids(c, grid, block)
    for m in range(ks.shape[2]):
        members = np.flatnonzero(bid == m)
        R = rotation(_centre(grid, block, m), D)
        assert np.allclose(ks[0, 0, m], R @ k[0, members, 0].mean(axis=0), atol=1e-12)
        assert np.allclose(vs[0, 0, m], v[0, members, 0].mean(axis=0), atol=1e-14)


def test_unit_blocks_equal_rotate_then_pool():
    grid, block = (3, 4, 5), (1, 1, 1)
    d, c, q, k, v = _setup(grid, block, B=2, H=2, D=24)
    slot, _, _ = oracle.index(d, c)
    kc, vc = oracle.summaries_centre(d, slot, k, v)
    kt, vt = oracle.summaries(d, slot, oracle.rope_axial(d, c, k), v)
    assert np.allclose(kc, kt, atol=1e-13)
    assert np.array_equal(vc, vt)


def test_within_block_swap_is_invisible_to_centre_summary():
    grid, block, D = (2, 2, 2), (2, 2, 2), 12
    d, c, q, k, v = _setup(grid, block, D=D, kind="raster")
    slot, _, _ = oracle.index(d, c)
    k2, v2 = k.copy(), v.copy()
    k2[:, [1, 6]] = k2[:, [6, 1]]
    v2[:, [1, 6]] = v2[:, [6, 1]]
    kc0, _ = oracle.summaries_centre(d, slot, k, v)
    kc1, _ = oracle.summaries_centre(d, slot, k2, v2)
    kt0, _ = oracle.summaries(d, slot, oracle.rope_axial(d, c, k), v)
    kt1, _ = oracle.summaries(d, slot, oracle.rope_axial(d, c, k2), v2)
    assert np.abs(kc1 - kc0).max() < 1e-14
    assert np.abs(kt1 - kt0).max() > 1e-3


def _drift(grid, block, base, D=24, seed=1, coherent=False):
    d, c, q, k, v = _setup(grid, block, D=D, base=base, seed=seed)
    if coherent:  # every token carries the same key: no within-block variation to average out
        k[:] = k[:, :1]
    slot, _, _ = oracle.index(d, c)
    qr = oracle.rope_axial(d, c, q)
    kc, _ = oracle.summaries_centre(d, slot, k, v)
    kt, _ = oracle.summaries(d, slot, oracle.rope_axial(d, c, k), v)
    bid = block_ids(c, grid, block)
    da, P = D // 3, D // 6
    errs, bounds = [], []
    rng = np.random.default_rng(seed)
    for i in rng.choice(c.shape[0], 24, replace=False):
        for m in range(kc.shape[2]):
            members = np.flatnonzero(bid == m)
            cm = _centre(grid, block, m)
            bound = 0.0
            for a in range(3):
                for p in range(P):
                    th = base ** (-2.0 * p / da)
                    ch = slice(a * da + 2 * p, a * da + 2 * p + 2)
                    shift = 2 * np.abs(np.sin(th * (cm[a] - c[members, a]) / 2))
                    bound += np.linalg.norm(qr[0, i, 0, ch]) * np.mean(
                        shift * np.linalg.norm(k[0, members, 0, ch], axis=1))
            errs.append(abs(qr[0, i, 0] @ kc[0, 0, m] - qr[0, i, 0] @ kt[0, 0, m]))
            bounds.append(bound)
    return np.array(errs), np.array(bounds)


def test_logit_drift_within_bound():
    for grid, block, base in [((4, 4, 8), (2, 2, 2), 10000.0), ((8, 8, 8), (4, 4, 4), 10000.0),
                              ((4, 4, 8), (2, 2, 4), 100.0)]:
        e, bnd = _drift(grid, block, base)
        assert (e <= bnd + 1e-12).all()
        assert e.max() > 0


def test_drift_grows_with_block_size_and_frequency():
    # the bound grows with block diameter and with rotary frequency (plane 0
    # turns at rate 1 whatever the base, so a higher-frequency base raises the
    # other planes' terms); with one key shared by every token the drift
    # itself grows with the block (with iid keys the mean over more members
    # averages it down)
    _, b_small = _drift((8, 8, 8), (2, 2, 2), 10000.0)
    _, b_large = _drift((8, 8, 8), (4, 4, 4), 10000.0)
    _, b_fast = _drift((8, 8, 8), (2, 2, 2), 10.0)
    assert b_large.mean() > 1.5 * b_small.mean()
    assert b_fast.mean() > 1.5 * b_small.mean()
    e_small, _ = _drift((8, 8, 8), (2, 2, 2), 10000.0, coherent=True)
    e_large, _ = _drift((8, 8, 8), (4, 4, 4), 10000.0, coherent=True)
    assert e_large.mean() > 2 * e_small.mean()


@pytest.mark.parametrize("a,b", [("raster", "morton"), ("block", "random")])
def test_centre_operator_permutes_bitwise(a, b):
    grid, block, D = (4, 6, 8), (2, 2, 2), 12
    w = pi.Workload(900, "t", grid, 1, 2, D, block, "f32", "iid", a, b)
    fields = pi.make_fields(w)
    d = oracle.make_desc(1, w.N, 2, D, grid, block)
    outs = []
    coords = []
    for kind in (a, b):
        c = pi.packing_coords(grid, kind, block=block, seed=7)
        q, k, v, g = pi.pack_fields(fields, c, grid)
        outs.append(oracle.forward(d, c, q, k, v, g, summary_rope="centre"))
        coords.append(c)
    p = pi.order_between(coords[0], coords[1], grid)
    assert np.array_equal(outs[0], outs[1][:, p])

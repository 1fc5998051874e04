"""Oracle pins for the local branch, the summaries, the global branch and the
mixer.

local     <- dense masked SDPA in float64 over all token pairs, mask from
             pairwise Chebyshev distance (project page Ch. 3, Contract 1)
summaries <- the block-weighted displacement identity (paper summary §B.5):
             <q~_i, ks_m> = mean_j <q_i, R(c_j - c_i) k_j>
global    <- torch scaled_dot_product_attention over the summaries; M = 1 and
             1x1x1 blocks reduce to textbook closed forms
mix       <- saturated and neutral gates
"""
import numpy as np
import pytest

import oracle
import pack3d_inputs as pi
from refs import (block_ids, chebyshev_mask, dense_masked_attention, rotate_all, rotation,
                  torch_sdpa)


def _setup(grid, block, B, H, D, kind="random", seed=0):
    c = pi.packing_coords(grid, kind, block=block, seed=seed + 100)
    rng = np.random.default_rng(seed)
    N = c.shape[0]
    q, k, v = (rng.standard_normal((B, N, H, D)) for _ in range(3))
    g = rng.standard_normal((B, N, H))
    d = oracle.make_desc(B, N, H, D, grid, block)
    return d, c, q, k, v, g


@pytest.mark.parametrize("grid,block,B,H,D,kind", [
    ((8, 8, 8), (2, 2, 2), 1, 1, 24, "raster"),
    ((3, 5, 7), (2, 2, 2), 2, 2, 12, "random"),
    ((4, 4, 4), (2, 2, 2), 1, 3, 48, "morton"),
])
def test_local_matches_dense_masked_sdpa(grid, block, B, H, D, kind):
    d, c, q, k, v, _ = _setup(grid, block, B, H, D, kind)
    slot, _, _ = oracle.index(d, c)
    ol = oracle.local(d, c, slot, oracle.rope_axial(d, c, q), oracle.rope_axial(d, c, k), v)
    ref = dense_masked_attention(rotate_all(c, q), rotate_all(c, k), v, chebyshev_mask(c),
                                 1 / np.sqrt(D))
    assert np.allclose(ol, ref, rtol=0, atol=1e-12)


def test_local_rows_subset_equals_full():
    d, c, q, k, v, _ = _setup((5, 6, 7), (2, 2, 2), 2, 2, 12)
    slot, _, _ = oracle.index(d, c)
    qr, kr = oracle.rope_axial(d, c, q), oracle.rope_axial(d, c, k)
    full = oracle.local(d, c, slot, qr, kr, v)
    rows = np.array([0, 17, 5, 209], dtype=np.int32)
    assert np.array_equal(oracle.local(d, c, slot, qr, kr, v, rows), full[:, rows])


def test_local_zero_query_is_neighbour_mean():
    d, c, q, k, v, _ = _setup((4, 5, 3), (2, 2, 2), 1, 2, 12)
    slot, _, _ = oracle.index(d, c)
    ol = oracle.local(d, c, slot, np.zeros_like(q), oracle.rope_axial(d, c, k), v)
    mask = chebyshev_mask(c)
    ref = np.einsum("nm,bmhd->bnhd", mask / mask.sum(axis=1, keepdims=True), v)
    assert np.allclose(ol, ref, atol=1e-13)


def test_local_single_token_returns_its_value():
    d, c, q, k, v, _ = _setup((1, 1, 1), (1, 1, 1), 2, 3, 6)
    slot, _, _ = oracle.index(d, c)
    ol = oracle.local(d, c, slot, oracle.rope_axial(d, c, q), oracle.rope_axial(d, c, k), v)
    assert np.array_equal(ol, v)


@pytest.mark.parametrize("grid,block", [((8, 8, 8), (2, 2, 2)), ((5, 6, 7), (2, 3, 4)),
                                        ((4, 4, 8), (2, 2, 4))])
def test_summary_logit_is_block_weighted_displacement_sum(grid, block):
    D = 24
    d, c, q, k, v, _ = _setup(grid, block, 1, 1, D)
    slot, _, _ = oracle.index(d, c)
    qr, kr = oracle.rope_axial(d, c, q), oracle.rope_axial(d, c, k)
    ks, vs = oracle.summaries(d, slot, kr, v)
    bid = block_ids(c, grid, block)
    rng = np.random.default_rng(3)
    for i in rng.choice(c.shape[0], 6, replace=False):
        for m in rng.choice(ks.shape[2], 5, replace=False):
            members = np.flatnonzero(bid == m)
            terms = [q[0, i, 0] @ (rotation(c[j] - c[i], D) @ k[0, j, 0]) for j in members]
            assert abs(qr[0, i, 0] @ ks[0, 0, m] - np.mean(terms)) < 1e-11
            assert np.allclose(vs[0, 0, m], v[0, members, 0].mean(axis=0), atol=1e-14)


def test_within_block_swap_moves_rotated_summary_only():
    # exchanging two token states inside a block keeps the pooled value and
    # the pooled unrotated key but moves the rotate-then-pool key (project
    # page, Ch. 3, "One block, two ways to summarize it")
    grid, block, D = (2, 2, 2), (2, 2, 2), 12
    d, c, q, k, v, _ = _setup(grid, block, 1, 1, D, "raster")
    slot, _, _ = oracle.index(d, c)
    ks0, vs0 = oracle.summaries(d, slot, oracle.rope_axial(d, c, k), v)
    k2, v2 = k.copy(), v.copy()
    k2[:, [1, 6]] = k2[:, [6, 1]]
    v2[:, [1, 6]] = v2[:, [6, 1]]
    ks1, vs1 = oracle.summaries(d, slot, oracle.rope_axial(d, c, k2), v2)
    assert np.abs(ks1 - ks0).max() > 1e-3
    assert np.allclose(vs1, vs0, atol=1e-15)
    assert np.allclose(k2.mean(axis=1), k.mean(axis=1), atol=1e-15)


@pytest.mark.parametrize("grid,block,B,H,D", [((8, 8, 8), (2, 2, 2), 1, 1, 24),
                                              ((6, 5, 4), (2, 2, 2), 2, 2, 12),
                                              ((4, 8, 8), (2, 2, 4), 1, 2, 48)])
def test_global_matches_torch_sdpa(grid, block, B, H, D):
    d, c, q, k, v, _ = _setup(grid, block, B, H, D)
    slot, _, _ = oracle.index(d, c)
    qr, kr = oracle.rope_axial(d, c, q), oracle.rope_axial(d, c, k)
    ks, vs = oracle.summaries(d, slot, kr, v)
    og = oracle.global_(d, c, qr, ks, vs)
    assert np.allclose(og, torch_sdpa(qr, ks, vs, 1 / np.sqrt(D)), rtol=0, atol=1e-12)


def test_global_is_invariant_to_summary_order():
    d, c, q, k, v, _ = _setup((6, 6, 6), (2, 2, 2), 1, 2, 12)
    slot, _, _ = oracle.index(d, c)
    qr, kr = oracle.rope_axial(d, c, q), oracle.rope_axial(d, c, k)
    ks, vs = oracle.summaries(d, slot, kr, v)
    perm = np.random.default_rng(0).permutation(ks.shape[2])
    a = oracle.global_(d, c, qr, ks, vs)
    b = oracle.global_(d, c, qr, ks[:, :, perm], vs[:, :, perm])
    assert np.allclose(a, b, atol=1e-13)


def test_global_single_summary_is_mean_of_values():
    grid = (3, 4, 5)
    d, c, q, k, v, _ = _setup(grid, grid, 1, 2, 12)
    slot, _, _ = oracle.index(d, c)
    qr, kr = oracle.rope_axial(d, c, q), oracle.rope_axial(d, c, k)
    ks, vs = oracle.summaries(d, slot, kr, v)
    assert ks.shape[2] == 1
    og = oracle.global_(d, c, qr, ks, vs)
    assert np.allclose(og, np.broadcast_to(v.mean(axis=1, keepdims=True), og.shape), atol=1e-14)


def test_global_unit_blocks_is_full_field_rope_attention():
    grid = (3, 3, 4)
    d, c, q, k, v, _ = _setup(grid, (1, 1, 1), 1, 2, 24, "morton")
    slot, _, _ = oracle.index(d, c)
    qr, kr = oracle.rope_axial(d, c, q), oracle.rope_axial(d, c, k)
    ks, vs = oracle.summaries(d, slot, kr, v)
    og = oracle.global_(d, c, qr, ks, vs)
    full = np.ones((c.shape[0], c.shape[0]), bool)
    ref = dense_masked_attention(rotate_all(c, q), rotate_all(c, k), v, full, 1 / np.sqrt(24))
    assert np.allclose(og, ref, atol=1e-12)


@pytest.mark.parametrize("mode", ["own_block", "neighbourhood_blocks"])
def test_global_exclusion_readings(mode):
    grid, block, D = (6, 4, 6), (2, 2, 2), 12
    d, c, q, k, v, _ = _setup(grid, block, 1, 2, D)
    d.exclusion = oracle.EXCLUSION[mode]
    slot, _, _ = oracle.index(d, c)
    qr, kr = oracle.rope_axial(d, c, q), oracle.rope_axial(d, c, k)
    ks, vs = oracle.summaries(d, slot, kr, v)
    og = oracle.global_(d, c, qr, ks, vs)
    bid = block_ids(c, grid, block)
    M = ks.shape[2]
    allowed = np.ones((c.shape[0], M), bool)
    if mode == "own_block":
        allowed[np.arange(c.shape[0]), bid] = False
    else:
        near = chebyshev_mask(c)
        for i in range(c.shape[0]):
            allowed[i, np.unique(bid[near[i]])] = False
    ref = torch_sdpa(qr, ks, vs, 1 / np.sqrt(D), mask=allowed)
    assert np.allclose(og, ref, atol=1e-12)


def test_global_everything_excluded_gives_zero():
    grid = (2, 2, 2)
    d, c, q, k, v, _ = _setup(grid, grid, 1, 1, 6)
    d.exclusion = oracle.EXCLUSION["own_block"]
    slot, _, _ = oracle.index(d, c)
    qr, kr = oracle.rope_axial(d, c, q), oracle.rope_axial(d, c, k)
    ks, vs = oracle.summaries(d, slot, kr, v)
    assert np.array_equal(oracle.global_(d, c, qr, ks, vs), np.zeros_like(q))


def test_mix_gates():
    d, c, q, k, v, g = _setup((4, 4, 4), (2, 2, 2), 1, 2, 12)
    o, parts = oracle.forward(d, c, q, k, v, g, return_parts=True)
    ol, og = parts["local"], parts["glob"]
    sig = 1 / (1 + np.exp(-g))[..., None]
    assert np.allclose(o, (1 - sig) * ol + sig * og, atol=1e-14)
    hi = oracle.forward(d, c, q, k, v, np.full_like(g, 40.0))
    lo = oracle.forward(d, c, q, k, v, np.full_like(g, -40.0))
    mid = oracle.forward(d, c, q, k, v, np.zeros_like(g))
    assert np.allclose(hi, og, atol=1e-15) and np.allclose(lo, ol, atol=1e-15)
    assert np.allclose(mid, 0.5 * (ol + og), atol=1e-15)
    # a closed gate is not the same intervention as a zeroed global output:
    # with the gate at 0 logits (g = 1/2) zeroing O_glob halves the local term
    zeroed = oracle.mix(d, np.zeros_like(g), ol, np.zeros_like(og))
    assert np.allclose(zeroed, 0.5 * ol, atol=1e-15)
    assert np.abs(zeroed - lo).max() > 1e-2

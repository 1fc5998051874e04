"""Oracle pins for the index step: neighbourhoods, blocks, slots.

Pinned by brute force over coordinate pairs, by closed-form counts and by the
layout facts the pages print (tests/golden/pages_facts.json).
"""
import json
import os

import numpy as np
import pytest

import oracle
import pack3d_inputs as pi
from refs import block_ids, chebyshev_mask

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_facts.json")))


def _desc(grid, block=(2, 2, 2), B=1, H=1, D=6):
    return oracle.make_desc(B, int(np.prod(grid)), H, D, grid, block)


GRIDS = [((1, 1, 1), "raster"), ((2, 2, 2), "morton"), ((3, 4, 5), "random"),
         ((8, 8, 8), "raster"), ((5, 3, 7), "morton"), ((4, 6, 2), "block")]


@pytest.mark.parametrize("grid,kind", GRIDS)
def test_neighbours_match_brute_force(grid, kind):
    c = pi.packing_coords(grid, kind, block=(2, 2, 2), seed=7)
    d = _desc(grid)
    slot, blk, rank = oracle.index(d, c)
    nbr = oracle.neighbours(d, c, slot)
    mask = chebyshev_mask(c)
    for i in range(c.shape[0]):
        got = sorted(j for j in nbr[i] if j >= 0)
        assert got == sorted(np.flatnonzero(mask[i]).tolist())
        # each entry sits at its own canonical offset; self is entry 13
        for kk in range(27):
            off = np.array([kk // 9 - 1, (kk // 3) % 3 - 1, kk % 3 - 1])
            if nbr[i, kk] >= 0:
                assert np.array_equal(c[nbr[i, kk]] - c[i], off)
        assert nbr[i, 13] == i


@pytest.mark.parametrize("grid", [(8, 8, 8), (3, 4, 5), (1, 1, 9), (16, 2, 3)])
def test_valid_pair_count_closed_form(grid):
    c = pi.raster_coords(grid)
    d = _desc(grid)
    slot, _, _ = oracle.index(d, c)
    nbr = oracle.neighbours(d, c, slot)
    # along each axis a site has 3 neighbours inside, 2 at an edge: 3n - 2 pairs
    assert int((nbr >= 0).sum()) == int(np.prod([3 * n - 2 for n in grid]))


def test_corner_edge_face_interior_counts_8cubed():
    g = GOLDEN["lab_field"]["grid"]
    c = pi.raster_coords(g)
    d = _desc(g)
    slot, _, _ = oracle.index(d, c)
    sizes = (oracle.neighbours(d, c, slot) >= 0).sum(axis=1)
    vals, counts = np.unique(sizes, return_counts=True)
    assert dict(zip(vals.tolist(), counts.tolist())) == {8: 8, 12: 72, 18: 216, 27: 216}
    assert sizes.max() == GOLDEN["neighbourhood_max"]["size"]


def test_raster_face_offsets_are_face_neighbours():
    f = GOLDEN["raster_face_offsets"]
    grid = f["grid"]
    c = pi.raster_coords(grid)
    d = _desc(grid)
    slot, _, _ = oracle.index(d, c)
    nbr = oracle.neighbours(d, c, slot)
    face = {4: -64, 22: 64, 10: -8, 16: 8, 12: -1, 14: 1}  # offset index -> delta seq
    assert sorted(abs(v) for v in face.values()) == sorted(f["delta_seq"] * 2)
    interior = np.flatnonzero(np.all((c > 0) & (c < 7), axis=1))
    for i in interior:
        for kk, ds in face.items():
            assert nbr[i, kk] == i + ds


def test_lab_query_offset_under_raster():
    f = GOLDEN["lab_query"]
    grid = GOLDEN["lab_field"]["grid"]
    c = pi.raster_coords(grid)
    d = _desc(grid)
    slot, _, _ = oracle.index(d, c)
    q = slot[(f["query"][0] * 8 + f["query"][1]) * 8 + f["query"][2]]
    nbr = oracle.neighbours(d, c, slot)
    kk = (f["offset"][0] + 1) * 9 + (f["offset"][1] + 1) * 3 + (f["offset"][2] + 1)
    assert nbr[q, kk] - q == 64


def test_summary_counts_from_pages():
    lab = GOLDEN["lab_field"]
    assert oracle.num_blocks(_desc(lab["grid"], lab["block"])) == 64
    # 1,024 summaries per head at 262,144 tokens and 4,096 at 2^20 tokens both
    # mean 256 tokens per summary; a 4x8x8 block realises that on both grids
    for fact, grid in zip(GOLDEN["summaries_per_kv_head"], [(64, 64, 64), (64, 128, 128)]):
        assert np.prod(grid) == fact["tokens"]
        assert oracle.num_blocks(_desc(grid, (4, 8, 8))) == fact["summaries"]


@pytest.mark.parametrize("grid,block", [((8, 8, 8), (2, 2, 2)), ((5, 7, 3), (2, 3, 2)),
                                        ((64, 64, 64), (4, 4, 4)), ((16, 64, 64), (2, 2, 4))])
def test_block_ids_and_ranks(grid, block):
    c = pi.packing_coords(grid, "random", seed=3)
    d = _desc(grid, block)
    slot, blk, rank = oracle.index(d, c)
    assert np.array_equal(blk, block_ids(c, grid, block))
    assert oracle.num_blocks(d) == int(np.prod([-(-g // b) for g, b in zip(grid, block)]))
    # within a block every member has a distinct canonical slot
    key = blk.astype(np.int64) * np.prod(block) + rank
    assert np.unique(key).size == c.shape[0]
    assert rank.min() >= 0 and rank.max() < np.prod(block)
    # slot map inverts the packing
    sites = pi.coords_to_sites(c, grid)
    assert np.array_equal(slot[sites], np.arange(c.shape[0]))


def test_index_rejects_bad_coordinates():
    grid = (3, 3, 3)
    c = pi.raster_coords(grid).copy()
    d = _desc(grid)
    bad = c.copy()
    bad[5] = [0, 3, 0]
    with pytest.raises(oracle.OracleError, match="range"):
        oracle.index(d, bad)
    bad = c.copy()
    bad[5] = [-1, 0, 0]
    with pytest.raises(oracle.OracleError, match="range"):
        oracle.index(d, bad)
    dup = c.copy()
    dup[7] = dup[3]
    with pytest.raises(oracle.OracleError, match="duplicate"):
        oracle.index(d, dup)

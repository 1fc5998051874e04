"""Packings of a Z x Y x X token grid into memory order.

A packing is returned as int32 coords[N, 3]: coords[i] = (z, y, x) of the token
stored at memory position i. Raster, Morton, block-contiguous and random orders
are the layouts the pages name (Geometry Matters in Packed 3D Attention, paper
summary §3.4 and project page Ch. 1); the group-permuted repack moves whole
summary groups and keeps every membership (project page, "Take it home").
"""
import numpy as np


def _grid_sites(grid):
    Z, Y, X = grid
    z, y, x = np.meshgrid(np.arange(Z), np.arange(Y), np.arange(X), indexing="ij")
    return np.stack([z.ravel(), y.ravel(), x.ravel()], axis=1).astype(np.int32)


def raster_coords(grid):
    """x fastest, then y, then z."""
    return _grid_sites(grid)


def _morton_code(c, nbits):
    code = np.zeros(c.shape[0], dtype=np.int64)
    for b in range(nbits):
        code |= ((c[:, 2].astype(np.int64) >> b) & 1) << (3 * b)
        code |= ((c[:, 1].astype(np.int64) >> b) & 1) << (3 * b + 1)
        code |= ((c[:, 0].astype(np.int64) >> b) & 1) << (3 * b + 2)
    return code


def morton_coords(grid):
    """Bit-interleaved order (x -> bit 3b, y -> 3b+1, z -> 3b+2), ranked, so
    anisotropic grids are handled too."""
    c = _grid_sites(grid)
    nbits = max(int(max(grid) - 1).bit_length(), 1)
    return c[np.argsort(_morton_code(c, nbits), kind="stable")]


def block_contiguous_coords(grid, block):
    """Blocks in raster order, each block's tokens contiguous and in raster
    order inside the block (the layout the main experiments use)."""
    c = _grid_sites(grid)
    Z, Y, X = grid
    bz, by, bx = block
    My, Mx = -(-Y // by), -(-X // bx)
    bid = ((c[:, 0] // bz) * My + (c[:, 1] // by)) * Mx + (c[:, 2] // bx)
    inner = ((c[:, 0] % bz) * by + (c[:, 1] % by)) * bx + (c[:, 2] % bx)
    return c[np.lexsort((inner, bid))]


def block_morton_coords(grid, block):
    """Blocks in Morton order of their block coordinate, raster inside."""
    c = _grid_sites(grid)
    bz, by, bx = block
    bc = np.stack([c[:, 0] // bz, c[:, 1] // by, c[:, 2] // bx], axis=1)
    nbits = max(int(max(bc.max(axis=0))).bit_length(), 1)
    code = _morton_code(bc, nbits)
    inner = ((c[:, 0] % bz) * by + (c[:, 1] % by)) * bx + (c[:, 2] % bx)
    return c[np.lexsort((inner, code))]


def random_coords(grid, seed):
    c = _grid_sites(grid)
    rng = np.random.Generator(np.random.PCG64(seed))
    return c[rng.permutation(c.shape[0])]


def group_permuted_coords(coords, block, seed):
    """Pure repack: memory is cut into its summary groups (maximal runs of
    tokens of one block, in the order they appear), and whole groups are
    permuted; tokens inside a group keep their relative order."""
    bz, by, bx = block
    key = np.stack([coords[:, 0] // bz, coords[:, 1] // by, coords[:, 2] // bx], axis=1)
    change = np.ones(coords.shape[0], dtype=bool)
    change[1:] = np.any(key[1:] != key[:-1], axis=1)
    starts = np.flatnonzero(change)
    ends = np.append(starts[1:], coords.shape[0])
    rng = np.random.Generator(np.random.PCG64(seed))
    perm = rng.permutation(len(starts))
    order = np.concatenate([np.arange(starts[g], ends[g]) for g in perm])
    return coords[order]


def packing_coords(grid, kind, block=(2, 2, 2), seed=0, base=None):
    if kind == "raster":
        return raster_coords(grid)
    if kind == "morton":
        return morton_coords(grid)
    if kind == "block":
        return block_contiguous_coords(grid, block)
    if kind == "block_morton":
        return block_morton_coords(grid, block)
    if kind in ("random", "random2"):
        return random_coords(grid, seed)
    if kind == "group":
        src = base if base is not None else block_contiguous_coords(grid, block)
        return group_permuted_coords(src, block, seed)
    raise ValueError(f"unknown packing {kind!r}")


def coords_to_sites(coords, grid):
    Z, Y, X = grid
    c = coords.astype(np.int64)
    return (c[:, 0] * Y + c[:, 1]) * X + c[:, 2]


def order_between(coords_a, coords_b, grid):
    """Index array p with coords_b[p] == coords_a (p maps packing A's
    positions to where the same token sits in packing B)."""
    sa = coords_to_sites(coords_a, grid)
    sb = coords_to_sites(coords_b, grid)
    pos_b = np.empty(sb.shape[0], dtype=np.int64)
    pos_b[sb] = np.arange(sb.shape[0])
    return pos_b[sa]

"""Seeded synthetic inputs for the PACK3D forward operator.

This module is shared by the CPU oracle's tests and the GPU path's tests and
bench. It holds input construction only (workload shapes, random draws,
packings of a 3D token grid into memory order); none of the operator's
arithmetic lives here.

Workloads follow the shapes of the pages' experiments (Geometry Matters in
Packed 3D Attention: project page Ch. 1 lab field of 8x8x8 tokens with 2x2x2
blocks; Ch. 9 65k-token and 262k-token layers). Every draw is NumPy PCG64 with
seed 1000*workload + {Q:0, K:1, V:2, gate:3, permutation:4}.
"""
from .configs import WORKLOADS, Workload, workload
from .packing import (packing_coords, raster_coords, morton_coords, block_contiguous_coords,
                      block_morton_coords, random_coords, group_permuted_coords,
                      coords_to_sites, order_between)
from .fields import make_dout, make_fields, pack_fields, round_bf16

__all__ = [
    "WORKLOADS", "Workload", "workload",
    "packing_coords", "raster_coords", "morton_coords", "block_contiguous_coords",
    "block_morton_coords", "random_coords", "group_permuted_coords", "coords_to_sites",
    "order_between", "make_dout", "make_fields", "pack_fields", "round_bf16",
]

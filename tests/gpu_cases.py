"""Shared helpers for the GPU parity tests: seeded cases, device transfer,
oracle calls and the error metrics of the parity bar.

Bar: integer / index work bit-exact; fp32 outputs within 1e-4 of the oracle
measured per output vector as max|g - r| / max(max|r|, 1e-6); bf16 outputs
within 2e-2 absolute. The oracle sees the exact values the GPU sees (bf16
inputs upcast exactly to float64).
"""
import numpy as np
import torch

import oracle
import pack3d_inputs as pi

FP32_REL = 1e-4
BF16_ABS = 2e-2


def tdtype(w):
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


def inputs(w, packing=None, seed_perm=None):
    """coords (int32 [N,3]) and packed q, k, v, gate as float32 numpy."""
    packing = packing or w.packing
    coords = pi.packing_coords(w.grid, packing, block=w.block,
                               seed=seed_perm if seed_perm is not None else w.seed("perm"))
    fields = pi.make_fields(w)
    return (coords,) + pi.pack_fields(fields, coords, w.grid)


def to_dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(dtype).contiguous()


def desc_pair(w, exclusion=0, validate=False):
    import geometry_aware_sparse_amd as gas
    d = gas.make_desc(w.B, w.N, w.H, w.D, w.grid, w.block,
                      dtype=gas.PACK3D_BF16 if w.dtype == "bf16" else gas.PACK3D_F32,
                      rope_base=w.rope_base, exclusion=exclusion, validate=validate,
                      kv_heads=w.kv_heads)
    od = oracle.make_desc(w.B, w.N, w.H, w.D, w.grid, w.block, rope_base=w.rope_base,
                          exclusion=exclusion, kv_heads=w.kv_heads)
    return d, od


def err_fp32(got, ref):
    """max over output vectors of ||g - r||_inf / max(||r||_inf, 1e-6)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.abs(got - ref).max(axis=-1)
    den = np.maximum(np.abs(ref).max(axis=-1), 1e-6)
    return float((num / den).max())


def err_abs(got, ref):
    return float(np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64)).max())


def assert_close(w, got, ref, what=""):
    if w.dtype == "bf16":
        e = err_abs(got, ref)
        assert e <= BF16_ABS, f"{what}: max abs error {e:.3e} > {BF16_ABS}"
    else:
        e = err_fp32(got, ref)
        assert e <= FP32_REL, f"{what}: max rel error {e:.3e} > {FP32_REL}"
    return e


def host(t):
    return t.float().cpu().numpy()

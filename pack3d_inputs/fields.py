"""Seeded Q/K/V/gate fields defined on grid sites, then packed.

Values are drawn per grid site (raster site order), so that a repack is a pure
permutation of the same tokens. "iid" draws N(0,1); "smooth" blurs N(0,1)
with a separable Gaussian (sigma 2 tokens, radius 8, reflect boundary) along
z, y and x and standardises each channel, to give peaked attention. bf16
workloads draw in fp32 and round to bf16 (round to nearest even).
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np


def round_bf16(a, chunk=1 << 26):
    """Round fp32 values to the nearest bf16 (ties to even); returns fp32.

    Works in uint32 and in chunks, so that multi-GB fields need little extra
    memory: for every non-NaN pattern u <= 0xFF800000 the sum u + 0x8000
    cannot wrap, and NaNs are restored explicitly."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty_like(a)
    src = a.reshape(-1).view(np.uint32)
    dst = out.reshape(-1).view(np.uint32)
    for s0 in range(0, src.size, chunk):
        u = src[s0:s0 + chunk]
        r = u + np.uint32(0x7FFF)
        r += (u >> np.uint32(16)) & np.uint32(1)
        r &= np.uint32(0xFFFF0000)
        nan = ((u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000))
        r[nan] = np.uint32(0x7FC00000)
        dst[s0:s0 + chunk] = r
    return out


def _blur_axis(f, axis, sigma=2.0, radius=8):
    t = np.arange(-radius, radius + 1, dtype=np.float64)
    w = np.exp(-0.5 * (t / sigma) ** 2)
    w /= w.sum()
    pad = [(0, 0)] * f.ndim
    pad[axis] = (radius, radius)
    fp = np.pad(f, pad, mode="reflect")
    out = np.zeros_like(f, dtype=np.float64)
    n = f.shape[axis]
    for o, wt in enumerate(w):
        sl = [slice(None)] * f.ndim
        sl[axis] = slice(o, o + n)
        out += wt * fp[tuple(sl)]
    return out


def _draw(rng, shape, values, grid):
    """shape = (B, Z*Y*X, H, D) or (B, Z*Y*X, H); returns fp32 in site order."""
    if values == "iid":
        return rng.standard_normal(shape, dtype=np.float32)
    if values == "smooth":
        Z, Y, X = grid
        f = rng.standard_normal(shape, dtype=np.float32).astype(np.float64)
        f = f.reshape((shape[0], Z, Y, X) + tuple(shape[2:]))
        for ax in (1, 2, 3):
            f = _blur_axis(f, ax)
        f = f.reshape(shape)
        mu = f.mean(axis=(0, 1), keepdims=True)
        sd = f.std(axis=(0, 1), keepdims=True)
        return ((f - mu) / sd).astype(np.float32)
    raise ValueError(values)


def make_fields(w, values=None, shape_override=None):
    """Q [B, sites, H, D], K and V [B, sites, Hkv, D] and gate logits G
    [B, sites, H], fp32 arrays in raster site order (bf16-representable when
    the workload is bf16). Gate logits are iid N(0,1) for every workload."""
    values = values or w.values
    B, H, D = w.B, w.H, w.D
    N = w.N

    def field(name):
        # each field has its own seeded stream, so the fields can be drawn
        # concurrently (numpy releases the GIL while filling) with the same
        # values as one after the other
        rng = np.random.Generator(np.random.PCG64(w.seed(name)))
        if name == "g":
            a = rng.standard_normal((B, N, H), dtype=np.float32)
        else:
            heads = H if name == "q" else w.kv_heads
            a = _draw(rng, (B, N, heads, D), values, w.grid)
        return round_bf16(a) if w.dtype == "bf16" else a

    with ThreadPoolExecutor(max_workers=4) as pool:
        return tuple(pool.map(field, ("q", "k", "v", "g")))


def make_dout(w):
    """Output gradient dO [B, sites, H, D] for the backward: iid N(0,1) in
    raster site order (bf16-representable when the workload is bf16)."""
    rng = np.random.Generator(np.random.PCG64(w.seed("dout")))
    d = rng.standard_normal((w.B, w.N, w.H, w.D), dtype=np.float32)
    return round_bf16(d) if w.dtype == "bf16" else d


def pack_fields(fields, coords, grid):
    """Reorder site-ordered fields into the memory order given by coords."""
    Z, Y, X = grid
    c = coords.astype(np.int64)
    sites = (c[:, 0] * Y + c[:, 1]) * X + c[:, 2]
    return tuple(np.ascontiguousarray(f[:, sites]) for f in fields)

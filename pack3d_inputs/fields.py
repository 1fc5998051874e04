"""Seeded Q/K/V/gate fields defined on grid sites, then packed.

Values are drawn per grid site (raster site order), so that a repack is a pure
permutation of the same tokens. "iid" draws N(0,1); "smooth" blurs N(0,1)
with a separable Gaussian (sigma 2 tokens, radius 8, reflect boundary) along
z, y and x and standardises each channel, to give peaked attention. bf16
workloads draw in fp32 and round to bf16 (round to nearest even).
"""
import numpy as np


def round_bf16(a):
    """Round fp32 values to the nearest bf16 (ties to even); returns fp32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)
    out = r.view(np.float32).copy()
    nan = np.isnan(a)
    out[nan] = np.nan
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
    out = []
    for name in ("q", "k", "v"):
        rng = np.random.Generator(np.random.PCG64(w.seed(name)))
        heads = H if name == "q" else w.kv_heads
        out.append(_draw(rng, (B, N, heads, D), values, w.grid))
    rng = np.random.Generator(np.random.PCG64(w.seed("g")))
    out.append(rng.standard_normal((B, N, H), dtype=np.float32))
    if w.dtype == "bf16":
        out = [round_bf16(a) for a in out]
    return tuple(out)


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

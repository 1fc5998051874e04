"""CPU oracle for the PACK3D forward operator (TEST INFRASTRUCTURE).

A ctypes wrapper around oracle/pack3d_oracle.c (plain fp64 C). Only the test
suite, the smoke entry point and the benchmark's CPU-baseline leg may import
this package; the GPU library never does, and this package never imports the
GPU library.

All float inputs are converted to float64 (bf16 inputs are exactly
representable), outputs are float64 numpy arrays. Layouts: Q [B,N,H,D] and
K/V [B,N,Hkv,D] in packed (memory) order, coords int32 [N,3] as (z,y,x), gate
[B,N,H], summaries [B,Hkv,M,D]; Hkv (key/value heads) equals H unless the
descriptor sets fewer, query head h reading KV head h // (H // Hkv).
"""
import contextlib
import ctypes as C
import os

import numpy as np

from . import build as _build

_lib = None


class _Desc(C.Structure):
    _fields_ = [("B", C.c_int32), ("N", C.c_int32), ("H", C.c_int32), ("D", C.c_int32),
                ("grid", C.c_int32 * 3), ("block", C.c_int32 * 3),
                ("rope_base", C.c_double), ("scale", C.c_double), ("exclusion", C.c_int32),
                ("Hkv", C.c_int32)]


EXCLUSION = {"none": 0, "own_block": 1, "neighbourhood_blocks": 2}


def _load(path):
    L = C.CDLL(path)
    P = C.c_void_p
    L.ork_num_threads.restype = C.c_int
    L.ork_num_blocks.restype = C.c_int
    L.ork_num_blocks.argtypes = [P]
    L.ork_index.restype = C.c_int
    L.ork_index.argtypes = [P, P, P, P, P]
    for name, n in [("ork_neighbours", 4), ("ork_rope_axial", 4), ("ork_rope_sequence", 3),
                    ("ork_summaries", 6), ("ork_summaries_centre", 6)]:
        getattr(L, name).restype = None
        getattr(L, name).argtypes = [P] * n
    L.ork_local.restype = None
    L.ork_local.argtypes = [P] * 7 + [C.c_int, P]
    L.ork_global.restype = None
    L.ork_global.argtypes = [P] * 6 + [C.c_int, P]
    L.ork_mix.restype = None
    L.ork_mix.argtypes = [P] * 5 + [C.c_int, P]
    L.ork_backward.restype = C.c_int
    L.ork_backward.argtypes = [P] * 7 + [C.c_int] + [P] * 4
    return L


def lib():
    global _lib
    if _lib is None:
        path = _build.LIB
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
            _build.build()
        _lib = _load(path)
    return _lib


@contextlib.contextmanager
def use_library(path):
    """Temporarily route every call to another build of the oracle source
    (used by the pin-sensitivity tests, which plant mistakes in a copy)."""
    global _lib
    saved = lib()
    _lib = _load(path)
    try:
        yield
    finally:
        _lib = saved


def num_threads() -> int:
    return lib().ork_num_threads()


class OracleError(RuntimeError):
    pass


def _ptr(a):
    return a.ctypes.data_as(C.c_void_p) if a is not None else None


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _i32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def make_desc(B, N, H, D, grid, block, rope_base=10000.0, scale=0.0, exclusion="none",
              kv_heads=None):
    if kv_heads is not None and (kv_heads < 1 or H % kv_heads):
        raise ValueError("kv_heads must divide H")
    d = _Desc()
    d.B, d.N, d.H, d.D = B, N, H, D
    d.Hkv = H if kv_heads is None else int(kv_heads)
    d.grid[:] = list(grid)
    d.block[:] = list(block)
    d.rope_base = float(rope_base)
    d.scale = float(scale)
    d.exclusion = EXCLUSION[exclusion] if isinstance(exclusion, str) else int(exclusion)
    return d


def num_blocks(desc) -> int:
    return lib().ork_num_blocks(C.byref(desc))


def index(desc, coords):
    """Returns (slot_map [Z*Y*X], block_id [N], block_rank [N]); raises
    OracleError on an out-of-range or duplicate coordinate."""
    coords = _i32(coords)
    S = int(np.prod(desc.grid))
    slot = np.empty(S, np.int32)
    blk = np.empty(desc.N, np.int32)
    rank = np.empty(desc.N, np.int32)
    rc = lib().ork_index(C.byref(desc), _ptr(coords), _ptr(slot), _ptr(blk), _ptr(rank))
    if rc == -2:
        raise OracleError("coordinate out of range")
    if rc == -3:
        raise OracleError("duplicate coordinate")
    if rc != 0:
        raise OracleError(f"index error {rc}")
    return slot, blk, rank


def neighbours(desc, coords, slot):
    coords = _i32(coords)
    nbr = np.empty((desc.N, 27), np.int32)
    lib().ork_neighbours(C.byref(desc), _ptr(coords), _ptr(_i32(slot)), _ptr(nbr))
    return nbr


def kv_heads(desc) -> int:
    return desc.Hkv if desc.Hkv > 0 else desc.H


def _with_heads(desc, heads):
    # the rotations act on each [D] row alone; a K/V tensor has Hkv rows per token
    if heads == desc.H:
        return desc
    d = _Desc.from_buffer_copy(desc)
    d.H = d.Hkv = heads
    return d


def rope_axial(desc, coords, x):
    """x: [B, N, heads, D] with heads H (queries) or Hkv (keys)."""
    x = _f64(x)
    y = np.empty_like(x)
    lib().ork_rope_axial(C.byref(_with_heads(desc, x.shape[2])), _ptr(_i32(coords)), _ptr(x),
                         _ptr(y))
    return y


def rope_sequence(desc, x):
    x = _f64(x)
    y = np.empty_like(x)
    lib().ork_rope_sequence(C.byref(_with_heads(desc, x.shape[2])), _ptr(x), _ptr(y))
    return y


def summaries(desc, slot, kr, v):
    kr, v = _f64(kr), _f64(v)
    _check_kv(desc, kr, v)
    M = num_blocks(desc)
    ks = np.empty((desc.B, kv_heads(desc), M, desc.D))
    vs = np.empty_like(ks)
    lib().ork_summaries(C.byref(desc), _ptr(_i32(slot)), _ptr(kr), _ptr(v), _ptr(ks), _ptr(vs))
    return ks, vs


def summaries_centre(desc, slot, k, v):
    """Summary-centre variant: mean of the UNROTATED keys k, rotated once at
    the block centre; values as in summaries()."""
    k, v = _f64(k), _f64(v)
    _check_kv(desc, k, v)
    M = num_blocks(desc)
    ks = np.empty((desc.B, kv_heads(desc), M, desc.D))
    vs = np.empty_like(ks)
    lib().ork_summaries_centre(C.byref(desc), _ptr(_i32(slot)), _ptr(k), _ptr(v), _ptr(ks),
                               _ptr(vs))
    return ks, vs


def _check_kv(desc, *xs):
    for x in xs:
        if x.shape != (desc.B, desc.N, kv_heads(desc), desc.D):
            raise ValueError(f"K/V shape {x.shape}: expected [B, N, Hkv, D]")


def _rows(rows, N):
    if rows is None:
        return None, N
    r = _i32(rows)
    return r, int(r.shape[0])


def local(desc, coords, slot, qr, kr, v, rows=None):
    r, n = _rows(rows, desc.N)
    kr, v = _f64(kr), _f64(v)
    _check_kv(desc, kr, v)
    out = np.empty((desc.B, n, desc.H, desc.D))
    lib().ork_local(C.byref(desc), _ptr(_i32(coords)), _ptr(_i32(slot)), _ptr(_f64(qr)),
                    _ptr(kr), _ptr(v), _ptr(r), n, _ptr(out))
    return out


def global_(desc, coords, qr, ks, vs, rows=None):
    r, n = _rows(rows, desc.N)
    ks, vs = _f64(ks), _f64(vs)
    M = num_blocks(desc)
    for x in (ks, vs):
        if x.shape != (desc.B, kv_heads(desc), M, desc.D):
            raise ValueError(f"summary shape {x.shape}: expected [B, Hkv, M, D]")
    out = np.empty((desc.B, n, desc.H, desc.D))
    lib().ork_global(C.byref(desc), _ptr(_i32(coords)), _ptr(_f64(qr)), _ptr(ks),
                     _ptr(vs), _ptr(r), n, _ptr(out))
    return out


def mix(desc, gate, oloc, oglob, rows=None):
    r, n = _rows(rows, desc.N)
    out = np.empty((desc.B, n, desc.H, desc.D))
    lib().ork_mix(C.byref(desc), _ptr(_f64(gate)), _ptr(_f64(oloc)), _ptr(_f64(oglob)),
                  _ptr(r), n, _ptr(out))
    return out


def forward(desc, coords, q, k, v, gate, rows=None, rope="axial", return_parts=False,
            summary_rope="token"):
    """The whole operator, steps 0-5 in order. rope: "axial" (grid
    coordinates), "sequence" (packed-index control) or "none". summary_rope:
    "token" (rotate every key, then pool) or "centre" (pool unrotated keys,
    rotate the mean at the block centre; axial RoPE only)."""
    slot, _, _ = index(desc, coords)
    if rope == "axial":
        qr, kr = rope_axial(desc, coords, q), rope_axial(desc, coords, k)
    elif rope == "sequence":
        qr, kr = rope_sequence(desc, q), rope_sequence(desc, k)
    elif rope == "none":
        qr, kr = _f64(q), _f64(k)
    else:
        raise ValueError(rope)
    if summary_rope == "token":
        ks, vs = summaries(desc, slot, kr, v)
    elif summary_rope == "centre" and rope == "axial":
        ks, vs = summaries_centre(desc, slot, k, v)
    else:
        raise ValueError(summary_rope)
    ol = local(desc, coords, slot, qr, kr, v, rows)
    og = global_(desc, coords, qr, ks, vs, rows)
    o = mix(desc, gate, ol, og, rows)
    if return_parts:
        return o, dict(slot=slot, qr=qr, kr=kr, ks=ks, vs=vs, local=ol, glob=og)
    return o


def backward(desc, coords, q, k, v, gate, dout, summary_rope="token"):
    """Gradients (dq, dk, dv, dgate) of sum(dout * forward(...)) with respect
    to the unrotated q, k, v and the gate logits, axial RoPE. summary_rope:
    "token" or "centre" as in forward()."""
    if summary_rope not in ("token", "centre"):
        raise ValueError(summary_rope)
    q, k, v, gate, dout = _f64(q), _f64(k), _f64(v), _f64(gate), _f64(dout)
    _check_kv(desc, k, v)
    for x, shp in ((q, (desc.B, desc.N, desc.H, desc.D)), (dout, (desc.B, desc.N, desc.H, desc.D)),
                   (gate, (desc.B, desc.N, desc.H))):
        if x.shape != shp:
            raise ValueError(f"shape {x.shape}: expected {shp}")
    dq, dout_ = np.empty_like(q), dout
    dk, dv = np.empty_like(k), np.empty_like(v)
    dgate = np.empty_like(gate)
    rc = lib().ork_backward(C.byref(desc), _ptr(_i32(coords)), _ptr(q), _ptr(k), _ptr(v),
                            _ptr(gate), _ptr(dout_), 1 if summary_rope == "centre" else 0,
                            _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dgate))
    if rc == -2:
        raise OracleError("coordinate out of range")
    if rc == -3:
        raise OracleError("duplicate coordinate")
    if rc != 0:
        raise OracleError(f"backward error {rc}")
    return dq, dk, dv, dgate

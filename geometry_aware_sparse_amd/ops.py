"""Torch-tensor front end of the C entry points (marshalling only)."""
import ctypes as C

import torch

from ._lib import (PACK3D_BF16, PACK3D_EXACT_SOFTMAX, PACK3D_F32, PACK3D_NUM_BWD_STAGES,
                   PACK3D_NUM_STAGES,
                   PACK3D_SUMMARY_CENTRE,
                   PACK3D_VALIDATE, Desc, Pack3DError, library)

_DTYPES = {PACK3D_F32: torch.float32, PACK3D_BF16: torch.bfloat16}


def make_desc(B, N, H, D, grid, block, dtype=PACK3D_BF16, rope_base=10000.0, scale=0.0,
              exclusion=0, validate=False, exact_softmax=False, summary_centre=False,
              kv_heads=None):
    """kv_heads: key/value heads (grouped-query attention); None means H.
    Query head h reads KV head h // (H // kv_heads)."""
    if isinstance(dtype, torch.dtype):
        dtype = {torch.float32: PACK3D_F32, torch.bfloat16: PACK3D_BF16}[dtype]
    d = Desc()
    d.B, d.N, d.H, d.D = int(B), int(N), int(H), int(D)
    d.grid[:] = [int(x) for x in grid]
    d.block[:] = [int(x) for x in block]
    d.rope_base = float(rope_base)
    d.scale = float(scale)
    d.dtype = int(dtype)
    d.exclusion = int(exclusion)
    d.flags = ((PACK3D_VALIDATE if validate else 0) | (PACK3D_EXACT_SOFTMAX if exact_softmax else 0)
               | (PACK3D_SUMMARY_CENTRE if summary_centre else 0))
    d.kv_heads = 0 if kv_heads is None else int(kv_heads)
    return d


def kv_heads(desc):
    return desc.kv_heads if desc.kv_heads > 0 else desc.H


def _check(rc, what):
    if rc != 0:
        raise Pack3DError(rc, what)


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return C.c_void_p(t.data_ptr()) if t is not None else None


def _need(t, name, desc, shape, dtype=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    want = dtype if dtype is not None else _DTYPES[desc.dtype]
    if t.dtype != want:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {want}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _bnhd(desc):
    return (desc.B, desc.N, desc.H, desc.D)


def _bnkd(desc):
    return (desc.B, desc.N, kv_heads(desc), desc.D)


def pack3d_num_summaries(desc):
    m = library().pack3d_num_summaries(C.byref(desc))
    _check(0 if m >= 0 else int(m), "pack3d_num_summaries")
    return int(m)


def pack3d_geometry_layout(desc):
    so, to, nb = C.c_size_t(), C.c_size_t(), C.c_size_t()
    _check(library().pack3d_geometry_layout(C.byref(desc), C.byref(so), C.byref(to), C.byref(nb)),
           "pack3d_geometry_layout")
    return so.value, to.value, nb.value


def pack3d_geometry_bytes(desc):
    n = C.c_size_t()
    _check(library().pack3d_geometry_bytes(C.byref(desc), C.byref(n)), "pack3d_geometry_bytes")
    return n.value


def pack3d_workspace_bytes(desc):
    n = C.c_size_t()
    _check(library().pack3d_workspace_bytes(C.byref(desc), C.byref(n)), "pack3d_workspace_bytes")
    return n.value


def _mp(M):
    return (M + 31) // 32 * 32


def ksum_shape(desc, M=None):
    """k_sum: [B, Hkv, Mp/32, Dp/8, 32, 8], Mp = 32*ceil(M/32), Dp = 8*ceil(D/8);
    key summary (m, d) of KV head h at [b, h, m // 32, d // 8, m % 32, d % 8]."""
    M = pack3d_num_summaries(desc) if M is None else M
    return (desc.B, kv_heads(desc), _mp(M) // 32, (desc.D + 7) // 8, 32, 8)


def vsum_shape(desc, M=None):
    """v_sum: [B, Hkv, Mp/8, D, 8]; value summary (m, d) at [b, h, m // 8, d, m % 8]."""
    M = pack3d_num_summaries(desc) if M is None else M
    return (desc.B, kv_heads(desc), _mp(M) // 8, desc.D, 8)


def ksum_to_rows(ks, M, D):
    """[B, H, Mp/32, Dp/8, 32, 8] -> [B, H, M, D]."""
    B, H, M32, D8, _, _ = ks.shape
    return ks.permute(0, 1, 2, 4, 3, 5).reshape(B, H, M32 * 32, D8 * 8)[:, :, :M, :D].contiguous()


def ksum_from_rows(k_rows):
    """[B, H, M, D] -> [B, H, Mp/32, Dp/8, 32, 8], zero padding."""
    B, H, M, D = k_rows.shape
    Dp = (D + 7) // 8 * 8
    pad = k_rows.new_zeros((B, H, _mp(M), Dp))
    pad[:, :, :M, :D] = k_rows
    return pad.view(B, H, _mp(M) // 32, 32, Dp // 8, 8).permute(0, 1, 2, 4, 3, 5).contiguous()


def vsum_to_rows(vs, M):
    """[B, H, Mp/8, D, 8] -> [B, H, M, D]."""
    B, H, M8, D, _ = vs.shape
    return vs.permute(0, 1, 2, 4, 3).reshape(B, H, M8 * 8, D)[:, :, :M].contiguous()


def vsum_from_rows(v_rows):
    """[B, H, M, D] -> [B, H, Mp/8, D, 8], zero past M."""
    B, H, M, D = v_rows.shape
    pad = v_rows.new_zeros((B, H, _mp(M), D))
    pad[:, :, :M] = v_rows
    return pad.view(B, H, _mp(M) // 8, 8, D).permute(0, 1, 2, 4, 3).contiguous()


def slot_map_view(desc, geom):
    """The int32 slot map inside a geometry buffer, as a tensor view."""
    so, _, _ = pack3d_geometry_layout(desc)
    S = desc.grid[0] * desc.grid[1] * desc.grid[2]
    return geom[so:so + 4 * S].view(torch.int32)


def pack3d_index_build(desc, coords, geom=None, neighbours=False, blocks=False, ranks=False):
    """Returns (geom, nbr, block, rank); the last three are None unless asked."""
    _need(coords, "coords", desc, (desc.N, 3), torch.int32)
    nb = pack3d_geometry_bytes(desc)
    if geom is None:
        geom = torch.empty(nb, dtype=torch.uint8, device=coords.device)
    elif geom.numel() * geom.element_size() < nb or not geom.is_cuda:
        raise ValueError("geometry buffer too small or not on the GPU")
    dev = coords.device
    nbr = torch.empty((desc.N, 27), dtype=torch.int32, device=dev) if neighbours else None
    blk = torch.empty(desc.N, dtype=torch.int32, device=dev) if blocks else None
    rank = torch.empty(desc.N, dtype=torch.int32, device=dev) if ranks else None
    _check(library().pack3d_index_build(C.byref(desc), _ptr(coords), _ptr(geom), _ptr(nbr),
                                        _ptr(blk), _ptr(rank), _stream()), "pack3d_index_build")
    return geom, nbr, blk, rank


def pack3d_rope_coords(desc, coords, x, out=None):
    """x: [B, N, H, D], or [B, N, Hkv, D] (keys; rotated through a descriptor
    whose head count is Hkv)."""
    _need(coords, "coords", desc, (desc.N, 3), torch.int32)
    if x.dim() == 4 and x.shape[2] == kv_heads(desc) and x.shape[2] != desc.H:
        d = Desc.from_buffer_copy(desc)
        d.H, d.kv_heads = kv_heads(desc), 0
        desc = d
    _need(x, "x", desc, _bnhd(desc))
    out = torch.empty_like(x) if out is None else out
    _need(out, "out", desc, _bnhd(desc))
    _check(library().pack3d_rope_coords(C.byref(desc), _ptr(coords), _ptr(x), _ptr(out),
                                        _stream()), "pack3d_rope_coords")
    return out


def pack3d_block_summarize(desc, geom, k, v):
    _need(k, "k", desc, _bnkd(desc))
    _need(v, "v", desc, _bnkd(desc))
    M = pack3d_num_summaries(desc)
    ks = torch.empty(ksum_shape(desc, M), dtype=k.dtype, device=k.device)
    vs = torch.empty(vsum_shape(desc, M), dtype=k.dtype, device=k.device)
    _check(library().pack3d_block_summarize(C.byref(desc), _ptr(geom), _ptr(k), _ptr(v), _ptr(ks),
                                            _ptr(vs), _stream()), "pack3d_block_summarize")
    return ks, vs


def pack3d_local_attn(desc, geom, q, k, v, out=None):
    _need(q, "q", desc, _bnhd(desc))
    _need(k, "k", desc, _bnkd(desc))
    _need(v, "v", desc, _bnkd(desc))
    out = torch.empty_like(q) if out is None else out
    _need(out, "out", desc, _bnhd(desc))
    _check(library().pack3d_local_attn(C.byref(desc), _ptr(geom), _ptr(q), _ptr(k), _ptr(v),
                                       _ptr(out), _stream()), "pack3d_local_attn")
    return out


def pack3d_global_attn(desc, geom, coords, q, ks, vs, out=None):
    _need(coords, "coords", desc, (desc.N, 3), torch.int32)
    _need(q, "q", desc, _bnhd(desc))
    M = pack3d_num_summaries(desc)
    _need(ks, "k_sum", desc, ksum_shape(desc, M))
    _need(vs, "v_sum", desc, vsum_shape(desc, M))
    out = torch.empty_like(q) if out is None else out
    _need(out, "out", desc, _bnhd(desc))
    _check(library().pack3d_global_attn(C.byref(desc), _ptr(geom), _ptr(coords), _ptr(q),
                                        _ptr(ks), _ptr(vs), _ptr(out), _stream()),
           "pack3d_global_attn")
    return out


def pack3d_mix(desc, gate, o_local, o_global, out=None):
    _need(gate, "gate", desc, (desc.B, desc.N, desc.H))
    _need(o_local, "o_local", desc, _bnhd(desc))
    _need(o_global, "o_global", desc, _bnhd(desc))
    out = torch.empty_like(o_local) if out is None else out
    _need(out, "out", desc, _bnhd(desc))
    _check(library().pack3d_mix(C.byref(desc), _ptr(gate), _ptr(o_local), _ptr(o_global),
                                _ptr(out), _stream()), "pack3d_mix")
    return out


def pack3d_forward(desc, coords, q, k, v, gate, out=None, workspace=None, stage_events=None):
    """The whole operator. stage_events: None or a list of
    2*PACK3D_NUM_STAGES torch.cuda.Event(enable_timing=True) objects (a None
    entry skips that mark; every recorded event adds stream time)."""
    _need(coords, "coords", desc, (desc.N, 3), torch.int32)
    _need(q, "q", desc, _bnhd(desc))
    _need(k, "k", desc, _bnkd(desc))
    _need(v, "v", desc, _bnkd(desc))
    _need(gate, "gate", desc, (desc.B, desc.N, desc.H))
    out = torch.empty_like(q) if out is None else out
    _need(out, "out", desc, _bnhd(desc))
    nb = pack3d_workspace_bytes(desc)
    if workspace is None:
        workspace = torch.empty(nb, dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    ev = _events(stage_events, PACK3D_NUM_STAGES)
    _check(library().pack3d_forward(C.byref(desc), _ptr(coords), _ptr(q), _ptr(k), _ptr(v),
                                    _ptr(gate), _ptr(out), _ptr(workspace), C.c_size_t(ws_bytes),
                                    _stream(), ev), "pack3d_forward")
    return out


def pack3d_forward_noalloc(desc, coords, q, k, v, gate, out):
    """The whole operator with the library's own per-GPU scratch array as the
    workspace: the C call allocates nothing (out is the caller's)."""
    _need(coords, "coords", desc, (desc.N, 3), torch.int32)
    _need(q, "q", desc, _bnhd(desc))
    _need(k, "k", desc, _bnkd(desc))
    _need(v, "v", desc, _bnkd(desc))
    _need(gate, "gate", desc, (desc.B, desc.N, desc.H))
    _need(out, "out", desc, _bnhd(desc))
    _check(library().pack3d_forward_noalloc(C.byref(desc), _ptr(coords), _ptr(q), _ptr(k),
                                            _ptr(v), _ptr(gate), _ptr(out), _stream()),
           "pack3d_forward_noalloc")
    return out


def _events(stage_events, n):
    if stage_events is None:
        return None
    if len(stage_events) != 2 * n:
        raise ValueError(f"stage_events needs {2 * n} events")
    return (C.c_void_p * len(stage_events))(
        *[C.c_void_p(None if e is None else e.cuda_event) for e in stage_events])


def pack3d_saved_bytes(desc):
    n = C.c_size_t()
    _check(library().pack3d_saved_bytes(C.byref(desc), C.byref(n)), "pack3d_saved_bytes")
    return n.value


def saved_views(desc, saved):
    """(O_glob [B, N, H, D] in the descriptor's dtype, lse [B, N, H] fp32):
    views into the buffer pack3d_forward_train fills."""
    es = 2 if desc.dtype == PACK3D_BF16 else 4
    nrow = desc.B * desc.N * desc.H
    ob = (nrow * desc.D * es + 255) // 256 * 256
    og = saved[:nrow * desc.D * es].view(_DTYPES[desc.dtype]).view(_bnhd(desc))
    lse = saved[ob:ob + 4 * nrow].view(torch.float32).view(desc.B, desc.N, desc.H)
    return og, lse


def pack3d_forward_train(desc, coords, q, k, v, gate, out=None, saved=None, workspace=None,
                         stage_events=None):
    """The forward, also filling the buffer the backward needs. Returns
    (out, saved)."""
    _need(coords, "coords", desc, (desc.N, 3), torch.int32)
    _need(q, "q", desc, _bnhd(desc))
    _need(k, "k", desc, _bnkd(desc))
    _need(v, "v", desc, _bnkd(desc))
    _need(gate, "gate", desc, (desc.B, desc.N, desc.H))
    out = torch.empty_like(q) if out is None else out
    _need(out, "out", desc, _bnhd(desc))
    sb = pack3d_saved_bytes(desc)
    if saved is None:
        saved = torch.empty(sb, dtype=torch.uint8, device=q.device)
    if workspace is None:
        workspace = torch.empty(pack3d_workspace_bytes(desc), dtype=torch.uint8, device=q.device)
    _check(library().pack3d_forward_train(
        C.byref(desc), _ptr(coords), _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(out),
        _ptr(saved), C.c_size_t(saved.numel() * saved.element_size()), _ptr(workspace),
        C.c_size_t(workspace.numel() * workspace.element_size()), _stream(),
        _events(stage_events, PACK3D_NUM_STAGES)), "pack3d_forward_train")
    return out, saved


def pack3d_backward_workspace_bytes(desc):
    n = C.c_size_t()
    _check(library().pack3d_backward_workspace_bytes(C.byref(desc), C.byref(n)),
           "pack3d_backward_workspace_bytes")
    return n.value


def pack3d_backward(desc, coords, q, k, v, gate, saved, dout, workspace=None, grads=None,
                    stage_events=None):
    """Gradients (dq, dk, dv, dgate) of sum(dout * O) with respect to the
    unrotated q, k, v and the gate logits. saved: from pack3d_forward_train
    on the same inputs. grads: optional preallocated (dq, dk, dv, dgate)."""
    _need(coords, "coords", desc, (desc.N, 3), torch.int32)
    _need(q, "q", desc, _bnhd(desc))
    _need(k, "k", desc, _bnkd(desc))
    _need(v, "v", desc, _bnkd(desc))
    _need(gate, "gate", desc, (desc.B, desc.N, desc.H))
    _need(dout, "dout", desc, _bnhd(desc))
    if grads is None:
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v),
                 torch.empty_like(gate))
    dq, dk, dv, dg = grads
    _need(dq, "dq", desc, _bnhd(desc))
    _need(dk, "dk", desc, _bnkd(desc))
    _need(dv, "dv", desc, _bnkd(desc))
    _need(dg, "dgate", desc, (desc.B, desc.N, desc.H))
    if workspace is None:
        workspace = torch.empty(pack3d_backward_workspace_bytes(desc), dtype=torch.uint8,
                                device=q.device)
    _check(library().pack3d_backward(
        C.byref(desc), _ptr(coords), _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(saved),
        C.c_size_t(saved.numel() * saved.element_size()), _ptr(dout), _ptr(dq), _ptr(dk),
        _ptr(dv), _ptr(dg), _ptr(workspace),
        C.c_size_t(workspace.numel() * workspace.element_size()), _stream(),
        _events(stage_events, PACK3D_NUM_BWD_STAGES)), "pack3d_backward")
    return dq, dk, dv, dg

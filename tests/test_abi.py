"""The C ABI without a GPU: the library loads, exports every entry point that
include/pack3d.h declares, and rejects bad descriptors on the host before
anything is launched (each case is forced from the host; no kernel runs)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pack3d.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(pack3d_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def gas():
    import geometry_aware_sparse_amd
    return geometry_aware_sparse_amd


def test_library_exports_every_declared_symbol(gas):
    lib = C.CDLL(gas.LIB_PATH)
    names = _declared()
    assert len(names) == 18
    for n in names:
        assert hasattr(lib, n), f"{n} declared in pack3d.h but not exported"
    assert sorted(gas.EXPORTED_SYMBOLS) == names


def test_debug_build_loads_and_exports_the_same_symbols(gas):
    """lib/libpack3d_debug.so (checked slot-map reads) is built beside the
    library and declares the same ABI; inside debug_library() the binding
    calls it."""
    from geometry_aware_sparse_amd import _lib
    assert os.path.exists(_lib.DEBUG_LIB_PATH)
    dbg = C.CDLL(_lib.DEBUG_LIB_PATH)
    for n in _declared():
        assert hasattr(dbg, n), f"{n} missing from the debug build"
    with _lib.debug_library() as L:
        assert gas.library() is L
        assert L.pack3d_abi_version() == 2
        assert L.pack3d_strerror(-7) and b"debug" in L.pack3d_strerror(-7)
    assert gas.library() is not L


def test_version_and_strerror(gas):
    lib = gas.library()
    assert lib.pack3d_abi_version() == 2
    # the ctypes descriptor matches the C struct: kv_heads is the last field
    assert C.sizeof(gas.Desc) == 4 * 4 + 4 * 6 + 4 * 2 + 4 * 4
    for code in (0, -1, -2, -3, -4, -5, -6, -7, -99):
        assert lib.pack3d_strerror(code)


def _desc(gas, **kw):
    base = dict(B=1, N=512, H=2, D=48, grid=(8, 8, 8), block=(2, 2, 2), dtype=gas.PACK3D_BF16)
    base.update(kw)
    d = gas.make_desc(base["B"], base["N"], base["H"], base["D"], base["grid"], base["block"],
                      dtype=base["dtype"], rope_base=base.get("rope_base", 10000.0),
                      exclusion=base.get("exclusion", 0))
    d.kv_heads = base.get("kv_heads", 0)
    return d


@pytest.mark.parametrize("kw,code", [
    (dict(N=500), -2), (dict(D=40), -2), (dict(block=(0, 2, 2)), -2), (dict(grid=(8, 8, -8)), -2),
    (dict(B=0), -1), (dict(H=-1), -1), (dict(dtype=7), -1), (dict(exclusion=5), -1),
    (dict(rope_base=0.0), -1), (dict(H=64, D=48), -2),
    (dict(H=6, kv_heads=4), -2), (dict(kv_heads=-1), -1),
])
def test_bad_descriptors_are_rejected(gas, kw, code):
    d = _desc(gas, **kw)
    lib = gas.library()
    n = C.c_size_t()
    assert lib.pack3d_workspace_bytes(C.byref(d), C.byref(n)) == code
    assert lib.pack3d_num_summaries(C.byref(d)) == code
    fake = C.c_void_p(16)
    assert lib.pack3d_forward(C.byref(d), fake, fake, fake, fake, fake, fake, fake,
                              C.c_size_t(1 << 40), None, None) == code


def test_null_pointers_small_workspace_and_unsupported_head_dim(gas):
    lib = gas.library()
    d = _desc(gas)
    fake = C.c_void_p(16)
    assert lib.pack3d_forward(C.byref(d), None, fake, fake, fake, fake, fake, fake,
                              C.c_size_t(1 << 40), None, None) == -1
    n = C.c_size_t()
    assert lib.pack3d_workspace_bytes(C.byref(d), C.byref(n)) == 0
    assert lib.pack3d_forward(C.byref(d), fake, fake, fake, fake, fake, fake, fake,
                              C.c_size_t(n.value - 1), None, None) == -3
    d18 = _desc(gas, D=18)
    assert lib.pack3d_workspace_bytes(C.byref(d18), C.byref(n)) == 0
    assert lib.pack3d_forward(C.byref(d18), fake, fake, fake, fake, fake, fake, fake,
                              C.c_size_t(n.value), None, None) == -4
    assert lib.pack3d_index_build(None, fake, fake, None, None, None, None) == -1
    assert lib.pack3d_block_summarize(C.byref(d), None, fake, fake, fake, fake, None) == -1


def test_geometry_and_workspace_sizes(gas):
    d = _desc(gas)
    so, to, nb = gas.pack3d_geometry_layout(d)
    assert so == 256 and so % 256 == 0 and to % 256 == 0
    assert to >= so + 4 * 512
    assert nb >= to + (8 + 8 + 8 + 1) * (48 // 6) * 8  # a row per coordinate, one half-angle row
    M = gas.pack3d_num_summaries(d)
    assert M == 64
    assert gas.pack3d_workspace_bytes(d) >= nb + 2 * (1 * 2 * M * 48 * 2)
    # summaries are stored per KV head: 4 query heads over 2 KV heads need
    # the workspace of 2 heads, less than 4
    ws = gas.pack3d_workspace_bytes
    assert ws(_desc(gas, H=4, kv_heads=2)) == ws(_desc(gas, H=2)) < ws(_desc(gas, H=4))
    assert ws(_desc(gas, H=4, kv_heads=4)) == ws(_desc(gas, H=4))
    with pytest.raises(gas.Pack3DError, match="SHAPE"):
        gas.pack3d_num_summaries(_desc(gas, N=7))


def test_binding_refuses_host_tensors(gas):
    import torch
    d = _desc(gas)
    with pytest.raises(ValueError, match="GPU"):
        gas.pack3d_rope_coords(d, torch.zeros((512, 3), dtype=torch.int32),
                               torch.zeros((1, 512, 2, 48), dtype=torch.bfloat16))


def test_training_entry_points_check_arguments_on_the_host(gas):
    # every failure below is decided before anything is enqueued
    lib = gas.library()
    d = _desc(gas)
    fake = C.c_void_p(16)
    n, sb, bn = C.c_size_t(), C.c_size_t(), C.c_size_t()
    assert lib.pack3d_workspace_bytes(C.byref(d), C.byref(n)) == 0
    assert lib.pack3d_saved_bytes(C.byref(d), C.byref(sb)) == 0
    assert lib.pack3d_backward_workspace_bytes(C.byref(d), C.byref(bn)) == 0
    # saved = O_glob [B,N,H,D] bf16 then lse [B,N,H] fp32, each 256-aligned
    rows = 1 * 512 * 2
    assert sb.value == (rows * 48 * 2 + 255) // 256 * 256 + (rows * 4 + 255) // 256 * 256
    assert bn.value > n.value
    # training forward: missing saved buffer, too small a saved buffer
    assert lib.pack3d_forward_train(C.byref(d), fake, fake, fake, fake, fake, fake, None,
                                    C.c_size_t(sb.value), fake, C.c_size_t(n.value), None,
                                    None) == -1
    assert lib.pack3d_forward_train(C.byref(d), fake, fake, fake, fake, fake, fake, fake,
                                    C.c_size_t(sb.value - 1), fake, C.c_size_t(n.value), None,
                                    None) == -3
    # backward: null gradient pointer, small saved buffer, small workspace, bad descriptor
    args = [fake] * 6
    assert lib.pack3d_backward(C.byref(d), *args, C.c_size_t(sb.value), fake, None, fake, fake,
                               fake, fake, C.c_size_t(bn.value), None, None) == -1
    assert lib.pack3d_backward(C.byref(d), *args, C.c_size_t(sb.value - 1), fake, fake, fake,
                               fake, fake, fake, C.c_size_t(bn.value), None, None) == -3
    assert lib.pack3d_backward(C.byref(d), *args, C.c_size_t(sb.value), fake, fake, fake, fake,
                               fake, fake, C.c_size_t(bn.value - 1), None, None) == -3
    bad = _desc(gas, N=500)
    assert lib.pack3d_backward(C.byref(bad), *args, C.c_size_t(sb.value), fake, fake, fake, fake,
                               fake, fake, C.c_size_t(bn.value), None, None) == -2
    # unsupported head dim
    d18 = _desc(gas, D=18)
    assert lib.pack3d_backward_workspace_bytes(C.byref(d18), C.byref(bn)) == 0
    assert lib.pack3d_saved_bytes(C.byref(d18), C.byref(sb)) == 0
    assert lib.pack3d_backward(C.byref(d18), *args, C.c_size_t(sb.value), fake, fake, fake, fake,
                               fake, fake, C.c_size_t(bn.value), None, None) == -4

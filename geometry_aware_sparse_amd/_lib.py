"""ctypes declarations of include/pack3d.h."""
import contextlib
import ctypes as C
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libpack3d.so")

ABI_VERSION = 2  # layout of Desc below; the library must report the same
PACK3D_F32 = 0
PACK3D_BF16 = 1
PACK3D_EXCL_NONE = 0
PACK3D_EXCL_OWN_BLOCK = 1
PACK3D_EXCL_NEIGHBOURHOOD_BLOCKS = 2
PACK3D_VALIDATE = 0x1
PACK3D_EXACT_SOFTMAX = 0x2
PACK3D_SUMMARY_CENTRE = 0x4
PACK3D_NUM_STAGES = 4
PACK3D_NUM_BWD_STAGES = 3
PACK3D_NOALLOC_SCRATCH_BYTES = 32 << 20

STATUS = {0: "PACK3D_OK", -1: "PACK3D_ERR_INVALID_ARG", -2: "PACK3D_ERR_SHAPE",
          -3: "PACK3D_ERR_WORKSPACE", -4: "PACK3D_ERR_UNSUPPORTED", -5: "PACK3D_ERR_HIP",
          -6: "PACK3D_ERR_COORDS", -7: "PACK3D_ERR_INTERNAL"}


class Pack3DError(RuntimeError):
    def __init__(self, status, what=""):
        self.status = status
        name = STATUS.get(status, str(status))
        msg = f"{what}: {name}" if what else name
        try:
            msg += f" ({library().pack3d_strerror(status).decode()})"
        except Exception:  # library not loadable
            pass
        super().__init__(msg)


class Desc(C.Structure):
    _fields_ = [("B", C.c_int32), ("N", C.c_int32), ("H", C.c_int32), ("D", C.c_int32),
                ("grid", C.c_int32 * 3), ("block", C.c_int32 * 3), ("rope_base", C.c_float),
                ("scale", C.c_float), ("dtype", C.c_int32), ("exclusion", C.c_int32),
                ("flags", C.c_uint32), ("kv_heads", C.c_int32)]


_P = C.c_void_p
_SIGS = {
    "pack3d_abi_version": (C.c_int, []),
    "pack3d_strerror": (C.c_char_p, [C.c_int]),
    "pack3d_num_summaries": (C.c_int64, [_P]),
    "pack3d_geometry_bytes": (C.c_int, [_P, C.POINTER(C.c_size_t)]),
    "pack3d_geometry_layout": (C.c_int, [_P, C.POINTER(C.c_size_t), C.POINTER(C.c_size_t),
                                         C.POINTER(C.c_size_t)]),
    "pack3d_index_build": (C.c_int, [_P, _P, _P, _P, _P, _P, _P]),
    "pack3d_rope_coords": (C.c_int, [_P, _P, _P, _P, _P]),
    "pack3d_block_summarize": (C.c_int, [_P, _P, _P, _P, _P, _P, _P]),
    "pack3d_local_attn": (C.c_int, [_P, _P, _P, _P, _P, _P, _P]),
    "pack3d_global_attn": (C.c_int, [_P, _P, _P, _P, _P, _P, _P, _P]),
    "pack3d_mix": (C.c_int, [_P, _P, _P, _P, _P, _P]),
    "pack3d_workspace_bytes": (C.c_int, [_P, C.POINTER(C.c_size_t)]),
    "pack3d_forward": (C.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, C.c_size_t, _P, _P]),
    "pack3d_forward_noalloc": (C.c_int, [_P, _P, _P, _P, _P, _P, _P, _P]),
    "pack3d_saved_bytes": (C.c_int, [_P, C.POINTER(C.c_size_t)]),
    "pack3d_forward_train": (C.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, C.c_size_t, _P, C.c_size_t,
                                       _P, _P]),
    "pack3d_backward_workspace_bytes": (C.c_int, [_P, C.POINTER(C.c_size_t)]),
    "pack3d_backward": (C.c_int, [_P, _P, _P, _P, _P, _P, _P, C.c_size_t, _P, _P, _P, _P, _P, _P,
                                  C.c_size_t, _P, _P]),
}
EXPORTED_SYMBOLS = tuple(_SIGS)

_lib = None
_debug_lib = None
_use_debug = False
DEBUG_LIB_PATH = os.path.join(os.path.dirname(LIB_PATH), "libpack3d_debug.so")


def _load(path):
    if not os.path.exists(path):
        raise ImportError(f"PACK3D HIP library not built: {path} is missing "
                          "(run geometry_aware_sparse_amd/build.py)")
    L = C.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    if L.pack3d_abi_version() != ABI_VERSION:
        raise ImportError(f"{path} reports ABI {L.pack3d_abi_version()}, the binding "
                          f"expects {ABI_VERSION}: rebuild the library")
    return L


def library():
    """Load lib/libpack3d.so once; raises when it is missing (no fallback).
    Inside `with debug_library():` the debug build is returned instead."""
    global _lib
    if _use_debug:
        return _debug_lib
    if _lib is None:
        _lib = _load(LIB_PATH)
    return _lib


@contextlib.contextmanager
def debug_library():
    """Route every call of the binding to lib/libpack3d_debug.so (the build
    with checked slot-map reads, `build.py --debug`) inside the block."""
    global _debug_lib, _use_debug
    if _debug_lib is None:
        _debug_lib = _load(DEBUG_LIB_PATH)
    prev, _use_debug = _use_debug, True
    try:
        yield _debug_lib
    finally:
        _use_debug = prev

"""Python binding of the PACK3D gfx950 library (include/pack3d.h).

Argument marshalling only: every step of the operator runs in the HIP kernels
of lib/libpack3d.so. Functions carry the C entry points' names, take torch
tensors that already live on the GPU, pass their data pointers plus torch's
current HIP stream, and raise Pack3DError on any non-zero status. Importing
this package loads the library and fails loudly when it has not been built
(there is no CPU fallback).
"""
from ._lib import (PACK3D_BF16, PACK3D_EXCL_NEIGHBOURHOOD_BLOCKS, PACK3D_EXCL_NONE,
                   PACK3D_EXCL_OWN_BLOCK, PACK3D_F32, PACK3D_NUM_STAGES, PACK3D_VALIDATE,
                   PACK3D_EXACT_SOFTMAX, PACK3D_SUMMARY_CENTRE, PACK3D_NUM_BWD_STAGES,
                   PACK3D_NOALLOC_SCRATCH_BYTES, EXPORTED_SYMBOLS, LIB_PATH, DEBUG_LIB_PATH, Desc,
                   Pack3DError, debug_library, library)
from .ops import (kv_heads, make_desc, pack3d_backward, pack3d_backward_workspace_bytes,
                  pack3d_forward_train, pack3d_saved_bytes, saved_views, pack3d_block_summarize,
                  pack3d_forward, pack3d_forward_noalloc, pack3d_geometry_bytes,
                  pack3d_geometry_layout, pack3d_global_attn, pack3d_index_build,
                  pack3d_local_attn, pack3d_mix, pack3d_num_summaries, pack3d_rope_coords,
                  pack3d_workspace_bytes, slot_map_view, ksum_from_rows, ksum_shape,
                  ksum_to_rows, vsum_from_rows, vsum_shape, vsum_to_rows)

library()  # load now: no silent fallback when the HIP library is absent

__all__ = [
    "PACK3D_BF16", "PACK3D_F32", "PACK3D_EXCL_NONE", "PACK3D_EXCL_OWN_BLOCK",
    "PACK3D_EXCL_NEIGHBOURHOOD_BLOCKS", "PACK3D_VALIDATE", "PACK3D_EXACT_SOFTMAX",
    "PACK3D_SUMMARY_CENTRE", "PACK3D_NUM_STAGES", "PACK3D_NOALLOC_SCRATCH_BYTES",
    "EXPORTED_SYMBOLS", "LIB_PATH", "DEBUG_LIB_PATH", "Desc", "Pack3DError", "debug_library",
    "library", "kv_heads", "make_desc",
    "pack3d_block_summarize", "pack3d_forward", "pack3d_forward_noalloc", "pack3d_geometry_bytes",
    "pack3d_geometry_layout", "pack3d_global_attn", "pack3d_index_build", "pack3d_local_attn",
    "pack3d_mix", "pack3d_num_summaries", "pack3d_rope_coords", "pack3d_workspace_bytes",
    "slot_map_view", "ksum_from_rows", "ksum_shape", "ksum_to_rows", "vsum_from_rows",
    "vsum_shape", "vsum_to_rows", "PACK3D_NUM_BWD_STAGES", "pack3d_backward",
    "pack3d_backward_workspace_bytes", "pack3d_forward_train", "pack3d_saved_bytes", "saved_views",
]

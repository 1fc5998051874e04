"""pack3d_forward_noalloc: the forward with the library's fixed per-GPU
scratch array as its workspace, for callers that cannot allocate. Called
through the C ABI and compared with pack3d_forward (its own workspace) on two
calls in a row, the second on a smaller input, so the second call runs over
what the first left in the array; the results must be the same bits."""
import numpy as np
import pytest
import torch

import pack3d_inputs as pi
from gpu_cases import assert_close, desc_pair, host, inputs, tdtype, to_dev

pytestmark = pytest.mark.gpu

W = pi.Workload
SEQUENCE = [
    pi.workload(3),  # 32x32x64 grid, 8 heads, head dim 48: 12.6 MB of summaries
    W(150, "noalloc_ragged_bf16_d96", (6, 9, 11), 1, 2, 96, (2, 3, 2), "bf16", "smooth",
      "morton", "raster"),
    W(151, "noalloc_small_f32_d24", (5, 7, 9), 2, 6, 24, (2, 2, 3), "f32", "iid", "block",
      "random", Hkv=3),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _run(w):
    import geometry_aware_sparse_amd as gas
    coords, q, k, v, g = inputs(w)
    d, _ = desc_pair(w)
    dt = tdtype(w)
    dev = [to_dev(coords, torch.int32)] + [to_dev(x, dt) for x in (q, k, v, g)]
    assert gas.pack3d_workspace_bytes(d) <= gas.PACK3D_NOALLOC_SCRATCH_BYTES
    ref = gas.pack3d_forward(d, *dev)
    out = torch.full_like(ref, float("nan"))
    gas.pack3d_forward_noalloc(d, *dev, out)
    torch.cuda.synchronize()
    return w, ref, out


def test_noalloc_matches_forward_on_consecutive_calls():
    sizes = []
    for w in SEQUENCE:
        w, ref, out = _run(w)
        assert torch.equal(out, ref), f"{w.name}: no-alloc forward differs from pack3d_forward"
        sizes.append(w.B * w.N * w.H * w.D)
    assert sizes[1] < sizes[0] and sizes[2] < sizes[0]


def test_noalloc_small_case_against_oracle():
    # the smaller call, after the large one, also meets the parity bar itself
    import oracle
    w = SEQUENCE[1]
    _run(SEQUENCE[0])
    _, _, out = _run(w)
    coords, q, k, v, g = inputs(w)
    _, od = desc_pair(w)
    assert_close(w, host(out), oracle.forward(od, coords, q, k, v, g), "noalloc forward")


def test_noalloc_rejects_a_workspace_beyond_the_array():
    import geometry_aware_sparse_amd as gas
    # 64^3 tokens, 8 heads, one summary per site: 400 MB of summaries
    w = W(152, "noalloc_too_big", (64, 64, 64), 1, 8, 48, (1, 1, 1), "bf16", "iid", "raster",
          "raster")
    d, _ = desc_pair(w)
    assert gas.pack3d_workspace_bytes(d) > gas.PACK3D_NOALLOC_SCRATCH_BYTES
    small = torch.empty(1, device="cuda")
    lib = gas.library()
    import ctypes as C
    p = C.c_void_p(small.data_ptr())
    rc = lib.pack3d_forward_noalloc(C.byref(d), p, p, p, p, p, p, None)
    assert rc == -3  # PACK3D_ERR_WORKSPACE, checked on the host before any launch

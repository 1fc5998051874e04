"""Coordinate errors (project page Ch. 4: every token carries its grid
coordinate; a full grid holds each site once). With PACK3D_VALIDATE an
off-grid or repeated coordinate makes every entry point that builds the
geometry return PACK3D_ERR_COORDS; without it the status word records the
error, the kernels' own checks keep every access in bounds, and an off-grid
token takes no part (its rows stay zero)."""
import numpy as np
import pytest
import torch

import pack3d_inputs as pi
from gpu_cases import desc_pair, inputs, tdtype, to_dev

pytestmark = pytest.mark.gpu

W = pi.Workload
CASES = [W(140, "valid_bf16_d48", (4, 6, 8), 1, 2, 48, (2, 2, 2), "bf16", "iid", "random", "raster"),
         W(141, "valid_f32_d12", (3, 4, 5), 1, 2, 12, (2, 2, 2), "f32", "iid", "random", "raster")]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _bad(coords, kind):
    c = coords.copy()
    if kind == "off_grid":
        c[5] = [c[5][0], c[5][1], 10_000]       # x far past the grid
    else:
        c[5] = c[9]                               # site of token 9 claimed twice
    return c


@pytest.mark.parametrize("kind,bit", [("off_grid", 1), ("duplicate", 2)])
@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_validate_reports_coordinate_errors(w, kind, bit):
    import geometry_aware_sparse_amd as gas
    coords, q, k, v, g = inputs(w)
    bad = _bad(coords, kind)
    dt = tdtype(w)
    dev = [to_dev(bad, torch.int32)] + [to_dev(x, dt) for x in (q, k, v, g)]
    dv, _ = desc_pair(w, validate=True)
    for call in (lambda: gas.pack3d_index_build(dv, dev[0]),
                 lambda: gas.pack3d_forward(dv, *dev),
                 lambda: gas.pack3d_forward_train(dv, *dev)):
        with pytest.raises(gas.Pack3DError, match="COORDS"):
            call()
    # the backward builds the geometry too
    good = [to_dev(coords, torch.int32)] + dev[1:]
    dn, _ = desc_pair(w)
    _, saved = gas.pack3d_forward_train(dn, *good)
    with pytest.raises(gas.Pack3DError, match="COORDS"):
        gas.pack3d_backward(dv, *dev, saved, dev[1])
    # without validation: the status word carries the error bit, nothing faults
    geom, _, _, _ = gas.pack3d_index_build(dn, dev[0])
    torch.cuda.synchronize()
    assert int(geom[:4].view(torch.int32).item()) == bit
    o = gas.pack3d_forward(dn, *dev)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()
    if kind == "off_grid":
        assert torch.count_nonzero(o[:, 5]).item() == 0


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_validate_passes_valid_coordinates(w):
    import geometry_aware_sparse_amd as gas
    coords, q, k, v, g = inputs(w)
    dt = tdtype(w)
    dev = [to_dev(coords, torch.int32)] + [to_dev(x, dt) for x in (q, k, v, g)]
    dv, _ = desc_pair(w, validate=True)
    dn, _ = desc_pair(w)
    assert torch.equal(gas.pack3d_forward(dv, *dev), gas.pack3d_forward(dn, *dev))

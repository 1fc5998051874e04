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
def test_repeated_coordinate_lowest_index_wins(w):
    """Without validation a site claimed twice goes to the lowest memory index,
    whatever order the claims arrive in, and the other token takes no part:
    its output and gradient rows are zero, and the whole result is bit for bit
    that of the same tokens with the loser moved off the grid."""
    import geometry_aware_sparse_amd as gas
    coords, q, k, v, g = inputs(w)
    dup = _bad(coords, "duplicate")         # token 5 takes token 9's site
    off = dup.copy()
    off[9] = [off[9][0], off[9][1], 10_000]  # the same, with token 9 off the grid
    dt = tdtype(w)
    dn, _ = desc_pair(w)
    vals = [to_dev(x, dt) for x in (q, k, v, g)]
    dout = to_dev(pi.pack_fields((pi.make_dout(w),), coords, w.grid)[0], dt)
    results = []
    for c in (dup, off, dup):
        dc = to_dev(c, torch.int32)
        geom, _, _, _ = gas.pack3d_index_build(dn, dc)
        slot = gas.slot_map_view(dn, geom).cpu().numpy()
        o, saved = gas.pack3d_forward_train(dn, dc, *vals)
        grads = gas.pack3d_backward(dn, dc, *vals, saved, dout)
        torch.cuda.synchronize()
        results.append((slot, o, grads))
    Z, Y, X = w.grid
    z, y, x = coords[9]
    assert results[0][0][(z * Y + y) * X + x] == 5
    assert np.array_equal(results[0][0], results[1][0])
    for slot, o, grads in results:
        assert torch.count_nonzero(o[:, 9]).item() == 0
        for gr in grads:
            assert torch.count_nonzero(gr[:, 9]).item() == 0
        assert torch.isfinite(o.float()).all()
    for a, b in ((results[0], results[1]), (results[0], results[2])):
        assert torch.equal(a[1], b[1])
        for ga, gb in zip(a[2], b[2]):
            assert torch.equal(ga, gb)


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_validate_passes_valid_coordinates(w):
    import geometry_aware_sparse_amd as gas
    coords, q, k, v, g = inputs(w)
    dt = tdtype(w)
    dev = [to_dev(coords, torch.int32)] + [to_dev(x, dt) for x in (q, k, v, g)]
    dv, _ = desc_pair(w, validate=True)
    dn, _ = desc_pair(w)
    assert torch.equal(gas.pack3d_forward(dv, *dev), gas.pack3d_forward(dn, *dev))


def test_stage_events_with_skipped_marks():
    """stage_events entries may be None (NULL in the C ABI): those marks are
    skipped, the others recorded; the result does not depend on them."""
    import geometry_aware_sparse_amd as gas
    w = pi.workload(2)
    coords, q, k, v, g = inputs(w)
    d, _ = desc_pair(w)
    dt = tdtype(w)
    dev = [to_dev(coords, torch.int32)] + [to_dev(a, dt) for a in (q, k, v, g)]
    ref = gas.pack3d_forward(d, *dev)
    n = 2 * gas.PACK3D_NUM_STAGES
    for only in (None, 2):  # every mark, then the global stage's two only
        evs = [torch.cuda.Event(enable_timing=True) if only is None or j // 2 == only else None
               for j in range(n)]
        for e in evs:
            if e is not None:
                e.record()
        out = gas.pack3d_forward(d, *dev, stage_events=evs)
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        for s in range(gas.PACK3D_NUM_STAGES):
            if evs[2 * s] is not None:
                assert evs[2 * s].elapsed_time(evs[2 * s + 1]) > 0


def test_backward_stage_events_with_skipped_marks():
    """The same for pack3d_backward: marks whose entries are None are
    skipped, including the two the global-branch dispatch records itself."""
    import geometry_aware_sparse_amd as gas
    w = pi.workload(2)
    coords, q, k, v, g = inputs(w)
    dout = pi.pack_fields((pi.make_dout(w),), coords, w.grid)[0]
    d, _ = desc_pair(w)
    dt = tdtype(w)
    dev = [to_dev(coords, torch.int32)] + [to_dev(a, dt) for a in (q, k, v, g)]
    ddo = to_dev(dout, dt)
    _, saved = gas.pack3d_forward_train(d, *dev)
    ref = gas.pack3d_backward(d, *dev, saved, ddo)
    n = 2 * gas.PACK3D_NUM_BWD_STAGES
    for only in (None, 0, 1, 2):
        evs = [torch.cuda.Event(enable_timing=True) if only is None or j // 2 == only else None
               for j in range(n)]
        for e in evs:
            if e is not None:
                e.record()
        grads = gas.pack3d_backward(d, *dev, saved, ddo, stage_events=evs)
        torch.cuda.synchronize()
        for a, b in zip(grads, ref):
            assert torch.equal(a, b)
        for s in range(gas.PACK3D_NUM_BWD_STAGES):
            if evs[2 * s] is not None:
                assert evs[2 * s].elapsed_time(evs[2 * s + 1]) > 0

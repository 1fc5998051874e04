"""Packing equivariance of the GPU operator, bit for bit (project page Ch. 4,
Prop. 2; paper summary §B.3), with the repack recipe of the project page's
"Take it home" section: repack the tokens with their coordinates, run the
same forward, restore spatial order, compare. Also: two runs of the same
input give the same bits.
"""
import numpy as np
import pytest
import torch

import pack3d_inputs as pi
from gpu_cases import desc_pair, tdtype, to_dev

pytestmark = pytest.mark.gpu

W = pi.Workload
SMALL = [
    (pi.workload(1), "raster", "morton"),
    (pi.workload(1), "raster", "random"),
    (pi.workload(2), "morton", "block"),
    (pi.workload(2), "block", "group"),
    (W(111, "ragged", (10, 13, 19), 2, 3, 48, (2, 2, 2), "bf16", "iid", "random", "raster"),
     "random", "block_morton"),
    (W(112, "d96", (6, 8, 12), 1, 2, 96, (2, 2, 4), "bf16", "smooth", "block", "raster"),
     "block", "raster"),
    # grouped key/value heads
    (W(113, "gqa4x2", (10, 13, 19), 1, 4, 48, (2, 2, 2), "bf16", "iid", "random", "raster", Hkv=2),
     "random", "block_morton"),
    (W(114, "mqa_f32", (6, 7, 9), 2, 3, 24, (2, 2, 2), "f32", "iid", "raster", "random", Hkv=1),
     "raster", "random"),
]


BY_ID = {f"{w.name}-{a}-{b}": (w, a, b) for w, a, b in SMALL}
assert len(BY_ID) == len(SMALL)
CENTRE = ["grid8_fp32-raster-random", "ragged-random-block_morton", "gqa4x2-random-block_morton",
          "mqa_f32-raster-random"]
assert any(BY_ID[n][0].kv_heads < BY_ID[n][0].H for n in CENTRE)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _forward_in(w, kind, fields, base=None, centre=False):
    import geometry_aware_sparse_amd as gas
    if kind == "group":
        coords = pi.group_permuted_coords(base, w.block, w.seed("perm2"))
    else:
        seed = w.seed("perm2") if kind == "random2" else w.seed("perm")
        coords = pi.packing_coords(w.grid, kind, block=w.block, seed=seed)
    q, k, v, g = pi.pack_fields(fields, coords, w.grid)
    d, _ = desc_pair(w)
    if centre:
        d.flags |= gas.PACK3D_SUMMARY_CENTRE
    dt = tdtype(w)
    o = gas.pack3d_forward(d, to_dev(coords, torch.int32), to_dev(q, dt), to_dev(k, dt),
                           to_dev(v, dt), to_dev(g, dt))
    return coords, o


def _check(w, a, b, centre=False):
    fields = pi.make_fields(w)
    ca, oa = _forward_in(w, a, fields, centre=centre)
    cb, ob = _forward_in(w, b, fields, base=ca, centre=centre)
    p = torch.from_numpy(pi.order_between(ca, cb, w.grid)).to("cuda")
    assert torch.equal(oa, ob[:, p]), f"{w.name}: {a} vs {b} differ"
    assert torch.isfinite(oa.float()).all()


@pytest.mark.parametrize("w,a,b", SMALL, ids=[f"{w.name}-{a}-{b}" for w, a, b in SMALL])
def test_repack_permutes_output_bitwise(w, a, b):
    _check(w, a, b)


def test_deterministic_replay():
    import geometry_aware_sparse_amd as gas
    w = BY_ID["ragged-random-block_morton"][0]
    fields = pi.make_fields(w)
    coords = pi.packing_coords(w.grid, "random", seed=3)
    q, k, v, g = pi.pack_fields(fields, coords, w.grid)
    d, _ = desc_pair(w)
    dt = tdtype(w)
    args = (to_dev(coords, torch.int32), to_dev(q, dt), to_dev(k, dt), to_dev(v, dt), to_dev(g, dt))
    o1 = gas.pack3d_forward(d, *args)
    o2 = gas.pack3d_forward(d, *args)
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("name", CENTRE)
def test_repack_permutes_output_bitwise_summary_centre(name):
    _check(*BY_ID[name], centre=True)

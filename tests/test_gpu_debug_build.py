"""The debug build, lib/libpack3d_debug.so: every slot-map read in every
kernel is checked against the grid, and one out of range would set bit 2 of
the status word, which the entry points report as PACK3D_ERR_INTERNAL under
PACK3D_VALIDATE. On cases that reach every kernel family -- both dtypes,
head dims 12 to 96, grouped KV heads, ragged grids with partial blocks, one
axis a single site long, a single site, the exclusion readings (the
vector-unit global branch) and the summary-centre variant -- each entry
point that reads the slot map runs validated without the check firing, and
its results meet the normal build's bars against the oracle (index work bit
for bit)."""
import numpy as np
import pytest
import torch

import oracle
import pack3d_inputs as pi
from gpu_cases import assert_close, desc_pair, host, inputs, tdtype, to_dev

pytestmark = pytest.mark.gpu

W = pi.Workload
# (workload, exclusion reading, summary RoPE)
CASES = [
    (pi.workload(2), 0, "token"),
    (W(201, "dbg_ragged_bf16_d48", (10, 13, 19), 2, 3, 48, (2, 2, 2), "bf16", "iid", "random",
       "raster"), 0, "token"),
    (W(202, "dbg_mqa_bf16_d96", (6, 9, 11), 1, 4, 96, (2, 3, 2), "bf16", "smooth", "morton",
       "raster", Hkv=1), 0, "token"),
    (W(203, "dbg_gqa_f32_d24", (5, 7, 9), 2, 6, 24, (2, 2, 3), "f32", "iid", "block", "raster",
       Hkv=3), 1, "token"),
    (W(204, "dbg_slab_bf16_d12", (1, 12, 21), 1, 2, 12, (1, 2, 2), "bf16", "iid", "random",
       "raster"), 2, "token"),
    (W(205, "dbg_centre_bf16_d48", (6, 8, 10), 1, 2, 48, (2, 2, 3), "bf16", "iid", "random",
       "raster"), 0, "centre"),
    (W(206, "dbg_single_site", (1, 1, 1), 1, 1, 48, (1, 1, 1), "bf16", "iid", "raster",
       "raster"), 0, "token"),
]
IDS = [w.name for w, _, _ in CASES]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import geometry_aware_sparse_amd  # noqa: F401


def _setup(w, excl, sr):
    import geometry_aware_sparse_amd as gas
    coords, q, k, v, g = inputs(w)
    d, od = desc_pair(w, exclusion=excl, validate=True)
    if sr == "centre":
        d.flags |= gas.PACK3D_SUMMARY_CENTRE
    dt = tdtype(w)
    dev = [to_dev(coords, torch.int32)] + [to_dev(x, dt) for x in (q, k, v, g)]
    return gas, d, od, coords, (q, k, v, g), dev


@pytest.mark.parametrize("w,excl,sr", CASES, ids=IDS)
def test_debug_build_stages_and_forward(w, excl, sr):
    gas, d, od, coords, (q, k, v, g), dev = _setup(w, excl, sr)
    dc, dq, dk, dv, dg = dev
    with gas.debug_library():
        geom, nbr, _, _ = gas.pack3d_index_build(d, dc, neighbours=True)
        ks, vs = gas.pack3d_block_summarize(d, geom, dk, dv)
        ol = gas.pack3d_local_attn(d, geom, dq, dk, dv)
        og = gas.pack3d_global_attn(d, geom, dc, dq, ks, vs)
        o = gas.pack3d_forward(d, dc, dq, dk, dv, dg)
        torch.cuda.synchronize()
    slot, _, _ = oracle.index(od, coords)
    assert np.array_equal(nbr.cpu().numpy(), oracle.neighbours(od, coords, slot))
    qr, kr = oracle.rope_axial(od, coords, q), oracle.rope_axial(od, coords, k)
    assert_close(w, host(ol), oracle.local(od, coords, slot, qr, kr, v), "debug local")
    if sr == "token":
        oks, ovs = oracle.summaries(od, slot, kr, v)
        assert_close(w, host(og), oracle.global_(od, coords, qr, oks, ovs), "debug global")
    assert_close(w, host(o), oracle.forward(od, coords, q, k, v, g, summary_rope=sr),
                 "debug forward")


BWD = [CASES[1], CASES[2], CASES[3], CASES[5]]


@pytest.mark.parametrize("w,excl,sr", BWD, ids=[w.name for w, _, _ in BWD])
def test_debug_build_backward(w, excl, sr):
    gas, d, od, coords, (q, k, v, g), dev = _setup(w, excl, sr)
    dout = pi.pack_fields((pi.make_dout(w),), coords, w.grid)[0]
    with gas.debug_library():
        o, saved = gas.pack3d_forward_train(d, *dev)
        grads = gas.pack3d_backward(d, *dev, saved, to_dev(dout, tdtype(w)))
        torch.cuda.synchronize()
    ref = oracle.backward(od, coords, q, k, v, g, dout, summary_rope=sr)
    tol = 1e-2 if w.dtype == "bf16" else 1e-4
    for name, gg, r in zip(("dq", "dk", "dv", "dgate"), grads, ref):
        bar = max(float(np.abs(r).max()), 1.0)
        err = float(np.abs(host(gg) - r).max())
        assert err <= tol * bar, f"debug {w.name} {name}: {err:.3e} > {tol} * {bar:.3f}"

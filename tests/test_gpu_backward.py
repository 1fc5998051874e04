"""GPU parity of the backward (pack3d_forward_train + pack3d_backward)
against the oracle's fp64 gradients, on seeded inputs spanning both dtypes,
every head-dim family, grouped KV heads, both summary RoPE variants and the
exclusion readings.

Bar (per gradient tensor, r = oracle, bar = max(max|r|, 1)):
  fp32: max|g - r| <= 1e-4 * bar
  bf16: max|g - r| <= 1e-2 * bar
The bf16 bar follows from the arithmetic: inputs are bf16 (exact in the
oracle), accumulation is fp32, and every gradient is rounded once to bf16
on output (relative 2^-9 = 2e-3 of its own size) after summing terms that
were formed from bf16 summaries (relative 2^-9 each); measured errors stay
below 5e-3 * bar. Gates saturated to one side isolate each branch (g = 1:
only the global branch and the pooling path carry gradient; g = 0: only
the local branch), so a dropped term cannot hide under the other branch.
"""
import numpy as np
import pytest
import torch

import oracle
import pack3d_inputs as pi
from gpu_cases import desc_pair, host, inputs, tdtype, to_dev

pytestmark = pytest.mark.gpu

W = pi.Workload
CASES = [
    (pi.workload(1), "token", 0),
    (W(120, "f32_d12_gqa", (5, 6, 7), 2, 4, 12, (2, 2, 3), "f32", "iid", "random", "raster", Hkv=2),
     "token", 0),
    (W(121, "bf16_d48_gqa", (6, 8, 10), 1, 4, 48, (2, 2, 2), "bf16", "iid", "block", "random",
       Hkv=2), "token", 0),
    (W(122, "bf16_d96_mqa", (4, 6, 8), 1, 2, 96, (2, 2, 4), "bf16", "smooth", "morton", "raster",
       Hkv=1), "token", 0),
    (W(123, "f32_d48_centre", (4, 5, 6), 1, 2, 48, (2, 2, 2), "f32", "iid", "random", "raster"),
     "centre", 0),
    (W(124, "f32_d96", (3, 4, 5), 1, 1, 96, (1, 2, 2), "f32", "iid", "random", "raster"), "token", 0),
    (W(125, "bf16_d24_centre", (5, 5, 9), 2, 2, 24, (3, 3, 3), "bf16", "iid", "random", "raster"),
     "centre", 0),
    (pi.workload(2), "token", 0),
    (W(126, "f32_d24_own_block", (4, 6, 5), 1, 2, 24, (2, 3, 2), "f32", "iid", "random", "raster",
       Hkv=1), "token", 1),
    (W(127, "bf16_d48_nbhd_blocks", (6, 6, 8), 1, 2, 48, (2, 2, 2), "bf16", "iid", "random",
       "raster"), "token", 2),
    (W(128, "bf16_d48_mha", (8, 12, 16), 2, 4, 48, (2, 2, 2), "bf16", "iid", "block", "random"),
     "token", 0),
    # 72 summaries: the matrix-core query side's last 64-summary tile is half full
    (W(129, "bf16_d48_m72_half_tile", (6, 8, 12), 1, 2, 48, (2, 2, 2), "bf16", "iid", "random",
       "raster"), "token", 0),
    (W(130, "bf16_d48_single_site", (1, 1, 1), 1, 2, 48, (1, 1, 1), "bf16", "iid", "raster",
       "raster", Hkv=1), "token", 0),
    # the query side's pipeline at head dim 48 runs iterations of eight
    # 32-summary sub-tiles: 288 summaries fill nine sub-tiles exactly (one
    # unmasked iteration, then a tail of one sub-tile); 300 end in a partial
    # sub-tile, with grouped KV heads
    (W(131, "bf16_d48_m288_nine_subtiles", (8, 12, 24), 1, 2, 48, (2, 2, 2), "bf16", "iid",
       "random", "raster"), "token", 0),
    (W(132, "bf16_d48_m300_ragged_tail", (10, 12, 20), 1, 4, 48, (2, 2, 2), "bf16", "iid", "block",
       "raster", Hkv=2), "token", 0),
    # the matrix-core local backward at head dim 48 with the summary-centre
    # variant (its key side routes dK~ through the block-centre rotation),
    # grouped heads and boxes cut by the grid edge
    (W(133, "bf16_d48_centre_gqa", (6, 9, 10), 1, 4, 48, (2, 3, 2), "bf16", "iid", "random",
       "raster", Hkv=2), "centre", 0),
]
IDS = [f"{w.name}-{sr}" for w, sr, _ in CASES]
BY_NAME = {w.name: (w, sr, excl) for w, sr, excl in CASES}
assert len(BY_NAME) == len(CASES), "case names are unique"
# gates saturated to one side: one grouped case per dtype, D = 96 multi-query,
# the centre variant in both dtypes
BRANCH_CASES = ["f32_d12_gqa", "bf16_d48_gqa", "bf16_d96_mqa", "f32_d48_centre",
                "bf16_d24_centre"]
REPACK_CASES = ["bf16_d48_gqa", "bf16_d24_centre"]
assert any(BY_NAME[n][0].kv_heads < BY_NAME[n][0].H for n in BRANCH_CASES)
assert {BY_NAME[n][1] for n in BRANCH_CASES} == {"token", "centre"}
assert {BY_NAME[n][0].dtype for n in BRANCH_CASES} == {"f32", "bf16"}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import geometry_aware_sparse_amd  # noqa: F401


def _run(w, sr, excl, gate_override=None, packing=None):
    import geometry_aware_sparse_amd as gas
    coords, q, k, v, g = inputs(w, packing=packing)
    if gate_override is not None:
        g = np.full_like(g, gate_override)
    dout = pi.pack_fields((pi.make_dout(w),), coords, w.grid)[0]
    d, od = desc_pair(w, exclusion=excl)
    if sr == "centre":
        d.flags |= gas.PACK3D_SUMMARY_CENTRE
    dt = tdtype(w)
    dev = [to_dev(coords, torch.int32)] + [to_dev(x, dt) for x in (q, k, v, g)]
    o, saved = gas.pack3d_forward_train(d, *dev)
    grads = gas.pack3d_backward(d, *dev, saved, to_dev(dout, dt))
    return gas, d, od, coords, (q, k, v, g, dout), dev, o, saved, grads


def _assert_grads(w, grads, ref, what):
    tol = 1e-2 if w.dtype == "bf16" else 1e-4
    for name, gg, r in zip(("dq", "dk", "dv", "dgate"), grads, ref):
        gh = host(gg)
        assert np.isfinite(gh).all(), f"{what} {name}: non-finite"
        bar = max(float(np.abs(r).max()), 1.0)
        err = float(np.abs(gh - r).max())
        assert err <= tol * bar, f"{what} {name}: {err:.3e} > {tol} * {bar:.3f}"


@pytest.mark.parametrize("w,sr,excl", CASES, ids=IDS)
def test_backward_matches_oracle(w, sr, excl):
    gas, d, od, coords, (q, k, v, g, dout), dev, o, saved, grads = _run(w, sr, excl)
    # the training forward gives the inference forward's output, bit for bit
    assert torch.equal(o, gas.pack3d_forward(d, *dev))
    og, lse = gas.saved_views(d, saved)
    assert torch.isfinite(og.float()).all() and not torch.isnan(lse).any()
    ref = oracle.backward(od, coords, q, k, v, g, dout, summary_rope=sr)
    _assert_grads(w, grads, ref, w.name)


@pytest.mark.parametrize("gate", [30.0, -30.0], ids=["global_only", "local_only"])
@pytest.mark.parametrize("name", BRANCH_CASES)
def test_backward_each_branch_alone(name, gate):
    w, sr, excl = BY_NAME[name]
    gas, d, od, coords, (q, k, v, g, dout), dev, o, saved, grads = _run(w, sr, excl,
                                                                       gate_override=gate)
    ref = oracle.backward(od, coords, q, k, v, g, dout, summary_rope=sr)
    _assert_grads(w, grads, ref, f"{w.name} gate {gate}")


def test_saved_lse_is_the_global_log_sum_exp():
    # lse = log2 sum_m exp2(t_m), t = <q~, k_sum_m> * scale * log2(e), per (b, i, h)
    w, sr, excl = BY_NAME["f32_d12_gqa"]
    gas, d, od, coords, (q, k, v, g, dout), dev, o, saved, grads = _run(w, sr, excl)
    _, lse = gas.saved_views(d, saved)
    slot, _, _ = oracle.index(od, coords)
    ks, _ = oracle.summaries(od, slot, oracle.rope_axial(od, coords, k), v)
    qr = oracle.rope_axial(od, coords, q)
    G = w.H // w.kv_heads
    t = np.einsum("bnhd,bhmd->bnhm", qr, np.repeat(ks, G, axis=1)) * (np.log2(np.e) / np.sqrt(w.D))
    ref = np.log2(np.exp2(t - t.max(-1, keepdims=True)).sum(-1)) + t.max(-1)
    assert np.abs(lse.cpu().numpy() - ref).max() < 1e-4


@pytest.mark.parametrize("name", REPACK_CASES)
def test_backward_repack_permutes_gradients_bitwise(name):
    w, sr, excl = BY_NAME[name]
    outs = []
    for packing in (w.packing, w.repack):
        gas, d, od, coords, _, dev, o, saved, grads = _run(w, sr, excl, packing=packing)
        outs.append((coords, grads))
    p = torch.from_numpy(pi.order_between(outs[0][0], outs[1][0], w.grid)).to("cuda")
    for a, b in zip(outs[0][1], outs[1][1]):
        assert torch.equal(a, b[:, p])


def test_backward_is_deterministic():
    import geometry_aware_sparse_amd as gas
    w, sr, excl = BY_NAME["grid16_bf16"]
    _, d, _, _, (_, _, _, _, dout), dev, o, saved, grads = _run(w, sr, excl)
    again = gas.pack3d_backward(d, *dev, saved, to_dev(dout, tdtype(w)))
    for a, b in zip(grads, again):
        assert torch.equal(a, b)

"""GPU parity: every C entry point against the CPU oracle on seeded inputs.

Sizes span several LDS tiles and query tiles with ragged tails (grids that
are not multiples of the 4x4x8 local tile, summary counts that are not
multiples of 32 or 64, partial edge blocks), both dtypes and every head dim
the library builds. Index work must match bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import pack3d_inputs as pi
from gpu_cases import assert_close, desc_pair, host, inputs, tdtype, to_dev

pytestmark = pytest.mark.gpu

W = pi.Workload
CASES = [
    pi.workload(1),
    pi.workload(2),
    W(101, "ragged_bf16_d48", (10, 13, 19), 2, 3, 48, (2, 2, 2), "bf16", "iid", "random", "morton"),
    W(102, "ragged_bf16_d96", (6, 9, 11), 1, 2, 96, (2, 3, 2), "bf16", "smooth", "morton", "raster"),
    W(103, "partial_blocks_f32_d48", (5, 7, 9), 1, 2, 48, (2, 2, 3), "f32", "iid", "block", "random"),
    W(104, "small_bf16_d12", (3, 4, 5), 2, 2, 12, (3, 2, 2), "bf16", "iid", "raster", "random"),
    W(105, "f32_d96", (4, 5, 6), 1, 1, 96, (2, 2, 2), "f32", "iid", "random", "raster"),
    W(106, "bf16_d24_peaked", (6, 6, 6), 1, 2, 24, (3, 3, 3), "bf16", "smooth", "block", "raster"),
    W(107, "single_site", (1, 1, 1), 1, 1, 48, (1, 1, 1), "bf16", "iid", "raster", "raster"),
    # one axis a single site long: no neighbour along it, no rotation step
    W(114, "slab_z1_bf16_d48", (1, 12, 21), 1, 2, 48, (1, 2, 2), "bf16", "iid", "random", "raster"),
    W(115, "slab_y1_bf16_d96", (5, 1, 17), 1, 2, 96, (2, 1, 3), "bf16", "smooth", "block", "random"),
    # grouped key/value heads (GQA, MQA): query head h reads KV head h // (H // Hkv)
    W(110, "gqa4x2_bf16_d48", (10, 13, 19), 1, 4, 48, (2, 2, 2), "bf16", "iid", "random", "morton",
      Hkv=2),
    W(111, "mqa4_bf16_d96", (6, 9, 11), 1, 4, 96, (2, 3, 2), "bf16", "smooth", "morton", "raster",
      Hkv=1),
    W(112, "gqa6x3_f32_d24", (5, 7, 9), 2, 6, 24, (2, 2, 3), "f32", "iid", "block", "random", Hkv=3),
    W(113, "gqa8x2_bf16_d48", (12, 16, 20), 1, 8, 48, (2, 2, 2), "bf16", "iid", "block", "random",
      Hkv=2),
    # bf16 token rows wider than 512 elements (12 heads x 48): the pooling
    # pass takes its generic form
    W(116, "wide_rows_bf16_h12_d48", (5, 6, 7), 1, 12, 48, (2, 2, 2), "bf16", "iid", "random",
      "raster"),
    # one block spans the whole grid (M = 1, padded to 32 summaries): the
    # pooling pass stages its 2,048 members in several passes
    W(117, "one_big_block_bf16_d48", (8, 16, 16), 1, 2, 48, (8, 16, 16), "bf16", "iid", "random",
      "raster"),
]
IDS = [c.name for c in CASES]
BY_NAME = {c.name: c for c in CASES}
assert len(BY_NAME) == len(CASES), "case names are unique"


def _pick(*names):
    """Cases by name, so inserting a case never shifts a cross-cutting list."""
    return [BY_NAME[n] for n in names]


def _ids(cases):
    return [c.name for c in cases]


# every summary-exclusion reading, crossed with fp32 and bf16, ragged grids,
# partial blocks and grouped KV heads (fp32 GQA with three KV heads included)
EXCLUSION_CASES = _pick("grid8_fp32", "ragged_bf16_d48", "partial_blocks_f32_d48",
                        "gqa4x2_bf16_d48", "gqa6x3_f32_d24", "gqa8x2_bf16_d48")
# bf16 with head dim 48 or 96 and no exclusion: the matrix-core global kernel
MFMA_CASES = _pick("grid16_bf16", "ragged_bf16_d48", "ragged_bf16_d96", "single_site",
                   "slab_z1_bf16_d48", "slab_y1_bf16_d96", "gqa4x2_bf16_d48", "mqa4_bf16_d96",
                   "gqa8x2_bf16_d48")
# summary-centre variant: even, odd and clipped block extents, fp32 and bf16
# (both pooling kernels), grouped KV heads in both dtypes
CENTRE_CASES = _pick("grid8_fp32", "grid16_bf16", "ragged_bf16_d48", "ragged_bf16_d96",
                     "partial_blocks_f32_d48", "small_bf16_d12", "gqa4x2_bf16_d48",
                     "gqa6x3_f32_d24", "gqa8x2_bf16_d48")
# grouped KV heads proper: more query heads than KV heads in every entry
GQA_CASES = _pick("gqa4x2_bf16_d48", "mqa4_bf16_d96", "gqa6x3_f32_d24", "gqa8x2_bf16_d48")

# each list's defining property, checked when the module is imported
assert all(c.kv_heads < c.H for c in GQA_CASES)
assert {c.kv_heads for c in GQA_CASES} >= {1, 2, 3} and any(c.dtype == "f32" for c in GQA_CASES)
assert any(c.H // c.kv_heads == 4 for c in GQA_CASES)
assert all(c.dtype == "bf16" and c.D in (48, 96) for c in MFMA_CASES)
assert any(c.kv_heads < c.H for c in MFMA_CASES)
assert any(c.kv_heads < c.H and c.dtype == "f32" for c in EXCLUSION_CASES)
assert any(c.kv_heads < c.H and c.dtype == "f32" for c in CENTRE_CASES)
assert {c.dtype for c in CENTRE_CASES} == {"f32", "bf16"}
assert {c.dtype for c in EXCLUSION_CASES} == {"f32", "bf16"}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import geometry_aware_sparse_amd  # noqa: F401  (fails loudly if not built)


def _setup(w):
    import geometry_aware_sparse_amd as gas
    coords, q, k, v, g = inputs(w)
    d, od = desc_pair(w)
    dt = tdtype(w)
    dev = dict(coords=to_dev(coords, torch.int32), q=to_dev(q, dt), k=to_dev(k, dt),
               v=to_dev(v, dt), g=to_dev(g, dt))
    geom, nbr, blk, rank = gas.pack3d_index_build(d, dev["coords"], neighbours=True, blocks=True,
                                                  ranks=True)
    return gas, w, d, od, coords, (q, k, v, g), dev, geom, (nbr, blk, rank)


@pytest.mark.parametrize("w", CASES, ids=IDS)
def test_index_build_bit_exact(w):
    gas, w, d, od, coords, _, dev, geom, (nbr, blk, rank) = _setup(w)
    slot, oblk, orank = oracle.index(od, coords)
    onbr = oracle.neighbours(od, coords, slot)
    torch.cuda.synchronize()
    assert np.array_equal(gas.slot_map_view(d, geom).cpu().numpy(), slot)
    assert np.array_equal(nbr.cpu().numpy(), onbr)
    assert np.array_equal(blk.cpu().numpy(), oblk)
    assert np.array_equal(rank.cpu().numpy(), orank)
    assert int(geom[:4].view(torch.int32).item()) == 0


@pytest.mark.parametrize("w", CASES, ids=IDS)
def test_rope_table(w):
    # rows (axis_start + c) * P + p hold (cos, sin) of c * base^(-2p/(D/3))
    # rounded from double to fp32; the last row holds the same at c = 1/2
    # (paper summary §3.1; the half row serves block centres of even extent)
    gas, w, d, od, coords, _, dev, geom, _ = _setup(w)
    _, to, nb = gas.pack3d_geometry_layout(d)
    Z, Y, X = w.grid
    P = w.D // 6
    rows = Z + Y + X + 1
    assert nb >= to + rows * P * 8
    tab = geom[to:to + rows * P * 8].view(torch.float32).cpu().numpy().reshape(rows, P, 2)
    c = np.concatenate([np.arange(Z), np.arange(Y), np.arange(X), [0.5]]).astype(np.float64)
    theta = float(w.rope_base) ** (-2.0 * np.arange(P) / (w.D // 3))
    ang = c[:, None] * theta[None, :]
    want = np.stack([np.cos(ang), np.sin(ang)], axis=-1).astype(np.float32)
    assert np.abs(tab.astype(np.float64) - want.astype(np.float64)).max() <= 2.0 ** -23


@pytest.mark.parametrize("w", CASES, ids=IDS)
def test_rope_coords(w):
    gas, w, d, od, coords, (q, k, v, g), dev, geom, _ = _setup(w)
    got = host(gas.pack3d_rope_coords(d, dev["coords"], dev["q"]))
    assert_close(w, got, oracle.rope_axial(od, coords, q), "rope")
    # in place
    x = dev["k"].clone()
    gas.pack3d_rope_coords(d, dev["coords"], x, out=x)
    assert_close(w, host(x), oracle.rope_axial(od, coords, k), "rope in place")


@pytest.mark.parametrize("w", CASES, ids=IDS)
def test_block_summarize(w):
    gas, w, d, od, coords, (q, k, v, g), dev, geom, _ = _setup(w)
    ks, vs = gas.pack3d_block_summarize(d, geom, dev["k"], dev["v"])
    slot, _, _ = oracle.index(od, coords)
    oks, ovs = oracle.summaries(od, slot, oracle.rope_axial(od, coords, k), v)
    M = oks.shape[2]
    assert_close(w, host(gas.ksum_to_rows(ks, M, w.D)), oks, "k_sum")
    assert_close(w, host(gas.vsum_to_rows(vs, M)), ovs, "v_sum")
    # padding slots of the blocked layouts are zero
    Mp, Dp = (M + 31) // 32 * 32, (w.D + 7) // 8 * 8
    krows = ks.permute(0, 1, 2, 4, 3, 5).reshape(w.B, w.kv_heads, Mp, Dp)
    assert torch.count_nonzero(krows[:, :, :, w.D:]).item() == 0
    vrows = vs.permute(0, 1, 2, 4, 3).reshape(w.B, w.kv_heads, Mp, w.D)
    assert torch.count_nonzero(krows[:, :, M:]).item() == 0
    assert torch.count_nonzero(vrows[:, :, M:]).item() == 0


@pytest.mark.parametrize("w", CASES, ids=IDS)
def test_local_attn(w):
    gas, w, d, od, coords, (q, k, v, g), dev, geom, _ = _setup(w)
    ol = gas.pack3d_local_attn(d, geom, dev["q"], dev["k"], dev["v"])
    slot, _, _ = oracle.index(od, coords)
    ref = oracle.local(od, coords, slot, oracle.rope_axial(od, coords, q),
                       oracle.rope_axial(od, coords, k), v)
    assert_close(w, host(ol), ref, "local")


@pytest.mark.parametrize("w", CASES, ids=IDS)
def test_global_attn(w):
    gas, w, d, od, coords, (q, k, v, g), dev, geom, _ = _setup(w)
    slot, _, _ = oracle.index(od, coords)
    kr = oracle.rope_axial(od, coords, k)
    oks, ovs = oracle.summaries(od, slot, kr, v)
    ref = oracle.global_(od, coords, oracle.rope_axial(od, coords, q), oks, ovs)
    # from the GPU summaries (the forward's data flow) ...
    ks, vs = gas.pack3d_block_summarize(d, geom, dev["k"], dev["v"])
    og = gas.pack3d_global_attn(d, geom, dev["coords"], dev["q"], ks, vs)
    assert_close(w, host(og), ref, "global")
    # ... and from the oracle's summaries rounded to the working dtype
    dt = tdtype(w)
    og2 = gas.pack3d_global_attn(d, geom, dev["coords"], dev["q"],
                                 gas.ksum_from_rows(to_dev(oks, dt)),
                                 gas.vsum_from_rows(to_dev(ovs, dt)))
    assert_close(w, host(og2), ref, "global(oracle summaries)")


@pytest.mark.parametrize("w", CASES, ids=IDS)
def test_mix(w):
    gas, w, d, od, coords, (q, k, v, g), dev, geom, _ = _setup(w)
    a, b = dev["q"], dev["q"].flip(1).contiguous()
    o = gas.pack3d_mix(d, dev["g"], a, b)
    assert_close(w, host(o), oracle.mix(od, g, q, q[:, ::-1]), "mix")
    # aliasing the output with an input is allowed
    a2 = a.clone()
    gas.pack3d_mix(d, dev["g"], a2, b, out=a2)
    assert torch.equal(a2, o)


@pytest.mark.parametrize("w", CASES, ids=IDS)
def test_forward(w):
    gas, w, d, od, coords, (q, k, v, g), dev, geom, _ = _setup(w)
    o = gas.pack3d_forward(d, dev["coords"], dev["q"], dev["k"], dev["v"], dev["g"])
    ref = oracle.forward(od, coords, q, k, v, g)
    assert_close(w, host(o), ref, "forward")
    # the staged entry points give the same bits as the fused forward
    ks, vs = gas.pack3d_block_summarize(d, geom, dev["k"], dev["v"])
    og = gas.pack3d_global_attn(d, geom, dev["coords"], dev["q"], ks, vs)
    ol = gas.pack3d_local_attn(d, geom, dev["q"], dev["k"], dev["v"])
    staged = gas.pack3d_mix(d, dev["g"], ol, og)
    assert_close(w, host(staged), ref, "staged")


@pytest.mark.parametrize("mode", [1, 2], ids=["own_block", "neighbourhood_blocks"])
@pytest.mark.parametrize("w", EXCLUSION_CASES, ids=_ids(EXCLUSION_CASES))
def test_global_exclusion_readings(w, mode):
    import geometry_aware_sparse_amd as gas
    coords, q, k, v, g = inputs(w)
    d, od = desc_pair(w, exclusion=mode)
    dt = tdtype(w)
    dc, dq, dk, dv, dg = (to_dev(coords, torch.int32), to_dev(q, dt), to_dev(k, dt),
                          to_dev(v, dt), to_dev(g, dt))
    o = gas.pack3d_forward(d, dc, dq, dk, dv, dg)
    assert_close(w, host(o), oracle.forward(od, coords, q, k, v, g), f"exclusion {mode}")


def test_all_summaries_excluded_gives_local_only_mix():
    import geometry_aware_sparse_amd as gas
    w = W(108, "one_block", (2, 2, 2), 1, 1, 12, (2, 2, 2), "f32", "iid", "raster", "raster")
    coords, q, k, v, g = inputs(w)
    d, od = desc_pair(w, exclusion=1)
    dt = tdtype(w)
    dc, dq = to_dev(coords, torch.int32), to_dev(q, dt)
    geom, _, _, _ = gas.pack3d_index_build(d, dc)
    ks, vs = gas.pack3d_block_summarize(d, geom, to_dev(k, dt), to_dev(v, dt))
    og = gas.pack3d_global_attn(d, geom, dc, dq, ks, vs)
    assert torch.count_nonzero(og).item() == 0


@pytest.mark.parametrize("w", MFMA_CASES, ids=_ids(MFMA_CASES))
def test_global_exact_softmax_flag(w):
    """Every query through the two-pass softmax (maximum first) matches the
    oracle, and so does the default path."""
    import geometry_aware_sparse_amd as gas
    coords, q, k, v, g = inputs(w)
    d, od = desc_pair(w)
    de = gas.make_desc(w.B, w.N, w.H, w.D, w.grid, w.block, dtype=gas.PACK3D_BF16,
                       exact_softmax=True, kv_heads=w.kv_heads)
    dt = tdtype(w)
    dc, dq = to_dev(coords, torch.int32), to_dev(q, dt)
    geom, _, _, _ = gas.pack3d_index_build(d, dc)
    ks, vs = gas.pack3d_block_summarize(d, geom, to_dev(k, dt), to_dev(v, dt))
    fast = gas.pack3d_global_attn(d, geom, dc, dq, ks, vs)
    exact = gas.pack3d_global_attn(de, geom, dc, dq, ks, vs)
    slot, _, _ = oracle.index(od, coords)
    oks, ovs = oracle.summaries(od, slot, oracle.rope_axial(od, coords, k), v)
    ref = oracle.global_(od, coords, oracle.rope_axial(od, coords, q), oks, ovs)
    assert_close(w, host(exact), ref, "exact softmax")
    assert_close(w, host(fast), ref, "default softmax")
    if w.N * w.H >= 64:
        # the one-pass path is really taken: its rounding differs from the
        # two-pass one, so nearly every output row differs in some bit
        differ = (fast.reshape(-1, w.D) != exact.reshape(-1, w.D)).any(dim=1).float().mean().item()
        assert differ > 0.5, f"only {differ:.2%} of rows took the one-pass softmax"


def test_global_overflowing_scores_fall_back_per_query():
    """Queries whose scores overflow exp2 without a maximum are redone by the
    two-pass softmax: every query whose largest score (log2 units) is at
    least 110 -- its denominator is then above 2^100 -- equals the forced
    two-pass row bit for bit; ordinary rows keep the one-pass result; nothing
    is non-finite."""
    import geometry_aware_sparse_amd as gas
    w = BY_NAME["ragged_bf16_d48"]
    coords, q, k, v, g = inputs(w)
    big = np.zeros(w.N, bool)
    big[::7] = True
    q = q.copy()
    q[:, big] *= 64.0  # scores far beyond 2^7 in log2 units for most of these tokens
    d, od = desc_pair(w)
    de = gas.make_desc(w.B, w.N, w.H, w.D, w.grid, w.block, dtype=gas.PACK3D_BF16,
                       exact_softmax=True)
    dt = tdtype(w)
    dc, dq = to_dev(coords, torch.int32), to_dev(q, dt)
    geom, _, _, _ = gas.pack3d_index_build(d, dc)
    ks, vs = gas.pack3d_block_summarize(d, geom, to_dev(k, dt), to_dev(v, dt))
    fast = gas.pack3d_global_attn(d, geom, dc, dq, ks, vs)
    exact = gas.pack3d_global_attn(de, geom, dc, dq, ks, vs)
    assert torch.isfinite(fast.float()).all()
    # largest score of every (b, i, h) in log2 units, from the oracle's values
    slot, _, _ = oracle.index(od, coords)
    oks, _ = oracle.summaries(od, slot, oracle.rope_axial(od, coords, k), v)
    qr = oracle.rope_axial(od, coords, q)
    smax = np.einsum("bnhd,bhmd->bnhm", qr, oks).max(axis=-1) * (np.log2(np.e) / np.sqrt(w.D))
    must = torch.from_numpy(smax >= 110.0).to("cuda")
    assert must.sum().item() > 100
    f, e = fast.float(), exact.float()
    assert torch.equal(f[must], e[must])
    ordinary = torch.from_numpy(np.broadcast_to(~big[None, :, None], smax.shape).copy()).to("cuda")
    assert (f[ordinary] - e[ordinary]).abs().max().item() < 2e-2


# Summary-centre variant (paper summary §B.7, §B.8): keys pooled unrotated,
# the mean rotated once at the block centre. Cases with even, odd and clipped
# block extents, fp32 and bf16 (both pooling kernels).


def _centre_pair(w):
    import geometry_aware_sparse_amd as gas
    d = gas.make_desc(w.B, w.N, w.H, w.D, w.grid, w.block,
                      dtype=gas.PACK3D_BF16 if w.dtype == "bf16" else gas.PACK3D_F32,
                      rope_base=w.rope_base, summary_centre=True, kv_heads=w.kv_heads)
    od = oracle.make_desc(w.B, w.N, w.H, w.D, w.grid, w.block, rope_base=w.rope_base,
                          kv_heads=w.kv_heads)
    return d, od


@pytest.mark.parametrize("w", CENTRE_CASES, ids=_ids(CENTRE_CASES))
def test_block_summarize_centre(w):
    import geometry_aware_sparse_amd as gas
    coords, q, k, v, g = inputs(w)
    d, od = _centre_pair(w)
    dt = tdtype(w)
    dc = to_dev(coords, torch.int32)
    geom, _, _, _ = gas.pack3d_index_build(d, dc)
    ks, vs = gas.pack3d_block_summarize(d, geom, to_dev(k, dt), to_dev(v, dt))
    slot, _, _ = oracle.index(od, coords)
    oks, ovs = oracle.summaries_centre(od, slot, k, v)
    M = oks.shape[2]
    assert_close(w, host(gas.ksum_to_rows(ks, M, w.D)), oks, "centre k_sum")
    assert_close(w, host(gas.vsum_to_rows(vs, M)), ovs, "centre v_sum")
    # and the summaries differ from rotate-then-pool unless every block is one site
    ks_t, _ = gas.pack3d_block_summarize(desc_pair(w)[0], geom, to_dev(k, dt), to_dev(v, dt))
    if w.block != (1, 1, 1):
        assert not torch.equal(ks, ks_t)


@pytest.mark.parametrize("w", CENTRE_CASES, ids=_ids(CENTRE_CASES))
def test_forward_centre(w):
    import geometry_aware_sparse_amd as gas
    coords, q, k, v, g = inputs(w)
    d, od = _centre_pair(w)
    dt = tdtype(w)
    o = gas.pack3d_forward(d, to_dev(coords, torch.int32), to_dev(q, dt), to_dev(k, dt),
                           to_dev(v, dt), to_dev(g, dt))
    ref = oracle.forward(od, coords, q, k, v, g, summary_rope="centre")
    assert_close(w, host(o), ref, "centre forward")


@pytest.mark.parametrize("w", GQA_CASES, ids=_ids(GQA_CASES))
@pytest.mark.parametrize("centre", [False, True], ids=["token", "centre"])
def test_gqa_equals_mha_over_repeated_kv_bitwise(w, centre):
    """GQA through the library gives the same bits as multi-head attention
    over K/V repeated per group (query head h -> KV head h // (H // Hkv)):
    the same members, in the same order, with the same arithmetic."""
    import geometry_aware_sparse_amd as gas
    coords, q, k, v, g = inputs(w)
    dt = tdtype(w)
    G = w.H // w.kv_heads
    dc, dq, dg = to_dev(coords, torch.int32), to_dev(q, dt), to_dev(g, dt)
    args = dict(dtype=gas.PACK3D_BF16 if w.dtype == "bf16" else gas.PACK3D_F32,
                rope_base=w.rope_base, summary_centre=centre)
    dg_ = gas.make_desc(w.B, w.N, w.H, w.D, w.grid, w.block, kv_heads=w.kv_heads, **args)
    dm = gas.make_desc(w.B, w.N, w.H, w.D, w.grid, w.block, **args)
    og = gas.pack3d_forward(dg_, dc, dq, to_dev(k, dt), to_dev(v, dt), dg)
    om = gas.pack3d_forward(dm, dc, dq, to_dev(np.repeat(k, G, axis=2), dt),
                            to_dev(np.repeat(v, G, axis=2), dt), dg)
    assert torch.equal(og, om)
    # and the summaries of the grouped call are the repeated call's, one per KV head
    geom, _, _, _ = gas.pack3d_index_build(dg_, dc)
    ks, vs = gas.pack3d_block_summarize(dg_, geom, to_dev(k, dt), to_dev(v, dt))
    ksm, vsm = gas.pack3d_block_summarize(dm, geom, to_dev(np.repeat(k, G, axis=2), dt),
                                          to_dev(np.repeat(v, G, axis=2), dt))
    assert ks.shape[1] == w.kv_heads and ksm.shape[1] == w.H
    assert torch.equal(ks, ksm[:, ::G]) and torch.equal(vs, vsm[:, ::G])

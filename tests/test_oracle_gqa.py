"""Oracle pins for grouped key/value heads (GQA/MQA): keys, values and the
block summaries exist per KV head (project page Ch. 3, Contract 2; paper
summary §D.1, KV groups), query head h reading KV head h // (H // Hkv).

global branch  <- torch SDPA with its own grouped-query head mapping
local branch   <- dense masked attention over K/V repeated per group
summaries      <- one set per KV head: the MHA summaries of those heads
grouping       <- zeroing one KV head's values silences exactly its group
whole operator <- GQA equals MHA over K/V repeated per group, bit for bit,
                  under both summary RoPE variants and every exclusion
                  reading; MQA with identical query heads gives identical
                  heads; packing equivariance holds bitwise
"""
import numpy as np
import pytest

import oracle
import pack3d_inputs as pi
from refs import chebyshev_mask, dense_masked_attention, rotate_all, torch_sdpa


def _setup(H, Hkv, grid=(4, 5, 6), block=(2, 2, 3), B=2, D=12, seed=0, exclusion="none"):
    c = pi.packing_coords(grid, "random", block=block, seed=seed + 11)
    rng = np.random.default_rng(seed)
    N = c.shape[0]
    q = rng.standard_normal((B, N, H, D))
    k, v = (rng.standard_normal((B, N, Hkv, D)) for _ in range(2))
    g = rng.standard_normal((B, N, H))
    d = oracle.make_desc(B, N, H, D, grid, block, kv_heads=Hkv, exclusion=exclusion)
    return d, c, q, k, v, g


@pytest.mark.parametrize("H,Hkv", [(4, 2), (6, 3), (4, 1), (3, 3)])
def test_global_matches_torch_gqa(H, Hkv):
    d, c, q, k, v, _ = _setup(H, Hkv)
    slot, _, _ = oracle.index(d, c)
    qr = oracle.rope_axial(d, c, q)
    ks, vs = oracle.summaries(d, slot, oracle.rope_axial(d, c, k), v)
    assert ks.shape == (d.B, Hkv, oracle.num_blocks(d), d.D)
    ref = torch_sdpa(qr, ks, vs, 1 / np.sqrt(d.D))
    assert np.allclose(oracle.global_(d, c, qr, ks, vs), ref, atol=1e-12)


@pytest.mark.parametrize("H,Hkv", [(4, 2), (4, 1)])
def test_local_matches_dense_over_repeated_kv(H, Hkv):
    d, c, q, k, v, _ = _setup(H, Hkv, B=1)
    slot, _, _ = oracle.index(d, c)
    G = H // Hkv
    ol = oracle.local(d, c, slot, oracle.rope_axial(d, c, q), oracle.rope_axial(d, c, k), v)
    ref = dense_masked_attention(rotate_all(c, q), rotate_all(c, np.repeat(k, G, axis=2)),
                                 np.repeat(v, G, axis=2), chebyshev_mask(c), 1 / np.sqrt(d.D))
    assert np.allclose(ol, ref, atol=1e-12)


def test_summaries_are_per_kv_head():
    d, c, q, k, v, _ = _setup(6, 2)
    slot, _, _ = oracle.index(d, c)
    ks, vs = oracle.summaries(d, slot, oracle.rope_axial(d, c, k), v)
    dm = oracle.make_desc(d.B, d.N, 2, d.D, tuple(d.grid), tuple(d.block))
    ks2, vs2 = oracle.summaries(dm, slot, oracle.rope_axial(dm, c, k), v)
    assert np.array_equal(ks, ks2) and np.array_equal(vs, vs2)


def test_zeroed_kv_head_silences_its_group():
    d, c, q, k, v, g = _setup(6, 3)
    v = v.copy()
    v[:, :, 1] = 0.0  # KV head 1 serves query heads 2 and 3
    _, parts = oracle.forward(d, c, q, k, v, g, return_parts=True)
    for h in range(6):
        silent = h in (2, 3)
        for part in ("local", "glob"):
            assert (np.abs(parts[part][:, :, h]).max() == 0.0) == silent, (part, h)


@pytest.mark.parametrize("summary_rope", ["token", "centre"])
@pytest.mark.parametrize("exclusion", ["none", "own_block", "neighbourhood_blocks"])
def test_gqa_equals_mha_over_repeated_kv(summary_rope, exclusion):
    H, Hkv = 6, 2
    d, c, q, k, v, g = _setup(H, Hkv, exclusion=exclusion)
    dm = oracle.make_desc(d.B, d.N, H, d.D, tuple(d.grid), tuple(d.block), exclusion=exclusion)
    o = oracle.forward(d, c, q, k, v, g, summary_rope=summary_rope)
    om = oracle.forward(dm, c, q, np.repeat(k, H // Hkv, axis=2), np.repeat(v, H // Hkv, axis=2),
                        g, summary_rope=summary_rope)
    assert np.array_equal(o, om)


def test_mqa_identical_query_heads_give_identical_heads():
    d, c, q, k, v, g = _setup(4, 1)
    q[:] = q[:, :, :1]
    g[:] = g[:, :, :1]
    o = oracle.forward(d, c, q, k, v, g)
    for h in range(1, 4):
        assert np.array_equal(o[:, :, h], o[:, :, 0])


def test_gqa_operator_permutes_bitwise():
    grid, block = (4, 6, 8), (2, 2, 2)
    w = pi.Workload(901, "t", grid, 1, 4, 12, block, "f32", "iid", "raster", "random", Hkv=2)
    fields = pi.make_fields(w)
    assert fields[1].shape[2] == 2 and fields[0].shape[2] == 4
    d = oracle.make_desc(1, w.N, 4, 12, grid, block, kv_heads=2)
    outs, coords = [], []
    for kind in ("raster", "random"):
        cc = pi.packing_coords(grid, kind, block=block, seed=3)
        q, k, v, g = pi.pack_fields(fields, cc, grid)
        outs.append(oracle.forward(d, cc, q, k, v, g))
        coords.append(cc)
    p = pi.order_between(coords[0], coords[1], grid)
    assert np.array_equal(outs[0], outs[1][:, p])


def test_kv_heads_must_divide_h():
    with pytest.raises(ValueError):
        oracle.make_desc(1, 8, 6, 12, (2, 2, 2), (1, 1, 1), kv_heads=4)
    d, c, q, k, v, g = _setup(4, 2)
    slot, _, _ = oracle.index(d, c)
    with pytest.raises(ValueError):
        oracle.summaries(d, slot, q, q)  # query-shaped keys

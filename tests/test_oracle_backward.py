"""Oracle pins for the backward of the operator (paper summary §1, §3.4: the
operator is trained end to end; its gradients are the chain rule through
the forward's steps).

finite differences <- central differences of the (pinned) forward, for every
                      entry of q, k, v and the gate, under grouped KV heads,
                      both summary RoPE variants and the exclusion readings
torch autograd     <- gradients of an independent dense torch formulation of
                      the operator (rotation matrices from the matrix
                      exponential, masked dense attention, an explicit
                      averaging matrix for the pooling, torch's own grouped
                      SDPA for the global branch)
identities         <- a saturated-off gate sends no gradient into the global
                      branch; the value gradient of each (b, KV head) sums
                      the output gradients it receives (rows of P sum to 1)
"""
import numpy as np
import pytest
import torch

import oracle
import pack3d_inputs as pi
from refs import block_ids, chebyshev_mask, rotation


def _case(grid, block, B, H, Hkv, D, seed, exclusion=0):
    c = pi.packing_coords(grid, "random", block=block, seed=seed + 3)
    rng = np.random.default_rng(seed)
    N = c.shape[0]
    q = rng.standard_normal((B, N, H, D))
    k, v = (rng.standard_normal((B, N, Hkv, D)) for _ in range(2))
    g = rng.standard_normal((B, N, H))
    dout = rng.standard_normal((B, N, H, D))
    d = oracle.make_desc(B, N, H, D, grid, block, kv_heads=Hkv, exclusion=exclusion)
    return d, c, q, k, v, g, dout


FD_CASES = [
    # (grid, block, B, H, Hkv, D, summary_rope, exclusion)
    ((3, 3, 4), (2, 2, 2), 1, 2, 1, 6, "token", 0),
    ((3, 4, 3), (2, 2, 3), 1, 2, 2, 6, "centre", 0),
    ((2, 3, 4), (2, 2, 2), 2, 2, 1, 6, "token", 2),
    ((3, 3, 3), (2, 2, 2), 1, 4, 2, 6, "centre", 1),
]


@pytest.mark.parametrize("grid,block,B,H,Hkv,D,sr,excl", FD_CASES,
                         ids=[f"{c[6]}-kv{c[4]}of{c[3]}-ex{c[7]}" for c in FD_CASES])
def test_backward_matches_central_differences(grid, block, B, H, Hkv, D, sr, excl):
    d, c, q, k, v, g, dout = _case(grid, block, B, H, Hkv, D, seed=len(sr) + excl, exclusion=excl)
    dq, dk, dv, dg = oracle.backward(d, c, q, k, v, g, dout, summary_rope=sr)
    eps = 1e-5

    def loss(q_, k_, v_, g_):
        return float((dout * oracle.forward(d, c, q_, k_, v_, g_, summary_rope=sr)).sum())

    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv), ("gate", g, dg)):
        fd = np.empty_like(x)
        flat, fdf = x.reshape(-1), fd.reshape(-1)
        for e in range(flat.size):
            keep = flat[e]
            flat[e] = keep + eps
            lp = loss(q, k, v, g)
            flat[e] = keep - eps
            lm = loss(q, k, v, g)
            flat[e] = keep
            fdf[e] = (lp - lm) / (2 * eps)
        scale = max(np.abs(fd).max(), 1e-3)
        err = np.abs(grad - fd).max() / scale
        assert err < 1e-7, f"d{name}: {err:.2e}"


def _torch_operator(d, c, q, k, v, g, summary_rope):
    """The forward as dense torch float64 algebra, written from the method's
    definition independently of the oracle's C code."""
    B, N, H, D = q.shape
    Hkv = k.shape[2]
    G = H // Hkv
    s = 1.0 / np.sqrt(D)
    grid, block = tuple(d.grid), tuple(d.block)
    R = torch.from_numpy(np.stack([rotation(ci, D) for ci in c]))          # [N, D, D]
    qr = torch.einsum("nde,bnhe->bnhd", R, q)
    kr = torch.einsum("nde,bnhe->bnhd", R, k)
    # local: dense attention under the Chebyshev-1 mask, K/V repeated per group
    mask = torch.from_numpy(chebyshev_mask(c))
    krg, vg = kr.repeat_interleave(G, dim=2), v.repeat_interleave(G, dim=2)
    sl = torch.einsum("bihd,bjhd->bhij", qr, krg) * s
    sl = sl.masked_fill(~mask, float("-inf"))
    ol = torch.einsum("bhij,bjhd->bihd", torch.softmax(sl, dim=-1), vg)
    # summaries: averaging matrix over each block's members
    bid = block_ids(c, grid, block)
    M = oracle.num_blocks(d)
    A = np.zeros((M, N))
    for m in range(M):
        mem = np.flatnonzero(bid == m)
        A[m, mem] = 1.0 / len(mem)
    A = torch.from_numpy(A)
    if summary_rope == "token":
        ks = torch.einsum("mn,bnhd->bhmd", A, kr)
    else:
        My, Mx = -(-grid[1] // block[1]), -(-grid[2] // block[2])
        Rc = []
        for m in range(M):
            o = np.array([(m // (My * Mx)) * block[0], ((m // Mx) % My) * block[1],
                          (m % Mx) * block[2]])
            Rc.append(rotation(o + 0.5 * (np.minimum(block, np.array(grid) - o) - 1), D))
        Rc = torch.from_numpy(np.stack(Rc))
        ks = torch.einsum("mde,bhme->bhmd", Rc, torch.einsum("mn,bnhd->bhmd", A, k))
    vs = torch.einsum("mn,bnhd->bhmd", A, v)
    # global: torch SDPA with its grouped-query mapping, exclusion as a mask
    allow = np.ones((N, M), bool)
    if d.exclusion == 1:
        allow[np.arange(N), bid] = False
    elif d.exclusion == 2:
        nb = chebyshev_mask(c)
        for i in range(N):
            allow[i, np.unique(bid[nb[i]])] = False
    am = torch.from_numpy(np.where(allow, 0.0, float("-inf")))
    og = torch.nn.functional.scaled_dot_product_attention(
        qr.transpose(1, 2), ks, vs, attn_mask=am, scale=s, enable_gqa=G > 1).transpose(1, 2)
    og = torch.where(torch.from_numpy(allow.any(axis=1))[None, :, None, None], og,
                     torch.zeros_like(og))
    gg = torch.sigmoid(g)[..., None]
    return (1 - gg) * ol + gg * og


@pytest.mark.parametrize("sr,excl,Hkv", [("token", 0, 2), ("centre", 0, 4), ("token", 1, 1),
                                         ("centre", 2, 2)])
def test_backward_matches_torch_autograd(sr, excl, Hkv):
    d, c, q, k, v, g, dout = _case((4, 5, 6), (2, 2, 3), 2, 4, Hkv, 12, seed=7 + excl,
                                   exclusion=excl)
    dq, dk, dv, dg = oracle.backward(d, c, q, k, v, g, dout, summary_rope=sr)
    tq, tk, tv, tg = (torch.from_numpy(x.copy()).requires_grad_() for x in (q, k, v, g))
    o = _torch_operator(d, c, tq, tk, tv, tg, sr)
    assert np.allclose(o.detach().numpy(), oracle.forward(d, c, q, k, v, g, summary_rope=sr),
                       atol=1e-12)
    (o * torch.from_numpy(dout)).sum().backward()
    for name, mine, ref in (("q", dq, tq.grad), ("k", dk, tk.grad), ("v", dv, tv.grad),
                            ("gate", dg, tg.grad)):
        assert np.allclose(mine, ref.numpy(), atol=1e-11), name


def test_closed_gate_sends_nothing_to_the_global_branch():
    # with g = sigmoid(G) exactly 0 the global branch receives no gradient:
    # the block shape (which only the global branch sees) then changes none
    # of the gradients, and the gate gradient g (1 - g) <dO, O_g - O_l> is 0
    d, c, q, k, v, g, dout = _case((4, 4, 4), (2, 2, 2), 1, 2, 2, 12, seed=3)
    g_closed = np.full_like(g, -800.0)  # sigmoid underflows to exactly 0
    d2 = oracle.make_desc(d.B, d.N, d.H, d.D, tuple(d.grid), (1, 2, 4), kv_heads=2)
    a = oracle.backward(d, c, q, k, v, g_closed, dout)
    b = oracle.backward(d2, c, q, k, v, g_closed, dout)
    assert np.abs(a[3]).max() == 0.0
    for x, y in zip(a[:3], b[:3]):
        assert np.array_equal(x, y)
    # while with an open gate they differ
    a = oracle.backward(d, c, q, k, v, g, dout)
    b = oracle.backward(d2, c, q, k, v, g, dout)
    assert np.abs(a[0] - b[0]).max() > 1e-3


def test_value_gradient_conserves_output_gradient():
    # every softmax row sums to 1, so sum_j dv_j (over a KV head's tokens)
    # equals the sum over its query heads of (1-g) dO + g dO = dO
    d, c, q, k, v, g, dout = _case((4, 5, 3), (2, 2, 2), 2, 6, 3, 12, seed=5)
    _, _, dv, _ = oracle.backward(d, c, q, k, v, g, dout)
    tot = dout.reshape(2, d.N, 3, 2, 12).sum(axis=(1, 3))   # [B, Hkv, D]
    assert np.allclose(dv.sum(axis=1), tot, atol=1e-11)

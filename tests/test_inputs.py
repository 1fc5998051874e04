"""Host-side checks of the seeded input generators shared by the tests and
the benchmark (no method arithmetic here)."""
import numpy as np
import torch

import pack3d_inputs as pi


def test_round_bf16_matches_torch_conversion():
    # torch's float -> bfloat16 conversion rounds to nearest even: an
    # independent implementation of the same rounding
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 2**32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    x = np.concatenate([bits.view(np.float32),
                        rng.standard_normal(200_000).astype(np.float32),
                        np.array([np.inf, -np.inf, 0.0, -0.0, 3.4e38, -3.4e38, 1e-45,
                                  1.0 + 2.0**-8, 1.0 + 3 * 2.0**-8], dtype=np.float32)])
    ours = pi.round_bf16(x, chunk=65_537)  # several chunks and a ragged last one
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    fin = ~np.isnan(x)
    assert np.array_equal(ours[fin].view(np.uint32), ref[fin].view(np.uint32))
    assert np.isnan(ours[~fin]).all()


def test_round_bf16_keeps_shape_and_is_idempotent():
    x = np.random.default_rng(3).standard_normal((2, 5, 3, 7)).astype(np.float32)
    r = pi.round_bf16(x)
    assert r.shape == x.shape and r.dtype == np.float32
    assert np.array_equal(pi.round_bf16(r), r)


def test_workload_sizes():
    # the million-token volumes: 2^20, 2^22 and 2^23 tokens
    for wid, n in ((6, 1 << 20), (7, 1 << 22), (8, 1 << 23)):
        w = pi.workload(wid)
        assert w.tokens == n
        bz, by, bx = w.block
        Z, Y, X = w.grid
        assert Z % bz == 0 and Y % by == 0 and X % bx == 0

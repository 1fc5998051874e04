"""The pins must catch plausible mistakes in the oracle.

Each case copies oracle/pack3d_oracle.c, plants one mistake by text
substitution (a flipped sign, a wrong index or stride, a dropped term, a
transposed operand), builds the copy with gcc in a temporary folder and shows
that the relevant pin (the same independent references the other oracle tests
use) now fails while the unmodified oracle passes it.
"""
import os
import subprocess

import numpy as np
import pytest

import oracle
import pack3d_inputs as pi
from refs import (block_ids, chebyshev_mask, dense_masked_attention, rotate_all, rotation,
                  sequence_rotate_all, torch_sdpa)

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                   "pack3d_oracle.c")


def _setup(grid=(4, 5, 6), block=(2, 2, 2), B=1, H=2, D=12, kind="random"):
    c = pi.packing_coords(grid, kind, block=block, seed=5)
    rng = np.random.default_rng(9)
    N = c.shape[0]
    q, k, v = (rng.standard_normal((B, N, H, D)) for _ in range(3))
    g = rng.standard_normal((B, N, H))
    return oracle.make_desc(B, N, H, D, grid, block), c, q, k, v, g


def pin_rope():
    d, c, q, _, _, _ = _setup()
    return np.allclose(oracle.rope_axial(d, c, q), rotate_all(c, q), atol=1e-12)


def pin_rope_sequence():
    rng = np.random.default_rng(12)
    x = rng.standard_normal((2, 30, 2, 24))
    d = oracle.make_desc(2, 30, 2, 24, (2, 3, 5), (2, 2, 2))
    return np.allclose(oracle.rope_sequence(d, x), sequence_rotate_all(x), rtol=0, atol=1e-10)


def pin_neighbours():
    d, c, *_ = _setup()
    slot, _, _ = oracle.index(d, c)
    nbr = oracle.neighbours(d, c, slot)
    mask = chebyshev_mask(c)
    return all(sorted(j for j in nbr[i] if j >= 0) == np.flatnonzero(mask[i]).tolist()
               for i in range(c.shape[0]))


def pin_local():
    d, c, q, k, v, _ = _setup()
    slot, _, _ = oracle.index(d, c)
    ol = oracle.local(d, c, slot, oracle.rope_axial(d, c, q), oracle.rope_axial(d, c, k), v)
    ref = dense_masked_attention(rotate_all(c, q), rotate_all(c, k), v, chebyshev_mask(c),
                                 1 / np.sqrt(d.D))
    return np.allclose(ol, ref, atol=1e-12)


def pin_summaries():
    d, c, q, k, v, _ = _setup(grid=(4, 4, 6), block=(2, 2, 3))
    slot, _, _ = oracle.index(d, c)
    qr = oracle.rope_axial(d, c, q)
    ks, vs = oracle.summaries(d, slot, oracle.rope_axial(d, c, k), v)
    bid = block_ids(c, d.grid, d.block)
    for i in (0, 7, 33):
        for m in range(ks.shape[2]):
            mem = np.flatnonzero(bid == m)
            t = np.mean([q[0, i, 1] @ (rotation(c[j] - c[i], d.D) @ k[0, j, 1]) for j in mem])
            if abs(qr[0, i, 1] @ ks[0, 1, m] - t) > 1e-11:
                return False
            if not np.allclose(vs[0, 1, m], v[0, mem, 1].mean(axis=0), atol=1e-14):
                return False
    return True


def pin_global():
    d, c, q, k, v, _ = _setup(B=2, H=3)
    slot, _, _ = oracle.index(d, c)
    qr = oracle.rope_axial(d, c, q)
    ks, vs = oracle.summaries(d, slot, oracle.rope_axial(d, c, k), v)
    return np.allclose(oracle.global_(d, c, qr, ks, vs), torch_sdpa(qr, ks, vs, 1 / np.sqrt(d.D)),
                       atol=1e-12)


def pin_mix():
    d, c, q, k, v, g = _setup()
    o, parts = oracle.forward(d, c, q, k, v, g, return_parts=True)
    sig = 1 / (1 + np.exp(-g))[..., None]
    return np.allclose(o, (1 - sig) * parts["local"] + sig * parts["glob"], atol=1e-14)


def pin_summary_centre():
    d, c, q, k, v, _ = _setup(grid=(5, 4, 6), block=(2, 2, 4))
    slot, _, _ = oracle.index(d, c)
    ks, vs = oracle.summaries_centre(d, slot, k, v)
    bid = block_ids(c, d.grid, d.block)
    My, Mx = -(-d.grid[1] // d.block[1]), -(-d.grid[2] // d.block[2])
    for m in range(ks.shape[2]):
        o = np.array([(m // (My * Mx)) * d.block[0], ((m // Mx) % My) * d.block[1],
                      (m % Mx) * d.block[2]])
        centre = o + 0.5 * (np.minimum(np.array(d.block), np.array(d.grid) - o) - 1)
        mem = np.flatnonzero(bid == m)
        if not np.allclose(ks[0, 1, m], rotation(centre, d.D) @ k[0, mem, 1].mean(axis=0),
                           atol=1e-12):
            return False
    return True


def pin_gqa():
    # H = 4 query heads over 2 KV heads: torch SDPA's grouped mapping for the
    # global branch, dense attention over K/V repeated per group for the local one
    d0, c, q, _, _, _ = _setup(H=4)
    rng = np.random.default_rng(3)
    k, v = (rng.standard_normal((1, d0.N, 2, d0.D)) for _ in range(2))
    d = oracle.make_desc(1, d0.N, 4, d0.D, tuple(d0.grid), tuple(d0.block), kv_heads=2)
    slot, _, _ = oracle.index(d, c)
    qr, kr = oracle.rope_axial(d, c, q), oracle.rope_axial(d, c, k)
    ks, vs = oracle.summaries(d, slot, kr, v)
    s = 1 / np.sqrt(d.D)
    if not np.allclose(oracle.global_(d, c, qr, ks, vs), torch_sdpa(qr, ks, vs, s), atol=1e-12):
        return False
    ref = dense_masked_attention(rotate_all(c, q), rotate_all(c, np.repeat(k, 2, axis=2)),
                                 np.repeat(v, 2, axis=2), chebyshev_mask(c), s)
    return np.allclose(oracle.local(d, c, slot, qr, kr, v), ref, atol=1e-12)


def pin_backward():
    # central differences of the forward on a tiny grouped case
    grid, block = (3, 3, 2), (2, 2, 2)
    c = pi.packing_coords(grid, "random", block=block, seed=2)
    rng = np.random.default_rng(4)
    N, H, Hkv, D = c.shape[0], 2, 1, 6
    q, dout = (rng.standard_normal((1, N, H, D)) for _ in range(2))
    k, v = (rng.standard_normal((1, N, Hkv, D)) for _ in range(2))
    g = rng.standard_normal((1, N, H))
    d = oracle.make_desc(1, N, H, D, grid, block, kv_heads=Hkv)
    grads = oracle.backward(d, c, q, k, v, g, dout)
    eps = 1e-5
    for x, grad in zip((q, k, v, g), grads):
        flat = x.reshape(-1)
        for e in range(0, flat.size, 5):
            keep = flat[e]
            flat[e] = keep + eps
            lp = float((dout * oracle.forward(d, c, q, k, v, g)).sum())
            flat[e] = keep - eps
            lm = float((dout * oracle.forward(d, c, q, k, v, g)).sum())
            flat[e] = keep
            if abs((lp - lm) / (2 * eps) - grad.reshape(-1)[e]) > 1e-7:
                return False
    return True


MUTANTS = [
    ("rope_sin_sign", "yr[c0 + 1] = x0 * sn + x1 * cs;", "yr[c0 + 1] = -x0 * sn + x1 * cs;", pin_rope),
    ("rope_frequency", "pow(d->rope_base, -2.0 * p / (double)da)", "pow(d->rope_base, -2.0 * p / (double)D)", pin_rope),
    ("rope_axis_chunk", "int c0 = a * da + 2 * p;", "int c0 = a * 2 + 2 * p * 3;", pin_rope),
    ("rope_coord_axis", "double phi = (double)coords[3 * i + a] * theta;", "double phi = (double)coords[3 * i + (2 - a)] * theta;", pin_rope),
    ("seq_rope_exponent", "double theta = pow(d->rope_base, -2.0 * p / (double)D);", "double theta = pow(d->rope_base, -1.0 * p / (double)D);", pin_rope_sequence),
    ("seq_rope_axis_exponent", "double theta = pow(d->rope_base, -2.0 * p / (double)D);", "double theta = pow(d->rope_base, -2.0 * p / (double)(D / 3));", pin_rope_sequence),
    ("seq_rope_sin_sign", "yr[2 * p + 1] = x0 * sn + x1 * cs;", "yr[2 * p + 1] = -x0 * sn + x1 * cs;", pin_rope_sequence),
    ("seq_rope_row_index", "double phi = (double)i * theta;", "double phi = (double)(row % d->N) * theta;", pin_rope_sequence),
    ("neighbour_offset", "*dx = k % 3 - 1;", "*dx = k % 3;", pin_neighbours),
    ("neighbour_edge_wrap", "if (z < 0 || y < 0 || x < 0 || z >= d->grid[0] || y >= d->grid[1] || x >= d->grid[2])\n    return -1;", "if (z < 0 || y < 0 || x < 0 || z >= d->grid[0] || y >= d->grid[1] || x >= d->grid[2])\n    return slot[site_of(d, (z + d->grid[0]) % d->grid[0], (y + d->grid[1]) % d->grid[1], (x + d->grid[2]) % d->grid[2])];", pin_neighbours),
    ("local_no_scale", "logit[k] = s * dot(", "logit[k] = dot(", pin_local),
    ("local_drop_self", "if (nb[k] < 0) continue;\n          logit[k]", "if (nb[k] < 0 || k == 13) continue;\n          logit[k]", pin_local),
    ("summary_count", "ko[c] /= count;", "ko[c] /= (count + 1);", pin_summaries),
    ("summary_block_origin", "int oz = (m / (My * Mx)) * bz, oy = ((m / Mx) % My) * by, ox = (m % Mx) * bx;", "int oz = (m / (My * Mx)) * bz, oy = (m % My) * by, ox = ((m / My) % Mx) * bx;", pin_summaries),
    ("global_summary_stride", "logit[m] = s * dot(q, ks + (((int64_t)b * Hk + kv_of(d, h)) * M + m) * D, D);", "logit[m] = s * dot(q, ks + (((int64_t)b * M + m) * Hk + kv_of(d, h)) * D, D);", pin_global),
    ("global_value_head", "const double *vm = vs + (((int64_t)b * Hk + kv_of(d, h)) * M + m) * D;", "const double *vm = vs + (((int64_t)b * Hk + 0) * M + m) * D;", pin_global),
    ("kv_group_modulo", "static int kv_of(const ork_desc *d, int h) { return h / (d->H / kv_heads(d)); }", "static int kv_of(const ork_desc *d, int h) { return h % kv_heads(d); }", pin_gqa),
    ("local_kv_head_ignored", "logit[k] = s * dot(q, kr + (((int64_t)b * d->N + nb[k]) * Hk + kv_of(d, h)) * D, D);", "logit[k] = s * dot(q, kr + (((int64_t)b * d->N + nb[k]) * Hk + 0) * D, D);", pin_gqa),
    ("centre_extent", "centre[a] = o[a] + 0.5 * (extent - 1);", "centre[a] = o[a] + 0.5 * extent;", pin_summary_centre),
    ("centre_unclipped", "int extent = d->grid[a] - o[a] < d->block[a] ? d->grid[a] - o[a] : d->block[a];", "int extent = d->block[a];", pin_summary_centre),
    ("bwd_local_no_delta", "const double ds = p[n] * (dp[n] - delta);", "const double ds = p[n] * dp[n];", pin_backward),
    ("bwd_global_value_weight", "dvs[(sb + m) * D + c] += pm * doi[c];", "dvs[(sb + m) * D + c] += doi[c];", pin_backward),
    ("bwd_rope_forward_turn", "rotate_rows(d, coords, H, dqr, dq, -1);", "rotate_rows(d, coords, H, dqr, dq, +1);", pin_backward),
    ("bwd_pool_no_count", "dkr[jo + c] += gk[c] / count;", "dkr[jo + c] += gk[c];", pin_backward),
    ("bwd_gate_derivative", "dgate[r] = g * (1.0 - g) * acc;", "dgate[r] = g * acc;", pin_backward),
    ("mix_swapped", "out[base + c] = (1.0 - g) * oloc[base + c] + g * oglob[base + c];", "out[base + c] = g * oloc[base + c] + (1.0 - g) * oglob[base + c];", pin_mix),
]


def test_unmodified_oracle_passes_every_pin():
    for f in (pin_rope, pin_rope_sequence, pin_neighbours, pin_local, pin_summaries, pin_global, pin_mix,
              pin_summary_centre, pin_gqa, pin_backward):
        assert f(), f.__name__


@pytest.mark.parametrize("name,old,new,pin", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, name, old, new, pin):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique"
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / f"{name}.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-shared", "-fPIC", str(path), "-o",
                    str(so), "-lm"], check=True)
    with oracle.use_library(str(so)):
        assert not pin(), f"pin {pin.__name__} did not catch {name}"

"""Independent formulations used to pin the oracle (test helpers).

None of these re-types the oracle's loops: rotations are built as the matrix
exponential of their skew-symmetric generator, neighbourhoods by brute-force
pairwise Chebyshev distance on coordinates, attention as a dense masked
softmax in float64 or through torch's scaled_dot_product_attention.
"""
import numpy as np
import scipy.linalg
import torch


def generator(coord, D, base=10000.0):
    """Skew-symmetric D x D generator of the axial rotation at coordinate
    (z, y, x): axis a owns channels [a*D/3, (a+1)*D/3), plane p is the pair
    (2p, 2p+1) of that chunk with angular rate theta_p = base^(-2p/(D/3));
    the rotation turns x0 towards x1 (counter-clockwise)."""
    da = D // 3
    G = np.zeros((D, D))
    for a in range(3):
        for p in range(da // 2):
            th = base ** (-2.0 * p / da)
            c0 = a * da + 2 * p
            G[c0 + 1, c0] += coord[a] * th
            G[c0, c0 + 1] -= coord[a] * th
    return G


def rotation(coord, D, base=10000.0):
    return scipy.linalg.expm(generator(coord, D, base))


def sequence_generator(pos, D, base=10000.0):
    """Skew-symmetric D x D generator of 1-D RoPE at a packed sequence index
    (the control of paper summary §B.4): plane p is the channel pair
    (2p, 2p+1) over all D channels, angular rate theta_p = base^(-2p/D)."""
    G = np.zeros((D, D))
    for p in range(D // 2):
        th = base ** (-2.0 * p / D)
        G[2 * p + 1, 2 * p] += pos * th
        G[2 * p, 2 * p + 1] -= pos * th
    return G


def sequence_rotate_all(x, base=10000.0):
    """x: [B, N, H, D] -> the 1-D rotation at packed index i of row i, via
    explicit matrices."""
    D = x.shape[-1]
    out = np.empty_like(x, dtype=np.float64)
    for i in range(x.shape[1]):
        R = scipy.linalg.expm(sequence_generator(i, D, base))
        out[:, i] = x[:, i].astype(np.float64) @ R.T
    return out


def rotate_all(coords, x, base=10000.0):
    """x: [B, N, H, D] -> R(c_i) x_i via explicit matrices."""
    D = x.shape[-1]
    out = np.empty_like(x, dtype=np.float64)
    for i, c in enumerate(coords):
        R = rotation(c, D, base)
        out[:, i] = x[:, i].astype(np.float64) @ R.T
    return out


def chebyshev_mask(coords):
    c = coords.astype(np.int64)
    dist = np.abs(c[:, None, :] - c[None, :, :]).max(axis=2)
    return dist <= 1


def dense_masked_attention(qr, kr, v, mask, scale):
    """qr, kr, v: [B, N, H, D] float64; mask [N, N] bool (query, key)."""
    B, N, H, D = qr.shape
    out = np.empty((B, N, H, D))
    for b in range(B):
        for h in range(H):
            S = scale * (qr[b, :, h] @ kr[b, :, h].T)
            S = np.where(mask, S, -np.inf)
            S = S - S.max(axis=1, keepdims=True)
            P = np.exp(S)
            P /= P.sum(axis=1, keepdims=True)
            out[b, :, h] = P @ v[b, :, h]
    return out


def torch_sdpa(qr, ks, vs, scale, mask=None):
    """qr [B,N,H,D], ks/vs [B,Hkv,M,D] -> [B,N,H,D] via torch SDPA in float64
    (with Hkv < H, torch's own grouped-query head mapping)."""
    q = torch.from_numpy(np.ascontiguousarray(qr.transpose(0, 2, 1, 3)))
    k = torch.from_numpy(np.ascontiguousarray(ks))
    v = torch.from_numpy(np.ascontiguousarray(vs))
    am = None if mask is None else torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=am, scale=scale,
                                                         enable_gqa=k.shape[1] != q.shape[1])
    return o.numpy().transpose(0, 2, 1, 3)


def block_ids(coords, grid, block):
    c = coords.astype(np.int64)
    Mb = [-(-grid[a] // block[a]) for a in range(3)]
    return ((c[:, 0] // block[0]) * Mb[1] + c[:, 1] // block[1]) * Mb[2] + c[:, 2] // block[2]

"""Quadratic-form brute force in numpy, independent of oracle/ (test pin).

Linear attention is an exact reassociation of a quadratic form.  This module
evaluates the quadratic form directly, token pair by token pair:

    o_i = sigmoid(g_i) * sum_j (R_i phi(q_i) . R_j phi(k_j)) v_j
                         / (sum_j phi(q_i) . phi(k_j) + eps)

with phi = ReLU and the rotation done as complex multiplication of the
interleaved pairs (x[2p] + i x[2p+1]) by exp(i * angle).  The oracle instead
forms S and z first and rotates with real cos/sin arithmetic, so a dropped
term, a wrong sign or a transposed operand in either shows up as a mismatch.
The angle convention (axis blocks t, y, x; omega_j = theta^(-2j / (2 Pa))) is
the reading both sides follow, written here a second time in vector form.
"""
from __future__ import annotations

import numpy as np


def axis_pairs(D: int):
    py = D // 6
    return D // 2 - 2 * py, py, py


def angles(D: int, T: int, Hh: int, W: int, theta: float = 10000.0, t0=0, y0=0, x0=0):
    """[N, D/2] rotation angles, tokens in row-major (t, y, x) order."""
    pt, py, px = axis_pairs(D)
    n = np.arange(T * Hh * W)
    t = n // (Hh * W) + t0
    y = (n // W) % Hh + y0
    x = n % W + x0
    cols = []
    for pos, pa in ((t, pt), (y, py), (x, px)):
        if pa == 0:
            continue
        omega = theta ** (-2.0 * np.arange(pa) / (2.0 * pa))
        cols.append(pos[:, None].astype(np.float64) * omega[None, :])
    return np.concatenate(cols, axis=1)


def rotate_complex(u: np.ndarray, ang: np.ndarray) -> np.ndarray:
    """Rotate interleaved pairs of u [..., N, D] by ang [N, D/2] via complex products."""
    c = u[..., 0::2] + 1j * u[..., 1::2]
    c = c * np.exp(1j * ang)
    out = np.empty_like(u)
    out[..., 0::2] = c.real
    out[..., 1::2] = c.imag
    return out


def forward(q, k, v, g, grid=None, eps: float = 1e-6) -> np.ndarray:
    """q, k, v, g: float64 [B, N, H, D]; grid: (T, Hh, W[, theta, t0, y0, x0]) or None."""
    B, N, H, D = q.shape
    fq = np.maximum(q, 0.0)
    fk = np.maximum(k, 0.0)
    if grid is not None:
        ang = angles(D, *grid)
        rq = rotate_complex(np.transpose(fq, (0, 2, 1, 3)), ang)
        rk = rotate_complex(np.transpose(fk, (0, 2, 1, 3)), ang)
    else:
        rq = np.transpose(fq, (0, 2, 1, 3))
        rk = np.transpose(fk, (0, 2, 1, 3))
    out = np.empty_like(q)
    for b in range(B):
        for h in range(H):
            num_w = rq[b, h] @ rk[b, h].T                 # [N, N] rotated weights
            den_w = fq[b, :, h, :] @ fk[b, :, h, :].T     # [N, N] unrotated weights
            num = num_w @ v[b, :, h, :]
            den = den_w.sum(axis=1) + eps
            gate = 1.0 / (1.0 + np.exp(-g[b, :, h, :]))
            out[b, :, h, :] = gate * num / den[:, None]
    return out


def row(q, k, v, g, b: int, h: int, i: int, grid=None, eps: float = 1e-6) -> np.ndarray:
    """One output row o_i of head (b, h) in O(N D): the quadratic form for a single i."""
    B, N, H, D = q.shape
    fq = np.maximum(q[b, i, h], 0.0)
    fk = np.maximum(k[b, :, h], 0.0)
    if grid is not None:
        ang = angles(D, *grid)
        rq = rotate_complex(fq[None, :], ang[i:i + 1])[0]
        rk = rotate_complex(fk, ang)
    else:
        rq, rk = fq, fk
    w = rk @ rq                        # [N] rotated weights
    num = w @ v[b, :, h]
    den = (fk @ fq).sum() + eps
    gate = 1.0 / (1.0 + np.exp(-g[b, i, h]))
    return gate * num / den


def forward_blocks(q, k, v, g, grid, L: int, S_in=None, z_in=None, eps: float = 1e-6):
    """Block-causal quadratic form with a carried state.  Token i sees the
    tokens j with j // L <= i // L (its own block and every earlier one), and
    the carried state adds (R_i phi(q_i))^T S_in to the numerator and
    phi(q_i) . z_in to the denominator.  S_in [B, H, D, D], z_in [B, H, D]."""
    B, N, H, D = q.shape
    fq = np.maximum(q, 0.0)
    fk = np.maximum(k, 0.0)
    if grid is not None:
        ang = angles(D, *grid)
        rq = rotate_complex(np.transpose(fq, (0, 2, 1, 3)), ang)
        rk = rotate_complex(np.transpose(fk, (0, 2, 1, 3)), ang)
    else:
        rq = np.transpose(fq, (0, 2, 1, 3))
        rk = np.transpose(fk, (0, 2, 1, 3))
    blk = np.arange(N) // L
    mask = (blk[None, :] <= blk[:, None]).astype(np.float64)   # [i, j]
    out = np.empty_like(q)
    for b in range(B):
        for h in range(H):
            num_w = (rq[b, h] @ rk[b, h].T) * mask
            den_w = (fq[b, :, h, :] @ fk[b, :, h, :].T) * mask
            num = num_w @ v[b, :, h, :]
            den = den_w.sum(axis=1) + eps
            if S_in is not None:
                num = num + rq[b, h] @ S_in[b, h]
            if z_in is not None:
                den = den + fq[b, :, h, :] @ z_in[b, h]
            gate = 1.0 / (1.0 + np.exp(-g[b, :, h, :]))
            out[b, :, h, :] = gate * num / den[:, None]
    return out


def softmax_attention(q, k, v, g, grid=None) -> np.ndarray:
    """Gated softmax attention in numpy: o = sigmoid(g) * softmax(rq rk^T /
    sqrt(D)) v, with RoPE on q and k done as complex rotation."""
    B, N, H, D = q.shape
    qt = np.transpose(q, (0, 2, 1, 3))
    kt = np.transpose(k, (0, 2, 1, 3))
    if grid is not None:
        ang = angles(D, *grid)
        qt = rotate_complex(qt, ang)
        kt = rotate_complex(kt, ang)
    out = np.empty_like(q)
    for b in range(B):
        for h in range(H):
            s = qt[b, h] @ kt[b, h].T / np.sqrt(D)
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p = p / p.sum(axis=1, keepdims=True)
            gate = 1.0 / (1.0 + np.exp(-g[b, :, h, :]))
            out[b, :, h, :] = gate * (p @ v[b, :, h, :])
    return out

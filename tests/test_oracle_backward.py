"""Pins of the oracle's backward pass of the bidirectional mixer (the exact
derivative of the forward form; see gla_oracle_backward).

Checked against things other than the oracle itself:
  - torch autograd in fp64 through an independently written quadratic form
    with the rotation done as complex products;
  - central finite differences of the numpy quadratic form (tests/brute.py);
  - Euler's theorem: with eps = 0 the output is homogeneous of degree 0 in
    q (per token) and in k (per head), and of degree 1 in v, so
    <q_n, dq_n> = 0, sum_m <k_m, dk_m> = 0, sum_m <v_m, dv_m> = sum_n <dout_n, o_n>;
    with eps > 0, <q_n, dq_n> = eps * <dout_n, o_n> / den_n;
  - the sigmoid gate: dg = dout * o * (1 - sigmoid(g)) with o from the
    forward oracle;
  - constant values without RoPE and eps = 0 make o = sigmoid(g) * c, so
    dq = dk = 0;
  - zero dout, linearity in dout, permutation of tokens, and the row/state
    helpers against the whole pass.
"""
import numpy as np
import pytest
import torch

import brute
import oracle
from workloads import random_grad, random_inputs


def f64(*ts):
    return tuple(t.double().numpy() for t in ts)


def rel(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def torch_forward(q, k, v, g, grid, eps):
    """The quadratic form in torch fp64: real dot products of interleaved
    pairs as Re(c1 conj(c2)) of complex numbers rotated by exp(i angle)."""
    fq, fk = torch.relu(q), torch.relu(k)
    B, N, H, D = q.shape
    cq = torch.complex(fq[..., 0::2], fq[..., 1::2])
    ck = torch.complex(fk[..., 0::2], fk[..., 1::2])
    if grid is not None:
        rot = torch.exp(1j * torch.from_numpy(brute.angles(D, *grid)))   # [N, D/2]
        cq = cq * rot[None, :, None, :]
        ck = ck * rot[None, :, None, :]
    cq, ck = cq.permute(0, 2, 1, 3), ck.permute(0, 2, 1, 3)             # [B, H, N, D/2]
    w_num = (cq @ ck.conj().transpose(-1, -2)).real                     # [B, H, N, N]
    w_den = fq.permute(0, 2, 1, 3) @ fk.permute(0, 2, 3, 1)
    num = w_num @ v.permute(0, 2, 1, 3)
    den = w_den.sum(-1, keepdim=True) + eps
    return (torch.sigmoid(g).permute(0, 2, 1, 3) * num / den).permute(0, 2, 1, 3)


def autograd_grads(q, k, v, g, dout, grid, eps):
    ts = [torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in f64(q, k, v, g)]
    o = torch_forward(*ts, grid, eps)
    (o * dout.double()).sum().backward()
    return tuple(t.grad.numpy() for t in ts)


CASES = [
    # B, H, D, grid or (None, N)
    (1, 2, 8, (2, 3, 4)),
    (2, 1, 16, (3, 2, 2)),
    (1, 3, 12, (2, 2, 5)),
    (2, 2, 8, None, 17),
    (1, 1, 32, (2, 4, 4)),
]


def shape(c):
    if c[3] is None:
        return c[0], c[4], c[1], c[2], None
    T, Hh, W = c[3]
    return c[0], T * Hh * W, c[1], c[2], c[3]


@pytest.mark.parametrize("case", CASES)
def test_backward_matches_autograd(case):
    B, N, H, D, grid = shape(case)
    q, k, v, g = random_inputs(B, N, H, D, seed=500 + N + D)
    dout = random_grad(B, N, H, D, seed=600 + N + D)
    og = oracle.Grid(*grid) if grid else None
    got = oracle.backward(q, k, v, g, dout, og)
    ref = autograd_grads(q, k, v, g, dout, grid, oracle.EPS)
    for name, a, b in zip("qkvg", got, ref):
        assert rel(a, b) < 1e-10, name


def test_backward_matches_finite_differences():
    B, N, H, D, grid = 1, 12, 2, 8, (2, 2, 3)
    q, k, v, g = random_inputs(B, N, H, D, seed=77)
    dout = random_grad(B, N, H, D, seed=78)
    grads = oracle.backward(q, k, v, g, dout, oracle.Grid(*grid))
    x = list(f64(q, k, v, g))
    dn = dout.double().numpy()

    def loss(xs):
        return float((brute.forward(*xs, grid) * dn).sum())

    rng = np.random.default_rng(5)
    for which in range(4):
        for _ in range(12):
            idx = tuple(int(rng.integers(0, s)) for s in x[which].shape)
            if abs(x[which][idx]) < 1e-3:     # keep off the ReLU kink
                continue
            h = 1e-6 * max(1.0, abs(x[which][idx]))
            xp = [a.copy() for a in x]
            xm = [a.copy() for a in x]
            xp[which][idx] += h
            xm[which][idx] -= h
            fd = (loss(xp) - loss(xm)) / (2 * h)
            scale = np.abs(grads[which]).max()
            assert abs(fd - grads[which][idx]) <= 1e-6 * scale, ("qkvg"[which], idx)


def positive_rows(q):
    """q with feature 0 of every row made positive, so phi(q).z > 0 without eps."""
    q = q.clone()
    q[..., 0] = q[..., 0].abs() + 0.5
    return q


@pytest.mark.parametrize("grid", [(2, 3, 4), None])
def test_euler_identities_without_eps(grid):
    B, N, H, D = 2, 24, 2, 16
    q, k, v, g = random_inputs(B, N, H, D, seed=91)
    q = positive_rows(q)
    dout = random_grad(B, N, H, D, seed=92)
    og = oracle.Grid(*grid) if grid else None
    dq, dk, dv, dg = oracle.backward(q, k, v, g, dout, og, eps=0.0)
    qf, kf, vf, _ = f64(q, k, v, g)
    o = brute.forward(*f64(q, k, v, g), grid, eps=0.0)
    dn = dout.double().numpy()
    # degree 0 in q_n: <q_n, dq_n> = 0 for every token
    per_token = (qf * dq).sum(-1)
    assert np.abs(per_token).max() < 1e-12 * np.abs(dq).max() * np.abs(qf).max() * D
    # degree 0 in k (per head): sum_m <k_m, dk_m> = 0
    per_head_k = (kf * dk).sum(axis=(1, 3))
    assert np.abs(per_head_k).max() < 1e-11 * np.abs(dk).max() * np.abs(kf).max() * N * D
    # degree 1 in v (per head): sum_m <v_m, dv_m> = sum_n <dout_n, o_n>
    lhs = (vf * dv).sum(axis=(1, 3))
    rhs = (dn * o).sum(axis=(1, 3))
    assert np.allclose(lhs, rhs, rtol=1e-10, atol=1e-12)


def test_euler_identity_q_with_eps():
    B, N, H, D, grid = 1, 24, 2, 16, (2, 3, 4)
    q, k, v, g = random_inputs(B, N, H, D, seed=93)
    q = positive_rows(q)
    dout = random_grad(B, N, H, D, seed=94)
    eps = 0.5   # large enough to matter
    dq, _, _, _ = oracle.backward(q, k, v, g, dout, oracle.Grid(*grid), eps=eps)
    qf, kf, _, _ = f64(q, k, v, g)
    o = brute.forward(*f64(q, k, v, g), grid, eps=eps)
    den = np.einsum("bnhd,bmhd->bnh", np.maximum(qf, 0), np.maximum(kf, 0)) + eps
    expect = eps * (dout.double().numpy() * o).sum(-1) / den
    got = (qf * dq).sum(-1)
    assert np.allclose(got, expect, rtol=1e-9, atol=1e-14)


def test_gate_gradient_closed_form():
    B, N, H, D, grid = 2, 30, 2, 8, (2, 3, 5)
    q, k, v, g = random_inputs(B, N, H, D, seed=95)
    dout = random_grad(B, N, H, D, seed=96)
    _, _, _, dg = oracle.backward(q, k, v, g, dout, oracle.Grid(*grid))
    o = oracle.forward(q, k, v, g, oracle.Grid(*grid))
    s = 1.0 / (1.0 + np.exp(-g.double().numpy()))
    assert rel(dg, dout.double().numpy() * o * (1.0 - s)) < 1e-13


def test_constant_values_give_zero_q_and_k_gradients():
    B, N, H, D = 1, 20, 2, 8
    q, k, _, g = random_inputs(B, N, H, D, seed=97)
    q = positive_rows(q)
    c = torch.tensor([0.5, -1.0, 2.0, 0.25, 1.5, -0.75, 3.0, 1.0], dtype=torch.bfloat16)
    v = c.expand(B, N, H, D).contiguous()
    dout = random_grad(B, N, H, D, seed=98)
    dq, dk, dv, dg = oracle.backward(q, k, v, g, dout, None, eps=0.0)
    assert np.abs(dq).max() < 1e-12 * np.abs(dv).max()
    assert np.abs(dk).max() < 1e-12 * np.abs(dv).max()
    s = 1.0 / (1.0 + np.exp(-g.double().numpy()))
    o = s * c.double().numpy()
    assert rel(dg, dout.double().numpy() * o * (1.0 - s)) < 1e-12


def test_zero_output_gradient():
    q, k, v, g = random_inputs(1, 24, 2, 8, seed=99)
    dout = torch.zeros_like(q)
    for t in oracle.backward(q, k, v, g, dout, oracle.Grid(2, 3, 4)):
        assert not np.any(t)


def test_linear_in_output_gradient():
    B, N, H, D, grid = 1, 24, 2, 8, oracle.Grid(2, 3, 4)
    q, k, v, g = random_inputs(B, N, H, D, seed=101)
    # few mantissa bits, so the bf16 sum is exact
    rng = np.random.default_rng(3)
    d1 = torch.tensor(rng.integers(-8, 9, (B, N, H, D)) / 8.0, dtype=torch.bfloat16)
    d2 = torch.tensor(rng.integers(-8, 9, (B, N, H, D)) / 4.0, dtype=torch.bfloat16)
    g1 = oracle.backward(q, k, v, g, d1, grid)
    g2 = oracle.backward(q, k, v, g, d2, grid)
    g12 = oracle.backward(q, k, v, g, d1 + d2, grid)
    for a, b, c in zip(g1, g2, g12):
        assert rel(a + b, c) < 1e-12


def test_token_permutation_without_rope():
    B, N, H, D = 2, 19, 2, 8
    q, k, v, g = random_inputs(B, N, H, D, seed=103)
    dout = random_grad(B, N, H, D, seed=104)
    perm = torch.from_numpy(np.random.default_rng(8).permutation(N))
    base = oracle.backward(q, k, v, g, dout, None)
    permuted = oracle.backward(*(t[:, perm] for t in (q, k, v, g, dout)), None)
    for a, b in zip(base, permuted):
        assert rel(a[:, perm.numpy()], b) < 1e-12


def test_row_and_state_helpers_match_whole_pass():
    B, N, H, D, grid = 2, 36, 3, 16, oracle.Grid(3, 3, 4)
    q, k, v, g = random_inputs(B, N, H, D, seed=105)
    dout = random_grad(B, N, H, D, seed=106)
    dq, dk, dv, dg = oracle.backward(q, k, v, g, dout, grid)
    S, z = oracle.state(k, v, grid)
    dS, dz = oracle.backward_state(q, g, dout, grid, S, z)
    rows = np.array([0, 5, 17, 35, 2])
    for b in range(B):
        for h in range(H):
            rq, rg = oracle.backward_q_rows(q, g, dout, grid, b, h, S[b, h], z[b, h], rows)
            assert np.array_equal(rq, dq[b, rows, h])
            assert np.array_equal(rg, dg[b, rows, h])
            rk, rv = oracle.backward_kv_rows(k, v, grid, b, h, dS[b, h], dz[b, h], rows)
            assert np.array_equal(rk, dk[b, rows, h])
            assert np.array_equal(rv, dv[b, rows, h])


def test_gradient_state_closed_form():
    """dS = sum_n rq_n a_n^T and dz = sum_n dden_n phi(q_n), assembled here
    in numpy from the forward pieces (rotation as complex products)."""
    B, N, H, D, grid = 1, 24, 2, 8, (2, 3, 4)
    q, k, v, g = random_inputs(B, N, H, D, seed=107)
    dout = random_grad(B, N, H, D, seed=108)
    og = oracle.Grid(*grid)
    S, z = oracle.state(k, v, og)
    dS, dz = oracle.backward_state(q, g, dout, og, S, z)
    qf, kf, vf, gf = f64(q, k, v, g)
    dn = dout.double().numpy()
    fq = np.maximum(qf, 0.0)
    rq = brute.rotate_complex(np.transpose(fq, (0, 2, 1, 3)), brute.angles(D, *grid))
    zk = np.maximum(kf, 0.0).sum(axis=1)                       # [B, H, D]
    for h in range(H):
        den = fq[0, :, h] @ zk[0, h] + oracle.EPS              # [N]
        s = 1.0 / (1.0 + np.exp(-gf[0, :, h]))
        a = dn[0, :, h] * s / den[:, None]                     # [N, D]
        o = brute.forward(qf, kf, vf, gf, grid)[0, :, h]
        dden = -(dn[0, :, h] * o).sum(-1) / den
        assert rel(dS[0, h], rq[0, h].T @ a) < 1e-12
        assert rel(dz[0, h], fq[0, :, h].T @ dden) < 1e-12

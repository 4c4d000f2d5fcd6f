"""Pins of the fp64 oracle against things other than itself (CPU only).

Each test names what it checks the oracle against:
  * quadratic-form brute force (tests/brute.py, complex-number rotation);
  * a hand-derived worked example (closed form written out below);
  * closed forms and special cases of the definition;
  * invariants of rotations (norm, identity, composition, relative position);
  * structural invariants (permutation, linearity, head independence).
The frequency constants of the 3D RoPE are a reading of the pages (they only
name "Wan 3D rotary position embeddings") and stay parity unpinned; what is
pinned is that the rotation is a proper position-dependent rotation applied
the same way to q and k.
"""
import math

import numpy as np
import pytest
import torch

import brute
import oracle
from oracle import Grid
from workloads import BY_NAME, random_inputs

EPS = 1e-6


def f64(t: torch.Tensor) -> np.ndarray:
    return t.double().numpy()


def rel_err(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def bf16(x) -> torch.Tensor:
    return torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)


# --------------------------------------------------------------------------
# input decoding


def test_bf16_widening_is_exact():
    """Every finite bf16 pattern widens to the value torch assigns it."""
    bits = np.arange(65536, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    got = np.array([oracle.bf16_to_f64(int(b)) for b in bits])
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite], ref[finite])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[np.isinf(ref)], ref[np.isinf(ref)])


# --------------------------------------------------------------------------
# rotation


@pytest.mark.parametrize("D,expect", [(2, (1, 0, 0)), (32, (6, 5, 5)), (64, (12, 10, 10)),
                                      (128, (22, 21, 21))])
def test_axis_split_reading(D, expect):
    """Wan-style split: y and x get floor(D/6) pairs each, t gets the rest."""
    assert oracle.axis_split(D) == expect
    assert sum(expect) == D // 2


def test_rotation_preserves_norm():
    rng = np.random.default_rng(1)
    grid = Grid(5, 7, 9)
    for D in (32, 64, 128):
        for n in (0, 1, 17, 200, 314):
            u = rng.standard_normal(D)
            r = oracle.rotate(u, grid, n)
            assert abs(np.linalg.norm(r) - np.linalg.norm(u)) < 1e-12 * np.linalg.norm(u)


def test_rotation_identity_at_origin():
    u = np.random.default_rng(2).standard_normal(128)
    assert np.array_equal(oracle.rotate(u, Grid(3, 4, 5), 0), u)


def test_rotation_composition():
    """R(p1 + p2) = R(p2) R(p1): grid offsets add to the token's own position."""
    rng = np.random.default_rng(3)
    D = 128
    u = rng.standard_normal(D)
    base = Grid(6, 5, 7)
    for n, off in ((0, (2, 3, 4)), (37, (1, 0, 0)), (150, (9, 11, 13)), (209, (0, 0, 5))):
        one_step = oracle.rotate(u, Grid(6, 5, 7, t0=off[0], y0=off[1], x0=off[2]), n)
        first = oracle.rotate(u, base, n)
        two_step = oracle.rotate(first, Grid(6, 5, 7, t0=off[0], y0=off[1], x0=off[2]), 0)
        assert np.allclose(one_step, two_step, rtol=0, atol=1e-12)
        # the rotation by minus the total position undoes it
        t, y, x = n // 35, (n // 7) % 5, n % 7
        inv = oracle.rotate(one_step, Grid(6, 5, 7, t0=-(t + off[0]), y0=-(y + off[1]),
                                           x0=-(x + off[2])), 0)
        assert np.allclose(inv, u, rtol=0, atol=1e-12)


def test_rotation_matches_complex_product():
    """Real cos/sin arithmetic equals multiplication of x[2p] + i x[2p+1] by e^{i angle}."""
    rng = np.random.default_rng(4)
    D = 64
    grid = Grid(4, 3, 5, theta=10000.0)
    for n in range(grid.N):
        u = rng.standard_normal(D)
        t, y, x = n // 15, (n // 5) % 3, n % 5
        ang = np.array([oracle.angle(D, 1e4, p, t, y, x) for p in range(D // 2)])
        c = (u[0::2] + 1j * u[1::2]) * np.exp(1j * ang)
        ref = np.empty(D)
        ref[0::2], ref[1::2] = c.real, c.imag
        assert np.allclose(oracle.rotate(u, grid, n), ref, rtol=0, atol=1e-13)


def test_rope_axis_blocks_follow_token_order():
    """Pair 0 of each axis block turns by exactly the token's t, y, x index
    (its frequency is theta^0 = 1), and moving along one axis only turns
    that axis's pairs."""
    D = 128
    pt, py, px = oracle.axis_split(D)
    for (t, y, x) in ((0, 0, 0), (3, 1, 2), (24, 21, 39), (180, 0, 7)):
        assert oracle.angle(D, 1e4, 0, t, y, x) == t
        assert oracle.angle(D, 1e4, pt, t, y, x) == y
        assert oracle.angle(D, 1e4, pt + py, t, y, x) == x
    a = np.array([oracle.angle(D, 1e4, p, 2, 3, 4) for p in range(D // 2)])
    for axis, (sl, d) in enumerate(((slice(0, pt), (1, 0, 0)), (slice(pt, pt + py), (0, 1, 0)),
                                    (slice(pt + py, None), (0, 0, 1)))):
        b = np.array([oracle.angle(D, 1e4, p, 2 + d[0], 3 + d[1], 4 + d[2])
                      for p in range(D // 2)])
        changed = np.nonzero(a != b)[0]
        assert set(changed) == set(range(D // 2)[sl])
    # frequencies fall monotonically within each axis block
    for sl in (slice(0, pt), slice(pt, pt + py), slice(pt + py, None)):
        w = np.array([oracle.angle(D, 1e4, p, 1, 1, 1) for p in range(D // 2)])[sl]
        assert np.all(np.diff(w) < 0)
    # token n = (t*Hh + y)*W + x of a grid sits at (t, y, x)
    u = np.zeros(D)
    u[0] = 1.0
    u[2 * pt] = 1.0
    u[2 * (pt + py)] = 1.0
    grid = Grid(3, 4, 5)
    for t in range(3):
        for y in range(4):
            for x in range(5):
                r = oracle.rotate(u, grid, (t * 4 + y) * 5 + x)
                assert math.isclose(math.atan2(r[1], r[0]), math.atan2(math.sin(t), math.cos(t)),
                                    abs_tol=1e-12)
                assert math.isclose(math.atan2(r[2 * pt + 1], r[2 * pt]),
                                    math.atan2(math.sin(y), math.cos(y)), abs_tol=1e-12)
                assert math.isclose(math.atan2(r[2 * (pt + py) + 1], r[2 * (pt + py)]),
                                    math.atan2(math.sin(x), math.cos(x)), abs_tol=1e-12)


# --------------------------------------------------------------------------
# brute force


TINY = [
    # B, H, D, grid or N
    (1, 1, 32, (1, 1, 1)),
    (1, 2, 32, (1, 1, 2)),
    (1, 1, 32, (1, 1, 7)),
    (2, 3, 32, (2, 3, 5)),
    (1, 2, 32, (4, 8, 8)),
    (1, 1, 64, (2, 4, 8)),
    (1, 2, 128, (4, 8, 8)),
    (2, 1, 128, (3, 5, 7)),
]


@pytest.mark.parametrize("B,H,D,g3", TINY)
@pytest.mark.parametrize("rope", [True, False])
def test_oracle_matches_quadratic_brute_force(B, H, D, g3, rope):
    N = g3[0] * g3[1] * g3[2]
    q, k, v, g = random_inputs(B, N, H, D, seed=100 + N + D + B * 7 + H)
    grid = Grid(*g3) if rope else None
    got = oracle.forward(q, k, v, g, grid)
    ref = brute.forward(f64(q), f64(k), f64(v), f64(g), g3 if rope else None)
    assert rel_err(got, ref) < 1e-12
    assert np.max(np.abs(got - ref)) < 1e-12 * max(1.0, np.max(np.abs(ref)))


def test_oracle_state_matches_direct_sums():
    """S and z equal their defining sums formed with complex rotation in numpy."""
    B, H, D, g3 = 1, 2, 32, (2, 3, 4)
    N = 24
    q, k, v, g = random_inputs(B, N, H, D, seed=7)
    S, z = oracle.state(k, v, Grid(*g3))
    fk = np.maximum(f64(k), 0)
    ang = brute.angles(D, *g3)
    for h in range(H):
        rk = brute.rotate_complex(fk[0, :, h], ang)
        assert np.allclose(S[0, h], rk.T @ f64(v)[0, :, h], rtol=0, atol=1e-12)
        assert np.allclose(z[0, h], fk[0, :, h].sum(0), rtol=0, atol=1e-12)


def test_spot_rows_at_full_size():
    """At the 5B 480p/81-frame shape, 64 sampled rows equal the O(N D) row form."""
    w = BY_NAME["5b_480p_81f"]
    q, k, v, g = random_inputs(w.B, w.N, w.H, w.D, seed=w.seed, qk_scale=w.qk_scale)
    grid = Grid(w.T, w.Hh, w.W)
    rng = np.random.default_rng(5)
    qd, kd, vd, gd = f64(q), f64(k), f64(v), f64(g)
    heads = sorted(set(int(x) for x in rng.integers(0, w.H, 4)))
    for h in heads:
        ks, vs = k[:, :, h:h + 1].contiguous(), v[:, :, h:h + 1].contiguous()
        S, z = oracle.state(ks, vs, grid)
        toks = rng.integers(0, w.N, 16)
        got = oracle.rows(q[:, :, h:h + 1].contiguous(), g[:, :, h:h + 1].contiguous(), grid,
                          0, 0, S[0, 0], z[0, 0], toks)
        for i, n in enumerate(toks):
            ref = brute.row(qd, kd, vd, gd, 0, h, int(n), (w.T, w.Hh, w.W))
            assert np.allclose(got[i], ref, rtol=1e-11, atol=1e-15)


# --------------------------------------------------------------------------
# hand-derived worked example


def test_hand_worked_example():
    """D = 2 (one pair, t axis, omega = 1), grid T=2, Hh=W=1 so token n turns by n rad.

    k0 = (1, 0), k1 = (1, 1), v0 = (1, 2), v1 = (3, -1), q0 = (2, 1), q1 = (-1, 1), g = 0.
    With c = cos 1, s = sin 1:
      R0 phi(k0) = (1, 0), R1 phi(k1) = (c - s, s + c), z = (2, 1);
      R0 phi(q0) = (2, 1), R1 phi(q1) = R1 (0, 1) = (-s, c);
      num0 = 2 v0 + (2(c - s) + (s + c)) v1 = 2 v0 + (3c - s) v1, den0 = 5 + eps;
      num1 = -s v0 + (-s(c - s) + c(s + c)) v1 = -s v0 + v1,       den1 = 1 + eps;
      o_n = num_n / (2 den_n).
    """
    c, s = math.cos(1.0), math.sin(1.0)
    v0, v1 = np.array([1.0, 2.0]), np.array([3.0, -1.0])
    o0 = (2 * v0 + (3 * c - s) * v1) / (2 * (5 + EPS))
    o1 = (-s * v0 + v1) / (2 * (1 + EPS))
    q = bf16([[[[2, 1]], [[-1, 1]]]])
    k = bf16([[[[1, 0]], [[1, 1]]]])
    v = bf16([[[[1, 2]], [[3, -1]]]])
    g = bf16(np.zeros((1, 2, 1, 2)))
    got = oracle.forward(q, k, v, g, Grid(2, 1, 1))
    assert np.allclose(got[0, 0, 0], o0, rtol=1e-15, atol=1e-16)
    assert np.allclose(got[0, 1, 0], o1, rtol=1e-15, atol=1e-16)


# --------------------------------------------------------------------------
# closed forms and special cases


def _const_v(B, N, H, D, seed):
    q, k, _, g = random_inputs(B, N, H, D, seed=seed)
    c = np.linspace(-2.0, 2.0, D).astype(np.float32)
    v = bf16(np.broadcast_to(c, (B, N, H, D)).copy())
    return q, k, v, g, f64(v)[0, 0, 0]


def test_constant_v_rope_off():
    """Every v row equal to c, no RoPE: o_n = sigma(g_n) c (phi(q_n).z) / (phi(q_n).z + eps)."""
    B, N, H, D = 1, 96, 2, 32
    q, k, v, g, c = _const_v(B, N, H, D, 11)
    got = oracle.forward(q, k, v, g, None)
    fq, fk = np.maximum(f64(q), 0), np.maximum(f64(k), 0)
    sg = 1 / (1 + np.exp(-f64(g)))
    for h in range(H):
        qz = fq[0, :, h] @ fk[0, :, h].sum(0)
        ref = sg[0, :, h] * c[None, :] * (qz / (qz + EPS))[:, None]
        assert np.allclose(got[0, :, h], ref, rtol=1e-13, atol=1e-15)


def test_constant_v_rope_on():
    """v = c with RoPE: o_n = sigma(g_n) c (R_n phi(q_n) . sum_m R_m phi(k_m)) / (phi(q_n).z + eps)."""
    B, H, D, g3 = 1, 2, 64, (3, 4, 5)
    N = 60
    q, k, v, g, c = _const_v(B, N, H, D, 12)
    grid = Grid(*g3)
    got = oracle.forward(q, k, v, g, grid)
    fq, fk = np.maximum(f64(q), 0), np.maximum(f64(k), 0)
    sg = 1 / (1 + np.exp(-f64(g)))
    for h in range(H):
        rk_sum = sum(oracle.rotate(fk[0, m, h], grid, m) for m in range(N))
        z = fk[0, :, h].sum(0)
        for n in range(N):
            w = oracle.rotate(fq[0, n, h], grid, n) @ rk_sum
            ref = sg[0, n, h] * c * w / (fq[0, n, h] @ z + EPS)
            assert np.allclose(got[0, n, h], ref, rtol=1e-12, atol=1e-15)


def test_nonpositive_q_rows_are_exactly_zero():
    B, N, H, D = 1, 40, 2, 32
    q, k, v, g = random_inputs(B, N, H, D, seed=13)
    qn = f64(q)
    qn[0, ::3] = -np.abs(qn[0, ::3])
    qn[0, 1, 0] = 0.0
    q = bf16(qn)
    got = oracle.forward(q, k, v, g, Grid(1, 5, 8))
    assert np.all(got[0, ::3] == 0.0)
    assert np.all(got[0, 1, 0] == 0.0)
    assert np.any(got[0, 2] != 0.0)


def test_all_k_nonpositive_gives_zero():
    B, N, H, D = 1, 30, 2, 32
    q, k, v, g = random_inputs(B, N, H, D, seed=14)
    k = bf16(-np.abs(f64(k)))
    got = oracle.forward(q, k, v, g, Grid(2, 3, 5))
    assert np.all(got == 0.0)


def test_single_token_q_equals_k():
    """N = 1, q = k: o = sigma(g) v |phi(q)|^2 / (|phi(q)|^2 + eps) (R_0 . R_0 cancels)."""
    D = 128
    q, _, v, g = random_inputs(1, 1, 1, D, seed=15)
    got = oracle.forward(q, q, v, g, Grid(1, 1, 1, t0=5, y0=6, x0=7))
    fq = np.maximum(f64(q)[0, 0, 0], 0)
    nn = fq @ fq
    ref = (1 / (1 + np.exp(-f64(g)[0, 0, 0]))) * f64(v)[0, 0, 0] * nn / (nn + EPS)
    assert np.allclose(got[0, 0, 0], ref, rtol=1e-14, atol=0)


def test_gate_zero_is_half_of_open_gate():
    B, N, H, D = 1, 48, 1, 32
    q, k, v, _ = random_inputs(B, N, H, D, seed=16)
    g0 = bf16(np.zeros((B, N, H, D)))
    g30 = bf16(np.full((B, N, H, D), 30.0))
    grid = Grid(2, 4, 6)
    a = oracle.forward(q, k, v, g0, grid)
    b = oracle.forward(q, k, v, g30, grid)
    assert np.allclose(a, 0.5 * b / (1.0 / (1.0 + math.exp(-30.0))), rtol=1e-14, atol=0)


def test_qk_scaling_only_moves_eps():
    """Scaling q by a and k by b (powers of two, exact in bf16) scales numerator and
    phi(q).z by a b, so o' = o_num a b / (a b Q + eps) with Q = phi(q).z."""
    B, N, H, D = 1, 64, 1, 32
    q, k, v, g = random_inputs(B, N, H, D, seed=17)
    grid = Grid(4, 4, 4)
    a, bsc = 0.25, 8.0
    o1 = oracle.forward(q, k, v, g, grid)
    o2 = oracle.forward(bf16(f64(q) * a), bf16(f64(k) * bsc), v, g, grid)
    fq, fk = np.maximum(f64(q), 0), np.maximum(f64(k), 0)
    Q = fq[0, :, 0] @ fk[0, :, 0].sum(0)
    ratio = (a * bsc * (Q + EPS)) / (a * bsc * Q + EPS)
    assert np.allclose(o2[0, :, 0], o1[0, :, 0] * ratio[:, None], rtol=1e-13, atol=0)


# --------------------------------------------------------------------------
# structure


def test_permutation_equivariance_without_rope():
    B, N, H, D = 1, 50, 2, 32
    q, k, v, g = random_inputs(B, N, H, D, seed=18)
    perm = torch.from_numpy(np.random.default_rng(0).permutation(N))
    S1, z1 = oracle.state(k, v, None)
    S2, z2 = oracle.state(k[:, perm].contiguous(), v[:, perm].contiguous(), None)
    assert np.allclose(S1, S2, rtol=1e-13, atol=1e-13)
    assert np.allclose(z1, z2, rtol=1e-13, atol=1e-13)
    o1 = oracle.forward(q, k, v, g, None)
    o2 = oracle.forward(*(t[:, perm].contiguous() for t in (q, k, v, g)), None)
    assert np.allclose(o1[:, perm.numpy()], o2, rtol=1e-12, atol=1e-15)


def test_linear_in_v():
    B, N, H, D = 1, 40, 1, 32
    q, k, v1, g = random_inputs(B, N, H, D, seed=19)
    _, _, v2, _ = random_inputs(B, N, H, D, seed=20)
    grid = Grid(2, 4, 5)
    vs = bf16(f64(v1) + 2.0 * f64(v2))  # may round; compare against the rounded sum
    o1 = oracle.forward(q, k, v1, g, grid)
    o2 = oracle.forward(q, k, v2, g, grid)
    o3 = oracle.forward(q, k, vs, g, grid)
    # the linear combination of outputs for the exact sum, minus its rounding
    dv = f64(vs) - (f64(v1) + 2.0 * f64(v2))
    o_dv = brute.forward(f64(q), f64(k), dv, f64(g), (2, 4, 5))
    assert np.allclose(o3, o1 + 2.0 * o2 + o_dv, rtol=1e-11, atol=1e-14)


def test_heads_and_batches_are_independent():
    B, N, H, D = 2, 30, 3, 32
    q, k, v, g = random_inputs(B, N, H, D, seed=21)
    grid = Grid(2, 3, 5)
    base = oracle.forward(q, k, v, g, grid)
    k2 = k.clone()
    k2[1, :, 2] = bf16(np.random.default_rng(1).standard_normal((N, D)))
    alt = oracle.forward(q, k2, v, g, grid)
    changed = np.zeros((B, H), bool)
    for b in range(B):
        for h in range(H):
            changed[b, h] = not np.array_equal(base[b, :, h], alt[b, :, h])
    assert changed[1, 2] and changed.sum() == 1


def test_relative_position_invariance():
    """Shifting every grid index by the same offset leaves o unchanged (R_a u . R_b w
    depends on b - a only)."""
    B, N, H, D = 1, 60, 2, 64
    q, k, v, g = random_inputs(B, N, H, D, seed=22)
    o1 = oracle.forward(q, k, v, g, Grid(3, 4, 5))
    o2 = oracle.forward(q, k, v, g, Grid(3, 4, 5, t0=17, y0=-3, x0=101))
    assert rel_err(o2, o1) < 1e-12


def test_empty_sequence_without_rope():
    q = torch.zeros((1, 0, 2, 32), dtype=torch.bfloat16)
    out = oracle.forward(q, q, q, q, None)
    assert out.shape == (1, 0, 2, 32)


def test_grid_mismatch_rejected():
    q, k, v, g = random_inputs(1, 10, 1, 32, seed=0)
    with pytest.raises(ValueError):
        oracle.forward(q, k, v, g, Grid(2, 2, 2))


# --------------------------------------------------------------------------
# regression snapshot


def test_golden_snapshot():
    """tests/golden/oracle_small.txt was written by tests/golden/make_golden.py from
    the oracle alone; this guards the oracle against accidental change."""
    import golden.make_golden as mg
    ref = mg.read()
    got = mg.compute()
    assert got.shape == ref.shape
    assert np.allclose(got, ref, rtol=1e-13, atol=1e-16)

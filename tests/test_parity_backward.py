"""GPU parity of the mixer's backward pass (through the C ABI) against the
fp64 oracle (oracle.backward and its row/state helpers).

Bar, per gradient (dq, dk, dv, dg): relative L2 error <= 5e-3 and max
absolute error <= 3e-2 against the oracle's fp64 gradients on the same bf16
inputs and output gradient.  The GPU rounds S, dS, the rotated features and
a = dout * sigmoid(g) / den to bf16 as MFMA operands, and the gradients to
bf16.  Every shape, the five layer shapes included, is compared element by
element over every gradient: the layer shapes a few heads at a time against
oracle.backward, with the errors taken over the whole tensors.
"""
import numpy as np
import pytest
import torch

import gated_linear_attention_forward_amd as gla
import oracle
from workloads import BY_NAME, WORKLOADS, make_inputs, random_grad, random_inputs

pytestmark = pytest.mark.gpu

REL_TOL = 5e-3
ABS_TOL = 3e-2
TERM_TOL = 2 * 3 * 2.0 ** -9   # two terms, three bf16 roundings each (see assert_cancelling)
DEV = torch.device("cuda:0")
NAMES = ("dq", "dk", "dv", "dg")


def say(msg):
    print(msg, flush=True)


def errs(got, ref):
    got = np.asarray(got, np.float64)
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    mx = float(np.max(np.abs(got - ref))) if got.size else 0.0
    return rel, mx


def assert_close(got, ref, what):
    rel, mx = errs(got, ref)
    say(f"  {what}: rel_l2={rel:.3e} max_abs={mx:.3e} max|ref|={np.max(np.abs(ref)):.3e}")
    assert rel <= REL_TOL, f"{what}: rel_l2 {rel}"
    assert mx <= ABS_TOL, f"{what}: max_abs {mx}"


def gpu_backward(q, k, v, g, dout, grid):
    """grid: (T, Hh, W) or None; the four bf16 gradients as CPU float64 arrays."""
    qd, kd, vd, gd, dd = (t.to(DEV) for t in (q, k, v, g, dout))
    rope = gla.gla_rope_create(*grid, q.shape[-1]) if grid is not None else None
    grads = gla.gla_backward(qd, kd, vd, gd, dd, rope)
    torch.cuda.synchronize()
    if rope is not None:
        rope.close()
    return tuple(t.double().cpu().numpy() for t in grads)


SMALL = [
    # B, H, D, grid (T, Hh, W)
    (1, 2, 32, (4, 8, 8)),      # the tiny workload
    (1, 1, 32, (1, 1, 1)),      # a single token
    (1, 3, 32, (1, 1, 7)),      # fewer tokens than one tile
    (2, 3, 64, (3, 5, 7)),      # D = 64, ragged
    (1, 2, 128, (2, 3, 43)),    # 258 tokens: a 2-token tail
    (2, 2, 128, (7, 11, 13)),   # 1001 tokens, B = 2
    (1, 1, 128, (1, 1, 65)),    # one past a tile
    (3, 1, 32, (5, 7, 11)),     # 385 tokens, D = 32, B = 3
]


@pytest.mark.parametrize("B,H,D,grid", SMALL)
@pytest.mark.parametrize("rope", [True, False])
def test_backward_small_shapes(B, H, D, grid, rope):
    N = grid[0] * grid[1] * grid[2]
    say(f"case backward B={B} H={H} D={D} grid={grid} rope={rope}")
    q, k, v, g = random_inputs(B, N, H, D, seed=700 + N + D + H)
    dout = random_grad(B, N, H, D, seed=800 + N + D + H)
    got = gpu_backward(q, k, v, g, dout, grid if rope else None)
    ref = oracle.backward(q, k, v, g, dout, oracle.Grid(*grid) if rope else None)
    if N == 1:
        # one token: R turns q and k alike, so dq's terms R^T (S a) = phi(k) (v . a)
        # and dden z cancel up to eps (dk's likewise)
        env = rounding_envelope(q, k, v, g, dout, grid if rope else None)
        assert_cancelling(got[:2], ref[:2], env)
        checked = ("dv", "dg")
    else:
        checked = NAMES
    for name, a, b in zip(NAMES, got, ref):
        if name in checked:
            assert_close(a, b, name)


@pytest.mark.parametrize("D", [32, 64])
def test_backward_long_ranges(D):
    """D = 32 and 64 over 100,000 tokens: every block's range spans several
    128-token steps of the query kernel's dS contraction (the layer shapes
    cover D = 128), with RoPE and a ragged tail, against the full oracle."""
    B, H, grid = 1, 2, (25, 40, 101)
    N = grid[0] * grid[1] * grid[2]
    say(f"case backward long ranges B={B} H={H} D={D} grid={grid} N={N}")
    q, k, v, g = random_inputs(B, N, H, D, seed=1300 + D)
    dout = random_grad(B, N, H, D, seed=1400 + D)
    got = gpu_backward(q, k, v, g, dout, grid)
    ref = oracle.backward(q, k, v, g, dout, oracle.Grid(*grid))
    for name, a, b in zip(NAMES, got, ref):
        assert_close(a, b, name)


def rounding_envelope(q, k, v, g, dout, grid):
    """Norms of the dot-product error envelopes of dq and dk: with operands
    rounded to bf16, a dot product sum_e x_e y_e is off by at most about
    u * sum_e |x_e| |y_e|.  dq's dot products are (S a)[d] and the dden z
    term, dk's (dS v)[d] and dz, so the envelopes are |S| |a| + |dden| |z|
    (where q > 0) and |dS| |v| + |dz| (where k > 0), with the oracle's S, z,
    dS, dz (R^T keeps 2-norms, so the norms hold with RoPE)."""
    og = oracle.Grid(*grid) if grid is not None else None
    S, z = oracle.state(k, v, og)
    dS, dz = oracle.backward_state(q, g, dout, og, S, z)
    o = oracle.forward(q, k, v, g, og)
    qf, kf, vf, gf, df = (t.double().numpy() for t in (q, k, v, g, dout))
    fq = np.maximum(qf, 0)
    den = np.einsum("bnhd,bhd->bnh", fq, z)[..., None] + oracle.EPS
    a = df / (1 + np.exp(-gf)) / den
    dden = -(df * o).sum(-1, keepdims=True) / den
    env_q = np.einsum("bhde,bnhe->bnhd", np.abs(S), np.abs(a)) + np.abs(dden) * np.abs(z)[:, None]
    env_k = np.einsum("bhde,bnhe->bnhd", np.abs(dS), np.abs(vf)) + np.abs(dz)[:, None]
    return np.linalg.norm(env_q * (qf > 0)), np.linalg.norm(env_k * (kf > 0))


def assert_cancelling(got, ref, envelopes, names=("dq", "dk")):
    """For gradients whose exact value vanishes up to eps (their two terms
    cancel), a relative error has no meaning: the absolute bar applies, and
    the error is bounded by the rounding envelope of the terms.  Each dot
    product carries the bf16 roundings of its operands and of the features
    behind them (S or dS, a, the rotated features: 3 * 2^-9), and the two
    terms add theirs: TERM_TOL = 2 * 3 * 2^-9 of the envelope."""
    for idx, name in enumerate(names):
        err = float(np.linalg.norm(got[idx] - ref[idx]) / envelopes[idx])
        mx = float(np.max(np.abs(got[idx] - ref[idx])))
        say(f"  {name} (terms cancel): err/envelope={err:.3e} max_abs={mx:.3e} "
            f"max|ref|={np.max(np.abs(ref[idx])):.3e}")
        assert err <= TERM_TOL and mx <= ABS_TOL


@pytest.mark.parametrize("name", [w.name for w in WORKLOADS])
def test_backward_workload(name):
    """The layer shapes: every element of dq, dk, dv and dg of every head."""
    w = BY_NAME[name]
    say(f"case backward workload {w.name} B={w.B} N={w.N} H={w.H} D={w.D}")
    q, k, v, g = make_inputs(w)
    dout = random_grad(w.B, w.N, w.H, w.D, seed=w.seed + 1000)
    qd, kd, vd, gd, dd = (t.to(DEV) for t in (q, k, v, g, dout))
    rope = gla.gla_rope_create(w.T, w.Hh, w.W, w.D, w.theta)
    grads = gla.gla_backward(qd, kd, vd, gd, dd, rope)
    torch.cuda.synchronize()
    rope.close()
    del qd, kd, vd, gd, dd
    grads = [t.cpu() for t in grads]
    grid = oracle.Grid(w.T, w.Hh, w.W, w.theta)
    d2 = {n: 0.0 for n in NAMES}
    r2 = {n: 0.0 for n in NAMES}
    mx = {n: 0.0 for n in NAMES}
    group = max(4, oracle.num_threads())  # the oracle runs one head per thread
    for b in range(w.B):
        for h0 in range(0, w.H, group):
            h1 = min(h0 + group, w.H)
            sl = lambda t: t[b:b + 1, :, h0:h1].contiguous()
            ref = oracle.backward(sl(q), sl(k), sl(v), sl(g), sl(dout), grid)
            for n, t, r in zip(NAMES, grads, ref):
                got = t[b:b + 1, :, h0:h1].double().numpy()
                d2[n] += float(np.sum((got - r) ** 2))
                r2[n] += float(np.sum(r ** 2))
                mx[n] = max(mx[n], float(np.max(np.abs(got - r))))
    for n in NAMES:
        rel = (d2[n] / r2[n]) ** 0.5
        say(f"  {w.name} all {n}: rel_l2={rel:.3e} max_abs={mx[n]:.3e}")
        assert rel <= REL_TOL, f"{n}: rel_l2 {rel}"
        assert mx[n] <= ABS_TOL, f"{n}: max_abs {mx[n]}"


def test_backward_constant_values_without_rope():
    """Constant v rows c make o = sigmoid(g) * c up to eps:
    dq_n = z (c . a_n) (1 - phi(q_n).z / den_n) and
    dk_m = sum_n phi(q_n) (c . a_n) (1 - phi(q_n).z / den_n) vanish up to eps
    (checked against the rounding envelope); dv and dg take the usual bar."""
    B, N, H, D = 1, 200, 2, 64
    say("case backward constant v")
    q, k, _, g = random_inputs(B, N, H, D, seed=901)
    c = torch.linspace(-2.0, 2.0, D).to(torch.bfloat16)
    v = c.expand(B, N, H, D).contiguous()
    dout = random_grad(B, N, H, D, seed=902)
    got = gpu_backward(q, k, v, g, dout, None)
    ref = oracle.backward(q, k, v, g, dout, None)
    assert_close(got[2], ref[2], "dv")
    assert_close(got[3], ref[3], "dg")
    assert_cancelling(got[:2], ref[:2], rounding_envelope(q, k, v, g, dout, None))


def test_backward_deterministic_and_workspace_entry_point():
    w = BY_NAME["5b_480p_81f"]
    say("case backward determinism")
    q, k, v, g = (t.to(DEV) for t in make_inputs(w))
    dout = random_grad(w.B, w.N, w.H, w.D, seed=5).to(DEV)
    rope = gla.gla_rope_create(w.T, w.Hh, w.W, w.D, w.theta)
    g1 = gla.gla_backward(q, k, v, g, dout, rope)
    ws = gla.alloc_workspace_backward(w.B, w.N, w.H, w.D, DEV)
    g2 = gla.gla_backward_ws(q, k, v, g, dout, rope, ws)
    g3 = gla.gla_backward_ws(q, k, v, g, dout, rope, ws)
    torch.cuda.synchronize()
    rope.close()
    for a, b, c in zip(g1, g2, g3):
        assert torch.equal(a, b) and torch.equal(b, c)


def test_backward_empty_and_errors():
    say("case backward empty / errors")
    x = torch.empty((1, 0, 2, 32), dtype=torch.bfloat16, device=DEV)
    outs = gla.gla_backward(x, x.clone(), x.clone(), x.clone(), x.clone())
    assert all(t.shape == x.shape for t in outs)
    y = torch.zeros((1, 8, 1, 48), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(gla.GlaError):
        gla.gla_backward(y, y.clone(), y.clone(), y.clone(), y.clone())  # D = 48 is not served
    z = torch.zeros((1, 8, 1, 32), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(gla.GlaError):
        gla.gla_backward(z, z.clone(), z.clone(), z.clone(), z.clone(), dq=z)  # dq aliases q

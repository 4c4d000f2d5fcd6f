"""GPU tests of the backward pass that takes the forward's state (S, z)
instead of recomputing it, through the C ABI.

With the state the forward returns (gla_forward_blocks with one attention
block, S_out and z_out), the gradients must equal gla_backward's bit for
bit: both form the same fp32 sums, and from there the passes are the same.
With any other state they are the chain rule at that state, checked
against the oracle's per-head helpers (backward_q_rows for dq and dg,
backward_state for dS and dz, backward_kv_rows for dk and dv) to the
backward pass's bar: relative L2 <= 5e-3 and max abs <= 3e-2.
"""
import numpy as np
import pytest
import torch

import gated_linear_attention_forward_amd as gla
import oracle
from workloads import BY_NAME, make_inputs, random_grad, random_inputs

pytestmark = pytest.mark.gpu

REL_TOL = 5e-3
ABS_TOL = 3e-2
DEV = torch.device("cuda:0")
NAMES = ("dq", "dk", "dv", "dg")


def say(msg):
    print(msg, flush=True)


def assert_close(got, ref, what):
    got = np.asarray(got, np.float64)
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    mx = float(np.max(np.abs(got - ref)))
    say(f"  {what}: rel_l2={rel:.3e} max_abs={mx:.3e}")
    assert rel <= REL_TOL, f"{what}: rel_l2 {rel}"
    assert mx <= ABS_TOL, f"{what}: max_abs {mx}"


def forward_state(q, k, v, g, rope):
    """The forward's output and its fp32 state from one attention block."""
    B, N, H, D = q.shape
    S = torch.empty((B, H, D, D), dtype=torch.float32, device=DEV)
    z = torch.empty((B, H, D), dtype=torch.float32, device=DEV)
    out = gla.gla_forward_blocks(q, k, v, g, rope, N, None, None, S, z)
    return out, S, z


CASES = [
    # B, H, D, grid (T, Hh, W)
    (1, 2, 32, (4, 8, 8)),
    (2, 3, 64, (3, 5, 7)),
    (1, 2, 128, (2, 3, 43)),
    (2, 2, 128, (7, 11, 13)),
    (1, 1, 128, (1, 1, 1)),
]


@pytest.mark.parametrize("B,H,D,grid", CASES)
@pytest.mark.parametrize("rope", [True, False])
def test_saved_state_matches_recompute_bitwise(B, H, D, grid, rope):
    N = grid[0] * grid[1] * grid[2]
    say(f"case saved-state backward B={B} H={H} D={D} grid={grid} rope={rope}")
    q, k, v, g = (t.to(DEV) for t in random_inputs(B, N, H, D, seed=900 + N + D))
    dout = random_grad(B, N, H, D, seed=950 + N + D).to(DEV)
    tables = gla.gla_rope_create(*grid, D) if rope else None
    out, S, z = forward_state(q, k, v, g, tables)
    assert torch.equal(out, gla.gla_forward(q, k, v, g, tables))
    ref = gla.gla_backward(q, k, v, g, dout, tables)
    got = gla.gla_backward_saved(q, k, v, g, dout, S, z, tables)
    ws = gla.alloc_workspace_backward(B, N, H, D, DEV)
    got_ws = gla.gla_backward_saved_ws(q, k, v, g, dout, S, z, tables, ws)
    torch.cuda.synchronize()
    for name, a, b, c in zip(NAMES, got, ref, got_ws):
        assert torch.equal(a, b), f"{name} differs from gla_backward"
        assert torch.equal(c, b), f"{name} (_ws) differs from gla_backward"
    if tables is not None:
        tables.close()


def test_saved_state_matches_recompute_at_layer_shape():
    w = BY_NAME["5b_720p_193f"]
    say(f"case saved-state backward {w.name}")
    q, k, v, g = (t.to(DEV) for t in make_inputs(w))
    dout = random_grad(w.B, w.N, w.H, w.D, seed=5).to(DEV)
    tables = gla.gla_rope_create(w.T, w.Hh, w.W, w.D, w.theta)
    _, S, z = forward_state(q, k, v, g, tables)
    ref = gla.gla_backward(q, k, v, g, dout, tables)
    got = gla.gla_backward_saved(q, k, v, g, dout, S, z, tables)
    torch.cuda.synchronize()
    for name, a, b in zip(NAMES, got, ref):
        assert torch.equal(a, b), f"{name} differs from gla_backward"
    tables.close()


@pytest.mark.parametrize("D,grid", [(32, (3, 4, 5)), (128, (2, 3, 43))])
def test_other_state_against_oracle(D, grid):
    """An S and z that are not k and v's: the gradients at that state."""
    B, H = 1, 2
    N = grid[0] * grid[1] * grid[2]
    say(f"case backward at a given state B={B} H={H} D={D} grid={grid}")
    q, k, v, g = random_inputs(B, N, H, D, seed=970 + N + D)
    dout = random_grad(B, N, H, D, seed=980 + N + D)
    gen = torch.Generator().manual_seed(990 + D)
    S = torch.randn((B, H, D, D), generator=gen, dtype=torch.float32) * 4.0
    z = torch.rand((B, H, D), generator=gen, dtype=torch.float32) * 20.0 + 1.0
    tables = gla.gla_rope_create(*grid, D)
    got = gla.gla_backward_saved(*(t.to(DEV) for t in (q, k, v, g, dout)), S.to(DEV), z.to(DEV),
                                 tables)
    torch.cuda.synchronize()
    got = [t.double().cpu().numpy() for t in got]
    tables.close()
    og = oracle.Grid(*grid)
    Sd, zd = S.double().numpy(), z.double().numpy()
    dS, dz = oracle.backward_state(q, g, dout, og, Sd, zd)
    rows = np.arange(N)
    ref = {n: np.empty((B, N, H, D)) for n in NAMES}
    for b in range(B):
        for h in range(H):
            dq, dg = oracle.backward_q_rows(q, g, dout, og, b, h, Sd[b, h], zd[b, h], rows)
            dk, dv = oracle.backward_kv_rows(k, v, og, b, h, dS[b, h], dz[b, h], rows)
            ref["dq"][b, :, h], ref["dg"][b, :, h] = dq, dg
            ref["dk"][b, :, h], ref["dv"][b, :, h] = dk, dv
    for name, a in zip(NAMES, got):
        assert_close(a, ref[name], name)


def test_saved_state_empty_and_errors():
    q = torch.zeros((1, 0, 2, 64), dtype=torch.bfloat16, device=DEV)
    S = torch.zeros((1, 2, 64, 64), dtype=torch.float32, device=DEV)
    z = torch.zeros((1, 2, 64), dtype=torch.float32, device=DEV)
    grads = gla.gla_backward_saved(q, q, q, q, q, S, z)
    assert all(t.shape == q.shape for t in grads)
    q = torch.zeros((1, 16, 2, 64), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):
        gla.gla_backward_saved(q, q, q, q, q, S[:, :1], z)
    with pytest.raises(ValueError):
        gla.gla_backward_saved(q, q, q, q, q, None, z)


@pytest.mark.parametrize("rope", [True, False])
def test_autograd_function_matches_the_entry_points(rope):
    """gated_linear_attention under torch.autograd: the forward equals
    gla_forward and the gradients equal gla_backward's, bit for bit."""
    B, H, D, grid = 2, 3, 64, (3, 5, 7)
    N = grid[0] * grid[1] * grid[2]
    say(f"case autograd function B={B} H={H} D={D} grid={grid} rope={rope}")
    q, k, v, g = (t.to(DEV) for t in random_inputs(B, N, H, D, seed=1500 + N))
    dout = random_grad(B, N, H, D, seed=1550 + N).to(DEV)
    tables = gla.gla_rope_create(*grid, D) if rope else None
    leaves = [t.clone().requires_grad_(True) for t in (q, k, v, g)]
    out = gla.gated_linear_attention(*leaves, tables)
    out.backward(dout)
    assert torch.equal(out.detach(), gla.gla_forward(q, k, v, g, tables))
    ref = gla.gla_backward(q, k, v, g, dout, tables)
    for name, leaf, r in zip(NAMES, leaves, ref):
        assert torch.equal(leaf.grad, r), f"{name} differs from gla_backward"
    if tables is not None:
        tables.close()

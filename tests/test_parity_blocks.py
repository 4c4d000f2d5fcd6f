"""GPU parity of the block-causal pass with a carried state (the
constant-memory KV cache for block linear attention, "SANA-Video_2B_720p"
model card, innovation (2)) against the fp64 oracle, through the C ABI.

Bar as for the bidirectional mixer: relative L2 <= 5e-3 and max abs <= 3e-2
on the bf16 output; the returned fp32 state within 3e-3 (S, summed from
bf16-rounded R phi(k)) and 1e-6 (z, exact features) relative L2.
"""
import numpy as np
import pytest
import torch

import gated_linear_attention_forward_amd as gla
import oracle
from workloads import BY_NAME, make_inputs, random_inputs

pytestmark = pytest.mark.gpu

REL_TOL = 5e-3
ABS_TOL = 3e-2
DEV = torch.device("cuda:0")


def say(msg):
    print(msg, flush=True)


def rel(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def assert_close(got, ref, what):
    got = np.asarray(got, np.float64)
    r, mx = rel(got, ref), float(np.max(np.abs(got - ref))) if got.size else 0.0
    say(f"  {what}: rel_l2={r:.3e} max_abs={mx:.3e}")
    assert r <= REL_TOL, f"{what}: rel_l2 {r}"
    assert mx <= ABS_TOL, f"{what}: max_abs {mx}"


def carried(B, H, D, seed):
    gen = torch.Generator().manual_seed(seed)
    S = torch.randn((B, H, D, D), generator=gen, dtype=torch.float32)
    z = torch.rand((B, H, D), generator=gen, dtype=torch.float32) * 50.0
    return S, z


def run_gpu(q, k, v, g, grid, L, S_in=None, z_in=None):
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, g))
    B, N, H, D = q.shape
    rope = gla.gla_rope_create(*grid, D) if grid is not None else None
    S_out = torch.empty((B, H, D, D), dtype=torch.float32, device=DEV)
    z_out = torch.empty((B, H, D), dtype=torch.float32, device=DEV)
    out = gla.gla_forward_blocks(qd, kd, vd, gd, rope, L,
                                 S_in.to(DEV) if S_in is not None else None,
                                 z_in.to(DEV) if z_in is not None else None, S_out, z_out)
    torch.cuda.synchronize()
    if rope is not None:
        rope.close()
    return out.double().cpu().numpy(), S_out.double().cpu().numpy(), z_out.double().cpu().numpy()


SMALL = [
    # B, H, D, grid
    (1, 2, 32, (4, 8, 8)),
    (2, 3, 64, (3, 5, 7)),
    (1, 2, 128, (2, 3, 43)),
    (2, 1, 128, (7, 11, 13)),
]


@pytest.mark.parametrize("B,H,D,grid", SMALL)
@pytest.mark.parametrize("L", [1, 7, 16, 37, 128, 10**6])
@pytest.mark.parametrize("state", [False, True])
def test_blocks_small_shapes(B, H, D, grid, L, state):
    N = grid[0] * grid[1] * grid[2]
    say(f"case blocks B={B} H={H} D={D} grid={grid} L={L} state={state}")
    q, k, v, g = random_inputs(B, N, H, D, seed=2000 + N + D + L)
    S_in, z_in = carried(B, H, D, seed=N + L) if state else (None, None)
    got, S_got, z_got = run_gpu(q, k, v, g, grid, L, S_in, z_in)
    ref, S_ref, z_ref = oracle.forward_blocks(
        q, k, v, g, oracle.Grid(*grid), L,
        S_in.double().numpy() if state else None, z_in.double().numpy() if state else None)
    assert_close(got, ref, "out")
    rs, rz = rel(S_got, S_ref), rel(z_got, z_ref)
    say(f"  state: S rel_l2={rs:.3e} z rel_l2={rz:.3e}")
    assert rs <= 3e-3 and rz <= 1e-6


def test_single_block_equals_bidirectional_bitwise():
    w = BY_NAME["5b_480p_81f"]
    say("case blocks single block == gla_forward")
    q, k, v, g = (t.to(DEV) for t in make_inputs(w))
    rope = gla.gla_rope_create(w.T, w.Hh, w.W, w.D)
    o1 = gla.gla_forward(q, k, v, g, rope)
    o2 = gla.gla_forward_blocks(q, k, v, g, rope, w.N)
    o3 = gla.gla_forward_blocks(q, k, v, g, rope, 10 * w.N)
    torch.cuda.synchronize()
    rope.close()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(o1.view(torch.int16), o3.view(torch.int16))


def test_two_calls_handing_over_the_state():
    """Frames 0-5 in one call, frames 6-10 in the next with the returned state
    and the RoPE frame offset: the same output and final state as one call."""
    w = BY_NAME["5b_480p_81f"]
    say("case blocks two calls")
    HW = w.Hh * w.W
    L = 2 * HW
    q, k, v, g = (t.to(DEV) for t in make_inputs(w))
    B, N, H, D = q.shape
    rope = gla.gla_rope_create(w.T, w.Hh, w.W, D)
    S_all = torch.empty((B, H, D, D), dtype=torch.float32, device=DEV)
    z_all = torch.empty((B, H, D), dtype=torch.float32, device=DEV)
    o_all = gla.gla_forward_blocks(q, k, v, g, rope, L, None, None, S_all, z_all)
    n1 = 6 * HW
    r1 = gla.gla_rope_create(6, w.Hh, w.W, D)
    r2 = gla.gla_rope_create(w.T - 6, w.Hh, w.W, D, 1e4, 6, 0, 0)
    cut = lambda t, a, b: t[:, a:b].contiguous()
    S = torch.empty_like(S_all)
    z = torch.empty_like(z_all)
    o1 = gla.gla_forward_blocks(*(cut(t, 0, n1) for t in (q, k, v, g)), r1, L, None, None, S, z)
    # the second call updates the state in place
    o2 = gla.gla_forward_blocks(*(cut(t, n1, N) for t in (q, k, v, g)), r2, L, S, z, S, z)
    torch.cuda.synchronize()
    for r in (rope, r1, r2):
        r.close()
    o_split = torch.cat([o1, o2], dim=1).double().cpu().numpy()
    r_out = rel(o_split, o_all.double().cpu().numpy())
    r_S = rel(S.double().cpu().numpy(), S_all.double().cpu().numpy())
    r_z = rel(z.double().cpu().numpy(), z_all.double().cpu().numpy())
    say(f"  split vs one call: out {r_out:.3e} S {r_S:.3e} z {r_z:.3e}")
    # the two runs chunk the sums differently (fp32 order), nothing more
    assert r_out <= 2e-3 and r_S <= 1e-5 and r_z <= 1e-6


def test_workload_720p_in_five_frame_blocks():
    """The 5B 720p layer in 5-frame blocks: every output of every head and
    every returned state against oracle.forward_blocks (a few heads at a time)."""
    w = BY_NAME["5b_720p_193f"]
    L = 5 * w.Hh * w.W
    say(f"case blocks {w.name} L={L}")
    q, k, v, g = make_inputs(w)
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, g))
    rope = gla.gla_rope_create(w.T, w.Hh, w.W, w.D)
    S_out = torch.empty((w.B, w.H, w.D, w.D), dtype=torch.float32, device=DEV)
    z_out = torch.empty((w.B, w.H, w.D), dtype=torch.float32, device=DEV)
    out = gla.gla_forward_blocks(qd, kd, vd, gd, rope, L, None, None, S_out, z_out).cpu()
    torch.cuda.synchronize()
    rope.close()
    del qd, kd, vd, gd
    S_gpu, z_gpu = S_out.double().cpu().numpy(), z_out.double().cpu().numpy()
    grid = oracle.Grid(w.T, w.Hh, w.W)
    d2 = r2 = 0.0
    mx = 0.0
    sd2 = sr2 = zd2 = zr2 = 0.0
    group = max(4, oracle.num_threads())  # the oracle runs one head per thread
    for b in range(w.B):
        for h0 in range(0, w.H, group):
            h1 = min(h0 + group, w.H)
            sl = lambda t: t[b:b + 1, :, h0:h1].contiguous()
            ref, S_ref, z_ref = oracle.forward_blocks(sl(q), sl(k), sl(v), sl(g), grid, L)
            got = out[b:b + 1, :, h0:h1].double().numpy()
            d2 += float(np.sum((got - ref) ** 2))
            r2 += float(np.sum(ref ** 2))
            mx = max(mx, float(np.max(np.abs(got - ref))))
            sd2 += float(np.sum((S_gpu[b, h0:h1] - S_ref[0]) ** 2))
            sr2 += float(np.sum(S_ref[0] ** 2))
            zd2 += float(np.sum((z_gpu[b, h0:h1] - z_ref[0]) ** 2))
            zr2 += float(np.sum(z_ref[0] ** 2))
    r_out, r_S, r_z = (d2 / r2) ** 0.5, (sd2 / sr2) ** 0.5, (zd2 / zr2) ** 0.5
    say(f"  all outputs: rel_l2={r_out:.3e} max_abs={mx:.3e}; final S rel_l2={r_S:.3e} "
        f"z rel_l2={r_z:.3e}")
    assert r_out <= REL_TOL and mx <= ABS_TOL
    assert r_S <= 3e-3 and r_z <= 1e-6


# Shapes sized so that the output half runs on the persistent kernel, one
# block per (attention block, G heads) walking only its attention block's
# tokens: the launch takes it for several attention blocks when those groups
# fill at least 7/8 of its rounds of 256 blocks (one round, or several with
# G > 1), and, for G > 1, each wave runs at least 16 steps.  B, H, grid, block tokens, RoPE, carried state, G:
PERSISTENT_BLOCKS = [
    (1, 3, (5, 20, 50), 1350, True, True),      # G = 1: 4 blocks x 3 heads x 21 ranges
    (1, 3, (5, 20, 50), 1350, False, False),    # G = 1 without RoPE
    (1, 2, (50, 50, 50), 62000, True, False),   # G = 2: a 1,000-token last block
    (1, 4, (40, 30, 52), 31000, True, True),    # G = 4 (fp16 table pairs, q tiles)
    (1, 4, (45, 40, 64), 257, True, False),     # G = 4, 449 groups in two rounds of blocks
]


@pytest.mark.parametrize("B,H,grid,L,rope,state", PERSISTENT_BLOCKS)
def test_blocks_on_the_persistent_output_kernel(B, H, grid, L, rope, state):
    """Every output and the returned state against oracle.forward_blocks."""
    D = 128
    N = grid[0] * grid[1] * grid[2]
    say(f"case blocks persistent B={B} H={H} grid={grid} L={L} rope={rope} state={state}")
    q, k, v, g = random_inputs(B, N, H, D, seed=3000 + H + L)
    S_in, z_in = carried(B, H, D, seed=L) if state else (None, None)
    got, S_got, z_got = run_gpu(q, k, v, g, grid if rope else None, L, S_in, z_in)
    ref, S_ref, z_ref = oracle.forward_blocks(
        q, k, v, g, oracle.Grid(*grid) if rope else None, L,
        S_in.double().numpy() if state else None, z_in.double().numpy() if state else None)
    assert_close(got, ref, "out")
    rs, rz = rel(S_got, S_ref), rel(z_got, z_ref)
    say(f"  state: S rel_l2={rs:.3e} z rel_l2={rz:.3e}")
    assert rs <= 3e-3 and rz <= 1e-6


def test_empty_sequence_returns_the_carried_state():
    say("case blocks empty")
    B, H, D = 2, 3, 64
    S_in, z_in = (t.to(DEV) for t in carried(B, H, D, seed=5))
    q = torch.empty((B, 0, H, D), dtype=torch.bfloat16, device=DEV)
    S_out = torch.full((B, H, D, D), 7.0, device=DEV)
    z_out = torch.full((B, H, D), 7.0, device=DEV)
    gla.gla_forward_blocks(q, q, q, q, None, 16, S_in, z_in, S_out, z_out)
    torch.cuda.synchronize()
    assert torch.equal(S_out, S_in) and torch.equal(z_out, z_in)
    gla.gla_forward_blocks(q, q, q, q, None, 16, None, None, S_out, z_out)
    torch.cuda.synchronize()
    assert torch.all(S_out == 0) and torch.all(z_out == 0)


def test_blocks_deterministic_and_in_place():
    w = BY_NAME["5b_480p_81f"]
    say("case blocks determinism / in place")
    q, k, v, g = (t.to(DEV) for t in make_inputs(w))
    B, N, H, D = q.shape
    S_in, z_in = (t.to(DEV) for t in carried(B, H, D, seed=9))
    rope = gla.gla_rope_create(w.T, w.Hh, w.W, D)
    L = 3 * w.Hh * w.W
    S1 = torch.empty_like(S_in)
    z1 = torch.empty_like(z_in)
    o1 = gla.gla_forward_blocks(q, k, v, g, rope, L, S_in, z_in, S1, z1)
    o2 = gla.gla_forward_blocks(q, k, v, g, rope, L, S_in, z_in)
    S2, z2 = S_in.clone(), z_in.clone()
    o3 = gla.gla_forward_blocks(q, k, v, g, rope, L, S2, z2, S2, z2)
    torch.cuda.synchronize()
    rope.close()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(o1.view(torch.int16), o3.view(torch.int16))
    assert torch.equal(S1, S2) and torch.equal(z1, z2)

"""GPU parity of the projection prologue fused with the mixer
(gla_forward_proj, through the C ABI) against the oracle: the projections
x W^T in fp64, rounded to bf16, then the fp64 mixer.

Bar: relative L2 error <= 5e-3 and max absolute error <= 3e-2 of the bf16
output.  The GPU accumulates the projections in fp32 before rounding them to
bf16 (a value next to a rounding boundary can land one bf16 step away from
the oracle's), then rounds as the mixer does.  Every shape is compared on
every output; at the layer shapes the oracle's projections of all heads come
from oracle.project_maps (numpy's fp64 product, chunked over tokens).
"""
import numpy as np
import pytest
import torch

import gated_linear_attention_forward_amd as gla
import oracle
from workloads import BY_NAME, PROJ_WORKLOADS, make_projection, random_projection

pytestmark = pytest.mark.gpu

REL_TOL = 5e-3
ABS_TOL = 3e-2
DEV = torch.device("cuda:0")


def say(msg):
    print(msg, flush=True)


def assert_close(got, ref, what):
    got = np.asarray(got, np.float64)
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    mx = float(np.max(np.abs(got - ref)))
    say(f"  {what}: rel_l2={rel:.3e} max_abs={mx:.3e} max|ref|={np.max(np.abs(ref)):.3e}")
    assert rel <= REL_TOL and mx <= ABS_TOL


SMALL = [
    # B, H, D, grid, C
    (1, 2, 32, (4, 8, 8), 128),
    (1, 1, 32, (1, 1, 1), 64),        # one token
    (2, 3, 64, (3, 5, 7), 192),       # ragged tile, D = 64
    (1, 2, 128, (2, 3, 43), 256),     # 258 tokens: two full tiles and a 2-token tail
    (2, 2, 128, (7, 11, 13), 128),    # 1001 tokens, B = 2
    (1, 1, 128, (1, 1, 129), 640),    # one past a tile, C = 640
]


@pytest.mark.parametrize("B,H,D,grid,C", SMALL)
@pytest.mark.parametrize("rope", [True, False])
def test_proj_small_shapes(B, H, D, grid, C, rope):
    N = grid[0] * grid[1] * grid[2]
    say(f"case proj B={B} N={N} H={H} D={D} C={C} rope={rope}")
    x, w = random_projection(B, N, C, H, D, seed=1000 + N + C + D)
    xd, wd = x.to(DEV), w.to(DEV)
    r = gla.gla_rope_create(*grid, D) if rope else None
    out = gla.gla_forward_proj(xd, wd, H, D, r)
    torch.cuda.synchronize()
    if r is not None:
        r.close()
    ref = oracle.projected_forward(x, w, H, D, oracle.Grid(*grid) if rope else None)
    assert_close(out.double().cpu().numpy(), ref, "out")


@pytest.mark.parametrize("name", [w.name for w in PROJ_WORKLOADS])
def test_proj_workload(name):
    """The layer shapes: every output of every head against the oracle's
    projections (oracle.project_maps, rounded to bf16) followed by the mixer
    oracle, a few heads at a time."""
    w = BY_NAME[name]
    say(f"case proj workload {w.name} B={w.B} N={w.N} C={w.C} H={w.H} D={w.D}")
    x, wt = make_projection(w)
    rope = gla.gla_rope_create(w.T, w.Hh, w.W, w.D, w.theta)
    out = gla.gla_forward_proj(x.to(DEV), wt.to(DEV), w.H, w.D, rope)
    torch.cuda.synchronize()
    rope.close()
    out = out.cpu()
    grid = oracle.Grid(w.T, w.Hh, w.W, w.theta)
    q, k, v, g = oracle.project_maps(x, wt, w.H, w.D)
    d2 = r2 = mx = 0.0
    group = max(4, oracle.num_threads())  # the oracle runs one head per thread
    for b in range(w.B):
        for h0 in range(0, w.H, group):
            h1 = min(h0 + group, w.H)
            sl = lambda t: np.ascontiguousarray(t[b:b + 1, :, h0:h1])
            ref = oracle.forward(sl(q), sl(k), sl(v), sl(g), grid)
            got = out[b:b + 1, :, h0:h1].double().numpy()
            d2 += float(np.sum((got - ref) ** 2))
            r2 += float(np.sum(ref ** 2))
            mx = max(mx, float(np.max(np.abs(got - ref))))
    rel = (d2 / r2) ** 0.5
    say(f"  {w.name} all outputs: rel_l2={rel:.3e} max_abs={mx:.3e}")
    assert rel <= REL_TOL and mx <= ABS_TOL


def test_proj_deterministic_and_workspace_entry_point():
    w = BY_NAME["proj_5b_480p_81f"]
    say("case proj determinism")
    x, wt = (t.to(DEV) for t in make_projection(w))
    rope = gla.gla_rope_create(w.T, w.Hh, w.W, w.D, w.theta)
    o1 = gla.gla_forward_proj(x, wt, w.H, w.D, rope)
    ws = gla.alloc_workspace_proj(w.B, w.N, w.C, w.H, w.D, DEV)
    o2 = gla.gla_forward_proj_ws(x, wt, w.H, w.D, rope, ws)
    o3 = gla.gla_forward_proj_ws(x, wt, w.H, w.D, rope, ws)
    torch.cuda.synchronize()
    rope.close()
    assert torch.equal(o1, o2) and torch.equal(o2, o3)


def test_proj_matches_mixer_on_its_own_projections():
    """Selection weights (C = 4 H D) make the projections exact copies of
    blocks of x: the fused path must then agree with gla_forward on those
    blocks up to the fp32 order of the state sums (the fused kernel adds a
    chunk's tokens in another order, which can move a bf16 rounding of S or
    of the output by one step)."""
    B, N, H, D = 1, 300, 2, 64
    say("case proj selection weights")
    q, k, v, g = (torch.randn(B, N, H, D, generator=torch.Generator().manual_seed(i))
                  .to(torch.bfloat16) for i in range(4))
    x = torch.cat([t.reshape(B, N, H * D) for t in (q, k, v, g)], dim=-1).contiguous()
    C = 4 * H * D
    wt = torch.zeros((4, H * D, C), dtype=torch.bfloat16)
    for m in range(4):
        wt[m, :, m * H * D:(m + 1) * H * D] = torch.eye(H * D, dtype=torch.bfloat16)
    rope = gla.gla_rope_create(3, 10, 10, D)
    fused = gla.gla_forward_proj(x.to(DEV), wt.to(DEV), H, D, rope)
    plain = gla.gla_forward(*(t.to(DEV) for t in (q, k, v, g)), rope)
    torch.cuda.synchronize()
    rope.close()
    f, pl = fused.double().cpu().numpy(), plain.double().cpu().numpy()
    rel = float(np.linalg.norm(f - pl) / np.linalg.norm(pl))
    say(f"  fused vs gla_forward: rel_l2={rel:.3e}")
    assert rel <= 2e-3


def test_proj_empty_and_errors():
    say("case proj empty / errors")
    x = torch.empty((1, 0, 64), dtype=torch.bfloat16, device=DEV)
    wt = torch.zeros((4, 64, 64), dtype=torch.bfloat16, device=DEV)
    assert gla.gla_forward_proj(x, wt, 2, 32).shape == (1, 0, 2, 32)
    x2 = torch.zeros((1, 8, 100), dtype=torch.bfloat16, device=DEV)
    w2 = torch.zeros((4, 64, 100), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(gla.GlaError):
        gla.gla_forward_proj(x2, w2, 2, 32)          # C = 100 is not a multiple of 64

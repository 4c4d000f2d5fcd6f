"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Bar (from the fixed form of the mixer): relative L2 error <= 5e-3 and max
absolute error <= 3e-2 of the bf16 output against the oracle's fp64 output
on the same bf16 inputs.  The GPU rounds R phi(k), R phi(q), S and the
output to bf16 (four roundings of ~1.7e-3 each), so ~2e-3 is expected.
Every shape, the five layer shapes included, is compared element by element
over every output: the layer shapes head group by head group (the oracle's
output for a few heads at a time), with the relative L2 and maximum
absolute errors taken over the whole tensor.
"""
import numpy as np
import pytest
import torch

import gated_linear_attention_forward_amd as gla
import oracle
from workloads import BY_NAME, WORKLOADS, make_inputs, random_inputs

pytestmark = pytest.mark.gpu

REL_TOL = 5e-3
ABS_TOL = 3e-2
DEV = torch.device("cuda:0")


def say(msg):
    print(msg, flush=True)


def to_dev(*ts):
    return tuple(t.to(DEV) for t in ts)


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


def gpu_forward(q, k, v, g, grid):
    """grid: (T, Hh, W) or None; returns the bf16 output as a CPU float64 array."""
    qd, kd, vd, gd = to_dev(q, k, v, g)
    rope = None
    if grid is not None:
        rope = gla.gla_rope_create(*grid, q.shape[-1])
    out = gla.gla_forward(qd, kd, vd, gd, rope)
    torch.cuda.synchronize()
    if rope is not None:
        rope.close()
    return out.double().cpu().numpy()


# ---------------------------------------------------------------------------
# small shapes: every output element


SMALL = [
    # B, H, D, grid (T, Hh, W)
    (1, 2, 32, (4, 8, 8)),      # the tiny workload
    (1, 1, 32, (1, 1, 1)),      # a single token
    (1, 3, 32, (1, 1, 7)),      # fewer tokens than one tile
    (2, 3, 64, (3, 5, 7)),      # D = 64, ragged
    (1, 2, 128, (2, 3, 43)),    # 258 tokens: four tiles and a 2-token tail
    (2, 2, 128, (7, 11, 13)),   # 1001 tokens, B = 2
    (1, 1, 128, (1, 1, 65)),    # one past a tile
    (3, 1, 32, (5, 7, 11)),     # 385 tokens, D = 32, B = 3
    (1, 4, 128, (2, 3, 43)),    # four heads, too short to group them (one per block)
    (1, 4, 128, (1, 1, 1)),     # four heads, a single token
    (1, 4, 128, (64, 32, 33)),  # 67,584 tokens: four heads to an output block, ragged
    (2, 8, 128, (16, 40, 103)), # 65,920 tokens, B = 2: two head groups per batch element
    (1, 4, 128, (200, 3, 110)), # four heads, a RoPE table too long for LDS beside the q tiles
                                # (16 or 17 steps per wave: one or two after the whole rounds)
    (1, 4, 128, (192, 16, 24)), # the same path with 18 steps per wave: whole rounds only
    (1, 6, 128, (45, 31, 32)),  # six heads: two to an output block
]


@pytest.mark.parametrize("B,H,D,grid", SMALL)
@pytest.mark.parametrize("rope", [True, False])
def test_forward_small_shapes(B, H, D, grid, rope):
    N = grid[0] * grid[1] * grid[2]
    say(f"case B={B} H={H} D={D} grid={grid} rope={rope}")
    q, k, v, g = random_inputs(B, N, H, D, seed=1000 + N + D + H + B)
    got = gpu_forward(q, k, v, g, grid if rope else None)
    ref = oracle.forward(q, k, v, g, oracle.Grid(*grid) if rope else None)
    assert_close(got, ref, "out")


def test_state_matches_oracle():
    w = BY_NAME["5b_480p_81f"]
    say(f"case state {w.name}")
    q, k, v, g = make_inputs(w)
    rope = gla.gla_rope_create(w.T, w.Hh, w.W, w.D)
    kd, vd = to_dev(k, v)
    S, z = gla.gla_state(kd, vd, rope)
    torch.cuda.synchronize()
    rope.close()
    heads = [0, 7, 19]
    Sr, zr = oracle.state(k[:, :, heads].contiguous(), v[:, :, heads].contiguous(),
                          oracle.Grid(w.T, w.Hh, w.W))
    Sg = S[:, heads].double().cpu().numpy()
    zg = z[:, heads].double().cpu().numpy()
    # S uses R phi(k) rounded to bf16; z sums exact features in fp32
    rel_s = float(np.linalg.norm(Sg - Sr) / np.linalg.norm(Sr))
    rel_z = float(np.linalg.norm(zg - zr) / np.linalg.norm(zr))
    say(f"  S rel_l2={rel_s:.3e}  z rel_l2={rel_z:.3e}")
    assert rel_s <= 3e-3
    assert rel_z <= 1e-6


# ---------------------------------------------------------------------------
# the five layer workloads


class ErrAccum:
    """Relative L2 and maximum absolute error over a tensor compared piece by
    piece: sums of squared differences and of squared references."""

    def __init__(self):
        self.d2 = 0.0
        self.r2 = 0.0
        self.mx = 0.0
        self.rmax = 0.0
        self.n = 0

    def add(self, got, ref):
        got = np.asarray(got, np.float64)
        diff = got - ref
        self.d2 += float(np.sum(diff * diff))
        self.r2 += float(np.sum(ref * ref))
        if diff.size:
            self.mx = max(self.mx, float(np.max(np.abs(diff))))
            self.rmax = max(self.rmax, float(np.max(np.abs(ref))))
        self.n += diff.size

    def check(self, what):
        rel = (self.d2 / max(self.r2, 1e-300)) ** 0.5
        say(f"  {what}: {self.n} outputs rel_l2={rel:.3e} max_abs={self.mx:.3e} "
            f"max|ref|={self.rmax:.3e}")
        assert rel <= REL_TOL, f"{what}: rel_l2 {rel}"
        assert self.mx <= ABS_TOL, f"{what}: max_abs {self.mx}"


def head_groups(H, size):
    return [(h0, min(h0 + size, H)) for h0 in range(0, H, size)]


def check_all_heads(w, out, q, k, v, g, what, group=None):
    """Every output of every (b, h) against oracle.forward, a few heads at a
    time (the oracle's fp64 output of a whole layer would not fit in memory
    at once at the 60 s shape), as many heads as the oracle has threads."""
    grid = oracle.Grid(w.T, w.Hh, w.W, w.theta)
    group = group or max(4, oracle.num_threads())  # the oracle runs one head per thread
    acc = ErrAccum()
    out = out.cpu()
    for b in range(w.B):
        for h0, h1 in head_groups(w.H, group):
            sl = (slice(b, b + 1), slice(None), slice(h0, h1))
            ref = oracle.forward(*(t[sl].contiguous() for t in (q, k, v, g)), grid)
            acc.add(out[sl].double().numpy(), ref)
    acc.check(what)


@pytest.mark.parametrize("name", [w.name for w in WORKLOADS])
def test_workload(name):
    """Full-size layer shapes through the split entry points bench.py times
    (gla_state_ws then gla_output_ws on one caller workspace), every output
    compared."""
    w = BY_NAME[name]
    say(f"case workload {name} B={w.B} N={w.N} H={w.H} D={w.D}")
    q, k, v, g = make_inputs(w)
    qd, kd, vd, gd = to_dev(q, k, v, g)
    rope = gla.gla_rope_create(w.T, w.Hh, w.W, w.D, w.theta)
    ws = gla.alloc_workspace(w.B, w.N, w.H, w.D, DEV)
    out = torch.empty_like(qd)
    gla.gla_state_ws(kd, vd, rope, ws)
    gla.gla_output_ws(qd, gd, rope, out, ws)
    torch.cuda.synchronize()
    rope.close()
    assert torch.isfinite(out.float()).all()
    del qd, kd, vd, gd
    check_all_heads(w, out, q, k, v, g, f"{name} all outputs")


# ---------------------------------------------------------------------------
# special cases, determinism, entry-point equivalence


def test_nonpositive_q_rows_are_zero_and_negative_k_gives_zero():
    B, H, D, grid = 1, 2, 128, (2, 5, 13)
    N = 130
    say("case special q<=0 / k<=0")
    q, k, v, g = random_inputs(B, N, H, D, seed=77)
    q = q.clone()
    q[0, ::3] = -q[0, ::3].abs()
    got = gpu_forward(q, k, v, g, grid)
    assert np.all(got[0, ::3] == 0.0)
    ref = oracle.forward(q, k, v, g, oracle.Grid(*grid))
    assert_close(got, ref, "out")
    got2 = gpu_forward(q, -k.abs(), v, g, grid)
    assert np.all(got2 == 0.0)


@pytest.mark.parametrize("rope", [True, False])
def test_saturated_gates(rope):
    """Gate logits at the saturated ends, exact in bf16 (+-30, +-88, +-100;
    exp(88) is near the fp32 limit and exp(100) overflows it): against the
    oracle, and without RoPE and with constant v against the closed form
    o = sigmoid(g) c (phi(q).z) / (phi(q).z + eps), where sigmoid(30) = 1 -
    9.4e-14 and sigmoid(-30) = 9.4e-14 in fp64."""
    B, N, H, D, grid = 1, 330, 2, 128, (3, 5, 22)
    say(f"case saturated gates rope={rope}")
    q, k, v, g = random_inputs(B, N, H, D, seed=81)
    levels = torch.tensor([30.0, -30.0, 88.0, -88.0, 100.0, -100.0])
    gen = torch.Generator().manual_seed(82)
    g = levels[torch.randint(0, 6, (B, N, H, D), generator=gen)].to(torch.bfloat16)
    assert torch.equal(g.float().abs().unique(), torch.tensor([30.0, 88.0, 100.0]))
    got = gpu_forward(q, k, v, g, grid if rope else None)
    assert np.isfinite(got).all()
    ref = oracle.forward(q, k, v, g, oracle.Grid(*grid) if rope else None)
    assert_close(got, ref, "out")
    neg = g.double().numpy() < 0
    # the negative gates leave at most sigmoid(-30) of the ungated output
    assert np.max(np.abs(got[neg])) <= 1e-10
    if not rope:
        c = torch.linspace(-2, 2, D).to(torch.bfloat16)
        vc = c.expand(B, N, H, D).contiguous()
        got_c = gpu_forward(q, k, vc, g, None)
        fq = np.maximum(q.double().numpy(), 0)
        z = np.maximum(k.double().numpy(), 0).sum(axis=1)  # [B, H, D]
        dot = np.einsum("bnhd,bhd->bnh", fq, z)[..., None]
        sig = 1.0 / (1.0 + np.exp(-g.double().numpy()))
        closed = sig * c.double().numpy() * dot / (dot + oracle.EPS)
        err = float(np.max(np.abs(got_c - closed)))
        say(f"  constant v closed form: max_abs={err:.3e}")
        # bf16 S (one rounding) and bf16 output: within 2^-7 of |c| <= 2
        assert err <= 2.0 * 2.0 ** -7


@pytest.mark.parametrize("rope", [True, False])
def test_single_token_with_q_equal_k(rope):
    """N = 1 and q = k: o = sigmoid(g) v |phi(q)|^2 / (|phi(q)|^2 + eps)
    (a single grid position has angle zero, so RoPE is the identity)."""
    B, H, D = 2, 3, 128
    say(f"case single token q=k rope={rope}")
    q, _, v, g = random_inputs(B, 1, H, D, seed=83)
    got = gpu_forward(q, q.clone(), v, g, (1, 1, 1) if rope else None)
    fq = np.maximum(q.double().numpy(), 0)
    nq = (fq * fq).sum(-1, keepdims=True)
    closed = v.double().numpy() / (1.0 + np.exp(-g.double().numpy())) * nq / (nq + oracle.EPS)
    rel = float(np.linalg.norm(got - closed) / np.linalg.norm(closed))
    mx = float(np.max(np.abs(got - closed)))
    say(f"  closed form: rel_l2={rel:.3e} max_abs={mx:.3e}")
    assert rel <= REL_TOL and mx <= ABS_TOL
    ref = oracle.forward(q, q.clone(), v, g, oracle.Grid(1, 1, 1) if rope else None)
    assert_close(got, ref, "out")


def test_constant_v_closed_form_without_rope():
    """v rows all equal c, no RoPE: o = sigma(g) c (phi(q).z)/(phi(q).z + eps)."""
    B, N, H, D = 1, 300, 2, 64
    say("case constant v")
    q, k, _, g = random_inputs(B, N, H, D, seed=78)
    c = torch.linspace(-2, 2, D).to(torch.bfloat16)
    v = c.expand(B, N, H, D).contiguous()
    got = gpu_forward(q, k, v, g, None)
    ref = oracle.forward(q, k, v, g, None)
    assert_close(got, ref, "out")


def test_bitwise_deterministic_and_entry_points_agree():
    w = BY_NAME["5b_480p_81f"]
    say("case determinism")
    q, k, v, g = to_dev(*make_inputs(w))
    rope = gla.gla_rope_create(w.T, w.Hh, w.W, w.D)
    o1 = gla.gla_forward(q, k, v, g, rope)
    o2 = gla.gla_forward(q, k, v, g, rope)
    ws = gla.alloc_workspace(w.B, w.N, w.H, w.D, DEV)
    o3 = torch.empty_like(q)
    gla.gla_forward_ws(q, k, v, g, rope, o3, ws)
    o4 = torch.empty_like(q)
    gla.gla_state_ws(k, v, rope, ws)
    gla.gla_output_ws(q, g, rope, o4, ws)
    torch.cuda.synchronize()
    rope.close()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(o1.view(torch.int16), o3.view(torch.int16))
    assert torch.equal(o1.view(torch.int16), o4.view(torch.int16))


def test_workspace_release_then_calls_allocate_again():
    """gla_workspace_release frees the cached workspaces (after a device
    synchronisation); calls before and after it give the same bits, twice in a
    row, and a release with nothing cached is a no-op."""
    w = BY_NAME["5b_480p_81f"]
    say("case workspace release")
    q, k, v, g = to_dev(*make_inputs(w))
    dout = torch.randn_like(q)
    rope = gla.gla_rope_create(w.T, w.Hh, w.W, w.D)
    o1 = gla.gla_forward(q, k, v, g, rope)
    d1 = gla.gla_backward(q, k, v, g, dout, rope)
    gla.gla_workspace_release()
    gla.gla_workspace_release()
    o2 = gla.gla_forward(q, k, v, g, rope)
    d2 = gla.gla_backward(q, k, v, g, dout, rope)
    gla.gla_workspace_release()
    torch.cuda.synchronize()
    rope.close()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    for a, b in zip(d1, d2):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("B,H,D,grid", [(1, 2, 32, (10, 12, 16)), (3, 1, 32, (9, 11, 12)),
                                        (1, 1, 32, (1, 1, 1100))])
@pytest.mark.parametrize("rope", [True, False])
def test_folded_reduction_matches_the_reduce_kernel(B, H, D, grid, rope):
    """D = 32 sequences of 1,100 to 1,920 tokens run the whole pass as two
    launches, the output kernel summing the 9 to 15 chunk partials itself;
    the two halves called separately run the reduce kernel in between.  Both
    sum in the same pairwise order, so the outputs are bitwise equal."""
    T, Hh, W = grid
    N = T * Hh * W
    say(f"case folded reduction B={B} H={H} D={D} grid={grid} rope={rope}")
    q, k, v, g = to_dev(*random_inputs(B, N, H, D, seed=91))
    r = gla.gla_rope_create(T, Hh, W, D) if rope else None
    ws = gla.alloc_workspace(B, N, H, D, DEV)
    o1 = torch.empty_like(q)
    gla.gla_forward_ws(q, k, v, g, r, o1, ws)
    o2 = torch.empty_like(q)
    gla.gla_state_ws(k, v, r, ws)
    gla.gla_output_ws(q, g, r, o2, ws)
    torch.cuda.synchronize()
    if r is not None:
        r.close()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


@pytest.mark.parametrize("B,H,D,grid", [(1, 2, 32, (4, 8, 8)), (3, 1, 32, (5, 7, 11)),
                                        (2, 3, 64, (3, 5, 7)), (1, 4, 64, (2, 16, 16)),
                                        (2, 2, 32, (4, 16, 16))])
@pytest.mark.parametrize("rope", [True, False])
def test_one_launch_pass_against_the_oracle_and_the_split_halves(B, H, D, grid, rope):
    """Short D <= 64 sequences (N D <= 32,768) run the whole pass in one
    launch, one block per head forming the state from all N tokens; its
    output meets the oracle's bar, and agrees with the separately called
    halves (state, reduce and output kernels) to bf16 rounding."""
    T, Hh, W = grid
    N = T * Hh * W
    say(f"case one-launch pass B={B} H={H} D={D} grid={grid} rope={rope}")
    q, k, v, g = random_inputs(B, N, H, D, seed=93)
    qd, kd, vd, gd = to_dev(q, k, v, g)
    r = gla.gla_rope_create(T, Hh, W, D) if rope else None
    ws = gla.alloc_workspace(B, N, H, D, DEV)
    o1 = torch.empty_like(qd)
    gla.gla_forward_ws(qd, kd, vd, gd, r, o1, ws)
    o2 = torch.empty_like(qd)
    gla.gla_state_ws(kd, vd, r, ws)
    gla.gla_output_ws(qd, gd, r, o2, ws)
    torch.cuda.synchronize()
    if r is not None:
        r.close()
    ref = oracle.forward(q, k, v, g, oracle.Grid(T, Hh, W) if rope else None)
    rel, mx = errs(o1.double().cpu().numpy(), ref)
    say(f"  vs oracle rel={rel:.3e} max_abs={mx:.3e}")
    assert rel <= REL_TOL and mx <= ABS_TOL
    rel2, mx2 = errs(o1.double().cpu().numpy(), o2.double().cpu().numpy())
    say(f"  vs split halves rel={rel2:.3e} max_abs={mx2:.3e}")
    assert rel2 <= REL_TOL and mx2 <= ABS_TOL


def test_relative_position_shift():
    """Tables built with shifted grid indices give the same output (RoPE is relative)."""
    B, H, D, grid = 1, 2, 128, (3, 6, 9)
    N = 162
    say("case rope shift")
    q, k, v, g = to_dev(*random_inputs(B, N, H, D, seed=79))
    r0 = gla.gla_rope_create(*grid, D)
    r1 = gla.gla_rope_create(*grid, D, 1e4, 11, -4, 23)
    o0 = gla.gla_forward(q, k, v, g, r0).double().cpu().numpy()
    o1 = gla.gla_forward(q, k, v, g, r1).double().cpu().numpy()
    r0.close()
    r1.close()
    rel, _ = errs(o1, o0)
    say(f"  shift rel={rel:.3e}")
    assert rel <= REL_TOL


def test_empty_inputs_are_noops():
    say("case empty")
    for shape in ((1, 0, 2, 128), (0, 10, 2, 128), (1, 10, 0, 64)):
        q = torch.empty(shape, dtype=torch.bfloat16, device=DEV)
        out = gla.gla_forward(q, q.clone(), q.clone(), q.clone(), None)
        assert out.shape == q.shape
    # no tokens: the state is exactly zero (written by a kernel, every element)
    for D in (32, 64, 128):
        k = torch.empty((2, 0, 3, D), dtype=torch.bfloat16, device=DEV)
        # freed NaN blocks of the same sizes, which torch's caching allocator
        # hands out again for S and z
        junk = (torch.full((2, 3, D, D), float("nan"), device=DEV),
                torch.full((2, 3, D), float("nan"), device=DEV))
        torch.cuda.synchronize()
        del junk
        S, z = gla.gla_state(k, k.clone())
        torch.cuda.synchronize()
        assert S.shape == (2, 3, D, D) and z.shape == (2, 3, D)
        assert torch.all(S == 0) and torch.all(z == 0)


def test_bad_calls_raise():
    say("case errors")
    q = torch.zeros((1, 64, 2, 128), dtype=torch.bfloat16, device=DEV)
    rope = gla.gla_rope_create(4, 4, 5, 128)
    with pytest.raises(gla.GlaError):
        gla.gla_forward(q, q.clone(), q.clone(), q.clone(), rope)  # 80-token grid for N = 64
    rope.close()
    small = torch.zeros(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(gla.GlaError):
        gla.gla_forward_ws(q, q.clone(), q.clone(), q.clone(), None, torch.empty_like(q), small)
    with pytest.raises(gla.GlaError):
        gla.gla_forward(q, q, q, q, None, out=q)  # out aliases the inputs

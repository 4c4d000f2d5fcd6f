"""GPU: gla_forward_noalloc (the entry point that allocates nothing, on the
library's fixed per-GPU scratch) against gla_forward_ws (caller workspace) on
two calls in a row, the second with a smaller input, through the C ABI.  The
two run the same kernels on the same plan, so the outputs must be bitwise
equal; the first case is also checked against the fp64 oracle."""
import numpy as np
import pytest
import torch

import gated_linear_attention_forward_amd as gla
import oracle
from workloads import BY_NAME, make_inputs, random_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def say(msg):
    print(msg, flush=True)


def run_both(q, k, v, g, rope):
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, g))
    B, N, H, D = q.shape
    ws = gla.alloc_workspace(B, N, H, D, DEV)
    ref = gla.gla_forward_ws(qd, kd, vd, gd, rope, torch.empty_like(qd), ws)
    got = gla.gla_forward_noalloc(qd, kd, vd, gd, rope)
    torch.cuda.synchronize()
    return got, ref


@pytest.mark.parametrize("use_rope", [True, False])
def test_noalloc_matches_workspace_entry_on_two_calls(use_rope):
    # first call: the 5B 480p layer; second call: a smaller ragged shape
    w = BY_NAME["5b_480p_81f"]
    say(f"case noalloc first {w.name} rope={use_rope}")
    q, k, v, g = make_inputs(w)
    rope = gla.gla_rope_create(w.T, w.Hh, w.W, w.D, w.theta) if use_rope else None
    got, ref = run_both(q, k, v, g, rope)
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    heads = [(0, 0), (0, w.H - 1)]
    grid = oracle.Grid(w.T, w.Hh, w.W, w.theta) if use_rope else None
    for b, h in heads:
        sl = (slice(b, b + 1), slice(None), slice(h, h + 1))
        o = oracle.forward(*(t[sl].contiguous() for t in (q, k, v, g)), grid)
        o_gpu = got[sl].double().cpu().numpy()
        rel = float(np.linalg.norm(o_gpu - o) / np.linalg.norm(o))
        say(f"  head ({b},{h}) rel_l2={rel:.3e}")
        assert rel <= 5e-3 and float(np.max(np.abs(o_gpu - o))) <= 3e-2
    if rope is not None:
        rope.close()

    grid2 = (3, 7, 11)
    N2 = grid2[0] * grid2[1] * grid2[2]
    say(f"case noalloc second B=1 N={N2} H=3 D=128 rope={use_rope}")
    q2, k2, v2, g2 = random_inputs(1, N2, 3, 128, seed=4242)
    rope2 = gla.gla_rope_create(*grid2, 128) if use_rope else None
    got2, ref2 = run_both(q2, k2, v2, g2, rope2)
    assert torch.equal(got2.view(torch.int16), ref2.view(torch.int16))
    o2 = oracle.forward(q2, k2, v2, g2, oracle.Grid(*grid2) if use_rope else None)
    rel2 = float(np.linalg.norm(got2.double().cpu().numpy() - o2) / np.linalg.norm(o2))
    say(f"  second rel_l2={rel2:.3e}")
    assert rel2 <= 5e-3
    if rope2 is not None:
        rope2.close()


def test_noalloc_d32_and_empty():
    say("case noalloc D=32 and empty")
    q, k, v, g = random_inputs(2, 300, 2, 32, seed=99)
    got, ref = run_both(q, k, v, g, None)
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    e = torch.empty((1, 0, 2, 128), dtype=torch.bfloat16, device=DEV)
    out = gla.gla_forward_noalloc(e, e.clone(), e.clone(), e.clone(), None)
    assert out.shape == e.shape

"""GPU: the forward pass captured into a HIP graph (torch.cuda.CUDAGraph on
ROCm) and replayed.

The library enqueues only kernel launches on the caller's stream (no
allocation once the workspace exists, no memset, no host synchronisation),
so a caller can capture a pass and replay it without the host launch cost.
Each replay must give the eager result bit for bit; replays are separated
by the program's own eager work and synchronisations, and every replay's
output is checked.
"""
import pytest
import torch

import gated_linear_attention_forward_amd as gla
from workloads import BY_NAME, make_inputs, random_inputs

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def say(msg):
    print(msg, flush=True)


def _inputs(case):
    if case in BY_NAME:
        w = BY_NAME[case]
        q, k, v, g = make_inputs(w)
        return [t.to(DEV) for t in (q, k, v, g)], (w.T, w.Hh, w.W)
    B, H, D, grid = case
    q, k, v, g = random_inputs(B, grid[0] * grid[1] * grid[2], H, D, seed=97)
    return [t.to(DEV) for t in (q, k, v, g)], grid


# the tiny layer (one launch), a short D = 32 sequence (two launches, the
# output kernel summing the partials), the 5B 480p/81f layer (three launches)
CASES = ["tiny_d32_4x8x8", (2, 3, 32, (10, 12, 16)), "5b_480p_81f"]


@pytest.mark.parametrize("case", CASES, ids=["tiny", "d32_two_launches", "5b_480p_81f"])
@pytest.mark.parametrize("entry", ["ws", "noalloc"])
def test_captured_pass_replays_bitwise(case, entry):
    (q, k, v, g), grid = _inputs(case)
    B, N, H, D = q.shape
    say(f"case graph {case} entry={entry} B={B} N={N} H={H} D={D}")
    rope = gla.gla_rope_create(*grid, D)
    ws = gla.alloc_workspace(B, N, H, D, DEV)
    out = torch.empty_like(q)

    def run():
        if entry == "ws":
            gla.gla_forward_ws(q, k, v, g, rope, out, ws)
        else:
            gla.gla_forward_noalloc(q, k, v, g, rope, out)

    # eager reference (also raises each kernel's LDS limit and looks up the
    # scratch address before the capture)
    run()
    torch.cuda.synchronize()
    ref = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()
    for rep in range(4):
        out.fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"replay {rep}"
        # and an eager pass on other inputs in between (the scratch or
        # workspace then holds another call's state)
        other = [t.flip(1).contiguous() for t in (q, k, v, g)]
        o2 = torch.empty_like(q)
        gla.gla_forward(*other, rope, o2) if entry == "ws" else gla.gla_forward_noalloc(
            *other, rope, o2)
        torch.cuda.synchronize()
    del graph
    rope.close()

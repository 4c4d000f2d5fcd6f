"""GPU parity at the largest size the library accepts: a batch element's
[N, H, D] slab just under 2 GiB (N H D 2 < 2^31), so the kernels' 32-bit
byte offsets reach the top of their range.

The inputs are zero except at a few tokens spread over the sequence, the
first and last ones included.  The ReLU features of a zero token vanish, so
it adds nothing to the state, the normaliser, dS or dz, and its output and
all four gradients are exactly zero (the q > 0 and k > 0 masks are off and
dout is zero there).  The nonzero tokens then see exactly the small problem
made of them alone; without RoPE their positions do not enter, so the
oracle solves that small problem.  Bar: as in the other parity tests,
relative L2 <= 5e-3 and max abs <= 3e-2 on the nonzero tokens, and exact
zeros on sampled zero tokens."""
import numpy as np
import pytest
import torch

import gated_linear_attention_forward_amd as gla
import oracle
from workloads import random_grad, random_inputs

pytestmark = pytest.mark.gpu

REL_TOL = 5e-3
ABS_TOL = 3e-2
DEV = torch.device("cuda:0")
D = 128
N_MAX = ((1 << 31) - 1) // (2 * D)  # H = 1: the largest N with N H D 2 < 2^31
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


def positions(N, count, seed):
    """Sorted distinct token positions: the first, middle and last tokens and
    random others."""
    rng = np.random.default_rng(seed)
    pos = np.concatenate([rng.integers(0, N, count), [0, 1, N // 2, N - 2, N - 1]])
    return np.unique(pos)


def zero_positions(N, pos, seed, count=4096):
    """Sampled token positions outside pos (the tail included)."""
    rng = np.random.default_rng(seed)
    cand = np.unique(np.concatenate([rng.integers(0, N, count), np.arange(N - 600, N)]))
    return torch.from_numpy(np.setdiff1d(cand, pos)).to(DEV)


def scatter(small, B, N, idx):
    """[B, N, 1, D] bf16 zeros on the device with the rows of small at idx."""
    big = torch.zeros((B, N, 1, D), dtype=torch.bfloat16, device=DEV)
    big[:, idx] = small.to(DEV)
    return big


def test_forward_at_the_slab_limit():
    B, N = 2, N_MAX
    say(f"case forward max slab B={B} N={N} H=1 D={D} ({N * D * 2} bytes per slab)")
    pos = positions(N, 60, 11)
    idx = torch.from_numpy(pos).to(DEV)
    small = random_inputs(B, len(pos), 1, D, seed=4000)
    q, k, v, g = (scatter(t, B, N, idx) for t in small)
    out = gla.gla_forward(q, k, v, g, None)
    torch.cuda.synchronize()
    got = out[:, idx].double().cpu().numpy()
    zeros = out[:, zero_positions(N, pos, 12)]
    nonzero = int(torch.count_nonzero(zeros))
    del q, k, v, g, out
    torch.cuda.empty_cache()
    ref = oracle.forward(*small, None)
    assert_close(got, ref, "nonzero tokens")
    assert nonzero == 0, f"{nonzero} nonzero outputs at zero tokens"


def test_backward_at_the_slab_limit():
    B, N = 1, N_MAX
    say(f"case backward max slab B={B} N={N} H=1 D={D}")
    pos = positions(N, 60, 21)
    idx = torch.from_numpy(pos).to(DEV)
    small = random_inputs(B, len(pos), 1, D, seed=4100)
    dsmall = random_grad(B, len(pos), 1, D, seed=4200)
    q, k, v, g, dout = (scatter(t, B, N, idx) for t in (*small, dsmall))
    grads = gla.gla_backward(q, k, v, g, dout, None)
    torch.cuda.synchronize()
    del q, k, v, g, dout
    zidx = zero_positions(N, pos, 22)
    got = [t[:, idx].double().cpu().numpy() for t in grads]
    nonzero = [int(torch.count_nonzero(t[:, zidx])) for t in grads]
    del grads
    torch.cuda.empty_cache()
    ref = oracle.backward(*small, dsmall, None)
    for name, a, r in zip(NAMES, got, ref):
        assert_close(a, r, f"nonzero tokens {name}")
    for name, c in zip(NAMES, nonzero):
        assert c == 0, f"{c} nonzero {name} at zero tokens"

"""Pins of the oracle's block-causal form with a carried state (the
constant-memory KV cache for block linear attention, "SANA-Video_2B_720p"
model card, innovation (2)).

Token n in block n // L sees every token up to the end of its own block and
a carried state (S_in, z_in); the state after the last block is returned for
the next call.  Checked against: the masked quadratic form in numpy
(tests/brute.py), the bidirectional mixer for a single block, a run split
into two calls that hand the state over, and the full-sequence state.
"""
import numpy as np
import pytest

import brute
import oracle
from workloads import random_inputs


def f64(*ts):
    return tuple(t.double().numpy() for t in ts)


def carried(B, H, D, seed):
    rng = np.random.default_rng(seed)
    S_in = rng.standard_normal((B, H, D, D))
    z_in = np.abs(rng.standard_normal((B, H, D))) * 3.0
    return S_in, z_in


def rel(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


CASES = [
    # B, H, D, grid (T, Hh, W) or None with N
    (1, 2, 32, (2, 3, 4)),
    (2, 1, 8, None, 20),
    (1, 1, 16, (2, 3, 5)),
    (1, 3, 8, (3, 1, 7)),
]


def case_shape(c):
    if c[3] is None:
        return c[0], c[4], c[1], c[2], None
    T, Hh, W = c[3]
    return c[0], T * Hh * W, c[1], c[2], c[3]


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("L", [1, 5, 12, 1000])
@pytest.mark.parametrize("with_state", [False, True])
def test_blocks_match_masked_quadratic_form(case, L, with_state):
    B, N, H, D, grid = case_shape(case)
    q, k, v, g = random_inputs(B, N, H, D, seed=300 + N + L + D)
    S_in, z_in = carried(B, H, D, seed=N + L) if with_state else (None, None)
    og = oracle.Grid(*grid) if grid else None
    got, _, _ = oracle.forward_blocks(q, k, v, g, og, L, S_in, z_in)
    ref = brute.forward_blocks(*f64(q, k, v, g), grid, L, S_in, z_in)
    assert rel(got, ref) < 1e-11


def test_single_block_is_the_bidirectional_mixer():
    q, k, v, g = random_inputs(2, 60, 2, 32, seed=41)
    grid = oracle.Grid(3, 4, 5)
    for L in (60, 61, 10**6):
        got, S, z = oracle.forward_blocks(q, k, v, g, grid, L)
        ref = oracle.forward(q, k, v, g, grid)
        assert np.array_equal(got, ref)
    S_ref, z_ref = oracle.state(k, v, grid)
    assert np.array_equal(S, S_ref) and np.array_equal(z, z_ref)


def test_state_out_is_the_whole_sequence_state_plus_the_carried_one():
    q, k, v, g = random_inputs(1, 48, 3, 16, seed=42)
    grid = oracle.Grid(4, 3, 4)
    S_in, z_in = carried(1, 3, 16, seed=7)
    _, S, z = oracle.forward_blocks(q, k, v, g, grid, 9, S_in, z_in)
    S_all, z_all = oracle.state(k, v, grid)
    assert rel(S, S_all + S_in) < 1e-13
    assert rel(z, z_all + z_in) < 1e-13


@pytest.mark.parametrize("rope", [True, False])
def test_two_calls_handing_over_the_state_equal_one_call(rope):
    """Frames 0-1 in one call, frames 2-4 in the next with the carried state
    and the RoPE frame offset: the same outputs and final state as one call."""
    T, Hh, W = 5, 3, 4
    HW = Hh * W
    q, k, v, g = random_inputs(2, T * HW, 2, 16, seed=43)
    L = HW  # one frame per block
    whole = oracle.Grid(T, Hh, W) if rope else None
    o_all, S_all, z_all = oracle.forward_blocks(q, k, v, g, whole, L)
    n1 = 2 * HW
    first = oracle.Grid(2, Hh, W) if rope else None
    second = oracle.Grid(T - 2, Hh, W, t0=2) if rope else None
    cut = lambda t, a, b: t[:, a:b].contiguous()
    o1, S1, z1 = oracle.forward_blocks(*(cut(t, 0, n1) for t in (q, k, v, g)), first, L)
    o2, S2, z2 = oracle.forward_blocks(*(cut(t, n1, T * HW) for t in (q, k, v, g)), second, L,
                                       S1, z1)
    assert rel(np.concatenate([o1, o2], axis=1), o_all) < 1e-13
    assert rel(S2, S_all) < 1e-13 and rel(z2, z_all) < 1e-13


def test_first_block_with_no_positive_keys_is_zero():
    q, k, v, g = random_inputs(1, 40, 1, 8, seed=44)
    k = k.clone()
    k[:, :10] = -k[:, :10].abs()
    o, _, _ = oracle.forward_blocks(q, k, v, g, None, 10)
    assert np.all(o[:, :10] == 0.0)
    assert np.any(o[:, 10:] != 0.0)


def test_token_causal_first_token_closed_form():
    """L = 1: token 0 sees only itself: o_0 = sigmoid(g_0) v_0 (rq.rk)/(fq.fk + eps)."""
    q, k, v, g = random_inputs(1, 6, 1, 8, seed=45)
    o, _, _ = oracle.forward_blocks(q, k, v, g, None, 1)
    fq = np.maximum(q[0, 0, 0].double().numpy(), 0)
    fk = np.maximum(k[0, 0, 0].double().numpy(), 0)
    w = fq @ fk
    ref = 1 / (1 + np.exp(-g[0, 0, 0].double().numpy())) * v[0, 0, 0].double().numpy() * w / (w + 1e-6)
    assert np.allclose(o[0, 0, 0], ref, rtol=1e-13, atol=1e-300)


def test_bad_block_length_is_rejected():
    q, k, v, g = random_inputs(1, 8, 1, 8, seed=46)
    with pytest.raises(Exception):
        oracle.forward_blocks(q, k, v, g, None, 0)

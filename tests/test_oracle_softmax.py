"""Pins of the oracle's gated softmax anchor attention ("SANA-Video 2.0",
NVlabs Sana docs, section Architecture: dense softmax anchor layers with Wan
3D rotary embeddings; mlsanity index, Abstract: gated-softmax anchors):

    o_n = sigmoid(g_n) * sum_m softmax_m(R_n q_n . R_m k_m / sqrt(D)) v_m

Checked against closed forms (identical keys, a dominant key, constant
values, a single token), invariances (a common shift of every key, the
order of the key/value pairs, RoPE's relative positions) and a numpy
quadratic form with complex-number rotation.
"""
import numpy as np
import pytest
import torch

import brute
import oracle
from workloads import random_inputs


def sig(x):
    return 1.0 / (1.0 + np.exp(-x))


def f64(t):
    return t.double().numpy()


@pytest.mark.parametrize("grid", [None, (2, 3, 4)])
@pytest.mark.parametrize("D", [32, 64])
def test_matches_numpy_quadratic_form(grid, D):
    N = 24
    q, k, v, g = random_inputs(2, N, 2, D, seed=500 + D)
    got = oracle.softmax_forward(q, k, v, g, oracle.Grid(*grid) if grid else None)
    ref = brute.softmax_attention(f64(q), f64(k), f64(v), f64(g), grid)
    assert np.max(np.abs(got - ref)) < 1e-12


def test_identical_keys_average_the_values():
    q, k, v, g = random_inputs(1, 30, 2, 32, seed=501)
    k = k[:, :1].expand(-1, 30, -1, -1).contiguous()
    got = oracle.softmax_forward(q, k, v, g, None)
    ref = sig(f64(g)) * f64(v).mean(axis=1, keepdims=True)
    assert np.max(np.abs(got - ref)) < 1e-12


def test_dominant_key_selects_its_value():
    N, D = 20, 32
    q, k, v, g = random_inputs(1, N, 1, D, seed=502)
    q0 = torch.linspace(0.5, 2.0, D).to(torch.bfloat16)
    q = q0.expand(1, N, 1, D).contiguous()
    k = k.clone()
    k[0, 7, 0] = (4.0 * q0).to(torch.bfloat16)
    got = oracle.softmax_forward(q, k, v, g, None)
    ref = sig(f64(g)) * f64(v)[:, 7:8]
    assert np.max(np.abs(got - ref)) < 1e-6


@pytest.mark.parametrize("grid", [None, (3, 2, 5)])
def test_constant_values_pass_through(grid):
    q, k, _, g = random_inputs(1, 30, 2, 32, seed=503)
    c = torch.linspace(-3, 3, 32).to(torch.bfloat16)
    v = c.expand(1, 30, 2, 32).contiguous()
    got = oracle.softmax_forward(q, k, v, g, oracle.Grid(*grid) if grid else None)
    assert np.max(np.abs(got - sig(f64(g)) * f64(c))) < 1e-12


def test_single_token():
    q, k, v, g = random_inputs(1, 1, 3, 64, seed=504)
    got = oracle.softmax_forward(q, k, v, g, oracle.Grid(1, 1, 1))
    assert np.max(np.abs(got - sig(f64(g)) * f64(v))) < 1e-12


def test_common_shift_of_every_key_changes_nothing():
    """k_m -> k_m + w adds q_n . w to every logit of query n; values on a
    1/8 grid keep the shifted keys exact in bf16."""
    rng = np.random.default_rng(505)
    N, D = 26, 32
    q = torch.from_numpy(rng.integers(-16, 17, (1, N, 1, D)) / 8.0).to(torch.bfloat16)
    k = torch.from_numpy(rng.integers(-16, 17, (1, N, 1, D)) / 8.0).to(torch.bfloat16)
    w = torch.from_numpy(rng.integers(-8, 9, (1, 1, 1, D)) / 8.0)
    k2 = (k.double() + w).to(torch.bfloat16)
    assert torch.equal(k2.double(), k.double() + w)
    _, _, v, g = random_inputs(1, N, 1, D, seed=506)
    o1 = oracle.softmax_forward(q, k, v, g, None)
    o2 = oracle.softmax_forward(q, k2, v, g, None)
    assert np.max(np.abs(o1 - o2)) < 1e-12


def test_order_of_key_value_pairs_changes_nothing():
    q, k, v, g = random_inputs(1, 40, 2, 32, seed=507)
    perm = torch.randperm(40, generator=torch.Generator().manual_seed(3))
    rows = np.arange(40)
    o1 = oracle.softmax_rows(q, k, v, g, None, 0, 1, rows)
    o2 = oracle.softmax_rows(q, k[:, perm].contiguous(), v[:, perm].contiguous(), g, None, 0, 1,
                             rows)
    assert np.max(np.abs(o1 - o2)) < 1e-12


def test_rope_sees_relative_positions_only():
    q, k, v, g = random_inputs(1, 60, 1, 64, seed=508)
    o1 = oracle.softmax_forward(q, k, v, g, oracle.Grid(3, 4, 5))
    o2 = oracle.softmax_forward(q, k, v, g, oracle.Grid(3, 4, 5, t0=9, y0=-2, x0=5))
    assert np.max(np.abs(o1 - o2)) < 1e-10


def test_rows_match_the_whole_pass():
    q, k, v, g = random_inputs(2, 36, 2, 32, seed=509)
    grid = oracle.Grid(2, 3, 6)
    whole = oracle.softmax_forward(q, k, v, g, grid)
    rows = np.array([35, 0, 17])
    part = oracle.softmax_rows(q, k, v, g, grid, 1, 0, rows)
    assert np.array_equal(part, whole[1, rows, 0])

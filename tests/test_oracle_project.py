"""Pins of the oracle's projection prologue (q, k, v, g = x W^T per map,
rounded to bf16, then the mixer).

Checked against: numpy's fp64 matrix product; torch's float32 -> bf16
rounding on values exactly representable in float32 (one rounding, nearest,
ties to even) and hand-made ties; and selection weights that copy blocks of
x into q, k, v, g, which must reproduce the mixer on those blocks exactly
(pins the stacking order q, k, v, g and the head split of the features).
"""
import numpy as np
import torch

import oracle
from workloads import random_inputs, random_projection


def test_project_matches_numpy_product():
    x, w = random_projection(2, 17, 96, 2, 8, seed=3)
    feats = np.arange(w.shape[0] * w.shape[1])
    got = oracle.project(x, w.reshape(-1, 96), feats)
    ref = x.double().numpy() @ w.reshape(-1, 96).double().numpy().T
    assert np.allclose(got, ref, rtol=1e-13, atol=1e-13)
    sub = np.array([5, 0, 63, 17])
    assert np.array_equal(oracle.project(x, w.reshape(-1, 96), sub), got[..., sub])


def test_round_bf16_matches_torch_on_float32_values():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 1.0, 37.0)])
    v = v.astype(np.float32).astype(np.float64)          # exactly representable in float32
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(oracle.round_bf16(v), ref.view(np.uint16))


def test_round_bf16_ties_go_to_even():
    ulp = 2.0 ** -7                       # bf16 spacing on [1, 2)
    cases = {1 + ulp / 2: 1.0, 1 + 1.5 * ulp: 1 + 2 * ulp, -(1 + ulp / 2): -1.0,
             1 + ulp / 2 + 2.0 ** -30: 1 + ulp}
    for x, want in cases.items():
        bits = int(oracle.round_bf16(np.array([x]))[0])
        got = np.array([bits << 16], np.uint32).view(np.float32)[0]
        assert got == want, (x, got, want)


def test_selection_weights_reproduce_the_mixer():
    """C = 4 H D and W_m copies block m of x: the projections are exactly
    q, k, v, g, so projected_forward must equal the mixer on them."""
    B, N, H, D = 1, 24, 2, 8
    grid = oracle.Grid(2, 3, 4)
    q, k, v, g = random_inputs(B, N, H, D, seed=41)
    x = torch.cat([t.reshape(B, N, H * D) for t in (q, k, v, g)], dim=-1).contiguous()
    C = 4 * H * D
    w = torch.zeros((4, H * D, C), dtype=torch.bfloat16)
    for m in range(4):
        w[m, :, m * H * D:(m + 1) * H * D] = torch.eye(H * D, dtype=torch.bfloat16)
    got = oracle.projected_forward(x, w.reshape(4 * H * D, C), H, D, grid)
    ref = oracle.forward(q, k, v, g, grid)
    assert np.array_equal(got, ref)
    heads = oracle.projected_heads(x, w.reshape(4 * H * D, C), H, D, [1])
    assert np.array_equal(heads["k"][:, :, 0], oracle.as_bits(k)[:, :, 1])
    assert np.array_equal(heads["g"][:, :, 0], oracle.as_bits(g)[:, :, 1])


def test_project_maps_matches_the_c_projection():
    """project_maps (numpy's product, chunked over tokens) against the C
    oracle's projected_heads for every map and head, bit for bit after the
    bf16 rounding (the fp64 sums differ only in order, far below a bf16
    rounding boundary except on exact ties, which random data does not hit)."""
    B, N, C, H, D = 2, 37, 128, 3, 32
    x, w = random_projection(B, N, C, H, D, seed=11)
    maps = oracle.project_maps(x, w, H, D, chunk=16)
    ref = oracle.projected_heads(x, w, H, D, range(H))
    for name, got in zip("qkvg", maps):
        assert got.shape == (B, N, H, D)
        assert np.array_equal(got, ref[name]), name

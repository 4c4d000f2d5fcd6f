"""Python wrapper of the fp64 CPU oracle (oracle/gla_oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg are its only callers.  The product package
never imports this module.

The oracle computes the gated bidirectional linear-attention token mixer of
"SANA-Video 2.0" (NVlabs Sana docs, section Architecture: gated bidirectional
linear attention with Wan 3D rotary position embeddings) in plain IEEE double
arithmetic, one (b, h) head at a time: first the state S and normaliser z,
then every token's output.  ``forward_blocks`` is the block-causal form with
a carried state; ``softmax_rows`` the gated softmax anchor attention;
``backward`` (and its state / row helpers) the exact derivative of the
bidirectional mixer given the output gradient; ``project`` the linear maps
producing q, k, v, g from the hidden states and ``projected_forward`` the
projections followed by the mixer.  See gla_oracle.c for the exact forms and the readings they
take where the pages are silent.

Inputs are bf16 bit patterns (numpy uint16 arrays, or torch bfloat16 CPU
tensors which are viewed as such), layout [B, N, H, D] contiguous.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gla_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libgla_oracle.so")
_lib = None

EPS = 1e-6


def build() -> str:
    """Compile gla_oracle.c into oracle/libgla_oracle.so with gcc (OpenMP)."""
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
           "-o", _LIB_PATH + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_SRC) > os.path.getmtime(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    u16p = ctypes.POINTER(ctypes.c_uint16)
    dp = ctypes.POINTER(ctypes.c_double)
    lp = ctypes.POINTER(ctypes.c_long)
    c_int, c_long, c_double = ctypes.c_int, ctypes.c_long, ctypes.c_double
    grid = [c_int, c_int, c_int, c_int, c_double, c_long, c_long, c_long]
    lib.gla_oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
    lib.gla_oracle_bf16_to_f64.restype = c_double
    lib.gla_oracle_num_threads.argtypes = []
    lib.gla_oracle_num_threads.restype = c_int
    lib.gla_oracle_axis_split.argtypes = [c_int] + [ctypes.POINTER(c_int)] * 3
    lib.gla_oracle_axis_split.restype = None
    lib.gla_oracle_angle.argtypes = [c_int, c_double, c_int, c_long, c_long, c_long]
    lib.gla_oracle_angle.restype = c_double
    lib.gla_oracle_rotate.argtypes = [c_int, c_int, c_int, c_int, c_double, c_long, c_long,
                                      c_long, c_long, dp, dp]
    lib.gla_oracle_rotate.restype = c_int
    lib.gla_oracle_state.argtypes = [u16p, u16p, c_int, c_int, c_int, c_int] + grid + [dp, dp]
    lib.gla_oracle_state.restype = c_int
    lib.gla_oracle_rows.argtypes = ([u16p, u16p, c_int, c_int, c_int, c_int] + grid +
                                    [c_int, c_int, dp, dp, c_double, lp, c_long, dp])
    lib.gla_oracle_rows.restype = c_int
    lib.gla_oracle_forward.argtypes = ([u16p] * 4 + [c_int] * 4 + grid + [c_double, dp])
    lib.gla_oracle_forward.restype = c_int
    lib.gla_oracle_forward_blocks.argtypes = ([u16p] * 4 + [c_int] * 4 + grid +
                                              [c_double, c_long, dp, dp, dp, dp, dp])
    lib.gla_oracle_forward_blocks.restype = c_int
    lib.gla_oracle_softmax_rows.argtypes = ([u16p] * 4 + [c_int] * 4 + grid +
                                            [c_int, c_int, lp, c_long, dp])
    lib.gla_oracle_softmax_rows.restype = c_int
    lib.gla_oracle_round_bf16.argtypes = [c_double]
    lib.gla_oracle_round_bf16.restype = ctypes.c_uint16
    lib.gla_oracle_round_bf16_array.argtypes = [dp, c_long, u16p]
    lib.gla_oracle_round_bf16_array.restype = None
    lib.gla_oracle_project.argtypes = [u16p, u16p, c_int, c_int, c_int, c_int,
                                       ctypes.POINTER(c_int), c_int, dp]
    lib.gla_oracle_project.restype = c_int
    lib.gla_oracle_backward.argtypes = ([u16p] * 5 + [c_int] * 4 + grid +
                                        [c_double, dp, dp, dp, dp])
    lib.gla_oracle_backward.restype = c_int
    lib.gla_oracle_backward_state.argtypes = ([u16p] * 3 + [c_int] * 4 + grid +
                                              [c_double, dp, dp, dp, dp])
    lib.gla_oracle_backward_state.restype = c_int
    lib.gla_oracle_backward_q_rows.argtypes = ([u16p] * 3 + [c_int] * 4 + grid +
                                               [c_double, c_int, c_int, dp, dp, lp, c_long, dp,
                                                dp])
    lib.gla_oracle_backward_q_rows.restype = c_int
    lib.gla_oracle_backward_kv_rows.argtypes = ([u16p] * 2 + [c_int] * 4 + grid +
                                                [c_int, c_int, dp, dp, lp, c_long, dp, dp])
    lib.gla_oracle_backward_kv_rows.restype = c_int
    _lib = lib
    return lib


@dataclass(frozen=True)
class Grid:
    """Latent grid (frames T, rows Hh, columns W) with RoPE base and index offsets."""
    T: int
    Hh: int
    W: int
    theta: float = 10000.0
    t0: int = 0
    y0: int = 0
    x0: int = 0

    @property
    def N(self) -> int:
        return self.T * self.Hh * self.W


def _grid_args(grid):
    if grid is None:
        return [0, 1, 1, 1, 10000.0, 0, 0, 0]
    return [1, grid.T, grid.Hh, grid.W, float(grid.theta), grid.t0, grid.y0, grid.x0]


def as_bits(a) -> np.ndarray:
    """bf16 data as a C-contiguous uint16 numpy array of its bit patterns."""
    if isinstance(a, np.ndarray):
        if a.dtype != np.uint16:
            raise TypeError("oracle inputs must be bf16 bit patterns (uint16)")
        return np.ascontiguousarray(a)
    import torch  # only to view a bfloat16 tensor's bits
    if a.dtype != torch.bfloat16:
        raise TypeError("oracle inputs must be bfloat16")
    return a.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _p(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _check(rc):
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (code {rc})")


def num_threads() -> int:
    return _load().gla_oracle_num_threads()


def bf16_to_f64(bits: int) -> float:
    return _load().gla_oracle_bf16_to_f64(int(bits))


def axis_split(D: int):
    """Pair counts (Pt, Py, Px) of the t/y/x axis blocks of RoPE."""
    a, b, c = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    _load().gla_oracle_axis_split(D, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c))
    return a.value, b.value, c.value


def angle(D: int, theta: float, p: int, t: int, y: int, x: int) -> float:
    return _load().gla_oracle_angle(D, float(theta), p, t, y, x)


def rotate(u, grid: Grid, n: int) -> np.ndarray:
    """R_n u for a length-D float vector u, token n of the grid."""
    u = np.ascontiguousarray(u, dtype=np.float64)
    out = np.empty_like(u)
    _check(_load().gla_oracle_rotate(u.shape[0], grid.T, grid.Hh, grid.W, float(grid.theta),
                                     grid.t0, grid.y0, grid.x0, n,
                                     _p(u, ctypes.c_double), _p(out, ctypes.c_double)))
    return out


def state(k, v, grid: Grid | None):
    """(S, z) of every head: S [B, H, D, D] (S[d, e]), z [B, H, D], fp64."""
    k, v = as_bits(k), as_bits(v)
    B, N, H, D = k.shape
    S = np.empty((B, H, D, D), np.float64)
    z = np.empty((B, H, D), np.float64)
    _check(_load().gla_oracle_state(_p(k, ctypes.c_uint16), _p(v, ctypes.c_uint16), B, N, H, D,
                                    *_grid_args(grid), _p(S, ctypes.c_double),
                                    _p(z, ctypes.c_double)))
    return S, z


def rows(q, g, grid: Grid | None, b: int, h: int, S_bh, z_bh, token_rows, eps: float = EPS):
    """Outputs [len(token_rows), D] of head (b, h) at the given tokens."""
    q, g = as_bits(q), as_bits(g)
    B, N, H, D = q.shape
    S_bh = np.ascontiguousarray(S_bh, dtype=np.float64)
    z_bh = np.ascontiguousarray(z_bh, dtype=np.float64)
    r = np.ascontiguousarray(token_rows, dtype=np.int64)
    out = np.empty((r.shape[0], D), np.float64)
    _check(_load().gla_oracle_rows(_p(q, ctypes.c_uint16), _p(g, ctypes.c_uint16), B, N, H, D,
                                   *_grid_args(grid), b, h, _p(S_bh, ctypes.c_double),
                                   _p(z_bh, ctypes.c_double), float(eps),
                                   _p(r, ctypes.c_long), r.shape[0], _p(out, ctypes.c_double)))
    return out


def forward(q, k, v, g, grid: Grid | None, eps: float = EPS) -> np.ndarray:
    """Whole forward pass: o [B, N, H, D] in fp64."""
    q, k, v, g = (as_bits(a) for a in (q, k, v, g))
    B, N, H, D = q.shape
    for a in (k, v, g):
        if a.shape != q.shape:
            raise ValueError("q, k, v, g must share one [B, N, H, D] shape")
    out = np.empty((B, N, H, D), np.float64)
    _check(_load().gla_oracle_forward(*(_p(a, ctypes.c_uint16) for a in (q, k, v, g)),
                                      B, N, H, D, *_grid_args(grid), float(eps),
                                      _p(out, ctypes.c_double)))
    return out


def forward_blocks(q, k, v, g, grid: Grid | None, block_tokens: int, S_in=None, z_in=None,
                   eps: float = EPS):
    """Block-causal pass with a carried state (see gla_oracle_forward_blocks):
    returns (o [B, N, H, D], S_out [B, H, D, D], z_out [B, H, D]) in fp64."""
    q, k, v, g = (as_bits(a) for a in (q, k, v, g))
    B, N, H, D = q.shape
    for a in (k, v, g):
        if a.shape != q.shape:
            raise ValueError("q, k, v, g must share one [B, N, H, D] shape")
    out = np.empty((B, N, H, D), np.float64)
    S_out = np.empty((B, H, D, D), np.float64)
    z_out = np.empty((B, H, D), np.float64)
    null = ctypes.POINTER(ctypes.c_double)()
    if S_in is not None:
        S_in = np.ascontiguousarray(S_in, dtype=np.float64).reshape(B, H, D, D)
    if z_in is not None:
        z_in = np.ascontiguousarray(z_in, dtype=np.float64).reshape(B, H, D)
    _check(_load().gla_oracle_forward_blocks(
        *(_p(a, ctypes.c_uint16) for a in (q, k, v, g)), B, N, H, D, *_grid_args(grid),
        float(eps), int(block_tokens),
        _p(S_in, ctypes.c_double) if S_in is not None else null,
        _p(z_in, ctypes.c_double) if z_in is not None else null,
        _p(out, ctypes.c_double), _p(S_out, ctypes.c_double), _p(z_out, ctypes.c_double)))
    return out, S_out, z_out


def softmax_rows(q, k, v, g, grid: Grid | None, b: int, h: int, token_rows) -> np.ndarray:
    """Gated softmax anchor attention (see gla_oracle_softmax_rows): outputs
    [len(token_rows), D] of head (b, h) at the given query tokens, fp64."""
    q, k, v, g = (as_bits(a) for a in (q, k, v, g))
    B, N, H, D = q.shape
    for a in (k, v, g):
        if a.shape != q.shape:
            raise ValueError("q, k, v, g must share one [B, N, H, D] shape")
    r = np.ascontiguousarray(token_rows, dtype=np.int64)
    out = np.empty((r.shape[0], D), np.float64)
    _check(_load().gla_oracle_softmax_rows(*(_p(a, ctypes.c_uint16) for a in (q, k, v, g)),
                                           B, N, H, D, *_grid_args(grid), b, h,
                                           _p(r, ctypes.c_long), r.shape[0],
                                           _p(out, ctypes.c_double)))
    return out


def softmax_forward(q, k, v, g, grid: Grid | None) -> np.ndarray:
    """Every output of the gated softmax anchor attention: [B, N, H, D] fp64."""
    q = as_bits(q)
    B, N, H, D = q.shape
    out = np.empty((B, N, H, D), np.float64)
    rows_all = np.arange(N)
    for b in range(B):
        for h in range(H):
            out[b, :, h] = softmax_rows(q, k, v, g, grid, b, h, rows_all)
    return out


def _same_shape(*arrays):
    shape = arrays[0].shape
    for a in arrays[1:]:
        if a.shape != shape:
            raise ValueError("inputs must share one [B, N, H, D] shape")
    return shape


def backward(q, k, v, g, dout, grid: Grid | None, eps: float = EPS):
    """Gradients (dq, dk, dv, dg), each [B, N, H, D] fp64, of the loss whose
    gradient with respect to the mixer's output is dout (see
    gla_oracle_backward for the chain-rule form)."""
    q, k, v, g, dout = (as_bits(a) for a in (q, k, v, g, dout))
    B, N, H, D = _same_shape(q, k, v, g, dout)
    outs = [np.empty((B, N, H, D), np.float64) for _ in range(4)]
    _check(_load().gla_oracle_backward(*(_p(a, ctypes.c_uint16) for a in (q, k, v, g, dout)),
                                       B, N, H, D, *_grid_args(grid), eps,
                                       *(_p(o, ctypes.c_double) for o in outs)))
    return tuple(outs)


def backward_state(q, g, dout, grid: Grid | None, S, z, eps: float = EPS):
    """dS [B, H, D, D] = sum_n rq_n a_n^T and dz [B, H, D] = sum_n dden_n phi(q_n),
    given the forward state S, z (as ``state`` returns)."""
    q, g, dout = (as_bits(a) for a in (q, g, dout))
    B, N, H, D = _same_shape(q, g, dout)
    S = np.ascontiguousarray(S, dtype=np.float64)
    z = np.ascontiguousarray(z, dtype=np.float64)
    if S.shape != (B, H, D, D) or z.shape != (B, H, D):
        raise ValueError("S must be [B, H, D, D] and z [B, H, D]")
    dS = np.empty((B, H, D, D), np.float64)
    dz = np.empty((B, H, D), np.float64)
    _check(_load().gla_oracle_backward_state(*(_p(a, ctypes.c_uint16) for a in (q, g, dout)),
                                             B, N, H, D, *_grid_args(grid), eps,
                                             _p(S, ctypes.c_double), _p(z, ctypes.c_double),
                                             _p(dS, ctypes.c_double), _p(dz, ctypes.c_double)))
    return dS, dz


def backward_q_rows(q, g, dout, grid: Grid | None, b: int, h: int, S_bh, z_bh, token_rows,
                    eps: float = EPS):
    """dq and dg rows [len(token_rows), D] of head (b, h), given its S [D, D], z [D]."""
    q, g, dout = (as_bits(a) for a in (q, g, dout))
    B, N, H, D = _same_shape(q, g, dout)
    S_bh = np.ascontiguousarray(S_bh, dtype=np.float64)
    z_bh = np.ascontiguousarray(z_bh, dtype=np.float64)
    if S_bh.shape != (D, D) or z_bh.shape != (D,):
        raise ValueError("S_bh must be [D, D] and z_bh [D]")
    r = np.ascontiguousarray(token_rows, dtype=np.int64)
    dq = np.empty((r.shape[0], D), np.float64)
    dg = np.empty((r.shape[0], D), np.float64)
    _check(_load().gla_oracle_backward_q_rows(*(_p(a, ctypes.c_uint16) for a in (q, g, dout)),
                                              B, N, H, D, *_grid_args(grid), eps, b, h,
                                              _p(S_bh, ctypes.c_double), _p(z_bh, ctypes.c_double),
                                              _p(r, ctypes.c_long), r.shape[0],
                                              _p(dq, ctypes.c_double), _p(dg, ctypes.c_double)))
    return dq, dg


def backward_kv_rows(k, v, grid: Grid | None, b: int, h: int, dS_bh, dz_bh, token_rows):
    """dk and dv rows [len(token_rows), D] of head (b, h), given its dS [D, D], dz [D]."""
    k, v = (as_bits(a) for a in (k, v))
    B, N, H, D = _same_shape(k, v)
    dS_bh = np.ascontiguousarray(dS_bh, dtype=np.float64)
    dz_bh = np.ascontiguousarray(dz_bh, dtype=np.float64)
    if dS_bh.shape != (D, D) or dz_bh.shape != (D,):
        raise ValueError("dS_bh must be [D, D] and dz_bh [D]")
    r = np.ascontiguousarray(token_rows, dtype=np.int64)
    dk = np.empty((r.shape[0], D), np.float64)
    dv = np.empty((r.shape[0], D), np.float64)
    _check(_load().gla_oracle_backward_kv_rows(*(_p(a, ctypes.c_uint16) for a in (k, v)),
                                               B, N, H, D, *_grid_args(grid), b, h,
                                               _p(dS_bh, ctypes.c_double),
                                               _p(dz_bh, ctypes.c_double),
                                               _p(r, ctypes.c_long), r.shape[0],
                                               _p(dk, ctypes.c_double), _p(dv, ctypes.c_double)))
    return dk, dv


def round_bf16(values) -> np.ndarray:
    """bf16 bit patterns (uint16) of doubles rounded to nearest, ties to even."""
    a = np.ascontiguousarray(values, dtype=np.float64)
    out = np.empty(a.shape, np.uint16)
    _load().gla_oracle_round_bf16_array(_p(a, ctypes.c_double), a.size, _p(out, ctypes.c_uint16))
    return out


def project(x, w, features) -> np.ndarray:
    """x [B, N, C] and w [P, C] bf16: the fp64 products x w[features]^T,
    [B, N, len(features)]."""
    x, w = as_bits(x), as_bits(w)
    if w.ndim == 3:                       # stacked [4, H*D, C]
        w = np.ascontiguousarray(w.reshape(-1, w.shape[-1]))
    if x.ndim != 3 or w.ndim != 2 or x.shape[2] != w.shape[1]:
        raise ValueError("x must be [B, N, C] and w [P, C] (or [4, H*D, C])")
    B, N, C = x.shape
    feat = np.ascontiguousarray(features, dtype=np.int32)
    out = np.empty((B, N, feat.shape[0]), np.float64)
    _check(_load().gla_oracle_project(_p(x, ctypes.c_uint16), _p(w, ctypes.c_uint16), B, N, C,
                                      w.shape[0], _p(feat, ctypes.c_int), feat.shape[0],
                                      _p(out, ctypes.c_double)))
    return out


def projected_heads(x, w, H: int, D: int, heads, which="qkvg"):
    """bf16 bit patterns of the projections of the given heads, each
    [B, N, len(heads), D]: dict map name -> array (maps stacked q, k, v, g)."""
    idx = {"q": 0, "k": 1, "v": 2, "g": 3}
    out = {}
    for name in which:
        feats = np.concatenate([idx[name] * H * D + h * D + np.arange(D) for h in heads])
        y = project(x, w, feats)
        B, N = y.shape[:2]
        out[name] = round_bf16(y).reshape(B, N, len(heads), D)
    return out


def project_maps(x, w, H: int, D: int, chunk: int = 8192):
    """All four projections of every head, rounded to bf16: (q, k, v, g) bit
    patterns, each [B, N, H, D].  The fp64 products x W^T come from numpy's
    matrix product (a library primitive: the same sums as project, in
    another order, exact to fp64 rounding), taken over chunks of tokens so
    that a layer's fp64 products never sit in memory at once."""
    xb, wb = as_bits(x), as_bits(w)
    if wb.ndim == 3:
        wb = wb.reshape(-1, wb.shape[-1])
    B, N, C = xb.shape
    if wb.shape != (4 * H * D, C):
        raise ValueError("w must be [4, H*D, C] (or [4*H*D, C])")
    wf = (wb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)  # exact widening
    outs = [np.empty((B, N, H, D), np.uint16) for _ in range(4)]
    for b in range(B):
        for n0 in range(0, N, chunk):
            n1 = min(n0 + chunk, N)
            xf = (xb[b, n0:n1].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            y = round_bf16(xf @ wf.T).reshape(n1 - n0, 4, H, D)
            for i in range(4):
                outs[i][b, n0:n1] = y[:, i]
    return tuple(outs)


def projected_forward(x, w, H: int, D: int, grid: Grid | None, eps: float = EPS) -> np.ndarray:
    """The projections rounded to bf16, then the mixer: [B, N, H, D] fp64."""
    t = projected_heads(x, w, H, D, range(H))
    return forward(t["q"], t["k"], t["v"], t["g"], grid, eps)

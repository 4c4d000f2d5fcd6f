"""C-ABI checks that need no GPU: the library loads, exports every function
include/gla.h declares, validates arguments before any HIP call, and builds
RoPE tables that agree with the oracle's fp64 rotation angles."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import gated_linear_attention_forward_amd as gla
import oracle
from gated_linear_attention_forward_amd import gla as glamod

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "gla.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gla_\w+)\s*\(", src)))


def test_library_exports_every_declared_function():
    lib = gla.load_library()
    names = header_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), f"{n} declared in gla.h but not exported"
    assert set(names) == set(gla.EXPORTS)


def test_strerror_covers_codes():
    for code in range(0, -11, -1):
        s = gla.gla_strerror(code)
        assert s and s != "unknown status"
    assert gla.gla_strerror(17) == "unknown status"


A = 1 << 20  # fake, 16-byte aligned "device" addresses: validation never dereferences them


def check(q=A, k=2 * A, v=3 * A, g=4 * A, rope=None, out=5 * A, B=1, N=64, H=2, D=128):
    return gla.gla_forward_check(q, k, v, g, rope, out, B, N, H, D)


def test_valid_arguments_pass_validation():
    assert check() == 0
    assert check(D=32) == 0 and check(D=64) == 0


@pytest.mark.parametrize("D", [0, 16, 48, 96, 127, 256])
def test_bad_head_dim(D):
    assert check(D=D) == glamod.GLA_ERR_DIM


def test_negative_and_oversized_shapes():
    assert check(B=-1) == glamod.GLA_ERR_DIM
    assert check(N=-5) == glamod.GLA_ERR_DIM
    assert check(H=-2) == glamod.GLA_ERR_DIM
    assert check(B=2, H=40000) == glamod.GLA_ERR_DIM  # B*H beyond the grid limit


def test_empty_calls_are_noops():
    assert check(N=0) == 0
    assert check(B=0) == 0
    assert check(H=0, q=0, k=0) == 0  # nothing to touch: pointers are not needed


def test_null_and_alignment():
    assert check(q=0) == glamod.GLA_ERR_NULL
    assert check(out=0) == glamod.GLA_ERR_NULL
    assert check(v=3 * A + 8) == glamod.GLA_ERR_ALIGN
    assert check(out=5 * A + 2) == glamod.GLA_ERR_ALIGN


def test_alias_detection():
    nbytes = 1 * 64 * 2 * 128 * 2
    assert check(out=A) == glamod.GLA_ERR_ALIAS
    assert check(out=4 * A + nbytes - 16) == glamod.GLA_ERR_ALIAS
    assert check(out=4 * A + nbytes) == 0


def _host_rope(T, Hh, W, D, cs=A):
    r = glamod.gla_rope_tables()
    r.T, r.Hh, r.W, r.D = T, Hh, W, D
    py = D // 6
    r.Pt, r.Py, r.Px = D // 2 - 2 * py, py, py
    r.theta = 1e4
    r.cs = cs
    r.cs_floats = gla.gla_rope_table_floats(T, Hh, W, D)
    r.device = 0
    return ctypes.pointer(r)


def test_rope_mismatch_rejected():
    assert check(N=64, rope=_host_rope(4, 4, 4, 128)) == 0
    assert check(N=64, rope=_host_rope(4, 4, 5, 128)) == glamod.GLA_ERR_ROPE
    assert check(N=64, D=64, rope=_host_rope(4, 4, 4, 128)) == glamod.GLA_ERR_ROPE
    assert check(N=64, rope=_host_rope(4, 4, 4, 128, cs=0)) == glamod.GLA_ERR_NULL
    # the kernels read the table in 16-byte loads
    assert check(N=64, rope=_host_rope(4, 4, 4, 128, cs=A + 8)) == glamod.GLA_ERR_ALIGN


def test_workspace_size_formula():
    # partials (C chunks x (D*D + D) fp32) + bf16 state + fp32 z, each 256-byte aligned
    for (B, N, H, D) in ((1, 256, 2, 32), (2, 22000, 20, 128), (1, 159280, 20, 128)):
        ws = gla.gla_workspace_bytes(B, N, H, D)
        bh = B * H
        assert ws >= bh * (D * D + D) * 4 + bh * D * D * 2 + bh * D * 4
        assert ws % 256 == 0
    assert gla.gla_workspace_bytes(0, 10, 2, 128) == 0
    assert gla.gla_workspace_bytes(1, 10, 2, 100) == 0


@pytest.mark.parametrize("D,grid,off", [(32, (4, 8, 8), (0, 0, 0)), (64, (3, 5, 7), (1, 2, 3)),
                                        (128, (25, 22, 40), (0, 0, 0)),
                                        (128, (181, 22, 40), (5, -3, 7))])
def test_rope_table_matches_oracle_angles(D, grid, off):
    """Every (cos, sin) entry equals the oracle's fp64 angle's cos/sin within 1e-6."""
    T, Hh, W = grid
    cs = gla.gla_rope_fill_host(T, Hh, W, D, 1e4, *off).astype(np.float64)
    pt, py, px = oracle.axis_split(D)
    assert cs.size == 2 * (T * pt + Hh * py + W * px)
    at = 0
    for axis, (n, pa, first) in enumerate(((T, pt, 0), (Hh, py, pt), (W, px, pt + py))):
        for pos in range(n):
            idx = [0, 0, 0]
            idx[axis] = pos + off[axis]
            ang = np.array([oracle.angle(D, 1e4, first + j, *idx) for j in range(pa)])
            got = cs[at:at + 2 * pa]
            assert np.max(np.abs(got[0::2] - np.cos(ang))) <= 1e-6
            assert np.max(np.abs(got[1::2] - np.sin(ang))) <= 1e-6
            at += 2 * pa
    assert at == cs.size


def test_rope_fill_rejects_bad_args():
    with pytest.raises(gla.GlaError):
        gla.gla_rope_fill_host(0, 1, 1, 128)
    with pytest.raises(gla.GlaError):
        gla.gla_rope_fill_host(2, 2, 2, 127)


# ---------------------------------------------------------------------------
# block-causal entry point: validation without a GPU

SB = 2 * 128 * 128 * 4  # S bytes for B=1, H=2, D=128
ZB = 2 * 128 * 4


def bcheck(block_tokens=16, S_in=0, z_in=0, S_out=0, z_out=0, **kw):
    args = dict(q=A, k=2 * A, v=3 * A, g=4 * A, rope=None, out=5 * A, B=1, N=64, H=2, D=128)
    args.update(kw)
    return gla.gla_forward_blocks_check(args["q"], args["k"], args["v"], args["g"], args["rope"],
                                        args["out"], args["B"], args["N"], args["H"], args["D"],
                                        block_tokens, S_in or None, z_in or None, S_out or None,
                                        z_out or None)


def test_blocks_valid_arguments():
    assert bcheck() == 0
    assert bcheck(block_tokens=1) == 0
    assert bcheck(block_tokens=10**6) == 0
    assert bcheck(S_in=8 * A, z_in=9 * A, S_out=10 * A, z_out=11 * A) == 0


def test_blocks_bad_block_length():
    assert bcheck(block_tokens=0) == glamod.GLA_ERR_DIM
    assert bcheck(block_tokens=-3) == glamod.GLA_ERR_DIM


def test_blocks_state_alignment_and_aliasing():
    assert bcheck(S_in=8 * A + 4) == glamod.GLA_ERR_ALIGN
    assert bcheck(z_out=11 * A + 8) == glamod.GLA_ERR_ALIGN
    # in-place update of the carried state is allowed
    assert bcheck(S_in=8 * A, S_out=8 * A, z_in=9 * A, z_out=9 * A) == 0
    # partial overlap of the returned and carried states is not
    assert bcheck(S_in=8 * A, S_out=8 * A + 16) == glamod.GLA_ERR_ALIAS
    # a state over a bf16 tensor, or the two returned states over each other
    assert bcheck(S_out=A + 64) == glamod.GLA_ERR_ALIAS
    assert bcheck(S_in=5 * A) == glamod.GLA_ERR_ALIAS
    assert bcheck(S_out=10 * A, z_out=10 * A + SB - 16) == glamod.GLA_ERR_ALIAS
    assert bcheck(S_out=10 * A, z_out=10 * A + SB) == 0


def test_blocks_empty_sequence_needs_no_tensors():
    # N == 0: nothing is read but the carried state
    assert bcheck(N=0, q=0, k=0, v=0, g=0, out=0, S_in=8 * A, S_out=10 * A) == 0
    assert bcheck(B=0) == 0


def test_blocks_limits():
    far = dict(q=100 * A, k=200 * A, v=300 * A, g=400 * A, out=500 * A)
    # 65536 blocks of one token each exceed the output grid (D = 32: the
    # partial states stay small)
    assert bcheck(N=65536, H=1, D=32, block_tokens=1, **far) == glamod.GLA_ERR_DIM
    assert bcheck(N=65535, H=1, D=32, block_tokens=1, **far) == 0
    # D = 128: 40000 one-token blocks need 2.6 GB of partial states per head
    assert bcheck(N=40000, H=1, block_tokens=1, **far) == glamod.GLA_ERR_DIM
    assert bcheck(N=40000, H=1, block_tokens=16, **far) == 0


def test_blocks_workspace_size():
    one = gla.gla_workspace_bytes_blocks(2, 22000, 20, 128, 22000)
    assert one == gla.gla_workspace_bytes(2, 22000, 20, 128)
    five = gla.gla_workspace_bytes_blocks(2, 22000, 20, 128, 4400)
    assert five >= 40 * 5 * (128 * 128 + 128) * 4 + 40 * 5 * 130 * 128 * 2
    assert five % 256 == 0
    assert gla.gla_workspace_bytes_blocks(2, 22000, 20, 128, 0) == 0


# ---------------------------------------------------------------------------
# softmax anchor attention: validation without a GPU


def scheck(**kw):
    args = dict(q=A, k=2 * A, v=3 * A, g=4 * A, rope=None, out=5 * A, B=1, N=64, H=2, D=256)
    args.update(kw)
    return gla.gla_softmax_forward_check(args["q"], args["k"], args["v"], args["g"],
                                         args["rope"], args["out"], args["B"], args["N"],
                                         args["H"], args["D"])


def test_softmax_validation():
    assert scheck() == 0 and scheck(D=128) == 0
    for D in (32, 64, 192, 512):
        assert scheck(D=D) == glamod.GLA_ERR_DIM
    assert scheck(q=0) == glamod.GLA_ERR_NULL
    assert scheck(v=3 * A + 4) == glamod.GLA_ERR_ALIGN
    assert scheck(out=2 * A) == glamod.GLA_ERR_ALIAS
    assert scheck(N=0) == 0
    assert scheck(N=64, rope=_host_rope(4, 4, 4, 256)) == 0
    assert scheck(N=64, rope=_host_rope(4, 4, 4, 128)) == glamod.GLA_ERR_ROPE


def test_softmax_workspace_size():
    assert gla.gla_softmax_workspace_bytes(2, 22000, 10, 256) >= 2 * 2 * 22000 * 10 * 256 * 2
    assert gla.gla_softmax_workspace_bytes(1, 10, 1, 64) == 0
    assert gla.gla_softmax_workspace_bytes(0, 10, 1, 256) == 0


# ---------------------------------------------------------------------------
# backward pass: validation without a GPU


def bcheck_bwd(**kw):
    args = dict(q=A, k=2 * A, v=3 * A, g=4 * A, dout=5 * A, rope=None, dq=6 * A, dk=7 * A,
                dv=8 * A, dg=9 * A, B=1, N=64, H=2, D=128)
    args.update(kw)
    return gla.gla_backward_check(*(args[n] for n in ("q", "k", "v", "g", "dout", "rope", "dq",
                                                      "dk", "dv", "dg", "B", "N", "H", "D")))


def test_backward_validation():
    assert bcheck_bwd() == 0 and bcheck_bwd(D=32) == 0 and bcheck_bwd(D=64) == 0
    for D in (16, 48, 256):
        assert bcheck_bwd(D=D) == glamod.GLA_ERR_DIM
    assert bcheck_bwd(dout=0) == glamod.GLA_ERR_NULL
    assert bcheck_bwd(dk=0) == glamod.GLA_ERR_NULL
    assert bcheck_bwd(dg=9 * A + 8) == glamod.GLA_ERR_ALIGN
    assert bcheck_bwd(N=0) == 0 and bcheck_bwd(B=0, q=0) == 0
    assert bcheck_bwd(N=64, rope=_host_rope(4, 4, 4, 128)) == 0
    assert bcheck_bwd(N=64, rope=_host_rope(4, 4, 4, 64)) == glamod.GLA_ERR_ROPE


def test_backward_alias_detection():
    nbytes = 1 * 64 * 2 * 128 * 2
    assert bcheck_bwd(dq=A) == glamod.GLA_ERR_ALIAS             # dq is q
    assert bcheck_bwd(dv=5 * A + nbytes - 16) == glamod.GLA_ERR_ALIAS  # dv overlaps dout
    assert bcheck_bwd(dk=6 * A) == glamod.GLA_ERR_ALIAS         # two outputs share memory
    assert bcheck_bwd(dg=6 * A + nbytes - 16) == glamod.GLA_ERR_ALIAS  # dg overlaps dq's end
    assert bcheck_bwd(dg=6 * A + nbytes) == 0                   # dg right after dq
    assert bcheck_bwd(dg=10 * A) == 0


def scheck_bwd(**kw):
    args = dict(q=A, k=2 * A, v=3 * A, g=4 * A, dout=5 * A, rope=None, S=11 * A, z=12 * A,
                dq=6 * A, dk=7 * A, dv=8 * A, dg=9 * A, B=1, N=64, H=2, D=128)
    args.update(kw)
    return gla.gla_backward_saved_check(*(args[n] for n in (
        "q", "k", "v", "g", "dout", "rope", "S", "z", "dq", "dk", "dv", "dg", "B", "N", "H", "D")))


def test_backward_saved_validation():
    assert scheck_bwd() == 0 and scheck_bwd(D=32) == 0
    # the gradient tensors are validated as for gla_backward
    assert scheck_bwd(D=48) == glamod.GLA_ERR_DIM
    assert scheck_bwd(dq=A) == glamod.GLA_ERR_ALIAS
    # the saved state: present, 16-byte aligned, overlapping no output
    assert scheck_bwd(S=0) == glamod.GLA_ERR_NULL and scheck_bwd(z=0) == glamod.GLA_ERR_NULL
    assert scheck_bwd(S=11 * A + 8) == glamod.GLA_ERR_ALIGN
    assert scheck_bwd(z=12 * A + 4) == glamod.GLA_ERR_ALIGN
    sbytes = 2 * 128 * 128 * 4
    assert scheck_bwd(S=6 * A - sbytes + 16) == glamod.GLA_ERR_ALIAS   # S's end in dq
    assert scheck_bwd(z=9 * A + 16) == glamod.GLA_ERR_ALIAS            # z inside dg
    assert scheck_bwd(S=6 * A - sbytes) == 0                           # S right before dq
    # reading the state where an input lies is allowed (both are read only)
    assert scheck_bwd(S=A, z=2 * A) == 0
    # nothing to do: no state needed
    assert scheck_bwd(N=0, S=0, z=0) == 0


def test_backward_saved_state_must_not_overlap_the_workspace():
    """The _ws entry point refuses a saved state inside its workspace before
    any HIP call (fake addresses: validation never dereferences them)."""
    lib = gla.load_library()
    B, N, H, D = 1, 64, 2, 128
    need = gla.gla_backward_workspace_bytes(B, N, H, D)
    ws = 64 * A                                   # 256-byte aligned
    args = [A, 2 * A, 3 * A, 4 * A, 5 * A, None]  # q, k, v, g, dout, rope
    outs = [6 * A, 7 * A, 8 * A, 9 * A]

    def call(S, z):
        return lib.gla_backward_saved_ws(*args, S, z, *outs, B, N, H, D, ws, need, None)

    assert call(ws + 256, 12 * A) == glamod.GLA_ERR_ALIAS          # S inside
    assert call(11 * A, ws + need - 16) == glamod.GLA_ERR_ALIAS    # z at the end


def test_backward_workspace_size():
    for (B, N, H, D) in ((1, 256, 2, 32), (2, 22000, 20, 128)):
        ws = gla.gla_backward_workspace_bytes(B, N, H, D)
        # the forward's workspace, the S rows operand, z, and at least one dS
        # and dz partial per head
        assert ws >= (gla.gla_workspace_bytes(B, N, H, D) + B * H * D * D * 2
                      + B * H * (D * D + D) * 4)
        assert ws % 256 == 0
    assert gla.gla_backward_workspace_bytes(1, 0, 2, 128) == 0
    assert gla.gla_backward_workspace_bytes(1, 10, 1, 48) == 0


# ---------------------------------------------------------------------------
# projection prologue: validation without a GPU


def pcheck(**kw):
    args = dict(x=A, w=8 * A, rope=None, out=16 * A, B=1, N=64, C=256, H=2, D=128)
    args.update(kw)
    return gla.gla_forward_proj_check(*(args[n] for n in ("x", "w", "rope", "out", "B", "N", "C",
                                                          "H", "D")))


def test_proj_validation():
    assert pcheck() == 0 and pcheck(D=32) == 0 and pcheck(D=64, C=64) == 0
    for C in (0, 32, 100, 2561):
        assert pcheck(C=C) == glamod.GLA_ERR_DIM
    assert pcheck(D=48) == glamod.GLA_ERR_DIM
    assert pcheck(x=0) == glamod.GLA_ERR_NULL and pcheck(w=0) == glamod.GLA_ERR_NULL
    assert pcheck(out=16 * A + 4) == glamod.GLA_ERR_ALIGN
    assert pcheck(out=A) == glamod.GLA_ERR_ALIAS                 # out is x
    assert pcheck(out=8 * A + 4 * 2 * 128 * 256 * 2 - 16) == glamod.GLA_ERR_ALIAS  # w's end
    assert pcheck(N=0) == 0
    assert pcheck(N=64, rope=_host_rope(4, 4, 4, 128)) == 0
    assert pcheck(N=64, rope=_host_rope(4, 4, 5, 128)) == glamod.GLA_ERR_ROPE
    # x slab beyond 2 GiB of 32-bit offsets
    assert pcheck(N=1 << 20, C=1024) == glamod.GLA_ERR_DIM
    # the qg kernel's 1-D grid: B H ceil(N / 256) blocks of 512 work-items
    # must stay within 2^32 work-items
    big = dict(N=65535 * 256, C=64, H=1, D=32)
    assert pcheck(B=129, **big) == glamod.GLA_ERR_DIM
    assert pcheck(B=128, **big) != glamod.GLA_ERR_DIM


def test_proj_workspace_size():
    ws = gla.gla_proj_workspace_bytes(2, 22000, 2560, 20, 128)
    assert ws >= gla.gla_workspace_bytes(2, 22000, 20, 128) + 2 * (2 * 22000 * 20 * 128 * 2)
    assert ws % 256 == 0
    assert gla.gla_proj_workspace_bytes(1, 0, 256, 2, 128) == 0
    assert gla.gla_proj_workspace_bytes(1, 10, 100, 2, 128) == 0


def test_noalloc_rejects_calls_beyond_its_scratch_before_any_hip_call():
    """gla_forward_noalloc's fixed scratch is 32 MiB; a call whose workspace
    would be larger is refused with GLA_ERR_SCRATCH during validation (the
    fake pointers are never used, and no GPU is needed)."""
    lib = gla.load_library()
    B, N, H, D = 1, 64, 600, 128  # one chunk per head: 600 fp32 partials of 66 KB
    assert gla.gla_workspace_bytes(B, N, H, D) > 32 << 20
    G = 1 << 30  # fake addresses far enough apart for 9.8 MB tensors
    rc = lib.gla_forward_noalloc(G, 2 * G, 3 * G, 4 * G, None, 5 * G, B, N, H, D, None)
    assert rc == glamod.GLA_ERR_SCRATCH
    # argument errors are still reported first
    rc = lib.gla_forward_noalloc(G, 2 * G, 3 * G, 4 * G, None, 5 * G, B, N, H, 96, None)
    assert rc == glamod.GLA_ERR_DIM


# ---------------------------------------------------------------------------
# caller workspaces: the used part may overlap no tensor of the call (checked
# before any HIP call, so these need no GPU)

def test_forward_workspaces_must_not_overlap_the_tensors():
    lib = gla.load_library()
    B, N, H, D = 1, 64, 2, 128
    nbytes = B * N * H * D * 2
    need = gla.gla_workspace_bytes(B, N, H, D)
    W = 64 * A  # a workspace far from every tensor

    def fwd(ws):
        return lib.gla_forward_ws(A, 2 * A, 3 * A, 4 * A, None, 5 * A, B, N, H, D, ws, need, None)

    def state(ws):
        return lib.gla_state_ws(2 * A, 3 * A, None, B, N, H, D, ws, need, None)

    def output(ws):
        return lib.gla_output_ws(A, 4 * A, None, 5 * A, B, N, H, D, ws, need, None)

    for call, tensors in ((fwd, (A, 2 * A, 3 * A, 4 * A, 5 * A)), (state, (2 * A, 3 * A)),
                          (output, (A, 4 * A, 5 * A))):
        for t in tensors:
            assert call(t) == glamod.GLA_ERR_ALIAS                    # starts on a tensor
            assert call(t + nbytes - 256) == glamod.GLA_ERR_ALIAS     # starts in its tail
            assert call(t - need + 256) == glamod.GLA_ERR_ALIAS       # ends inside it
    # too small a workspace is reported as such
    assert need % 256 == 0
    assert lib.gla_forward_ws(A, 2 * A, 3 * A, 4 * A, None, 5 * A, B, N, H, D, W,
                              need - 256, None) == glamod.GLA_ERR_WORKSPACE


def test_block_workspace_must_not_overlap_tensors_or_states():
    lib = gla.load_library()
    B, N, H, D, L = 1, 64, 2, 128, 16
    need = gla.gla_workspace_bytes_blocks(B, N, H, D, L)

    def call(ws, S_in=8 * A, z_in=9 * A, S_out=10 * A, z_out=11 * A):
        return lib.gla_forward_blocks_ws(A, 2 * A, 3 * A, 4 * A, None, 5 * A, B, N, H, D, L,
                                         S_in, z_in, S_out, z_out, ws, need, None)

    assert call(3 * A + 512) == glamod.GLA_ERR_ALIAS        # inside v
    assert call(8 * A) == glamod.GLA_ERR_ALIAS              # on the carried state
    assert call(11 * A - need + 256) == glamod.GLA_ERR_ALIAS  # ends on the returned z


def test_stream_probe_validates_before_launching():
    lib = gla.load_library()
    assert lib.gla_stream_probe(0, 2 * A, 3 * A, 1 << 20, 0, None) == glamod.GLA_ERR_NULL
    assert lib.gla_stream_probe(A, 2 * A, 0, 1 << 20, 1, None) == glamod.GLA_ERR_NULL
    assert lib.gla_stream_probe(A + 8, 2 * A, 3 * A, 1 << 20, 0, None) == glamod.GLA_ERR_ALIGN
    assert lib.gla_stream_probe(A, 2 * A, 3 * A, 0, 0, None) == glamod.GLA_ERR_DIM
    assert lib.gla_stream_probe(A, 2 * A, 3 * A, 1000, 0, None) == glamod.GLA_ERR_DIM
    assert lib.gla_stream_probe(A, 2 * A, 3 * A, 1 << 31, 0, None) == glamod.GLA_ERR_DIM
    assert lib.gla_stream_probe(A, 2 * A, 3 * A, 1 << 20, 2, None) == glamod.GLA_ERR_DIM


def test_stream_probe_mix_validates_before_launching():
    lib = gla.load_library()
    vp = ctypes.c_void_p

    def arr(*ptrs):
        return (vp * len(ptrs))(*ptrs)

    ok_s, ok_d = arr(A, 2 * A, 3 * A), arr(4 * A, 5 * A)
    mix = lib.gla_stream_probe_mix
    assert mix(None, 3, ok_d, 2, 1 << 20, None) == glamod.GLA_ERR_NULL
    assert mix(ok_s, 3, None, 2, 1 << 20, None) == glamod.GLA_ERR_NULL
    for ns, nd in ((0, 1), (4, 1), (1, 0), (1, 3), (-1, 1)):
        assert mix(ok_s, ns, ok_d, nd, 1 << 20, None) == glamod.GLA_ERR_DIM
    assert mix(arr(A, 0, 3 * A), 3, ok_d, 2, 1 << 20, None) == glamod.GLA_ERR_NULL
    assert mix(ok_s, 3, arr(4 * A, 0), 2, 1 << 20, None) == glamod.GLA_ERR_NULL
    assert mix(arr(A, 2 * A + 8, 3 * A), 3, ok_d, 2, 1 << 20, None) == glamod.GLA_ERR_ALIGN
    assert mix(ok_s, 3, arr(4 * A, 5 * A + 4), 2, 1 << 20, None) == glamod.GLA_ERR_ALIGN
    for nbytes in (0, 1000, 1 << 31):
        assert mix(ok_s, 3, ok_d, 2, nbytes, None) == glamod.GLA_ERR_DIM
    # only the first nsrc / ndst entries are read: a null past them is fine
    # for validation, which then fails on the size
    assert mix(arr(A, 0, 0), 1, arr(4 * A, 0), 1, 1000, None) == glamod.GLA_ERR_DIM

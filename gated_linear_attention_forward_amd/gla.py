"""Python binding of libgla.so (include/gla.h): argument marshalling only.

Every step of the mixer runs in the library's HIP kernels; PyTorch only
provides device memory and the current stream.  The functions carry the C
names.  If the library has not been built the first call raises -- there is
no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgla.so")

GLA_OK = 0
GLA_ERR_NULL = -1
GLA_ERR_ALIGN = -2
GLA_ERR_DIM = -3
GLA_ERR_ROPE = -4
GLA_ERR_ALLOC = -5
GLA_ERR_LAUNCH = -6
GLA_ERR_ALIAS = -7
GLA_ERR_WORKSPACE = -8
GLA_ERR_HIP = -9
GLA_ERR_SCRATCH = -10

EXPORTS = (
    "gla_strerror", "gla_rope_table_floats", "gla_rope_fill_host", "gla_rope_create",
    "gla_rope_destroy", "gla_workspace_bytes", "gla_workspace_release", "gla_forward",
    "gla_forward_ws",
    "gla_forward_check", "gla_forward_noalloc", "gla_state_ws", "gla_output_ws", "gla_state",
    "gla_forward_blocks", "gla_forward_blocks_ws", "gla_workspace_bytes_blocks",
    "gla_forward_blocks_check", "gla_softmax_forward", "gla_softmax_forward_ws",
    "gla_softmax_workspace_bytes", "gla_softmax_forward_check", "gla_backward",
    "gla_backward_ws", "gla_backward_workspace_bytes", "gla_backward_check",
    "gla_backward_saved", "gla_backward_saved_ws", "gla_backward_saved_check",
    "gla_forward_proj", "gla_forward_proj_ws", "gla_proj_workspace_bytes",
    "gla_forward_proj_check", "gla_stream_probe", "gla_stream_probe_mix",
)


class GlaError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {gla_strerror(code)} (status {code})")


class gla_rope_tables(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int32), ("Hh", ctypes.c_int32), ("W", ctypes.c_int32),
        ("D", ctypes.c_int32),
        ("Pt", ctypes.c_int32), ("Py", ctypes.c_int32), ("Px", ctypes.c_int32),
        ("t0", ctypes.c_int32), ("y0", ctypes.c_int32), ("x0", ctypes.c_int32),
        ("theta", ctypes.c_double),
        ("cs", ctypes.c_void_p),
        ("cs_floats", ctypes.c_size_t),
        ("device", ctypes.c_int32),
    ]


_lib = None


def load_library():
    """Loads libgla.so once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it first "
                           "(python -m gated_linear_attention_forward_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, sz, dbl = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_double
    rp = ctypes.POINTER(gla_rope_tables)
    sig = {
        "gla_strerror": ([i32], ctypes.c_char_p),
        "gla_rope_table_floats": ([i32] * 4, sz),
        "gla_rope_fill_host": ([i32] * 4 + [dbl] + [i32] * 3 + [vp, sz], i32),
        "gla_rope_create": ([i32] * 4 + [dbl] + [i32] * 3 + [vp, ctypes.POINTER(rp)], i32),
        "gla_rope_destroy": ([rp], i32),
        "gla_workspace_bytes": ([i32] * 4, sz),
        "gla_workspace_release": ([], i32),
        "gla_forward": ([vp] * 4 + [rp, vp] + [i32] * 4 + [vp], i32),
        "gla_forward_ws": ([vp] * 4 + [rp, vp] + [i32] * 4 + [vp, sz, vp], i32),
        "gla_forward_check": ([vp] * 4 + [rp, vp] + [i32] * 4, i32),
        "gla_forward_noalloc": ([vp] * 4 + [rp, vp] + [i32] * 4 + [vp], i32),
        "gla_state_ws": ([vp, vp, rp] + [i32] * 4 + [vp, sz, vp], i32),
        "gla_output_ws": ([vp, vp, rp, vp] + [i32] * 4 + [vp, sz, vp], i32),
        "gla_state": ([vp, vp, rp, vp, vp] + [i32] * 4 + [vp], i32),
        "gla_forward_blocks": ([vp] * 4 + [rp, vp] + [i32] * 5 + [vp] * 4 + [vp], i32),
        "gla_forward_blocks_ws": ([vp] * 4 + [rp, vp] + [i32] * 5 + [vp] * 4 + [vp, sz, vp], i32),
        "gla_workspace_bytes_blocks": ([i32] * 5, sz),
        "gla_forward_blocks_check": ([vp] * 4 + [rp, vp] + [i32] * 5 + [vp] * 4, i32),
        "gla_softmax_forward": ([vp] * 4 + [rp, vp] + [i32] * 4 + [vp], i32),
        "gla_softmax_forward_ws": ([vp] * 4 + [rp, vp] + [i32] * 4 + [vp, sz, vp], i32),
        "gla_softmax_workspace_bytes": ([i32] * 4, sz),
        "gla_softmax_forward_check": ([vp] * 4 + [rp, vp] + [i32] * 4, i32),
        "gla_backward": ([vp] * 5 + [rp] + [vp] * 4 + [i32] * 4 + [vp], i32),
        "gla_backward_ws": ([vp] * 5 + [rp] + [vp] * 4 + [i32] * 4 + [vp, sz, vp], i32),
        "gla_backward_workspace_bytes": ([i32] * 4, sz),
        "gla_backward_check": ([vp] * 5 + [rp] + [vp] * 4 + [i32] * 4, i32),
        "gla_backward_saved": ([vp] * 5 + [rp] + [vp] * 6 + [i32] * 4 + [vp], i32),
        "gla_backward_saved_ws": ([vp] * 5 + [rp] + [vp] * 6 + [i32] * 4 + [vp, sz, vp], i32),
        "gla_backward_saved_check": ([vp] * 5 + [rp] + [vp] * 6 + [i32] * 4, i32),
        "gla_forward_proj": ([vp, vp, rp, vp] + [i32] * 5 + [vp], i32),
        "gla_forward_proj_ws": ([vp, vp, rp, vp] + [i32] * 5 + [vp, sz, vp], i32),
        "gla_proj_workspace_bytes": ([i32] * 5, sz),
        "gla_forward_proj_check": ([vp, vp, rp, vp] + [i32] * 5, i32),
        "gla_stream_probe": ([vp, vp, vp, sz, i32, vp], i32),
        "gla_stream_probe_mix": ([ctypes.POINTER(vp), i32, ctypes.POINTER(vp), i32, sz, vp], i32),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    _lib = lib
    return lib


def _ok(code: int, where: str):
    if code != GLA_OK:
        raise GlaError(code, where)


def gla_strerror(code: int) -> str:
    return load_library().gla_strerror(int(code)).decode()


# ---------------------------------------------------------------------------
# RoPE tables


class RopeTables:
    """Owner of a library-built gla_rope_tables descriptor (device memory)."""

    def __init__(self, ptr):
        self._ptr = ptr

    @property
    def ptr(self):
        if self._ptr is None:
            raise ValueError("RoPE tables already destroyed")
        return self._ptr

    @property
    def desc(self) -> gla_rope_tables:
        return self.ptr.contents

    def close(self):
        if self._ptr is not None and _lib is not None:
            _ok(_lib.gla_rope_destroy(self._ptr), "gla_rope_destroy")
        self._ptr = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _stream_handle(stream, device=None):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def gla_rope_table_floats(T: int, Hh: int, W: int, D: int) -> int:
    return load_library().gla_rope_table_floats(T, Hh, W, D)


def gla_rope_fill_host(T, Hh, W, D, theta=10000.0, t0=0, y0=0, x0=0) -> np.ndarray:
    """The (cos, sin) table as the library builds it, on the host (no GPU)."""
    n = gla_rope_table_floats(T, Hh, W, D)
    if n == 0:
        raise GlaError(GLA_ERR_DIM, "gla_rope_fill_host")
    buf = np.empty(n, np.float32)
    _ok(load_library().gla_rope_fill_host(T, Hh, W, D, float(theta), t0, y0, x0,
                                          buf.ctypes.data_as(ctypes.c_void_p), n),
        "gla_rope_fill_host")
    return buf


def gla_rope_create(T, Hh, W, D, theta=10000.0, t0=0, y0=0, x0=0, stream=None) -> RopeTables:
    ptr = ctypes.POINTER(gla_rope_tables)()
    _ok(load_library().gla_rope_create(T, Hh, W, D, float(theta), t0, y0, x0,
                                       _stream_handle(stream), ctypes.byref(ptr)),
        "gla_rope_create")
    return RopeTables(ptr)


def gla_rope_destroy(tables: RopeTables):
    tables.close()


# ---------------------------------------------------------------------------
# forward pass


def _check_bf16(name, t, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
    if t.dim() != 4:
        raise ValueError(f"{name} must be [B, N, H, D], got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _rope_ptr(rope):
    """RopeTables, a raw ctypes pointer to gla_rope_tables, or None (RoPE off)."""
    if rope is None:
        return None
    if isinstance(rope, RopeTables):
        return rope.ptr
    return rope


def gla_workspace_bytes(B: int, N: int, H: int, D: int) -> int:
    return load_library().gla_workspace_bytes(B, N, H, D)


def gla_workspace_release(device=None) -> None:
    """Frees the library-owned workspaces of `device` (default: the current
    one) after synchronising it; later calls allocate new ones.  Not while a
    stream of that device is being captured into a graph."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    with torch.cuda.device(dev):
        _ok(load_library().gla_workspace_release(), "gla_workspace_release")


def alloc_workspace(B: int, N: int, H: int, D: int, device=None) -> torch.Tensor:
    """A torch-owned uint8 device buffer large enough for gla_forward_ws."""
    return torch.empty(max(gla_workspace_bytes(B, N, H, D), 256), dtype=torch.uint8,
                       device=device)


def gla_forward_check(q, k, v, g, rope, out, B, N, H, D) -> int:
    """Status the library's own argument validation gives (no GPU needed).
    Pointers are passed as plain integers here."""
    return load_library().gla_forward_check(q, k, v, g, _rope_ptr(rope), out, B, N, H, D)


def gla_forward(q, k, v, g, rope=None, out=None, stream=None) -> torch.Tensor:
    """out = sigmoid(g) * (R phi(q))^T S / (phi(q).z + eps) per head; bf16 [B, N, H, D]."""
    _check_bf16("q", q)
    for name, t in (("k", k), ("v", v), ("g", g)):
        _check_bf16(name, t, q.shape)
        if t.device != q.device:
            raise ValueError(f"{name} is on {t.device}, q on {q.device}")
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_bf16("out", out, q.shape)
    B, N, H, D = q.shape
    with torch.cuda.device(q.device):
        _ok(load_library().gla_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(),
                                       _rope_ptr(rope), out.data_ptr(), B, N, H, D,
                                       _stream_handle(stream, q.device)),
            "gla_forward")
    return out


def gla_forward_noalloc(q, k, v, g, rope=None, out=None, stream=None) -> torch.Tensor:
    """gla_forward on the library's fixed per-GPU scratch (no device allocation
    by the library).  Calls on one GPU share that scratch: do not overlap them."""
    _check_bf16("q", q)
    for name, t in (("k", k), ("v", v), ("g", g)):
        _check_bf16(name, t, q.shape)
        if t.device != q.device:
            raise ValueError(f"{name} is on {t.device}, q on {q.device}")
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_bf16("out", out, q.shape)
    B, N, H, D = q.shape
    with torch.cuda.device(q.device):
        _ok(load_library().gla_forward_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                               g.data_ptr(), _rope_ptr(rope), out.data_ptr(),
                                               B, N, H, D, _stream_handle(stream, q.device)),
            "gla_forward_noalloc")
    return out


def gla_forward_ws(q, k, v, g, rope, out, ws: torch.Tensor, stream=None) -> torch.Tensor:
    _check_bf16("q", q)
    for name, t in (("k", k), ("v", v), ("g", g), ("out", out)):
        _check_bf16(name, t, q.shape)
    B, N, H, D = q.shape
    with torch.cuda.device(q.device):
        _ok(load_library().gla_forward_ws(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                          g.data_ptr(), _rope_ptr(rope), out.data_ptr(),
                                          B, N, H, D, ws.data_ptr(), ws.numel() * ws.element_size(),
                                          _stream_handle(stream, q.device)),
            "gla_forward_ws")
    return out


def gla_state_ws(k, v, rope, ws: torch.Tensor, stream=None):
    _check_bf16("k", k)
    _check_bf16("v", v, k.shape)
    B, N, H, D = k.shape
    with torch.cuda.device(k.device):
        _ok(load_library().gla_state_ws(k.data_ptr(), v.data_ptr(), _rope_ptr(rope), B, N, H, D,
                                        ws.data_ptr(), ws.numel() * ws.element_size(),
                                        _stream_handle(stream, k.device)),
            "gla_state_ws")


def gla_output_ws(q, g, rope, out, ws: torch.Tensor, stream=None) -> torch.Tensor:
    _check_bf16("q", q)
    _check_bf16("g", g, q.shape)
    _check_bf16("out", out, q.shape)
    B, N, H, D = q.shape
    with torch.cuda.device(q.device):
        _ok(load_library().gla_output_ws(q.data_ptr(), g.data_ptr(), _rope_ptr(rope),
                                         out.data_ptr(), B, N, H, D, ws.data_ptr(),
                                         ws.numel() * ws.element_size(),
                                         _stream_handle(stream, q.device)),
            "gla_output_ws")
    return out


def gla_state(k, v, rope=None, stream=None):
    """(S [B, H, D, D] fp32 with S[d, e], z [B, H, D] fp32) from the state kernels."""
    _check_bf16("k", k)
    _check_bf16("v", v, k.shape)
    B, N, H, D = k.shape
    S = torch.empty((B, H, D, D), dtype=torch.float32, device=k.device)
    z = torch.empty((B, H, D), dtype=torch.float32, device=k.device)
    with torch.cuda.device(k.device):
        _ok(load_library().gla_state(k.data_ptr(), v.data_ptr(), _rope_ptr(rope), S.data_ptr(),
                                     z.data_ptr(), B, N, H, D, _stream_handle(stream, k.device)),
            "gla_state")
    return S, z


# ---------------------------------------------------------------------------
# block-causal pass with a carried state


def _check_state(name, t, shape, device):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or t.dtype != torch.float32:
        raise TypeError(f"{name} must be a float32 torch.Tensor")
    if tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {tuple(shape)} tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, q on {device}")
    return t.data_ptr()


def gla_workspace_bytes_blocks(B: int, N: int, H: int, D: int, block_tokens: int) -> int:
    return load_library().gla_workspace_bytes_blocks(B, N, H, D, block_tokens)


def alloc_workspace_blocks(B, N, H, D, block_tokens, device=None) -> torch.Tensor:
    """A torch-owned uint8 device buffer large enough for gla_forward_blocks_ws."""
    return torch.empty(max(gla_workspace_bytes_blocks(B, N, H, D, block_tokens), 256),
                       dtype=torch.uint8, device=device)


def gla_forward_blocks_check(q, k, v, g, rope, out, B, N, H, D, block_tokens,
                             S_in=None, z_in=None, S_out=None, z_out=None) -> int:
    """Status of the library's argument validation (pointers as integers)."""
    return load_library().gla_forward_blocks_check(q, k, v, g, _rope_ptr(rope), out, B, N, H, D,
                                                   block_tokens, S_in, z_in, S_out, z_out)


def _blocks_args(q, k, v, g, out, S_in, z_in, S_out, z_out):
    _check_bf16("q", q)
    for name, t in (("k", k), ("v", v), ("g", g)):
        _check_bf16(name, t, q.shape)
        if t.device != q.device:
            raise ValueError(f"{name} is on {t.device}, q on {q.device}")
    B, N, H, D = q.shape
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_bf16("out", out, q.shape)
    ptrs = [_check_state("S_in", S_in, (B, H, D, D), q.device),
            _check_state("z_in", z_in, (B, H, D), q.device),
            _check_state("S_out", S_out, (B, H, D, D), q.device),
            _check_state("z_out", z_out, (B, H, D), q.device)]
    return out, ptrs


def gla_forward_blocks(q, k, v, g, rope, block_tokens: int, S_in=None, z_in=None,
                       S_out=None, z_out=None, out=None, stream=None):
    """Block-causal pass: token n of block n // block_tokens sees its own and
    every earlier block plus the carried state (S_in, z_in); the state after
    the last block goes to S_out, z_out (fp32; S_out may be S_in for an
    in-place update).  Returns out (bf16 [B, N, H, D])."""
    out, ptrs = _blocks_args(q, k, v, g, out, S_in, z_in, S_out, z_out)
    B, N, H, D = q.shape
    with torch.cuda.device(q.device):
        _ok(load_library().gla_forward_blocks(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                              g.data_ptr(), _rope_ptr(rope), out.data_ptr(),
                                              B, N, H, D, int(block_tokens), *ptrs,
                                              _stream_handle(stream, q.device)),
            "gla_forward_blocks")
    return out


def gla_forward_blocks_ws(q, k, v, g, rope, block_tokens: int, ws: torch.Tensor, S_in=None,
                          z_in=None, S_out=None, z_out=None, out=None, stream=None):
    out, ptrs = _blocks_args(q, k, v, g, out, S_in, z_in, S_out, z_out)
    B, N, H, D = q.shape
    with torch.cuda.device(q.device):
        _ok(load_library().gla_forward_blocks_ws(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                                 g.data_ptr(), _rope_ptr(rope), out.data_ptr(),
                                                 B, N, H, D, int(block_tokens), *ptrs,
                                                 ws.data_ptr(), ws.numel() * ws.element_size(),
                                                 _stream_handle(stream, q.device)),
            "gla_forward_blocks_ws")
    return out


# ---------------------------------------------------------------------------
# gated softmax anchor attention


def gla_softmax_workspace_bytes(B: int, N: int, H: int, D: int) -> int:
    return load_library().gla_softmax_workspace_bytes(B, N, H, D)


def alloc_workspace_softmax(B, N, H, D, device=None) -> torch.Tensor:
    """A torch-owned uint8 device buffer large enough for gla_softmax_forward_ws."""
    return torch.empty(max(gla_softmax_workspace_bytes(B, N, H, D), 256), dtype=torch.uint8,
                       device=device)


def gla_softmax_forward_check(q, k, v, g, rope, out, B, N, H, D) -> int:
    """Status of the library's argument validation (pointers as integers)."""
    return load_library().gla_softmax_forward_check(q, k, v, g, _rope_ptr(rope), out,
                                                    B, N, H, D)


def _softmax_args(q, k, v, g, out):
    _check_bf16("q", q)
    for name, t in (("k", k), ("v", v), ("g", g)):
        _check_bf16(name, t, q.shape)
        if t.device != q.device:
            raise ValueError(f"{name} is on {t.device}, q on {q.device}")
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_bf16("out", out, q.shape)
    return out


def gla_softmax_forward(q, k, v, g, rope=None, out=None, stream=None) -> torch.Tensor:
    """o = sigmoid(g) * softmax(R q . R k / sqrt(D)) v per head; bf16 [B, N, H, D]."""
    out = _softmax_args(q, k, v, g, out)
    B, N, H, D = q.shape
    with torch.cuda.device(q.device):
        _ok(load_library().gla_softmax_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                               g.data_ptr(), _rope_ptr(rope), out.data_ptr(),
                                               B, N, H, D, _stream_handle(stream, q.device)),
            "gla_softmax_forward")
    return out


def gla_softmax_forward_ws(q, k, v, g, rope, ws: torch.Tensor, out=None, stream=None):
    out = _softmax_args(q, k, v, g, out)
    B, N, H, D = q.shape
    with torch.cuda.device(q.device):
        _ok(load_library().gla_softmax_forward_ws(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                                  g.data_ptr(), _rope_ptr(rope), out.data_ptr(),
                                                  B, N, H, D, ws.data_ptr(),
                                                  ws.numel() * ws.element_size(),
                                                  _stream_handle(stream, q.device)),
            "gla_softmax_forward_ws")
    return out


# ---------------------------------------------------------------------------
# backward pass of the bidirectional mixer


def gla_backward_workspace_bytes(B: int, N: int, H: int, D: int) -> int:
    return load_library().gla_backward_workspace_bytes(B, N, H, D)


def alloc_workspace_backward(B, N, H, D, device=None) -> torch.Tensor:
    """A torch-owned uint8 device buffer large enough for gla_backward_ws."""
    return torch.empty(max(gla_backward_workspace_bytes(B, N, H, D), 256), dtype=torch.uint8,
                       device=device)


def gla_backward_check(q, k, v, g, dout, rope, dq, dk, dv, dg, B, N, H, D) -> int:
    """Status of the library's argument validation (pointers as integers)."""
    return load_library().gla_backward_check(q, k, v, g, dout, _rope_ptr(rope), dq, dk, dv, dg,
                                             B, N, H, D)


def _backward_args(q, k, v, g, dout, grads):
    _check_bf16("q", q)
    for name, t in (("k", k), ("v", v), ("g", g), ("dout", dout)):
        _check_bf16(name, t, q.shape)
        if t.device != q.device:
            raise ValueError(f"{name} is on {t.device}, q on {q.device}")
    out = []
    for name, t in zip(("dq", "dk", "dv", "dg"), grads):
        if t is None:
            t = torch.empty_like(q)
        else:
            _check_bf16(name, t, q.shape)
        out.append(t)
    return out


def gla_backward(q, k, v, g, dout, rope=None, dq=None, dk=None, dv=None, dg=None, stream=None):
    """(dq, dk, dv, dg), bf16 [B, N, H, D]: gradients of the mixer given dout."""
    grads = _backward_args(q, k, v, g, dout, (dq, dk, dv, dg))
    B, N, H, D = q.shape
    with torch.cuda.device(q.device):
        _ok(load_library().gla_backward(q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(),
                                        dout.data_ptr(), _rope_ptr(rope),
                                        *(t.data_ptr() for t in grads), B, N, H, D,
                                        _stream_handle(stream, q.device)),
            "gla_backward")
    return tuple(grads)


def gla_backward_ws(q, k, v, g, dout, rope, ws: torch.Tensor, dq=None, dk=None, dv=None, dg=None,
                    stream=None):
    grads = _backward_args(q, k, v, g, dout, (dq, dk, dv, dg))
    B, N, H, D = q.shape
    with torch.cuda.device(q.device):
        _ok(load_library().gla_backward_ws(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                           g.data_ptr(), dout.data_ptr(), _rope_ptr(rope),
                                           *(t.data_ptr() for t in grads), B, N, H, D,
                                           ws.data_ptr(), ws.numel() * ws.element_size(),
                                           _stream_handle(stream, q.device)),
            "gla_backward_ws")
    return tuple(grads)


def gla_backward_saved_check(q, k, v, g, dout, rope, S, z, dq, dk, dv, dg, B, N, H, D) -> int:
    """Status of the library's argument validation (pointers as integers)."""
    return load_library().gla_backward_saved_check(q, k, v, g, dout, _rope_ptr(rope), S, z, dq,
                                                   dk, dv, dg, B, N, H, D)


def _saved_state_ptrs(q, S, z):
    B, N, H, D = q.shape
    if S is None or z is None:
        raise ValueError("S and z are required (the forward's fp32 state)")
    return (_check_state("S", S, (B, H, D, D), q.device),
            _check_state("z", z, (B, H, D), q.device))


def gla_backward_saved(q, k, v, g, dout, S, z, rope=None, dq=None, dk=None, dv=None, dg=None,
                       stream=None):
    """gla_backward with the forward's fp32 state S [B, H, D, D] and z [B, H, D]
    (S_out and z_out of gla_forward_blocks with block_tokens >= N)."""
    grads = _backward_args(q, k, v, g, dout, (dq, dk, dv, dg))
    sp, zp = _saved_state_ptrs(q, S, z)
    B, N, H, D = q.shape
    with torch.cuda.device(q.device):
        _ok(load_library().gla_backward_saved(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                              g.data_ptr(), dout.data_ptr(), _rope_ptr(rope), sp,
                                              zp, *(t.data_ptr() for t in grads), B, N, H, D,
                                              _stream_handle(stream, q.device)),
            "gla_backward_saved")
    return tuple(grads)


def gla_backward_saved_ws(q, k, v, g, dout, S, z, rope, ws: torch.Tensor, dq=None, dk=None,
                          dv=None, dg=None, stream=None):
    grads = _backward_args(q, k, v, g, dout, (dq, dk, dv, dg))
    sp, zp = _saved_state_ptrs(q, S, z)
    B, N, H, D = q.shape
    with torch.cuda.device(q.device):
        _ok(load_library().gla_backward_saved_ws(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                                 g.data_ptr(), dout.data_ptr(), _rope_ptr(rope),
                                                 sp, zp, *(t.data_ptr() for t in grads), B, N, H,
                                                 D, ws.data_ptr(), ws.numel() * ws.element_size(),
                                                 _stream_handle(stream, q.device)),
            "gla_backward_saved_ws")
    return tuple(grads)


# ---------------------------------------------------------------------------
# projection prologue fused with the mixer


def gla_proj_workspace_bytes(B: int, N: int, C: int, H: int, D: int) -> int:
    return load_library().gla_proj_workspace_bytes(B, N, C, H, D)


def alloc_workspace_proj(B, N, C, H, D, device=None) -> torch.Tensor:
    """A torch-owned uint8 device buffer large enough for gla_forward_proj_ws."""
    return torch.empty(max(gla_proj_workspace_bytes(B, N, C, H, D), 256), dtype=torch.uint8,
                       device=device)


def gla_forward_proj_check(x, w, rope, out, B, N, C, H, D) -> int:
    """Status of the library's argument validation (pointers as integers)."""
    return load_library().gla_forward_proj_check(x, w, _rope_ptr(rope), out, B, N, C, H, D)


def _proj_args(x, w, out):
    for name, t, nd in (("x", x, 3), ("w", w, 3)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16:
            raise TypeError(f"{name} must be a bfloat16 tensor")
        if t.dim() != nd or not t.is_contiguous() or t.device.type != "cuda":
            raise ValueError(f"{name} must be a contiguous {nd}-d GPU tensor")
    B, N, C = x.shape
    if w.shape[0] != 4 or w.shape[2] != C or w.device != x.device:
        raise ValueError(f"w must be [4, H*D, {C}] on {x.device}, got {tuple(w.shape)}")
    return B, N, C


def gla_forward_proj(x, w, H: int, D: int, rope=None, out=None, stream=None) -> torch.Tensor:
    """The mixer on q, k, v, g = bf16(x W^T) per map; x [B, N, C], w [4, H*D, C];
    returns bf16 [B, N, H, D]."""
    B, N, C = _proj_args(x, w, out)
    if out is None:
        out = torch.empty((B, N, H, D), dtype=torch.bfloat16, device=x.device)
    else:
        _check_bf16("out", out, (B, N, H, D))
    with torch.cuda.device(x.device):
        _ok(load_library().gla_forward_proj(x.data_ptr(), w.data_ptr(), _rope_ptr(rope),
                                            out.data_ptr(), B, N, C, H, D,
                                            _stream_handle(stream, x.device)),
            "gla_forward_proj")
    return out


def gla_forward_proj_ws(x, w, H: int, D: int, rope, ws: torch.Tensor, out=None, stream=None):
    B, N, C = _proj_args(x, w, out)
    if out is None:
        out = torch.empty((B, N, H, D), dtype=torch.bfloat16, device=x.device)
    else:
        _check_bf16("out", out, (B, N, H, D))
    with torch.cuda.device(x.device):
        _ok(load_library().gla_forward_proj_ws(x.data_ptr(), w.data_ptr(), _rope_ptr(rope),
                                               out.data_ptr(), B, N, C, H, D, ws.data_ptr(),
                                               ws.numel() * ws.element_size(),
                                               _stream_handle(stream, x.device)),
            "gla_forward_proj_ws")
    return out


# ---------------------------------------------------------------------------
# autograd: the forward keeps its fp32 state for the backward pass


class GatedLinearAttention(torch.autograd.Function):
    """o = mixer(q, k, v, g) with gradients through the library: the forward
    runs gla_forward_blocks over one attention block (the bidirectional mixer)
    and keeps S and z (fp32, B*H*(D*D + D) floats); the backward runs
    gla_backward_saved on them.  rope: RopeTables or None, not differentiated."""

    @staticmethod
    def forward(ctx, q, k, v, g, rope=None):
        B, N, H, D = q.shape
        S = torch.empty((B, H, D, D), dtype=torch.float32, device=q.device)
        z = torch.empty((B, H, D), dtype=torch.float32, device=q.device)
        out = gla_forward_blocks(q, k, v, g, rope, max(N, 1), None, None, S, z)
        ctx.save_for_backward(q, k, v, g, S, z)
        ctx.rope = rope
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v, g, S, z = ctx.saved_tensors
        grads = gla_backward_saved(q, k, v, g, dout.contiguous(), S, z, ctx.rope)
        return (*grads, None)


def gated_linear_attention(q, k, v, g, rope=None) -> torch.Tensor:
    """The mixer as a differentiable torch op (see GatedLinearAttention)."""
    return GatedLinearAttention.apply(q, k, v, g, rope)


def gla_stream_probe(src0: torch.Tensor, src1: torch.Tensor, dst: torch.Tensor, mode: int,
                     stream=None):
    """Streams src0 and src1 (and writes dst in mode 1) through the library's
    bandwidth probe kernel; all three same-sized contiguous device tensors."""
    nbytes = src0.numel() * src0.element_size()
    for t in (src0, src1, dst):
        if t.numel() * t.element_size() != nbytes or not t.is_contiguous():
            raise ValueError("probe buffers must be contiguous and of one size")
    with torch.cuda.device(src0.device):
        _ok(load_library().gla_stream_probe(src0.data_ptr(), src1.data_ptr(), dst.data_ptr(),
                                            nbytes, int(mode), _stream_handle(stream, src0.device)),
            "gla_stream_probe")


def gla_stream_probe_mix(srcs, dsts, stream=None):
    """Streams every tensor of `srcs` (1 to 3) and writes every tensor of
    `dsts` (1 or 2) with their XOR, through the library's bandwidth probe;
    all same-sized contiguous device tensors."""
    bufs = list(srcs) + list(dsts)
    nbytes = bufs[0].numel() * bufs[0].element_size()
    for t in bufs:
        if t.numel() * t.element_size() != nbytes or not t.is_contiguous():
            raise ValueError("probe buffers must be contiguous and of one size")
    vp = ctypes.c_void_p
    sarr = (vp * max(len(srcs), 1))(*[t.data_ptr() for t in srcs])
    darr = (vp * max(len(dsts), 1))(*[t.data_ptr() for t in dsts])
    with torch.cuda.device(bufs[0].device):
        _ok(load_library().gla_stream_probe_mix(sarr, len(srcs), darr, len(dsts), nbytes,
                                                _stream_handle(stream, bufs[0].device)),
            "gla_stream_probe_mix")

"""Python binding of libmmssd.so (C ABI in include/mm_ssd.h).

Argument marshalling only: every function takes torch tensors that already
live on the GPU, passes their data pointers, row strides and the current HIP
stream to the C entry point of the same name, and raises on a non-zero
status.  Outputs and the workspace are allocated with torch (device memory is
plumbing here); every step of the computation runs in the HIP kernels.

There is no fallback: if the shared library is missing the call raises.
Build it with ``python -m selective_state_space_12_amd._build`` (or
``__graft_entry__.build()``).
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmmssd.so")

MM_OK = 0
MM_F32 = 0
MM_BF16 = 1
STATUS = {
    0: "MM_OK", -1: "MM_ERR_NULL", -2: "MM_ERR_SHAPE", -3: "MM_ERR_SLICE",
    -4: "MM_ERR_DTYPE", -5: "MM_ERR_UNSUPPORTED", -6: "MM_ERR_ALIGN",
    -7: "MM_ERR_WORKSPACE", -8: "MM_ERR_HIP",
}

_lock = threading.Lock()
_lib = None

_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
_int = ctypes.c_int


class MMError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: {msg}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libmmssd.so (once).  Raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build it with "
                    "`python -m selective_state_space_12_amd._build`")
            L = ctypes.CDLL(LIB_PATH)
            L.mm_abi_version.argtypes = []
            L.mm_abi_version.restype = _int
            L.mm_status_string.argtypes = [_int]
            L.mm_status_string.restype = ctypes.c_char_p
            L.mm_heads_for_dim.argtypes = [_i64, _i64, _i64, _i64, ctypes.POINTER(_i64)]
            L.mm_heads_for_dim.restype = _int
            L.mm_conv1d_silu.argtypes = [_vp, _i64, _vp, _i64, _vp, _vp, _vp, _i64, _i64,
                                         _i64, _i64, _i64, _i64, _i64, _vp, _int, _vp]
            L.mm_conv1d_silu.restype = _int
            L.mm_ssd_forward_workspace_size.argtypes = [_i64, _i64, _i64, _i64, _i64, _i64,
                                                        _i64, _i64, _int,
                                                        ctypes.POINTER(ctypes.c_size_t)]
            L.mm_ssd_forward_workspace_size.restype = _int
            L.mm_ssd_forward_segments.argtypes = [_i64, _i64, _i64, _i64, _i64, _i64, _i64,
                                                  _i64, _int, ctypes.POINTER(_int)]
            L.mm_ssd_forward_segments.restype = _int
            L.mm_ssd_forward.argtypes = [_vp, _i64, _vp, _i64, _vp, _vp, _i64, _vp, _i64, _vp,
                                         _vp, _i64, _vp, _vp, _i64, _i64, _i64, _i64, _i64,
                                         _i64, _i64, _i64, _int, _vp, ctypes.c_size_t, _vp]
            L.mm_ssd_forward.restype = _int
            L.mm_ssd_forward_nested.argtypes = [_vp, _i64, _vp, _i64, _vp, _vp, _i64, _vp, _i64,
                                                _vp, _vp, _i64, _vp, _vp, _i64, _i64, _i64, _i64,
                                                _i64, _i64, _i64, _i64, _i64, _int, _vp,
                                                ctypes.c_size_t, _vp]
            L.mm_ssd_forward_nested.restype = _int
            L.mm_ssd_forward_noalloc.argtypes = [_vp, _i64, _vp, _i64, _vp, _vp, _i64, _vp, _i64,
                                                 _vp, _vp, _i64, _vp, _vp, _i64, _i64, _i64, _i64,
                                                 _i64, _i64, _i64, _i64, _int, _vp]
            L.mm_ssd_forward_noalloc.restype = _int
            L.mm_ssd_forward_fused_workspace_size.argtypes = [_i64, _i64, _i64, _i64, _i64, _i64,
                                                              _i64, _i64, _int,
                                                              ctypes.POINTER(ctypes.c_size_t)]
            L.mm_ssd_forward_fused_workspace_size.restype = _int
            L.mm_ssd_forward_fused.argtypes = [_vp, _i64, _vp, _vp, _vp, _vp, _i64, _vp, _int, _vp,
                                               _vp, _vp, _i64, _vp, _vp, _i64, _i64, _i64, _i64,
                                               _i64, _i64, _i64, _i64, _int, _vp, ctypes.c_size_t,
                                               _vp]
            L.mm_ssd_forward_fused.restype = _int
            L.mm_ssd_forward_mixed_workspace_size.argtypes = [_i64, _i64, _i64, _i64, _i64, _i64,
                                                              _vp, _i64, _int,
                                                              ctypes.POINTER(ctypes.c_size_t)]
            L.mm_ssd_forward_mixed_workspace_size.restype = _int
            L.mm_ssd_forward_mixed.argtypes = [_vp, _i64, _vp, _i64, _vp, _vp, _i64, _vp, _i64, _vp,
                                               _vp, _i64, _vp, _vp, _i64, _i64, _i64, _i64, _i64,
                                               _i64, _vp, _i64, _int, _vp, ctypes.c_size_t, _vp]
            L.mm_ssd_forward_mixed.restype = _int
            L.mm_ssd_step_multi.argtypes = [_vp, _vp, _vp, _i64, _vp, _i64, _vp, _vp, _i64, _vp,
                                            _i64, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64,
                                            _i64, _i64, _vp, _vp, _int, _vp]
            L.mm_ssd_step_multi.restype = _int
            # state, cs_in, cs_out, xbc, xbcs, w, bias, dt, dts, A, D, y, ys,
            # batch, n_heads, d_head, d_state, ngroups, active, per_seq, dtype, stream
            L.mm_ssd_step_fused.argtypes = [_vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _i64, _vp,
                                            _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _i64,
                                            _vp, _int, _vp]
            L.mm_ssd_step_fused.restype = _int
            L.mm_conv_state_advance.argtypes = [_vp, _vp, _i64, _i64, _i64, _vp, _i64, _i64, _i64,
                                                _i64, _i64, _int, _vp]
            L.mm_conv_state_advance.restype = _int
            L.mm_gated_rmsnorm.argtypes = [_vp, _i64, _vp, _i64, _vp, ctypes.c_float, _vp, _i64,
                                           _i64, _i64, _int, _vp]
            L.mm_gated_rmsnorm.restype = _int
            L.mm_ssd_step.argtypes = [_vp, _vp, _i64, _vp, _i64, _vp, _vp, _i64, _vp, _i64,
                                      _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _i64,
                                      _vp, _int, _vp]
            L.mm_ssd_step.restype = _int
            L.mm_ssd_backward_workspace_size.argtypes = [_i64, _i64, _i64, _i64, _i64, _i64, _i64,
                                                         _int, ctypes.POINTER(ctypes.c_size_t)]
            L.mm_ssd_backward_workspace_size.restype = _int
            L.mm_ssd_backward.argtypes = ([_vp, _i64, _vp, _i64, _vp, _vp, _i64, _vp, _i64, _vp,
                                           _vp, _vp, _i64, _vp, _vp, _i64, _vp, _i64, _vp, _vp,
                                           _i64, _vp, _i64, _vp, _vp] + [_i64] * 7
                                          + [_int, _int, _vp, ctypes.c_size_t, _vp])
            L.mm_ssd_backward.restype = _int
            L.mm_ssd_backward_segments.argtypes = [_i64] * 7 + [_int, ctypes.POINTER(_int)]
            L.mm_ssd_backward_segments.restype = _int
            L.mm_conv1d_silu_backward.argtypes = ([_vp, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _vp,
                                                   _vp, _vp, _vp] + [_i64] * 7
                                                  + [_int, _int, _vp])
            L.mm_conv1d_silu_backward.restype = _int
            _lib = L
    return _lib


def _check(fn: str, status: int) -> None:
    if status != MM_OK:
        msg = lib().mm_status_string(status).decode()
        raise MMError(fn, status, msg)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MM_F32
    if t.dtype == torch.bfloat16:
        return MM_BF16
    raise TypeError(f"unsupported storage dtype {t.dtype} (float32 or bfloat16)")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _row_stride(t: torch.Tensor, name: str, inner: Tuple[int, ...]) -> int:
    """Token-row stride of a (batch, seqlen, *inner) view whose inner block is
    contiguous and whose batches are seqlen rows apart."""
    if t.dim() != 2 + len(inner) or tuple(t.shape[2:]) != tuple(inner):
        raise ValueError(f"{name}: expected shape (batch, seqlen, {inner}), got {tuple(t.shape)}")
    expect = 1
    for d in range(t.dim() - 1, 1, -1):
        if t.shape[d] > 1 and t.stride(d) != expect:
            raise ValueError(f"{name}: inner dimensions must be contiguous")
        expect *= t.shape[d]
    rs = t.stride(1) if t.shape[1] > 1 else (t.stride(0) if t.shape[0] > 1 else expect)
    if t.shape[0] > 1 and t.shape[1] > 1 and t.stride(0) != t.shape[1] * t.stride(1):
        raise ValueError(f"{name}: batches must be seqlen rows apart")
    return rs


def _batch_row_stride(t: torch.Tensor, name: str, inner: Tuple[int, ...]) -> int:
    """Row stride of a (batch, *inner) view of one token per sequence whose
    inner block is contiguous."""
    if tuple(t.shape[1:]) != tuple(inner):
        raise ValueError(f"{name}: expected (batch, {inner}), got {tuple(t.shape)}")
    expect = 1
    for d in range(t.dim() - 1, 0, -1):
        if t.shape[d] > 1 and t.stride(d) != expect:
            raise ValueError(f"{name}: inner dimensions must be contiguous")
        expect *= t.shape[d]
    return t.stride(0) if t.shape[0] > 1 else expect


def abi_version() -> int:
    return lib().mm_abi_version()


def heads_for_dim(d_model: int, d_inner: int, d_head: int, m: int) -> int:
    """h_i for Matryoshka width m (raises MMError on an invalid width)."""
    out = _i64(0)
    _check("mm_heads_for_dim", lib().mm_heads_for_dim(d_model, d_inner, d_head, m, ctypes.byref(out)))
    return out.value


def conv1d_silu(xbc: torch.Tensor, w: torch.Tensor, bias: Optional[torch.Tensor] = None,
                conv_state: Optional[torch.Tensor] = None, *, d_inner: int, d_head: int,
                d_state: int, ngroups: int = 1, n_heads_active: Optional[int] = None,
                heads_per_seq: Optional[torch.Tensor] = None,
                out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Causal depthwise conv (kernel 4) + SiLU on xbc (batch, seqlen, conv_dim)
    -> out (same layout; only active channels written).  conv_state
    (batch, 3, conv_dim) fp32 is read and updated in place."""
    conv_dim = d_inner + 2 * ngroups * d_state
    batch, seqlen = xbc.shape[0], xbc.shape[1]
    n_heads = d_inner // d_head
    h_act = n_heads if n_heads_active is None else int(n_heads_active)
    if out is None:
        out = torch.empty((batch, seqlen, conv_dim), dtype=xbc.dtype, device=xbc.device)
    if out.dtype != xbc.dtype:
        raise TypeError("out must have the input's dtype")
    rs_in = _row_stride(xbc, "xbc", (conv_dim,))
    rs_out = _row_stride(out, "out", (conv_dim,))
    if w.dtype != torch.float32 or not w.is_contiguous() or w.numel() != conv_dim * 4:
        raise ValueError("w must be a contiguous fp32 (conv_dim, 4) tensor")
    if conv_state is not None and (conv_state.dtype != torch.float32 or not conv_state.is_contiguous()
                                   or tuple(conv_state.shape) != (batch, 3, conv_dim)):
        raise ValueError("conv_state must be a contiguous fp32 (batch, 3, conv_dim) tensor")
    if heads_per_seq is not None and (heads_per_seq.dtype != torch.int32 or not heads_per_seq.is_contiguous()):
        raise ValueError("heads_per_seq must be a contiguous int32 tensor")
    st = lib().mm_conv1d_silu(_ptr(xbc), rs_in, _ptr(out), rs_out, _ptr(w), _ptr(bias),
                              _ptr(conv_state), batch, seqlen, d_inner, d_head, d_state,
                              ngroups, h_act, _ptr(heads_per_seq), _dtype_code(xbc), _stream())
    _check("mm_conv1d_silu", st)
    return out


def ssd_forward_workspace_size(batch: int, seqlen: int, n_heads: int, d_head: int,
                               d_state: int, ngroups: int, n_heads_active: int, chunk: int,
                               dtype: torch.dtype) -> int:
    out = ctypes.c_size_t(0)
    code = MM_F32 if dtype == torch.float32 else MM_BF16
    _check("mm_ssd_forward_workspace_size",
           lib().mm_ssd_forward_workspace_size(batch, seqlen, n_heads, d_head, d_state, ngroups,
                                               n_heads_active, chunk, code, ctypes.byref(out)))
    return out.value


def ssd_forward_segments(batch: int, seqlen: int, n_heads: int, d_head: int, d_state: int,
                         ngroups: int, n_heads_active: int, chunk: int,
                         dtype: torch.dtype) -> int:
    out = _int(0)
    code = MM_F32 if dtype == torch.float32 else MM_BF16
    _check("mm_ssd_forward_segments",
           lib().mm_ssd_forward_segments(batch, seqlen, n_heads, d_head, d_state, ngroups,
                                         n_heads_active, chunk, code, ctypes.byref(out)))
    return out.value


def ssd_forward(x: torch.Tensor, dt: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
                C: torch.Tensor, D: Optional[torch.Tensor] = None, *,
                n_heads_active: Optional[int] = None, chunk: int = 256,
                initial_state: Optional[torch.Tensor] = None,
                final_state: Optional[torch.Tensor] = None,
                y: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None,
                plan_heads: Optional[int] = None) -> torch.Tensor:
    """Chunked selective scan over heads [0, n_heads_active).

    x (batch, seqlen, n_heads, d_head), dt (batch, seqlen, n_heads),
    B, C (batch, seqlen, ngroups, d_state) -- each may be a strided view
    whose token rows are wider (e.g. column ranges of the conv output).
    Returns y: the given buffer (batch, seqlen, n_heads, d_head) with the
    active prefix written, or a new (batch, seqlen, n_heads_active, d_head)
    tensor.  final_state (batch, n_heads, d_head, d_state) fp32, if given, is
    written for the active heads.  plan_heads (mm_ssd_forward_nested): cut
    the sequences as for that many active heads, so that calls with the same
    plan_heads agree bit for bit on their common heads."""
    batch, seqlen, n_heads, d_head = x.shape
    if B.dim() == 3:
        B = B.unsqueeze(2)
        C = C.unsqueeze(2)
    ngroups, d_state = B.shape[2], B.shape[3]
    h_act = n_heads if n_heads_active is None else int(n_heads_active)
    if y is None:
        y = torch.empty((batch, seqlen, h_act, d_head), dtype=x.dtype, device=x.device)
    code = _dtype_code(x)
    for name, t in (("dt", dt), ("B", B), ("C", C), ("y", y)):
        if t.dtype != x.dtype:
            raise TypeError(f"{name} must have x's dtype")
    xs = _row_stride(x, "x", (n_heads, d_head))
    ys = _row_stride(y, "y", (y.shape[2], d_head))
    dts = _row_stride(dt, "dt", (n_heads,))
    bs = _row_stride(B, "B", (ngroups, d_state))
    cs = _row_stride(C, "C", (ngroups, d_state))
    for name, t in (("A", A), ("D", D), ("initial_state", initial_state), ("final_state", final_state)):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous fp32 tensor")
    need = ssd_forward_workspace_size(batch, seqlen, n_heads, d_head, d_state, ngroups,
                                      h_act if plan_heads is None else int(plan_heads), chunk,
                                      x.dtype)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if plan_heads is None:
        st = lib().mm_ssd_forward(_ptr(x), xs, _ptr(dt), dts, _ptr(A), _ptr(B), bs, _ptr(C), cs,
                                  _ptr(D), _ptr(y), ys, _ptr(initial_state), _ptr(final_state),
                                  batch, seqlen, n_heads, d_head, d_state, ngroups, h_act, chunk,
                                  code, _ptr(workspace), wbytes, _stream())
        _check("mm_ssd_forward", st)
    else:
        st = lib().mm_ssd_forward_nested(_ptr(x), xs, _ptr(dt), dts, _ptr(A), _ptr(B), bs, _ptr(C),
                                         cs, _ptr(D), _ptr(y), ys, _ptr(initial_state),
                                         _ptr(final_state), batch, seqlen, n_heads, d_head, d_state,
                                         ngroups, h_act, int(plan_heads), chunk, code,
                                         _ptr(workspace), wbytes, _stream())
        _check("mm_ssd_forward_nested", st)
    return y


def ssd_forward_noalloc(x: torch.Tensor, dt: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
                        C: torch.Tensor, D: Optional[torch.Tensor] = None, *,
                        n_heads_active: Optional[int] = None, chunk: int = 256,
                        initial_state: Optional[torch.Tensor] = None,
                        final_state: Optional[torch.Tensor] = None,
                        y: torch.Tensor) -> torch.Tensor:
    """ssd_forward through mm_ssd_forward_noalloc: no workspace argument and
    no device allocation anywhere in the call (the library's fixed device
    array serves as workspace), so ``y`` must be given.  Same layouts as
    ssd_forward."""
    batch, seqlen, n_heads, d_head = x.shape
    if B.dim() == 3:
        B = B.unsqueeze(2)
        C = C.unsqueeze(2)
    ngroups, d_state = B.shape[2], B.shape[3]
    h_act = n_heads if n_heads_active is None else int(n_heads_active)
    code = _dtype_code(x)
    for name, t in (("dt", dt), ("B", B), ("C", C), ("y", y)):
        if t.dtype != x.dtype:
            raise TypeError(f"{name} must have x's dtype")
    xs = _row_stride(x, "x", (n_heads, d_head))
    ys = _row_stride(y, "y", (y.shape[2], d_head))
    dts = _row_stride(dt, "dt", (n_heads,))
    bs = _row_stride(B, "B", (ngroups, d_state))
    cs = _row_stride(C, "C", (ngroups, d_state))
    for name, t in (("A", A), ("D", D), ("initial_state", initial_state), ("final_state", final_state)):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous fp32 tensor")
    st = lib().mm_ssd_forward_noalloc(_ptr(x), xs, _ptr(dt), dts, _ptr(A), _ptr(B), bs, _ptr(C),
                                      cs, _ptr(D), _ptr(y), ys, _ptr(initial_state),
                                      _ptr(final_state), batch, seqlen, n_heads, d_head, d_state,
                                      ngroups, h_act, chunk, code, _stream())
    _check("mm_ssd_forward_noalloc", st)
    return y


def conv1d_silu_backward(xbc: torch.Tensor, w: torch.Tensor, dout: torch.Tensor,
                         bias: Optional[torch.Tensor] = None,
                         conv_state: Optional[torch.Tensor] = None, *, d_inner: int, d_head: int,
                         d_state: int, ngroups: int = 1, n_heads_active: Optional[int] = None,
                         grads: Optional[dict] = None, accumulate: bool = False,
                         want_dbias: bool = False, want_dstate: bool = False) -> dict:
    """Gradients of sum(dout * conv1d_silu(xbc)) for the active channels:
    dxbc (like xbc), dw (conv_dim, 4) fp32 and, if asked, dbias (conv_dim)
    and dconv_state (batch, 3, conv_dim) fp32.  conv_state is the history the
    forward read (its value before the forward's in-place update).  `grads`
    may hold any of these buffers to write (or, with accumulate=True, add)
    into."""
    batch, seqlen, width = xbc.shape
    conv_dim = d_inner + 2 * ngroups * d_state
    h_act = d_inner // d_head if n_heads_active is None else int(n_heads_active)
    dev = xbc.device
    g = dict(grads or {})
    if "dxbc" not in g:
        g["dxbc"] = torch.empty((batch, seqlen, conv_dim), dtype=xbc.dtype, device=dev)
    if "dw" not in g:
        g["dw"] = torch.empty((conv_dim, 4), dtype=torch.float32, device=dev)
    if want_dbias and "dbias" not in g:
        g["dbias"] = torch.empty(conv_dim, dtype=torch.float32, device=dev)
    if want_dstate and "dconv_state" not in g:
        g["dconv_state"] = torch.empty((batch, 3, conv_dim), dtype=torch.float32, device=dev)
    for name, t in (("dout", dout), ("dxbc", g["dxbc"])):
        if t.dtype != xbc.dtype:
            raise TypeError(f"{name} must have xbc's dtype")
    xs = _row_stride(xbc, "xbc", (width,))
    ds = _row_stride(dout, "dout", (dout.shape[2],))
    gs = _row_stride(g["dxbc"], "dxbc", (g["dxbc"].shape[2],))
    for name, t in (("w", w), ("bias", bias), ("conv_state", conv_state), ("dw", g["dw"]),
                    ("dbias", g.get("dbias")), ("dconv_state", g.get("dconv_state"))):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous fp32 tensor")
    st = lib().mm_conv1d_silu_backward(_ptr(xbc), xs, _ptr(dout), ds, _ptr(g["dxbc"]), gs,
                                       _ptr(w), _ptr(bias), _ptr(conv_state), _ptr(g["dw"]),
                                       _ptr(g.get("dbias")), _ptr(g.get("dconv_state")), batch,
                                       seqlen, d_inner, d_head, d_state, ngroups, h_act,
                                       _dtype_code(xbc), int(bool(accumulate)), _stream())
    _check("mm_conv1d_silu_backward", st)
    return g


def ssd_backward_workspace_size(batch: int, seqlen: int, n_heads: int, d_head: int,
                                d_state: int, ngroups: int, n_heads_active: int,
                                dtype: torch.dtype) -> int:
    out = ctypes.c_size_t(0)
    code = MM_F32 if dtype == torch.float32 else MM_BF16
    _check("mm_ssd_backward_workspace_size",
           lib().mm_ssd_backward_workspace_size(batch, seqlen, n_heads, d_head, d_state, ngroups,
                                                n_heads_active, code, ctypes.byref(out)))
    return out.value


def ssd_backward_segments(batch: int, seqlen: int, n_heads: int, d_head: int, d_state: int,
                          ngroups: int, n_heads_active: int, dtype: torch.dtype) -> int:
    out = _int(0)
    code = MM_F32 if dtype == torch.float32 else MM_BF16
    _check("mm_ssd_backward_segments",
           lib().mm_ssd_backward_segments(batch, seqlen, n_heads, d_head, d_state, ngroups,
                                          n_heads_active, code, ctypes.byref(out)))
    return out.value


def ssd_backward(x: torch.Tensor, dt: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
                 C: torch.Tensor, D: Optional[torch.Tensor], dy: torch.Tensor, *,
                 n_heads_active: Optional[int] = None,
                 initial_state: Optional[torch.Tensor] = None,
                 dfinal_state: Optional[torch.Tensor] = None,
                 grads: Optional[dict] = None, accumulate: bool = False,
                 want_dD: bool = True, want_dinitial: bool = False,
                 workspace: Optional[torch.Tensor] = None) -> dict:
    """Gradients of sum(dy * y) + sum(dfinal_state * final_state) for
    ssd_forward over heads [0, n_heads_active).  Inputs as ssd_forward; dy
    like y (batch, seqlen, n_heads or n_heads_active, d_head).  Returns a dict
    of dx, ddt (x's dtype, shaped like x and dt: inactive heads of a new
    tensor are uninitialised), dA, dD (n_heads fp32), dB, dC (batch, seqlen,
    ngroups, d_state fp32) and dinitial_state (batch, n_heads, d_head,
    d_state fp32) if asked.  `grads` may hold any of these buffers to write
    (or, with accumulate=True, add) into."""
    batch, seqlen, n_heads, d_head = x.shape
    if B.dim() == 3:
        B = B.unsqueeze(2)
        C = C.unsqueeze(2)
    ngroups, d_state = B.shape[2], B.shape[3]
    h_act = n_heads if n_heads_active is None else int(n_heads_active)
    code = _dtype_code(x)
    dev = x.device
    g = dict(grads or {})
    if "dx" not in g:
        g["dx"] = torch.empty((batch, seqlen, n_heads, d_head), dtype=x.dtype, device=dev)
    if "ddt" not in g:
        g["ddt"] = torch.empty((batch, seqlen, n_heads), dtype=x.dtype, device=dev)
    for k, shape in (("dA", (n_heads,)), ("dB", (batch, seqlen, ngroups, d_state)),
                     ("dC", (batch, seqlen, ngroups, d_state))):
        if k not in g:
            g[k] = torch.empty(shape, dtype=torch.float32, device=dev)
    if want_dD and "dD" not in g:
        g["dD"] = torch.empty(n_heads, dtype=torch.float32, device=dev)
    if want_dinitial and "dinitial_state" not in g:
        g["dinitial_state"] = torch.empty((batch, n_heads, d_head, d_state), dtype=torch.float32,
                                          device=dev)
    for name, t in (("dt", dt), ("B", B), ("C", C), ("dy", dy), ("dx", g["dx"]),
                    ("ddt", g["ddt"])):
        if t.dtype != x.dtype:
            raise TypeError(f"{name} must have x's dtype")
    xs = _row_stride(x, "x", (n_heads, d_head))
    dys = _row_stride(dy, "dy", (dy.shape[2], d_head))
    dxs = _row_stride(g["dx"], "dx", (g["dx"].shape[2], d_head))
    dts = _row_stride(dt, "dt", (n_heads,))
    ddts = _row_stride(g["ddt"], "ddt", (g["ddt"].shape[2],))
    bs = _row_stride(B, "B", (ngroups, d_state))
    cs = _row_stride(C, "C", (ngroups, d_state))
    dbs = _row_stride(g["dB"], "dB", (ngroups, d_state))
    dcs = _row_stride(g["dC"], "dC", (ngroups, d_state))
    for name, t in (("A", A), ("D", D), ("initial_state", initial_state),
                    ("dfinal_state", dfinal_state), ("dA", g["dA"]), ("dB", g["dB"]),
                    ("dC", g["dC"]), ("dD", g.get("dD")), ("dinitial_state", g.get("dinitial_state"))):
        if t is not None and t.dtype != torch.float32:
            raise ValueError(f"{name} must be fp32")
    for name, t in (("A", A), ("D", D), ("initial_state", initial_state),
                    ("dfinal_state", dfinal_state), ("dA", g["dA"]), ("dD", g.get("dD")),
                    ("dinitial_state", g.get("dinitial_state"))):
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    need = ssd_backward_workspace_size(batch, seqlen, n_heads, d_head, d_state, ngroups, h_act,
                                       x.dtype)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wbytes = workspace.numel() * workspace.element_size()
    st = lib().mm_ssd_backward(_ptr(x), xs, _ptr(dt), dts, _ptr(A), _ptr(B), bs, _ptr(C), cs,
                               _ptr(D), _ptr(initial_state), _ptr(dy), dys, _ptr(dfinal_state),
                               _ptr(g["dx"]), dxs, _ptr(g["ddt"]), ddts, _ptr(g["dA"]),
                               _ptr(g["dB"]), dbs, _ptr(g["dC"]), dcs, _ptr(g.get("dD")),
                               _ptr(g.get("dinitial_state")), batch, seqlen, n_heads, d_head,
                               d_state, ngroups, h_act, code, int(bool(accumulate)),
                               _ptr(workspace), wbytes, _stream())
    _check("mm_ssd_backward", st)
    return g


def _host_heads(heads_per_seq, batch: int):
    """Per-sequence head counts as a host int32 array (kept alive by the caller)."""
    if len(heads_per_seq) != batch:
        raise ValueError(f"heads_per_seq must have {batch} entries")
    return (ctypes.c_int32 * batch)(*[int(v) for v in heads_per_seq])


def ssd_forward_mixed_workspace_size(batch: int, seqlen: int, n_heads: int, d_head: int,
                                     d_state: int, ngroups: int, heads_per_seq, chunk: int,
                                     dtype: torch.dtype) -> int:
    out = ctypes.c_size_t(0)
    code = MM_F32 if dtype == torch.float32 else MM_BF16
    hp = _host_heads(heads_per_seq, batch)
    _check("mm_ssd_forward_mixed_workspace_size",
           lib().mm_ssd_forward_mixed_workspace_size(batch, seqlen, n_heads, d_head, d_state,
                                                     ngroups, ctypes.cast(hp, ctypes.c_void_p),
                                                     chunk, code, ctypes.byref(out)))
    return out.value


def ssd_forward_mixed(x: torch.Tensor, dt: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
                      C: torch.Tensor, D: Optional[torch.Tensor] = None, *, heads_per_seq,
                      chunk: int = 256, initial_state: Optional[torch.Tensor] = None,
                      final_state: Optional[torch.Tensor] = None,
                      y: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """ssd_forward with a width per sequence: sequence b runs heads
    [0, heads_per_seq[b]) (a list or CPU tensor of ints).  Returns y
    (batch, seqlen, n_heads, d_head) -- the given buffer, or a new one whose
    inactive heads are uninitialised."""
    batch, seqlen, n_heads, d_head = x.shape
    if B.dim() == 3:
        B = B.unsqueeze(2)
        C = C.unsqueeze(2)
    ngroups, d_state = B.shape[2], B.shape[3]
    hps = [int(v) for v in (heads_per_seq.tolist() if torch.is_tensor(heads_per_seq)
                            else heads_per_seq)]
    hp = _host_heads(hps, batch)
    if y is None:
        y = torch.empty((batch, seqlen, n_heads, d_head), dtype=x.dtype, device=x.device)
    code = _dtype_code(x)
    for name, t in (("dt", dt), ("B", B), ("C", C), ("y", y)):
        if t.dtype != x.dtype:
            raise TypeError(f"{name} must have x's dtype")
    xs = _row_stride(x, "x", (n_heads, d_head))
    ys = _row_stride(y, "y", (y.shape[2], d_head))
    dts = _row_stride(dt, "dt", (n_heads,))
    bs = _row_stride(B, "B", (ngroups, d_state))
    cs = _row_stride(C, "C", (ngroups, d_state))
    for name, t in (("A", A), ("D", D), ("initial_state", initial_state), ("final_state", final_state)):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous fp32 tensor")
    need = ssd_forward_mixed_workspace_size(batch, seqlen, n_heads, d_head, d_state, ngroups, hps,
                                            chunk, x.dtype)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().mm_ssd_forward_mixed(_ptr(x), xs, _ptr(dt), dts, _ptr(A), _ptr(B), bs, _ptr(C), cs,
                                    _ptr(D), _ptr(y), ys, _ptr(initial_state), _ptr(final_state),
                                    batch, seqlen, n_heads, d_head, d_state, ngroups,
                                    ctypes.cast(hp, ctypes.c_void_p), chunk, code, _ptr(workspace),
                                    wbytes, _stream())
    _check("mm_ssd_forward_mixed", st)
    return y


def ssd_forward_fused_workspace_size(batch: int, seqlen: int, n_heads: int, d_head: int,
                                     d_state: int, ngroups: int, n_heads_active: int, chunk: int,
                                     dtype: torch.dtype) -> int:
    out = ctypes.c_size_t(0)
    code = MM_F32 if dtype == torch.float32 else MM_BF16
    _check("mm_ssd_forward_fused_workspace_size",
           lib().mm_ssd_forward_fused_workspace_size(batch, seqlen, n_heads, d_head, d_state,
                                                     ngroups, n_heads_active, chunk, code,
                                                     ctypes.byref(out)))
    return out.value


def ssd_forward_fused(xbc: torch.Tensor, conv_w: torch.Tensor, dt: torch.Tensor, A: torch.Tensor,
                      D: Optional[torch.Tensor] = None, *, d_head: int, d_state: int,
                      ngroups: int = 1, conv_bias: Optional[torch.Tensor] = None,
                      conv_state: Optional[torch.Tensor] = None,
                      dt_bias: Optional[torch.Tensor] = None, dt_softplus: bool = False,
                      n_heads_active: Optional[int] = None, chunk: int = 256,
                      initial_state: Optional[torch.Tensor] = None,
                      final_state: Optional[torch.Tensor] = None,
                      y: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Conv1d (kernel 4) + SiLU, dt transform and chunked scan in one call, on
    the raw conv input xbc (batch, seqlen, conv_dim) with conv_dim =
    n_heads*d_head + 2*ngroups*d_state; dt (batch, seqlen, n_heads) is the raw
    dt (dt_bias added, then softplus if dt_softplus).  conv_state
    (batch, 3, conv_dim) fp32, if given, is read and rolled in place.  Returns
    y as ssd_forward does."""
    batch, seqlen, n_heads = dt.shape
    conv_dim = n_heads * d_head + 2 * ngroups * d_state
    h_act = n_heads if n_heads_active is None else int(n_heads_active)
    if y is None:
        y = torch.empty((batch, seqlen, h_act, d_head), dtype=xbc.dtype, device=xbc.device)
    code = _dtype_code(xbc)
    for name, t in (("dt", dt), ("y", y)):
        if t.dtype != xbc.dtype:
            raise TypeError(f"{name} must have xbc's dtype")
    xs = _row_stride(xbc, "xbc", (conv_dim,))
    ys = _row_stride(y, "y", (y.shape[2], d_head))
    dts = _row_stride(dt, "dt", (n_heads,))
    if conv_w.dtype != torch.float32 or not conv_w.is_contiguous() or conv_w.numel() != conv_dim * 4:
        raise ValueError("conv_w must be a contiguous fp32 (conv_dim, 4) tensor")
    if conv_state is not None and (conv_state.dtype != torch.float32 or not conv_state.is_contiguous()
                                   or tuple(conv_state.shape) != (batch, 3, conv_dim)):
        raise ValueError("conv_state must be a contiguous fp32 (batch, 3, conv_dim) tensor")
    for name, t in (("A", A), ("D", D), ("conv_bias", conv_bias), ("dt_bias", dt_bias),
                    ("initial_state", initial_state), ("final_state", final_state)):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous fp32 tensor")
    need = ssd_forward_fused_workspace_size(batch, seqlen, n_heads, d_head, d_state, ngroups,
                                            h_act, chunk, xbc.dtype)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=xbc.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().mm_ssd_forward_fused(_ptr(xbc), xs, _ptr(conv_w), _ptr(conv_bias), _ptr(conv_state),
                                    _ptr(dt), dts, _ptr(dt_bias), int(bool(dt_softplus)), _ptr(A),
                                    _ptr(D), _ptr(y), ys, _ptr(initial_state), _ptr(final_state),
                                    batch, seqlen, n_heads, d_head, d_state, ngroups, h_act, chunk,
                                    code, _ptr(workspace), wbytes, _stream())
    _check("mm_ssd_forward_fused", st)
    return y


def gated_rmsnorm(y: torch.Tensor, z: torch.Tensor, w: torch.Tensor, eps: float = 1e-5, *,
                  d: Optional[int] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out = (y * SiLU(z)) * w / sqrt(mean((y * SiLU(z))^2) + eps) over the
    first d channels of every row.  y, z: (..., width) with contiguous rows of
    width >= d (views of wider rows allowed: the rows may be strided); w fp32.
    Returns out (..., d) (or writes the given out, which may be y)."""
    width = y.shape[-1]
    d = width if d is None else int(d)

    def rows_of(t, name):
        """(rows, row stride) of a (..., width) tensor whose leading
        dimensions collapse to evenly strided rows of unit-stride values."""
        if t.shape[-1] < d or (t.shape[-1] > 1 and t.stride(-1) != 1):
            raise ValueError(f"{name}: rows must be unit-stride with at least d={d} values")
        if t.dim() == 1:
            return 1, t.shape[-1]
        rs = t.stride(-2)
        for k in range(t.dim() - 3, -1, -1):
            if t.shape[k] > 1 and t.stride(k) != t.stride(k + 1) * t.shape[k + 1]:
                raise ValueError(f"{name}: leading dimensions must collapse to evenly strided rows")
        n = 1
        for v in t.shape[:-1]:
            n *= v
        return n, (rs if n > 1 else t.shape[-1])

    rows, ys = rows_of(y, "y")
    rz, zs = rows_of(z, "z")
    if rz != rows or z.dtype != y.dtype:
        raise ValueError("z must have y's rows and dtype")
    if out is None:
        out = torch.empty(tuple(y.shape[:-1]) + (d,), dtype=y.dtype, device=y.device)
    ro, os_ = rows_of(out, "out")
    if ro != rows or out.dtype != y.dtype:
        raise ValueError("out must have y's rows and dtype")
    if w.dtype != torch.float32 or not w.is_contiguous() or w.numel() < d:
        raise ValueError("w must be a contiguous fp32 tensor of at least d values")
    st = lib().mm_gated_rmsnorm(_ptr(y), ys, _ptr(z), zs, _ptr(w), float(eps), _ptr(out), os_,
                                rows, d, _dtype_code(y), _stream())
    _check("mm_gated_rmsnorm", st)
    return out


def _dev_i32(t: Optional[torch.Tensor], name: str):
    if t is not None and (t.dtype != torch.int32 or not t.is_contiguous() or t.device.type != "cuda"):
        raise ValueError(f"{name} must be a contiguous int32 device tensor")
    return _ptr(t)


def ssd_step_multi(state: torch.Tensor, x: torch.Tensor, dt: torch.Tensor, A: torch.Tensor,
                   B: torch.Tensor, C: torch.Tensor, D: Optional[torch.Tensor] = None, *,
                   state_out: Optional[torch.Tensor] = None,
                   n_heads_active: Optional[int] = None,
                   heads_per_seq: Optional[torch.Tensor] = None,
                   tokens_per_seq: Optional[torch.Tensor] = None,
                   y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """ntok decode tokens per sequence in one pass over the states.  x
    (batch, ntok, n_heads, d_head), dt (batch, ntok, n_heads), B, C
    (batch, ntok, [ngroups,] d_state).  state (batch, n_heads, d_head,
    d_state) fp32 is read; the advanced state goes to state_out (pass the
    state itself to update it in place; None: outputs only).  Returns y
    (batch, ntok, n_heads, d_head); rows past a sequence's token count and
    inactive heads are left untouched."""
    batch, n_heads, d_head, d_state = state.shape
    ntok = x.shape[1]
    if B.dim() == 3:
        B = B.unsqueeze(2)
        C = C.unsqueeze(2)
    ngroups = B.shape[2]
    h_act = n_heads if n_heads_active is None else int(n_heads_active)
    if y is None:
        y = torch.empty((batch, ntok, n_heads, d_head), dtype=x.dtype, device=x.device)
    for name, t in (("state", state), ("state_out", state_out)):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous fp32 tensor")
    xs = _row_stride(x, "x", (n_heads, d_head))
    ys = _row_stride(y, "y", (n_heads, d_head))
    dts = _row_stride(dt, "dt", (n_heads,))
    bs = _row_stride(B, "B", (ngroups, d_state))
    cs = _row_stride(C, "C", (ngroups, d_state))
    st = lib().mm_ssd_step_multi(_ptr(state), _ptr(state_out), _ptr(x), xs, _ptr(dt), dts, _ptr(A),
                                 _ptr(B), bs, _ptr(C), cs, _ptr(D), _ptr(y), ys, batch, ntok,
                                 n_heads, d_head, d_state, ngroups, h_act,
                                 _dev_i32(heads_per_seq, "heads_per_seq"),
                                 _dev_i32(tokens_per_seq, "tokens_per_seq"), _dtype_code(x),
                                 _stream())
    _check("mm_ssd_step_multi", st)
    return y


def conv_state_advance(conv_state: torch.Tensor, xbc: torch.Tensor, *, d_inner: int, d_head: int,
                       d_state: int, ngroups: int = 1, n_heads_active: Optional[int] = None,
                       tokens_per_seq: Optional[torch.Tensor] = None) -> torch.Tensor:
    """conv_state (batch, 3, conv_dim) fp32 advanced in place by each
    sequence's first tokens of xbc (batch, ntok, conv_dim) raw conv input."""
    batch, ntok = xbc.shape[0], xbc.shape[1]
    conv_dim = d_inner + 2 * ngroups * d_state
    if conv_state.dtype != torch.float32 or not conv_state.is_contiguous() or \
            tuple(conv_state.shape) != (batch, 3, conv_dim):
        raise ValueError("conv_state must be a contiguous fp32 (batch, 3, conv_dim) tensor")
    xs = _row_stride(xbc, "xbc", (conv_dim,))
    h_act = d_inner // d_head if n_heads_active is None else int(n_heads_active)
    st = lib().mm_conv_state_advance(_ptr(conv_state), _ptr(xbc), xs, batch, ntok,
                                     _dev_i32(tokens_per_seq, "tokens_per_seq"), d_inner, d_head,
                                     d_state, ngroups, h_act, _dtype_code(xbc), _stream())
    _check("mm_conv_state_advance", st)
    return conv_state


def ssd_step(state: torch.Tensor, x_t: torch.Tensor, dt_t: torch.Tensor, A: torch.Tensor,
             B_t: torch.Tensor, C_t: torch.Tensor, D: Optional[torch.Tensor] = None, *,
             n_heads_active: Optional[int] = None,
             heads_per_seq: Optional[torch.Tensor] = None,
             y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One decode token, in place on state (batch, n_heads, d_head, d_state)
    fp32.  x_t (batch, n_heads, d_head), dt_t (batch, n_heads),
    B_t, C_t (batch, ngroups, d_state) -- rows may be strided.  Returns y_t
    (batch, n_heads, d_head); inactive heads are left untouched."""
    batch, n_heads, d_head, d_state = state.shape
    if B_t.dim() == 2:
        B_t = B_t.unsqueeze(1)
        C_t = C_t.unsqueeze(1)
    ngroups = B_t.shape[1]
    h_act = n_heads if n_heads_active is None else int(n_heads_active)
    if y is None:
        y = torch.empty((batch, n_heads, d_head), dtype=x_t.dtype, device=x_t.device)
    if state.dtype != torch.float32 or not state.is_contiguous():
        raise ValueError("state must be a contiguous fp32 tensor")

    xs = _batch_row_stride(x_t, "x_t", (n_heads, d_head))
    ys = _batch_row_stride(y, "y", (n_heads, d_head))
    dts = _batch_row_stride(dt_t, "dt_t", (n_heads,))
    bs = _batch_row_stride(B_t, "B_t", (ngroups, d_state))
    cs = _batch_row_stride(C_t, "C_t", (ngroups, d_state))
    if heads_per_seq is not None and (heads_per_seq.dtype != torch.int32 or not heads_per_seq.is_contiguous()):
        raise ValueError("heads_per_seq must be a contiguous int32 tensor")
    st = lib().mm_ssd_step(_ptr(state), _ptr(x_t), xs, _ptr(dt_t), dts, _ptr(A), _ptr(B_t), bs,
                           _ptr(C_t), cs, _ptr(D), _ptr(y), ys, batch, n_heads, d_head, d_state,
                           ngroups, h_act, _ptr(heads_per_seq), _dtype_code(x_t), _stream())
    _check("mm_ssd_step", st)
    return y


def ssd_step_fused(state: torch.Tensor, conv_state_in: torch.Tensor, conv_state_out: torch.Tensor,
                   xbc_t: torch.Tensor, conv_w: torch.Tensor, dt_t: torch.Tensor, A: torch.Tensor,
                   D: Optional[torch.Tensor] = None, conv_bias: Optional[torch.Tensor] = None, *,
                   n_heads_active: Optional[int] = None,
                   heads_per_seq: Optional[torch.Tensor] = None,
                   y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One decode token with the conv folded in (mm_ssd_step_fused): the
    token's raw [x | B | C] row xbc_t (batch, conv_dim); the conv history is
    read from conv_state_in and the advanced one written to conv_state_out
    (both (batch, 3, conv_dim) fp32, disjoint); state (batch, n_heads, d_head,
    d_state) fp32 is updated in place.  Returns y_t (batch, n_heads, d_head)."""
    batch, n_heads, d_head, d_state = state.shape
    conv_dim = n_heads * d_head + 2 * d_state
    h_act = n_heads if n_heads_active is None else int(n_heads_active)
    if state.dtype != torch.float32 or not state.is_contiguous():
        raise ValueError("state must be a contiguous fp32 tensor")
    for name, t in (("conv_state_in", conv_state_in), ("conv_state_out", conv_state_out)):
        if t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != (batch, 3, conv_dim):
            raise ValueError(f"{name} must be a contiguous fp32 (batch, 3, conv_dim) tensor")
    if conv_w.dtype != torch.float32 or not conv_w.is_contiguous() or conv_w.numel() != conv_dim * 4:
        raise ValueError("conv_w must be a contiguous fp32 (conv_dim, 4) tensor")
    if y is None:
        y = torch.empty((batch, n_heads, d_head), dtype=xbc_t.dtype, device=xbc_t.device)
    xs = _batch_row_stride(xbc_t, "xbc_t", (conv_dim,))
    ys = _batch_row_stride(y, "y", (n_heads, d_head))
    dts = _batch_row_stride(dt_t, "dt_t", (n_heads,))
    if heads_per_seq is not None and (heads_per_seq.dtype != torch.int32 or not heads_per_seq.is_contiguous()):
        raise ValueError("heads_per_seq must be a contiguous int32 tensor")
    st = lib().mm_ssd_step_fused(_ptr(state), _ptr(conv_state_in), _ptr(conv_state_out), _ptr(xbc_t),
                                 xs, _ptr(conv_w), _ptr(conv_bias), _ptr(dt_t), dts, _ptr(A), _ptr(D),
                                 _ptr(y), ys, batch, n_heads, d_head, d_state, 1, h_act,
                                 _ptr(heads_per_seq), _dtype_code(xbc_t), _stream())
    _check("mm_ssd_step_fused", st)
    return y

"""fp64 CPU oracle for the Matryoshka-sliced conv1d+SiLU, selective scan and
gated RMSNorm epilogue.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no
code with the HIP library in ``selective_state_space_12_amd`` and never imports
it; the two meet only on the seeded inputs from ``synth``.

The arithmetic lives in ``mm_oracle.c`` (plain C, fp64, token-by-token
recurrence, OpenMP over independent (sequence, head) units).  This module
compiles it with gcc when the shared object is missing or older than the
source, converts arguments to contiguous fp64 numpy arrays and returns fp64
results.  Every function states the passage it follows.

Pins: every function here is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_pins.py`` (brute force, closed forms, textbook routines,
invariants) and, for the backward functions, ``tests/test_oracle_backward_pins.py``
(finite differences of the pinned forward functions, a one-token closed form)
-- see the docstrings there.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mm_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile ``mm_oracle.c`` with gcc (-O2, OpenMP, no fast-math)."""
    if (not force and os.path.exists(_LIB_PATH)
            and os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC)):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB_PATH)
            dp = ctypes.POINTER(ctypes.c_double)
            ip = ctypes.POINTER(ctypes.c_int64)
            i64 = ctypes.c_int64
            lib.oracle_conv1d_silu.argtypes = [dp, dp, dp, dp, dp, i64, i64, i64,
                                               i64, i64, ip]
            lib.oracle_conv1d_silu.restype = None
            lib.oracle_ssd_forward.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, dp,
                                               i64, i64, i64, i64, i64, i64, ip, dp]
            lib.oracle_ssd_forward.restype = None
            lib.oracle_ssd_step.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, i64, i64,
                                            i64, i64, i64, ip]
            lib.oracle_ssd_step.restype = None
            lib.oracle_gated_rmsnorm.argtypes = [dp, dp, dp, ctypes.c_double, dp, i64, i64]
            lib.oracle_gated_rmsnorm.restype = None
            lib.oracle_ssd_backward.argtypes = [dp] * 16 + [i64] * 6 + [ip]
            lib.oracle_ssd_backward.restype = None
            lib.oracle_conv1d_silu_backward.argtypes = [dp] * 9 + [i64] * 5 + [ip]
            lib.oracle_conv1d_silu_backward.restype = None
            _lib = lib
    return _lib


def _f64(a):
    if a is None:
        return None
    if hasattr(a, "detach"):  # torch tensor (CPU or device) -> numpy
        a = a.detach().float().cpu().numpy() if a.dtype.is_floating_point else a.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _heads_vec(heads_active, batch, n_heads):
    if heads_active is None:
        hv = np.full(batch, n_heads, dtype=np.int64)
    elif np.isscalar(heads_active):
        hv = np.full(batch, int(heads_active), dtype=np.int64)
    else:
        hv = np.ascontiguousarray(np.asarray(heads_active, dtype=np.int64))
    if hv.shape != (batch,) or (hv < 0).any() or (hv > n_heads).any():
        raise ValueError("heads_active must give 0..n_heads heads per sequence")
    return hv


def heads_for_dim(d_model: int, d_inner: int, d_head: int, m: int) -> int:
    """Matryoshka slice resolution (MatMamba page, nesting paragraph and the
    Mix'n'Match paragraph): with e = d_inner / d_model, d_i = e*m_i and
    h_i = d_i / d_head, valid only when d_i mod d_head == 0.  The trained list
    includes m_i = d_model, so 0 < m_i <= d_model is accepted."""
    if d_model <= 0 or d_inner <= 0 or d_head <= 0:
        raise ValueError("dimensions must be positive")
    if d_inner % d_model != 0:
        raise ValueError("expansion e = d_inner / d_model must be an integer")
    if not (0 < m <= d_model):
        raise ValueError("m_i must satisfy 0 < m_i <= d_model")
    d_i = (d_inner // d_model) * m
    if d_i % d_head != 0:
        raise ValueError("e * m_i must be a multiple of d_head")
    return d_i // d_head


def conv1d_silu(u, w, bias=None, conv_state=None, *, d_inner, d_head,
                heads_active=None):
    """Causal depthwise conv (kernel 4) + SiLU over the [x | B | C] channels
    (MatMamba page, block paragraph: concatenated W_conv_x, W_conv_B, W_conv_C,
    sigma = SiLU).  u: (batch, seqlen, conv_dim).  Returns (out, new_state);
    channels outside the slice are NaN in ``out`` (never computed) and keep
    their old value in the returned state."""
    lib = _load()
    u = _f64(u)
    batch, seqlen, conv_dim = u.shape
    n_heads = d_inner // d_head
    hv = _heads_vec(heads_active, batch, n_heads)
    w = _f64(w).reshape(conv_dim, 4)
    bias = _f64(bias)
    out = np.full_like(u, np.nan)
    st = None
    if conv_state is not None:
        st = _f64(conv_state).reshape(batch, conv_dim, 3).copy()
    lib.oracle_conv1d_silu(_ptr(u), _ptr(out), _ptr(w), _ptr(bias), _ptr(st),
                           batch, seqlen, conv_dim, d_inner, d_head,
                           hv.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)))
    return out, st


def ssd_forward(x, dt, A, B, C, D=None, h0=None, *, heads_active=None,
                return_state=True):
    """Token-by-token selective scan over the first heads_active[b] heads
    (recurrence in ``mm_oracle.c``'s header).  x: (batch, seqlen, n_heads, P);
    dt: (batch, seqlen, n_heads); B, C: (batch, seqlen, ngroups, N).
    Returns (y, h_final); inactive heads are NaN (never computed)."""
    lib = _load()
    x = _f64(x)
    batch, seqlen, n_heads, P = x.shape
    dt = _f64(dt).reshape(batch, seqlen, n_heads)
    B = _f64(B)
    C = _f64(C)
    if B.ndim == 3:
        B = B[:, :, None, :]
        C = C[:, :, None, :]
    ngroups, N = B.shape[2], B.shape[3]
    if n_heads % ngroups:
        raise ValueError("n_heads must be a multiple of ngroups")
    A = _f64(A).reshape(n_heads)
    D = _f64(D)
    if D is not None:
        D = D.reshape(n_heads)
    h0 = _f64(h0)
    if h0 is not None:
        h0 = h0.reshape(batch, n_heads, P, N)
    hv = _heads_vec(heads_active, batch, n_heads)
    y = np.full((batch, seqlen, n_heads, P), np.nan)
    hf = np.full((batch, n_heads, P, N), np.nan) if return_state else None
    scratch = np.empty((batch, n_heads, P, N))
    lib.oracle_ssd_forward(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                           _ptr(h0), _ptr(y), _ptr(hf), batch, seqlen, n_heads, P,
                           N, ngroups,
                           hv.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                           _ptr(scratch))
    return y, hf


def ssd_step(state, x_t, dt_t, A, B_t, C_t, D=None, *, heads_active=None):
    """One decode token of the recurrence (Mamba page, Strengths: linear-time
    recurrent inference).  state: (batch, n_heads, P, N), updated copy returned
    with y_t (batch, n_heads, P); inactive heads keep their state, y is NaN."""
    lib = _load()
    st = _f64(state).copy()
    batch, n_heads, P, N = st.shape
    x_t = _f64(x_t).reshape(batch, n_heads, P)
    dt_t = _f64(dt_t).reshape(batch, n_heads)
    B_t = _f64(B_t)
    C_t = _f64(C_t)
    if B_t.ndim == 2:
        B_t = B_t[:, None, :]
        C_t = C_t[:, None, :]
    ngroups = B_t.shape[1]
    A = _f64(A).reshape(n_heads)
    D = _f64(D)
    hv = _heads_vec(heads_active, batch, n_heads)
    y = np.full((batch, n_heads, P), np.nan)
    lib.oracle_ssd_step(_ptr(st), _ptr(x_t), _ptr(dt_t), _ptr(A), _ptr(B_t),
                        _ptr(C_t), _ptr(D), _ptr(y), batch, n_heads, P, N, ngroups,
                        hv.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)))
    return y, st


def ssd_backward(x, dt, A, B, C, D=None, h0=None, dy=None, dhT=None, *, heads_active=None):
    """Gradients of L = sum(dy * y) + sum(dhT * h_final) for ssd_forward, by
    reverse-mode differentiation of the recurrence token by token (the joint
    training of the nested sub-blocks, MatMamba page, training paragraph,
    needs the backward pass of every granularity; the chain rule is written
    out in ``mm_oracle.c``).  Shapes as ssd_forward; dy like y, dhT like the
    final state (None = 0).  Returns a dict with dx, ddt (NaN for inactive
    heads), dA, dD (n_heads; NaN for heads active in no sequence), dB, dC
    (batch, seqlen, ngroups, N; summed over the active heads of the group) and
    dh0 (batch, n_heads, P, N; NaN for inactive heads)."""
    lib = _load()
    x = _f64(x)
    batch, seqlen, n_heads, P = x.shape
    dt = _f64(dt).reshape(batch, seqlen, n_heads)
    B = _f64(B)
    C = _f64(C)
    if B.ndim == 3:
        B = B[:, :, None, :]
        C = C[:, :, None, :]
    ngroups, N = B.shape[2], B.shape[3]
    if n_heads % ngroups:
        raise ValueError("n_heads must be a multiple of ngroups")
    A = _f64(A).reshape(n_heads)
    D = _f64(D)
    if D is not None:
        D = D.reshape(n_heads)
    h0 = _f64(h0)
    if h0 is not None:
        h0 = h0.reshape(batch, n_heads, P, N)
    dy = _f64(dy).reshape(batch, seqlen, n_heads, P)
    dhT = _f64(dhT)
    if dhT is not None:
        dhT = dhT.reshape(batch, n_heads, P, N)
    hv = _heads_vec(heads_active, batch, n_heads)
    out = {
        "dx": np.full((batch, seqlen, n_heads, P), np.nan),
        "ddt": np.full((batch, seqlen, n_heads), np.nan),
        "dA": np.full(n_heads, np.nan),
        "dB": np.empty((batch, seqlen, ngroups, N)),
        "dC": np.empty((batch, seqlen, ngroups, N)),
        "dD": np.full(n_heads, np.nan),
        "dh0": np.full((batch, n_heads, P, N), np.nan),
    }
    lib.oracle_ssd_backward(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(h0),
                            _ptr(dy), _ptr(dhT), _ptr(out["dx"]), _ptr(out["ddt"]),
                            _ptr(out["dA"]), _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["dD"]),
                            _ptr(out["dh0"]), batch, seqlen, n_heads, P, N, ngroups,
                            hv.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)))
    return out


def conv1d_silu_backward(u, w, dout, bias=None, conv_state=None, *, d_inner, d_head,
                         heads_active=None):
    """Gradients of L = sum(dout * conv1d_silu(u)) (the returned new conv state
    is not differentiated): du (batch, seqlen, conv_dim; NaN outside the
    slice), dw (conv_dim, 4) and dbias (conv_dim) summed over the sequences in
    which each channel is active (NaN for channels active in none), dstate
    (batch, conv_dim, 3) for the given initial conv state (None without one).
    Chain rule in ``mm_oracle.c``."""
    lib = _load()
    u = _f64(u)
    batch, seqlen, conv_dim = u.shape
    n_heads = d_inner // d_head
    hv = _heads_vec(heads_active, batch, n_heads)
    w = _f64(w).reshape(conv_dim, 4)
    bias = _f64(bias)
    st = None if conv_state is None else _f64(conv_state).reshape(batch, conv_dim, 3)
    dout = _f64(dout).reshape(batch, seqlen, conv_dim)
    du = np.full_like(u, np.nan)
    dw = np.full((conv_dim, 4), np.nan)
    db = np.full(conv_dim, np.nan)
    dst = None if st is None else np.full((batch, conv_dim, 3), np.nan)
    lib.oracle_conv1d_silu_backward(_ptr(u), _ptr(w), _ptr(bias), _ptr(st), _ptr(dout),
                                    _ptr(du), _ptr(dw), _ptr(db), _ptr(dst), batch, seqlen,
                                    conv_dim, d_inner, d_head,
                                    hv.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)))
    return {"du": du, "dw": dw, "dbias": db, "dstate": dst}


def softplus(v):
    """softplus(v) = log(1 + e^v), the map from the raw W_dt projection (plus
    its bias) to the step size dt (MatMamba page, block paragraph: W_dt is one
    of the input projections; the workloads draw dt as softplus of a Gaussian).
    Written as log(e^0 + e^v) with numpy's logaddexp, which evaluates it
    without overflow."""
    return np.logaddexp(0.0, _f64(v))


def ssd_forward_fused(xbc, w, dt, A, D=None, *, d_inner, d_head, conv_bias=None,
                      conv_state=None, dt_bias=None, dt_softplus=False, h0=None,
                      heads_active=None):
    """The block's prefill path as one composition (MatMamba page, block
    paragraph: the conv over the concatenated x, B, C streams feeds the chunk +
    selective scan): u = conv1d_silu(xbc); x, B, C = the d_inner, d_state and
    d_state column ranges of u; dt' = dt + dt_bias, through softplus if asked;
    then ssd_forward.  xbc: (batch, seqlen, conv_dim) raw conv input; dt:
    (batch, seqlen, n_heads) raw.  conv_state in this module's layout
    (batch, conv_dim, 3).  Returns (y, h_final, new_conv_state)."""
    xbc = _f64(xbc)
    batch, seqlen, conv_dim = xbc.shape
    n_heads = d_inner // d_head
    N = (conv_dim - d_inner) // 2
    u, new_state = conv1d_silu(xbc, w, conv_bias, conv_state, d_inner=d_inner, d_head=d_head,
                               heads_active=heads_active)
    x = u[:, :, :d_inner].reshape(batch, seqlen, n_heads, d_head)
    B = u[:, :, d_inner:d_inner + N][:, :, None, :]
    C = u[:, :, d_inner + N:d_inner + 2 * N][:, :, None, :]
    d = _f64(dt).reshape(batch, seqlen, n_heads)
    if dt_bias is not None:
        d = d + _f64(dt_bias).reshape(1, 1, n_heads)
    if dt_softplus:
        d = softplus(d)
    y, hf = ssd_forward(x, d, A, B, C, D, h0, heads_active=heads_active)
    return y, hf, new_state


def gated_rmsnorm(y, z, w, eps, *, d):
    """Gated RMSNorm over the first d channels of each token (MatMamba page,
    block paragraph: sigma = SiLU gates the scan output with z, Norm =
    RMSNorm; gate before norm, the Mamba2 order):
    out = (y * SiLU(z)) * w / sqrt(mean((y * SiLU(z))^2) + eps).
    y, z: (..., >= d) -- the first d channels are used; w: (>= d,).  Returns
    (..., d) fp64."""
    lib = _load()
    y = _f64(y)
    z = _f64(z)
    lead = y.shape[:-1]
    yy = np.ascontiguousarray(y[..., :d].reshape(-1, d))
    zz = np.ascontiguousarray(z[..., :d].reshape(-1, d))
    ww = np.ascontiguousarray(_f64(w).reshape(-1)[:d])
    out = np.empty_like(yy)
    lib.oracle_gated_rmsnorm(_ptr(yy), _ptr(zz), _ptr(ww), float(eps), _ptr(out), yy.shape[0], d)
    return out.reshape(*lead, d)


def rel_l2(a, b) -> float:
    """Relative L2 distance ||a - b|| / ||b|| in fp64 (b is the reference)."""
    a = _f64(a)
    b = _f64(b)
    den = np.linalg.norm(b.ravel())
    num = np.linalg.norm((a - b).ravel())
    if den == 0.0:
        return float(num)
    return float(num / den)

"""Seeded synthetic inputs shaped like the pages' models.

This module holds the workload shapes and the random-input recipe, and nothing
of the method's arithmetic: it is the one piece of code that both the oracle
side (tests, CPU baseline) and the HIP side (tests, bench) take inputs from.
Every tensor is drawn on the CPU from its own ``torch.Generator`` seeded with
``1000 + 16*config_index + tensor_index`` (device independent), in fp32, and
then rounded once to the storage dtype.  Consumers copy it to the device.

Shapes follow the MatMamba page (block paragraph: (b, l, d) in and out,
e = d_inner / d_model, heads of d_head channels; nesting paragraph: m_i, d_i,
h_i; training paragraph: m_i in [d, d/2, d/4, d/8]); the page's own model
tables did not survive, so the sizes below are the workload definitions this
library is measured on.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import torch

# tensor indices inside a config's seed block
(_X, _B, _C, _DT, _A, _D, _CONVW, _XBC, _H0, _CS0, _DTSTEP, _XBCSTEP, _CONVB, _DTRAW, _DTB, _Z, _NW,
 _YN, _DY, _DHT, _DOUT) = range(21)


@dataclass(frozen=True)
class Workload:
    name: str
    index: int
    batch: int
    seqlen: int
    d_model: int
    d_inner: int
    d_head: int
    d_state: int
    ngroups: int
    chunk: int
    slices: List[int]          # Matryoshka dims m_i
    dtype: torch.dtype          # storage dtype of x, dt, B, C, y
    dt_mode: str                # "softplus" or "loguniform"
    bc_scale: float
    steps: int = 0              # decode only
    extra: Dict[str, object] = field(default_factory=dict)

    @property
    def n_heads(self) -> int:
        return self.d_inner // self.d_head

    @property
    def conv_dim(self) -> int:
        return self.d_inner + 2 * self.ngroups * self.d_state

    def heads(self, m: int) -> int:
        e = self.d_inner // self.d_model
        return e * m // self.d_head


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", 0, 1, 256, 64, 128, 32, 16, 1, 64, [16, 32, 64],
                     torch.float32, "softplus", 1.0 / math.sqrt(16)),
    "130m": Workload("130m", 1, 8, 2048, 768, 1536, 64, 128, 1, 256,
                     [96, 192, 384, 768], torch.bfloat16, "softplus",
                     1.0 / math.sqrt(128)),
    "1.4b": Workload("1.4b", 2, 4, 8192, 2048, 4096, 64, 128, 1, 256,
                     [256, 512, 1024, 2048], torch.bfloat16, "loguniform",
                     1.0 / math.sqrt(128)),
    "long": Workload("long", 3, 1, 131072, 1024, 2048, 64, 128, 1, 256,
                     [256, 512, 1024], torch.bfloat16, "softplus",
                     1.0 / math.sqrt(128)),
    "decode": Workload("decode", 4, 256, 1, 2048, 4096, 64, 128, 1, 256,
                       [512, 1024, 2048], torch.float32, "softplus",
                       1.0 / math.sqrt(128), steps=1024),
}


def _gen(w: Workload, idx: int, salt: int = 0) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(1000 + 16 * w.index + idx + 7919 * salt)
    return g


def _normal(shape, g, scale=1.0):
    t = torch.randn(*shape, generator=g, dtype=torch.float32)
    if scale != 1.0:
        t.mul_(scale)
    return t


def _dt(shape, w: Workload, g):
    if w.dt_mode == "loguniform":
        u = torch.rand(*shape, generator=g, dtype=torch.float32)
        return torch.exp(math.log(1e-3) + u * (math.log(1e-1) - math.log(1e-3)))
    return torch.nn.functional.softplus(_normal(shape, g) - 4.0)


def draw_A(w: Workload, n_heads: Optional[int] = None) -> torch.Tensor:
    """A_h = -exp(U(0, ln 16)) in [-16, -1], fp32, one real scalar per head."""
    n = n_heads or w.n_heads
    u = torch.rand(n, generator=_gen(w, _A), dtype=torch.float32)
    return -torch.exp(u * math.log(16.0))


def draw_D(w: Workload, n_heads: Optional[int] = None) -> torch.Tensor:
    n = n_heads or w.n_heads
    return _normal((n,), _gen(w, _D))


def draw_conv_w(w: Workload) -> torch.Tensor:
    """(conv_dim, 4) fp32, 0.5 * N(0, 1); tap 3 multiplies the current token."""
    return _normal((w.conv_dim, 4), _gen(w, _CONVW), 0.5)


def draw_conv_bias(w: Workload) -> torch.Tensor:
    """(conv_dim,) fp32, 0.5 * N(0, 1).  The workloads run without a conv bias;
    this draw exercises the optional bias argument."""
    return _normal((w.conv_dim,), _gen(w, _CONVB), 0.5)


def forward_inputs(w: Workload, batch: Optional[int] = None,
                   seqlen: Optional[int] = None, salt: int = 0,
                   with_state: bool = False) -> Dict[str, torch.Tensor]:
    """Dense CPU tensors for the scan: x (b,l,H,P), dt (b,l,H), B, C (b,l,G,N)
    in the workload's storage dtype; A, D (H) fp32; optional h0 (b,H,P,N) fp32
    drawn N(0,1).  ``batch``/``seqlen`` override the workload's size (the
    recipe is unchanged); ``salt`` gives an independent draw."""
    b = batch or w.batch
    l = seqlen or w.seqlen
    H, P, G, N = w.n_heads, w.d_head, w.ngroups, w.d_state
    out = {
        "x": _normal((b, l, H, P), _gen(w, _X, salt)).to(w.dtype),
        "B": _normal((b, l, G, N), _gen(w, _B, salt), w.bc_scale).to(w.dtype),
        "C": _normal((b, l, G, N), _gen(w, _C, salt), w.bc_scale).to(w.dtype),
        "dt": _dt((b, l, H), w, _gen(w, _DT, salt)).to(w.dtype),
        "A": draw_A(w),
        "D": draw_D(w),
    }
    if with_state:
        out["h0"] = _normal((b, H, P, N), _gen(w, _H0, salt))
    return out


def cotangents(w: Workload, batch: Optional[int] = None, seqlen: Optional[int] = None,
               salt: int = 0) -> Dict[str, torch.Tensor]:
    """Cotangents for a backward pass of the scan: dy (b, l, H, P) ~ N(0, 1)
    in the storage dtype (the gradient arriving at y) and dhT (b, H, P, N)
    ~ N(0, 1) fp32 (arriving at the final state)."""
    b = batch or w.batch
    l = seqlen or w.seqlen
    H, P, N = w.n_heads, w.d_head, w.d_state
    return {
        "dy": _normal((b, l, H, P), _gen(w, _DY, salt)).to(w.dtype),
        "dhT": _normal((b, H, P, N), _gen(w, _DHT, salt)),
    }


def conv_cotangent(w: Workload, batch: Optional[int] = None, seqlen: Optional[int] = None,
                   salt: int = 0) -> torch.Tensor:
    """Cotangent of the conv output (b, l, conv_dim) ~ N(0, 1) in the storage
    dtype."""
    b = batch or w.batch
    l = seqlen or w.seqlen
    return _normal((b, l, w.conv_dim), _gen(w, _DOUT, salt)).to(w.dtype)


def xbc_inputs(w: Workload, batch: Optional[int] = None,
               seqlen: Optional[int] = None, salt: int = 0,
               with_state: bool = False) -> Dict[str, torch.Tensor]:
    """Raw conv input (b, l, conv_dim) ~ N(0,1) in the storage dtype, its
    weights, and optionally a conv state (b, 3, conv_dim) ~ N(0,1) fp32
    (oldest tap first)."""
    b = batch or w.batch
    l = seqlen or w.seqlen
    out = {
        "xbc": _normal((b, l, w.conv_dim), _gen(w, _XBC, salt)).to(w.dtype),
        "w": draw_conv_w(w),
    }
    if with_state:
        out["conv_state"] = _normal((b, 3, w.conv_dim), _gen(w, _CS0, salt))
    return out


def pipeline_dt(w: Workload, batch: Optional[int] = None,
                seqlen: Optional[int] = None, salt: int = 0) -> torch.Tensor:
    """dt (b, l, H) for the conv -> scan pipeline (same recipe as the scan)."""
    b = batch or w.batch
    l = seqlen or w.seqlen
    return _dt((b, l, w.n_heads), w, _gen(w, _DT, salt + 1)).to(w.dtype)


def raw_dt(w: Workload, batch: Optional[int] = None, seqlen: Optional[int] = None,
           salt: int = 0) -> torch.Tensor:
    """Raw dt (b, l, H) before bias and softplus, N(0,1) - 4 in the storage
    dtype: through softplus with no bias it follows the softplus(N(0,1) - 4)
    recipe of the workloads."""
    b = batch or w.batch
    l = seqlen or w.seqlen
    return (_normal((b, l, w.n_heads), _gen(w, _DTRAW, salt)) - 4.0).to(w.dtype)


def draw_dt_bias(w: Workload) -> torch.Tensor:
    """(n_heads,) fp32, 0.5 * N(0, 1): exercises the optional dt bias."""
    return _normal((w.n_heads,), _gen(w, _DTB), 0.5)


def gate_inputs(w: Workload, batch: Optional[int] = None, seqlen: Optional[int] = None,
                salt: int = 0) -> Dict[str, torch.Tensor]:
    """Inputs of the gated RMSNorm epilogue: a scan output stand-in y and the
    gate z, both (b, l, d_inner) ~ N(0,1) in the storage dtype, and the norm
    weight (d_inner,) = 1 + 0.1 * N(0,1) fp32."""
    b = batch or w.batch
    l = seqlen or w.seqlen
    return {
        "y": _normal((b, l, w.d_inner), _gen(w, _YN, salt)).to(w.dtype),
        "z": _normal((b, l, w.d_inner), _gen(w, _Z, salt)).to(w.dtype),
        "w": 1.0 + _normal((w.d_inner,), _gen(w, _NW), 0.1),
    }


def decode_pool(w: Workload, pool: int = 64, batch: Optional[int] = None,
                salt: int = 0) -> Dict[str, torch.Tensor]:
    """A pool of per-step decode inputs, cycled by the decode loop:
    xbc_t (pool, b, conv_dim) ~ N(0,1) and dt_t (pool, b, H) = softplus(N(0,1)-4)."""
    b = batch or w.batch
    return {
        "xbc_t": _normal((pool, b, w.conv_dim), _gen(w, _XBCSTEP, salt)).to(w.dtype),
        "dt_t": torch.nn.functional.softplus(
            _normal((pool, b, w.n_heads), _gen(w, _DTSTEP, salt)) - 4.0).to(w.dtype),
    }


def decode_heads(w: Workload, batch: Optional[int] = None) -> torch.Tensor:
    """Mixed slices across the decode batch: sequence i runs m[i mod 3]."""
    b = batch or w.batch
    hs = [w.heads(w.slices[i % len(w.slices)]) for i in range(b)]
    return torch.tensor(hs, dtype=torch.int32)

"""GPU parity of the conv backward (mm_conv1d_silu_backward) through the C
ABI against the fp64 oracle's reverse-mode gradients
(oracle.conv1d_silu_backward): relative L2 per gradient, 1e-4 for fp32
storage and 2e-2 for bf16; channels outside the slice stay untouched."""
import numpy as np
import pytest
import torch

import oracle
import selective_state_space_12_amd as mm
import synth
from gpu_cases import DEV, TOL, conv_state_from_oracle, conv_state_to_oracle, f64, rel_l2, say

pytestmark = pytest.mark.gpu

TINY = synth.WORKLOADS["tiny"]
M130 = synth.WORKLOADS["130m"]
B14 = synth.WORKLOADS["1.4b"]


def _inputs(w, b, l, salt=0):
    xi = synth.xbc_inputs(w, batch=b, seqlen=l, salt=salt, with_state=True)
    return {"xbc": xi["xbc"], "w": xi["w"], "cs": xi["conv_state"],
            "cb": synth.draw_conv_bias(w), "dout": synth.conv_cotangent(w, batch=b, seqlen=l, salt=salt)}


def _nan_grads(w, b, l):
    return {"dxbc": torch.full((b, l, w.conv_dim), float("nan"), dtype=w.dtype, device=DEV),
            "dw": torch.full((w.conv_dim, 4), float("nan"), device=DEV),
            "dbias": torch.full((w.conv_dim,), float("nan"), device=DEV),
            "dconv_state": torch.full((b, 3, w.conv_dim), float("nan"), device=DEV)}


def _run(w, inp, h, *, bias=True, state=True, grads=None, accumulate=False):
    b, l = inp["xbc"].shape[:2]
    g = grads if grads is not None else _nan_grads(w, b, l)
    if not state:
        g.pop("dconv_state", None)
    mm.conv1d_silu_backward(inp["xbc"].to(DEV), inp["w"].to(DEV), inp["dout"].to(DEV),
                            inp["cb"].to(DEV) if bias else None,
                            inp["cs"].to(DEV) if state else None, d_inner=w.d_inner,
                            d_head=w.d_head, d_state=w.d_state, n_heads_active=h, grads=g,
                            accumulate=accumulate, want_dbias=bias)
    torch.cuda.synchronize()
    return g


def _oracle(w, inp, h, *, bias=True, state=True):
    r = oracle.conv1d_silu_backward(inp["xbc"], inp["w"], inp["dout"], inp["cb"] if bias else None,
                                    conv_state_to_oracle(inp["cs"]) if state else None,
                                    d_inner=w.d_inner, d_head=w.d_head, heads_active=h)
    if r["dstate"] is not None:
        r["dstate"] = conv_state_from_oracle(r["dstate"])
    return r


def _active(w, h):
    return np.r_[0:h * w.d_head, w.d_inner:w.conv_dim]


def _check(w, g, r, h, tol, *, bias=True, state=True):
    act = _active(w, h)
    ina = np.r_[h * w.d_head:w.d_inner]
    pairs = [("dxbc", "du", lambda t: t[..., act], lambda t: t[..., ina]),
             ("dw", "dw", lambda t: t[act], lambda t: t[ina])]
    if bias:
        pairs.append(("dbias", "dbias", lambda t: t[act], lambda t: t[ina]))
    if state:
        pairs.append(("dconv_state", "dstate", lambda t: t[..., act], lambda t: t[..., ina]))
    errs = {}
    for gk, rk, on, off in pairs:
        got = f64(g[gk])
        errs[gk] = oracle.rel_l2(on(got), on(r[rk]))
        assert np.isnan(off(got)).all(), gk
    say("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v < tol}
    assert not bad, bad


@pytest.mark.parametrize("seqlen", [1, 2, 5, 64, 100, 256])
def test_conv_backward_tiny_fp32(seqlen):
    """fp32, 128 + 32 channels: sequences shorter than the window, one run,
    several runs with a ragged tail; every slice."""
    w = TINY
    inp = _inputs(w, 1, seqlen)
    for m in w.slices:
        h = w.heads(m)
        say(f"conv backward tiny fp32 l={seqlen} heads={h}")
        _check(w, _run(w, inp, h), _oracle(w, inp, h), h, TOL[torch.float32])


@pytest.mark.parametrize("seqlen", [3, 65, 600])
def test_conv_backward_130m_bf16(seqlen):
    """bf16, 1536 + 256 channels, two sequences; smallest and full slice."""
    w = M130
    inp = _inputs(w, 2, seqlen, salt=1)
    for h in (3, 24):
        say(f"conv backward 130m bf16 l={seqlen} heads={h}")
        _check(w, _run(w, inp, h), _oracle(w, inp, h), h, TOL[torch.bfloat16])


def test_conv_backward_without_bias_and_state():
    w = M130
    inp = _inputs(w, 2, 300, salt=2)
    say("conv backward 130m bf16 no bias, no state")
    g = _run(w, inp, 12, bias=False, state=False)
    _check(w, g, _oracle(w, inp, 12, bias=False, state=False), 12, TOL[torch.bfloat16], bias=False,
           state=False)


def test_conv_backward_accumulates():
    """Two granularities into the same buffers: the sum of the oracle's."""
    w = M130
    inp = _inputs(w, 2, 200, salt=3)
    g = _run(w, inp, 24)
    g = _run(w, inp, 6, grads=g, accumulate=True)
    r24, r6 = _oracle(w, inp, 24), _oracle(w, inp, 6)
    act6 = _active(w, 6)
    tot = {k: r24[k].copy() for k in ("du", "dw", "dbias", "dstate")}
    tot["du"][..., act6] += r6["du"][..., act6]
    tot["dw"][act6] += r6["dw"][act6]
    tot["dbias"][act6] += r6["dbias"][act6]
    tot["dstate"][..., act6] += r6["dstate"][..., act6]
    say("conv backward accumulate heads=24 then 6")
    _check(w, g, tot, 24, TOL[torch.bfloat16])


def test_conv_backward_1p4b_full_size():
    """The 1.4B-scale rows (b=4, l=8192, 4352 channels) at the full slice."""
    w = B14
    inp = _inputs(w, None, None)
    say("conv backward 1.4b full size")
    g = _run(w, inp, w.n_heads, bias=False)
    _check(w, g, _oracle(w, inp, w.n_heads, bias=False), w.n_heads, TOL[torch.bfloat16], bias=False)


def test_conv_backward_rejects_bad_arguments():
    w = M130
    inp = {k: v.to(DEV) for k, v in _inputs(w, 1, 64).items()}
    with pytest.raises(mm.MMError):  # dxbc overlapping dout
        mm.conv1d_silu_backward(inp["xbc"], inp["w"], inp["dout"], d_inner=w.d_inner,
                                d_head=w.d_head, d_state=w.d_state, grads={"dxbc": inp["dout"]})

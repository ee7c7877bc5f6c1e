"""GPU parity of the scan backward (mm_ssd_backward) through the C ABI
against the fp64 oracle's reverse-mode gradients (oracle.ssd_backward).

Every gradient is compared as one tensor by relative L2: 1e-4 for fp32
storage, 2e-2 for bf16 storage with fp32 accumulation (the forward's bars:
the backward rounds the same kinds of operands -- x, dy, B, C, the chunk
states and dL/dH -- to the storage type before each MFMA).  Entries of heads
outside the slice must be left untouched (NaN sentinels)."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import selective_state_space_12_amd as mm
import synth
from gpu_cases import DEV, TOL, f64, rel_l2, say

pytestmark = pytest.mark.gpu

TINY = synth.WORKLOADS["tiny"]
M130 = synth.WORKLOADS["130m"]
B14 = synth.WORKLOADS["1.4b"]
M130_N64 = dataclasses.replace(M130, name="130m-n64", d_state=64)
# 80 heads: more than one launch's worth (64) of heads in the chunk kernel
M130_H80 = dataclasses.replace(M130, name="130m-h80", d_model=2560, d_inner=5120)

NAMES = ("dx", "ddt", "dA", "dB", "dC", "dD", "dinitial_state")


def _inputs(w, b, l, salt=0):
    inp = synth.forward_inputs(w, batch=b, seqlen=l, salt=salt, with_state=True)
    inp.update(synth.cotangents(w, batch=b, seqlen=l, salt=salt))
    return inp


def _nan_grads(w, b, l):
    H, P, N = w.n_heads, w.d_head, w.d_state
    return {
        "dx": torch.full((b, l, H, P), float("nan"), dtype=w.dtype, device=DEV),
        "ddt": torch.full((b, l, H), float("nan"), dtype=w.dtype, device=DEV),
        "dA": torch.full((H,), float("nan"), device=DEV),
        "dB": torch.full((b, l, 1, N), float("nan"), device=DEV),
        "dC": torch.full((b, l, 1, N), float("nan"), device=DEV),
        "dD": torch.full((H,), float("nan"), device=DEV),
        "dinitial_state": torch.full((b, H, P, N), float("nan"), device=DEV),
    }


def _run(w, inp, h, grads=None, accumulate=False, h0=True, dhT=True, D=True):
    b, l = inp["x"].shape[:2]
    d = {k: v.to(DEV) for k, v in inp.items()}
    g = grads if grads is not None else _nan_grads(w, b, l)
    mm.ssd_backward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"] if D else None, d["dy"],
                    n_heads_active=h, initial_state=d["h0"] if h0 else None,
                    dfinal_state=d["dhT"] if dhT else None, grads=g, accumulate=accumulate)
    torch.cuda.synchronize()
    return g


def _oracle(inp, h, h0=True, dhT=True, D=True):
    r = oracle.ssd_backward(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"],
                            inp["D"] if D else None, inp["h0"] if h0 else None, inp["dy"],
                            inp["dhT"] if dhT else None, heads_active=h)
    r["dinitial_state"] = r.pop("dh0")
    return r


def _check(g, ref, h, tol, names=NAMES, skip_dD=False):
    errs = {}
    for k in names:
        if skip_dD and k == "dD":
            continue
        got, want = g[k], ref[k]
        if k in ("dx", "ddt"):
            errs[k] = rel_l2(got[:, :, :h], want[:, :, :h])
            assert torch.isnan(got[:, :, h:]).all(), k
        elif k in ("dA", "dD"):
            errs[k] = rel_l2(got[:h], want[:h])
            assert torch.isnan(got[h:]).all(), k
        elif k == "dinitial_state":
            errs[k] = rel_l2(got[:, :h], want[:, :h])
            assert torch.isnan(got[:, h:]).all(), k
        else:
            errs[k] = rel_l2(got, want)
    say("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v < tol}
    assert not bad, bad


@pytest.mark.parametrize("seqlen", [1, 63, 100, 256])
def test_backward_tiny_fp32_all_slices(seqlen):
    """fp32, d_head 32, d_state 16: one chunk, a ragged chunk, several chunks."""
    w = TINY
    inp = _inputs(w, 1, seqlen)
    for m in w.slices:
        h = w.heads(m)
        say(f"backward tiny fp32 l={seqlen} heads={h}")
        _check(_run(w, inp, h), _oracle(inp, h), h, TOL[torch.float32])


@pytest.mark.parametrize("seqlen", [1, 5, 64, 129, 600])
def test_backward_130m_bf16(seqlen):
    """bf16, d_head 64, d_state 128, two sequences; the smallest and the full
    slice; a sequence shorter than a 16-token block, one exact chunk, a ragged
    tail and ten chunks."""
    w = M130
    inp = _inputs(w, 2, seqlen, salt=1)
    for h in (w.heads(w.slices[0]), w.n_heads):
        say(f"backward 130m bf16 l={seqlen} heads={h}")
        _check(_run(w, inp, h), _oracle(inp, h), h, TOL[torch.bfloat16])


@pytest.mark.parametrize("w,b,l,h", [(M130, 1, 2048, 3), (M130, 2, 1000, 12), (TINY, 1, 1024, 1)])
def test_backward_split_sequences(w, b, l, h):
    """Few (sequence, head) walks: the sequences are split into segments
    walked in parallel, each from its own boundary value, chained by a
    combine and corrected in the chunk kernel; the result matches the oracle
    as an unsplit call does."""
    nseg = mm.ssd_backward_segments(b, l, w.n_heads, w.d_head, w.d_state, 1, h, w.dtype)
    assert nseg > 1
    inp = _inputs(w, b, l, salt=7)
    say(f"backward split {w.name} b={b} l={l} heads={h} segments={nseg}")
    _check(_run(w, inp, h), _oracle(inp, h), h, TOL[w.dtype])


def test_backward_long_context_many_segments():
    """Long-context shape (32 heads of 64, d_state 128) at its narrowest slice,
    one 16384-token sequence: 8 walks, split into 16 segments of 1024 tokens
    (the oracle keeps every state of a walk, so the sequence is a 16384-token
    prefix of the workload's 131072)."""
    w = synth.WORKLOADS["long"]
    h, l = w.heads(w.slices[0]), 16384
    nseg = mm.ssd_backward_segments(1, l, w.n_heads, w.d_head, w.d_state, 1, h, w.dtype)
    assert nseg == 16
    inp = _inputs(w, 1, l, salt=8)
    say(f"backward long bf16 l={l} heads={h} segments={nseg}")
    _check(_run(w, inp, h), _oracle(inp, h), h, TOL[torch.bfloat16])


def test_backward_dstate64_bf16():
    """bf16 with d_state 64 (the other supported bf16 shape)."""
    w = M130_N64
    inp = _inputs(w, 2, 300, salt=2)
    for h in (3, 24):
        say(f"backward 130m d_state=64 bf16 heads={h}")
        _check(_run(w, inp, h), _oracle(inp, h), h, TOL[torch.bfloat16])


@pytest.mark.parametrize("h", [64, 70, 80])
def test_backward_more_heads_than_one_launch(h):
    """80 heads of 64: the chunk kernel takes at most 64 heads per launch
    (their per-head values live in LDS), so 70 and 80 active heads run as
    two launches whose dB, dC add up; 64 is exactly one."""
    w = M130_H80
    inp = _inputs(w, 1, 300, salt=9)
    say(f"backward 80-head bf16 l=300 heads={h}")
    _check(_run(w, inp, h), _oracle(inp, h), h, TOL[torch.bfloat16])


def test_backward_without_optional_inputs():
    """No D, no initial state, no final-state cotangent."""
    w = M130
    inp = _inputs(w, 1, 200, salt=3)
    say("backward 130m bf16 without D, h0, dhT")
    g = _run(w, inp, 12, h0=False, dhT=False, D=False)
    _check(g, _oracle(inp, 12, h0=False, dhT=False, D=False), 12, TOL[torch.bfloat16])


def test_backward_accumulates_over_granularities():
    """The joint training's pattern: one backward per granularity into the
    same gradient buffers (accumulate=1 after the first) equals the sum of the
    oracle's gradients of each granularity."""
    w = M130
    inp = _inputs(w, 2, 150, salt=4)
    hs = [w.heads(m) for m in w.slices]
    g = None
    total = None
    for i, h in enumerate(sorted(hs, reverse=True)):
        say(f"backward accumulate heads={h}")
        g = _run(w, inp, h, grads=g, accumulate=i > 0)
        r = _oracle(inp, h)
        if total is None:
            total = r
        else:
            for k in NAMES:
                if k in ("dB", "dC"):
                    total[k] = total[k] + r[k]
                elif k in ("dA", "dD"):
                    total[k][:h] += r[k][:h]
                elif k == "dinitial_state":
                    total[k][:, :h] += r[k][:, :h]
                else:
                    total[k][:, :, :h] += r[k][:, :, :h]
    _check(g, total, max(hs), TOL[torch.bfloat16])


def test_backward_deterministic_parts_repeat_bitwise():
    """dx, ddt, dB, dC and dinitial_state are each formed by one workgroup in
    a fixed order (dB and dC summed over the heads in registers): two calls
    give the same bits."""
    w = M130
    inp = _inputs(w, 2, 300, salt=5)
    g1 = _run(w, inp, 24)
    g2 = _run(w, inp, 24)
    for k in ("dx", "ddt", "dB", "dC", "dinitial_state"):
        a, b = g1[k], g2[k]
        assert torch.equal(torch.nan_to_num(a, nan=7.0), torch.nan_to_num(b, nan=7.0)), k


@pytest.mark.parametrize("m", [256, 2048])
def test_backward_1p4b_full_size_sequence0(m):
    """The full 1.4B-scale call (b=4, l=8192) at the smallest and the full
    slice; the oracle recomputes sequence 0 (every gradient of that sequence
    depends on it alone; dA and dD sum over the batch and are left to the
    smaller cases)."""
    w = B14
    h = w.heads(m)
    inp = _inputs(w, None, None)
    say(f"backward 1.4b full size heads={h}")
    g = _run(w, inp, h)
    one = {k: (v[:1] if v.dim() > 1 else v) for k, v in inp.items()}
    r = _oracle(one, h)
    sub = {k: (g[k][:1] if g[k].dim() > 1 else g[k]) for k in NAMES}
    _check(sub, r, h, TOL[torch.bfloat16], names=("dx", "ddt", "dB", "dC", "dinitial_state"))


def test_backward_rejects_bad_arguments():
    w = M130
    inp = {k: v.to(DEV) for k, v in _inputs(w, 1, 64).items()}
    with pytest.raises(mm.MMError):  # dx overlapping x
        mm.ssd_backward(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["dy"],
                        grads={"dx": inp["x"]})
    with pytest.raises(mm.MMError):  # fp32 with d_head 64 is not a backward shape
        f = {k: (v.float() if v.dtype == torch.bfloat16 else v) for k, v in inp.items()}
        mm.ssd_backward(f["x"], f["dt"], f["A"], f["B"], f["C"], f["D"], f["dy"])


def test_backward_accumulates_on_split_sequences():
    """Accumulating over granularities where the calls split the sequence:
    the second call's segment walks, combine (which writes dinitial_state),
    boundary corrections and segment-parallel dx read-modify-writes must add
    into the first call's gradients."""
    w = M130
    b, l = 1, 2048
    hs = (24, 3)
    nseg = [mm.ssd_backward_segments(b, l, w.n_heads, w.d_head, w.d_state, 1, h, w.dtype)
            for h in hs]
    assert max(nseg) > 1, nseg
    inp = _inputs(w, b, l, salt=11)
    g = None
    total = None
    for i, h in enumerate(hs):
        say(f"backward accumulate split heads={h} segments={nseg[i]}")
        g = _run(w, inp, h, grads=g, accumulate=i > 0)
        r = _oracle(inp, h)
        if total is None:
            total = r
        else:
            for k in NAMES:
                if k in ("dB", "dC"):
                    total[k] = total[k] + r[k]
                elif k in ("dA", "dD"):
                    total[k][:h] += r[k][:h]
                elif k == "dinitial_state":
                    total[k][:, :h] += r[k][:, :h]
                else:
                    total[k][:, :, :h] += r[k][:, :, :h]
    _check(g, total, max(hs), TOL[torch.bfloat16])

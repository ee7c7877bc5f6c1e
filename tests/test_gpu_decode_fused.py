"""GPU tests of the fused decode step (mm_ssd_step_fused): the conv step and
the SSD step in one launch.

- Bit for bit against the two-call path (mm_conv1d_silu's decode step, then
  mm_ssd_step) over several tokens: y, the SSD state and the conv state,
  with mixed widths per sequence, with and without a conv bias, fp32 and bf16.
- Against the fp64 oracle's conv step followed by its recurrent step over
  64 tokens, on sequences covering every width class of the decode workload.
- Sequences with no active head still advance their B and C taps.
- Replays of a HIP graph of fused tokens equal the eager run.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
import selective_state_space_12_amd as mm
from gpu_cases import DEV, TOL, conv_state_from_oracle, conv_state_to_oracle, f64, say

pytestmark = pytest.mark.gpu

DEC = synth.WORKLOADS["decode"]
TINY = synth.WORKLOADS["tiny"]


def _inputs(w, steps, dtype, batch, heads_per_seq, with_bias, seed=77):
    pool = synth.decode_pool(w, pool=steps, batch=batch)
    A, D, cw = synth.draw_A(w), synth.draw_D(w), synth.draw_conv_w(w)
    cb = synth.draw_conv_bias(w) if with_bias else None
    rng = torch.Generator().manual_seed(seed)
    st0 = torch.randn(batch, w.n_heads, w.d_head, w.d_state, generator=rng)
    cs0 = torch.randn(batch, 3, w.conv_dim, generator=rng)
    return dict(xbc=pool["xbc_t"].to(dtype), dt=pool["dt_t"].to(dtype), A=A, D=D, cw=cw, cb=cb,
                st0=st0, cs0=cs0, hv=heads_per_seq)


def _two_call(w, inp, steps, dtype):
    """conv decode step (in place on the conv state), then mm_ssd_step."""
    b, H, P, N = inp["st0"].shape
    st, cs = inp["st0"].clone().to(DEV), inp["cs0"].clone().to(DEV)
    hv = inp["hv"].to(DEV)
    cw, A, D = inp["cw"].to(DEV), inp["A"].to(DEV), inp["D"].to(DEV)
    cb = inp["cb"].to(DEV) if inp["cb"] is not None else None
    ys = []
    for k in range(steps):
        u = torch.empty((b, 1, w.conv_dim), dtype=dtype, device=DEV)
        mm.conv1d_silu(inp["xbc"][k].unsqueeze(1).to(DEV), cw, cb, cs, d_inner=w.d_inner, d_head=P,
                       d_state=N, n_heads_active=H, heads_per_seq=hv, out=u)
        u2 = u[:, 0]
        y = torch.full((b, H, P), float("nan"), dtype=dtype, device=DEV)
        mm.ssd_step(st, u2[:, :w.d_inner].view(b, H, P), inp["dt"][k].to(DEV), A,
                    u2[:, w.d_inner:w.d_inner + N], u2[:, w.d_inner + N:], D,
                    n_heads_active=H, heads_per_seq=hv, y=y)
        ys.append(y)
    torch.cuda.synchronize()
    return ys, st, cs


def _fused(w, inp, steps, dtype):
    """mm_ssd_step_fused with two conv-state buffers used in turn."""
    b, H, P, N = inp["st0"].shape
    st = inp["st0"].clone().to(DEV)
    cs = [inp["cs0"].clone().to(DEV), torch.full_like(inp["cs0"], float("nan")).to(DEV)]
    hv = inp["hv"].to(DEV)
    cw, A, D = inp["cw"].to(DEV), inp["A"].to(DEV), inp["D"].to(DEV)
    cb = inp["cb"].to(DEV) if inp["cb"] is not None else None
    ys = []
    for k in range(steps):
        y = torch.full((b, H, P), float("nan"), dtype=dtype, device=DEV)
        mm.ssd_step_fused(st, cs[k % 2], cs[(k + 1) % 2], inp["xbc"][k].to(DEV), cw,
                          inp["dt"][k].to(DEV), A, D, cb, n_heads_active=H, heads_per_seq=hv, y=y)
        ys.append(y)
    torch.cuda.synchronize()
    return ys, st, cs[steps % 2]


def _same_nan(a: torch.Tensor, b: torch.Tensor) -> bool:
    """Bitwise equality that also matches NaN slots (untouched outputs)."""
    return torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))


@pytest.mark.parametrize("dtype,with_bias", [(torch.bfloat16, False), (torch.bfloat16, True),
                                              (torch.float32, True)])
def test_fused_step_equals_two_calls(dtype, with_bias):
    w, steps = DEC, 5
    hv = synth.decode_heads(w)
    say(f"fused decode vs two calls: batch={w.batch} steps={steps} dtype={dtype} bias={with_bias}")
    inp = _inputs(w, steps, dtype, w.batch, hv, with_bias)
    y2, st2, cs2 = _two_call(w, inp, steps, dtype)
    say("  fused run")
    yf, stf, csf = _fused(w, inp, steps, dtype)
    for k in range(steps):
        assert _same_nan(yf[k], y2[k]), k
    assert torch.equal(stf, st2)
    assert torch.equal(csf, cs2)


def test_fused_step_small_state_and_idle_sequences():
    """d_state 16 (4 lanes per state row), 32-wide heads, widths 0..4 per
    sequence: sequences with no active head still advance B and C."""
    w, steps, b = TINY, 4, 10
    hv = torch.tensor([i % 5 for i in range(b)], dtype=torch.int32)
    say(f"fused decode tiny fp32 batch={b} heads={hv.tolist()}")
    inp = _inputs(w, steps, torch.float32, b, hv, True)
    y2, st2, cs2 = _two_call(w, inp, steps, torch.float32)
    yf, stf, csf = _fused(w, inp, steps, torch.float32)
    for k in range(steps):
        assert _same_nan(yf[k], y2[k]), k
    assert torch.equal(stf, st2)
    assert torch.equal(csf, cs2)
    # a sequence without active heads: x taps unchanged, B/C taps advanced
    cs0 = inp["cs0"]
    assert torch.equal(csf[0, :, :w.d_inner].cpu(), cs0[0, :, :w.d_inner])
    raw = inp["xbc"][steps - 1][0, w.d_inner:].float()
    assert torch.equal(csf[0, 2, w.d_inner:].cpu(), raw)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_fused_step_64_tokens_against_oracle(dtype):
    """64 tokens on 24 sequences of the decode workload (widths 16/32/64 heads
    in turn) against the oracle's conv step and recurrent step in fp64."""
    w, steps, b = DEC, 64, 24
    hv = synth.decode_heads(w, batch=b)
    say(f"fused decode vs oracle: batch={b} steps={steps} dtype={dtype}")
    inp = _inputs(w, steps, dtype, b, hv, True, seed=91)
    yf, stf, csf = _fused(w, inp, steps, dtype)
    H, P, N = w.n_heads, w.d_head, w.d_state
    ost = f64(inp["st0"])
    ocs = conv_state_to_oracle(inp["cs0"])
    A, D = f64(inp["A"]), f64(inp["D"])
    yo = []
    for k in range(steps):
        u, ocs = oracle.conv1d_silu(f64(inp["xbc"][k]).reshape(b, 1, w.conv_dim), f64(inp["cw"]),
                                    f64(inp["cb"]), ocs, d_inner=w.d_inner, d_head=P,
                                    heads_active=hv.numpy())
        u = u[:, 0]
        yk, ost = oracle.ssd_step(ost, np.nan_to_num(u[:, :w.d_inner]).reshape(b, H, P),
                                  f64(inp["dt"][k]), A, u[:, w.d_inner:w.d_inner + N],
                                  u[:, w.d_inner + N:], D, heads_active=hv.numpy())
        yo.append(yk)
    tol = TOL[dtype]
    mask = np.zeros((b, H), bool)
    for bb in range(b):
        mask[bb, :int(hv[bb])] = True
    got = np.stack([f64(yf[k])[mask] for k in range(steps)])
    want = np.stack([yo[k][mask] for k in range(steps)])
    assert oracle.rel_l2(got, want) < tol
    for k in (0, steps // 2, steps - 1):  # every token checked alone too, at a few points
        assert oracle.rel_l2(f64(yf[k])[mask], yo[k][mask]) < tol
    assert oracle.rel_l2(f64(stf)[mask], ost[mask]) < tol
    ocs_t = conv_state_from_oracle(ocs)
    gcs = f64(csf)
    for bb in range(b):
        act = np.zeros(w.conv_dim, bool)
        act[:int(hv[bb]) * P] = True
        act[w.d_inner:] = True
        assert oracle.rel_l2(gcs[bb][:, act], ocs_t[bb][:, act]) < 1e-6


def test_fused_step_in_a_graph_replays():
    """Four fused tokens captured in a HIP graph (conv-state buffers in
    turn), replayed three times with eager work between the replays: every
    replay equals the same four tokens run eagerly from the same start."""
    w, steps, b = DEC, 4, 48
    hv = synth.decode_heads(w, batch=b)
    inp = _inputs(w, steps, torch.float32, b, hv, True, seed=5)
    say(f"fused decode in a graph: batch={b} steps={steps}")
    want_y, want_st, want_cs = _fused(w, inp, steps, torch.float32)
    H, P = w.n_heads, w.d_head
    st = torch.empty_like(want_st)
    cs = [torch.empty_like(want_cs), torch.empty_like(want_cs)]
    ys = [torch.empty((b, H, P), device=DEV) for _ in range(steps)]
    xbc = [inp["xbc"][k].to(DEV) for k in range(steps)]
    dts = [inp["dt"][k].to(DEV) for k in range(steps)]
    hvd = hv.to(DEV)
    cw, A, D, cb = inp["cw"].to(DEV), inp["A"].to(DEV), inp["D"].to(DEV), inp["cb"].to(DEV)

    def reset():
        st.copy_(inp["st0"])
        cs[0].copy_(inp["cs0"])
        for y in ys:
            y.fill_(float("nan"))

    def run():
        for k in range(steps):
            mm.ssd_step_fused(st, cs[k % 2], cs[(k + 1) % 2], xbc[k], cw, dts[k], A, D, cb,
                              n_heads_active=H, heads_per_seq=hvd, y=ys[k])

    reset()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(3):
        reset()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in range(steps):
            assert _same_nan(ys[k], want_y[k]), (rep, k)
        assert torch.equal(st, want_st), rep
        assert torch.equal(cs[steps % 2], want_cs), rep
        _ = (st * 2).sum().item()  # eager work between replays

"""Device canaries: every output and workspace buffer of the entry points is
placed between two guard regions filled with a sentinel, and each call must
leave both guards untouched (no write before the start or past the end of any
buffer it is given), at ragged lengths and at the split-sequence plans where
the workspace is used.  Outputs are also checked to be finite where written."""
import math

import pytest
import torch

import selective_state_space_12_amd as mm
import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
GUARD = 4096            # elements on each side (keeps 16-byte alignment)
SENT = 7776.0           # exact in bf16 and fp32
SENT_U8 = 0xA5          # workspace (byte) buffers


class Guarded:
    """A tensor of `shape` in the middle of a larger buffer whose two guard
    regions hold SENT."""

    def __init__(self, shape, dtype, fill=None):
        n = math.prod(shape)
        self.n = n
        self.sent = SENT_U8 if dtype == torch.uint8 else SENT
        self.buf = torch.full((n + 2 * GUARD,), self.sent, dtype=dtype, device=DEV)
        self.t = self.buf[GUARD:GUARD + n].view(shape)
        if fill is not None:
            self.t.copy_(fill)

    def check(self, name):
        torch.cuda.synchronize()
        lo, hi = self.buf[:GUARD], self.buf[GUARD + self.n:]
        assert bool((lo == self.sent).all()), f"{name}: write before the buffer"
        assert bool((hi == self.sent).all()), f"{name}: write past the buffer"


def _bytes_buf(nbytes):
    return Guarded((max(int(nbytes), 1),), torch.uint8)


def _ws_check(g):
    g.check("workspace")


@pytest.mark.parametrize("wname,b,l,m", [("130m", 2, 700, 192), ("130m", 1, 1500, 96),
                                         ("long", 1, 4000, 256), ("tiny", 1, 200, 32)])
def test_forward_guards(wname, b, l, m):
    """mm_ssd_forward: y, final_state and the workspace (used by the split
    plans of the few-unit cases)."""
    w = synth.WORKLOADS[wname]
    h = w.heads(m)
    inp = {k: v.to(DEV) for k, v in synth.forward_inputs(w, batch=b, seqlen=l, with_state=True).items()}
    H, P, N = w.n_heads, w.d_head, w.d_state
    y = Guarded((b, l, H, P), w.dtype)
    hf = Guarded((b, H, P, N), torch.float32)
    ws = _bytes_buf(mm.ssd_forward_workspace_size(b, l, H, P, N, 1, h, w.chunk, w.dtype))
    mm.ssd_forward(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], n_heads_active=h,
                   chunk=w.chunk, initial_state=inp["h0"], final_state=hf.t, y=y.t, workspace=ws.t)
    y.check("y")
    hf.check("final_state")
    _ws_check(ws)
    assert torch.isfinite(y.t[:, :, :h].float()).all()
    assert torch.isfinite(hf.t[:, :h]).all()


def test_fused_and_mixed_guards():
    """mm_ssd_forward_fused (conv state, final state, y, workspace) and
    mm_ssd_forward_mixed (y, workspace) at a ragged length."""
    w = synth.WORKLOADS["130m"]
    b, l = 3, 777
    H, P, N, cd = w.n_heads, w.d_head, w.d_state, w.conv_dim
    xi = synth.xbc_inputs(w, batch=b, seqlen=l)
    xbc, cw = xi["xbc"].to(DEV), xi["w"].to(DEV)
    dt = synth.pipeline_dt(w, batch=b, seqlen=l).to(DEV)
    A, D = synth.draw_A(w).to(DEV), synth.draw_D(w).to(DEV)
    h = w.heads(384)
    y = Guarded((b, l, H, P), w.dtype)
    hf = Guarded((b, H, P, N), torch.float32)
    cs = Guarded((b, 3, cd), torch.float32, fill=torch.zeros((b, 3, cd)))
    ws = _bytes_buf(mm.ssd_forward_fused_workspace_size(b, l, H, P, N, 1, h, w.chunk, w.dtype))
    mm.ssd_forward_fused(xbc, cw, dt, A, D, d_head=P, d_state=N, n_heads_active=h, chunk=w.chunk,
                         conv_state=cs.t, final_state=hf.t, y=y.t, workspace=ws.t)
    for g, name in ((y, "y"), (hf, "final_state"), (cs, "conv_state")):
        g.check(name)
    _ws_check(ws)
    inp = {k: v.to(DEV) for k, v in synth.forward_inputs(w, batch=b, seqlen=l).items()}
    hps = [w.heads(m) for m in (96, 768, 192)]
    y2 = Guarded((b, l, H, P), w.dtype)
    ws2 = _bytes_buf(mm.ssd_forward_mixed_workspace_size(b, l, H, P, N, 1, hps, w.chunk, w.dtype))
    mm.ssd_forward_mixed(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"],
                         heads_per_seq=hps, chunk=w.chunk, y=y2.t, workspace=ws2.t)
    y2.check("mixed y")
    _ws_check(ws2)


@pytest.mark.parametrize("accumulate", [False, True])
def test_backward_guards(accumulate):
    """mm_ssd_backward: every gradient and the workspace, at a ragged length
    with a split-sequence plan (few walks)."""
    w = synth.WORKLOADS["130m"]
    b, l, m = 1, 1900, 96
    h = w.heads(m)
    H, P, N = w.n_heads, w.d_head, w.d_state
    inp = {k: v.to(DEV) for k, v in synth.forward_inputs(w, batch=b, seqlen=l, with_state=True).items()}
    dy = synth.cotangents(w, batch=b, seqlen=l)["dy"].to(DEV)
    dhT = torch.randn((b, H, P, N), generator=torch.Generator().manual_seed(3)).to(DEV)
    z = lambda shape, dt: torch.zeros(shape, dtype=dt) if accumulate else None
    g = {"dx": Guarded((b, l, H, P), w.dtype, fill=z((b, l, H, P), w.dtype)),
         "ddt": Guarded((b, l, H), w.dtype, fill=z((b, l, H), w.dtype)),
         "dA": Guarded((H,), torch.float32, fill=z((H,), torch.float32)),
         "dB": Guarded((b, l, 1, N), torch.float32, fill=z((b, l, 1, N), torch.float32)),
         "dC": Guarded((b, l, 1, N), torch.float32, fill=z((b, l, 1, N), torch.float32)),
         "dD": Guarded((H,), torch.float32, fill=z((H,), torch.float32)),
         "dinitial_state": Guarded((b, H, P, N), torch.float32, fill=z((b, H, P, N), torch.float32))}
    assert mm.ssd_backward_segments(b, l, H, P, N, 1, h, w.dtype) > 1
    ws = _bytes_buf(mm.ssd_backward_workspace_size(b, l, H, P, N, 1, h, w.dtype))
    out = mm.ssd_backward(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], dy,
                          n_heads_active=h, initial_state=inp["h0"], dfinal_state=dhT,
                          grads={k: v.t for k, v in g.items()}, accumulate=accumulate,
                          want_dinitial=True, workspace=ws.t)
    for k, v in g.items():
        v.check(k)
    _ws_check(ws)
    assert torch.isfinite(out["dx"][:, :, :h].float()).all()
    assert torch.isfinite(out["dB"]).all() and torch.isfinite(out["dC"]).all()


def test_decode_conv_norm_guards():
    """mm_conv1d_silu (out, conv state), mm_ssd_step (state, y) at mixed
    widths, mm_conv1d_silu_backward (dxbc, dw) and mm_gated_rmsnorm (out)."""
    d = synth.WORKLOADS["decode"]
    bsz, H, P, N, cd, di = 24, d.n_heads, d.d_head, d.d_state, d.conv_dim, d.d_inner
    pool = synth.decode_pool(d, pool=2, batch=bsz)
    hv = synth.decode_heads(d, batch=bsz).to(DEV)
    A, D, cw = synth.draw_A(d).to(DEV), synth.draw_D(d).to(DEV), synth.draw_conv_w(d).to(DEV)
    st = Guarded((bsz, H, P, N), torch.float32, fill=torch.zeros((bsz, H, P, N)))
    cs = Guarded((bsz, 3, cd), torch.float32, fill=torch.zeros((bsz, 3, cd)))
    u = Guarded((bsz, 1, cd), torch.float32)
    yt = Guarded((bsz, H, P), torch.float32)
    for k in range(2):
        mm.conv1d_silu(pool["xbc_t"][k].to(DEV).unsqueeze(1), cw, None, cs.t, d_inner=di, d_head=P,
                       d_state=N, n_heads_active=H, heads_per_seq=hv, out=u.t)
        u2 = u.t[:, 0]
        mm.ssd_step(st.t, u2[:, :di].view(bsz, H, P), pool["dt_t"][k].to(DEV), A, u2[:, di:di + N],
                    u2[:, di + N:], D, n_heads_active=H, heads_per_seq=hv, y=yt.t)
    for g, name in ((st, "state"), (cs, "conv_state"), (u, "conv out"), (yt, "y")):
        g.check(name)
    w = synth.WORKLOADS["130m"]
    b, l = 2, 333
    xi = synth.xbc_inputs(w, batch=b, seqlen=l)
    xbc, cw2 = xi["xbc"].to(DEV), xi["w"].to(DEV)
    dout = synth.conv_cotangent(w, batch=b, seqlen=l).to(DEV)
    dx = Guarded(tuple(xbc.shape), xbc.dtype)
    dw = Guarded((w.conv_dim, 4), torch.float32)
    mm.conv1d_silu_backward(xbc, cw2, dout, d_inner=w.d_inner, d_head=w.d_head, d_state=w.d_state,
                            grads={"dxbc": dx.t, "dw": dw.t})
    dx.check("dxbc")
    dw.check("dw")
    gi = synth.gate_inputs(w, batch=b, seqlen=l)
    gy, gz, gw = gi["y"].to(DEV), gi["z"].to(DEV), gi["w"].to(DEV)
    out = Guarded(tuple(gy.shape), gy.dtype)
    mm.gated_rmsnorm(gy, gz, gw, 1e-5, d=gy.shape[-1], out=out.t)
    out.check("gated_rmsnorm out")


def test_fused_decode_guards():
    """mm_ssd_step_fused: state, both conv-state buffers (the one read must
    stay unchanged) and y, at mixed widths including sequences with no active
    head, over two tokens with the buffers swapped."""
    d = synth.WORKLOADS["decode"]
    bsz, H, P, N, cd = 24, d.n_heads, d.d_head, d.d_state, d.conv_dim
    pool = synth.decode_pool(d, pool=2, batch=bsz)
    hv = synth.decode_heads(d, batch=bsz)
    hv[::5] = 0
    hv = hv.to(DEV)
    A, D, cw = synth.draw_A(d).to(DEV), synth.draw_D(d).to(DEV), synth.draw_conv_w(d).to(DEV)
    st = Guarded((bsz, H, P, N), torch.float32, fill=torch.zeros((bsz, H, P, N)))
    cs = [Guarded((bsz, 3, cd), torch.float32, fill=torch.randn(bsz, 3, cd)),
          Guarded((bsz, 3, cd), torch.float32, fill=torch.full((bsz, 3, cd), float("nan")))]
    yt = Guarded((bsz, H, P), torch.float32)
    for k in range(2):
        before = cs[k % 2].t.clone()
        mm.ssd_step_fused(st.t, cs[k % 2].t, cs[(k + 1) % 2].t, pool["xbc_t"][k].to(DEV), cw,
                          pool["dt_t"][k].to(DEV), A, D, n_heads_active=H, heads_per_seq=hv, y=yt.t)
        torch.cuda.synchronize()
        assert torch.equal(cs[k % 2].t, before), "conv_state_in written"
        assert bool(torch.isfinite(cs[(k + 1) % 2].t).all()), "conv_state_out not fully written"
    for g, name in ((st, "state"), (cs[0], "conv_state a"), (cs[1], "conv_state b"), (yt, "y")):
        g.check(name)

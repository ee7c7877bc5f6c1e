"""GPU parity: the HIP kernels, called through the C ABI (ctypes binding),
against the fp64 oracle on the same seeded inputs.

Bars (relative L2 over the whole active slice): 1e-4 for fp32 storage, 2e-2
for bf16 storage with fp32 accumulation.  Small cases compare every element;
full-size workloads run the whole problem on the GPU and compare sampled
(sequence, head) units that the oracle recomputes over the full length.
"""
import numpy as np
import pytest
import torch

import oracle
import selective_state_space_12_amd as mm
import synth
from gpu_cases import (DEV, TOL, conv_state_from_oracle, conv_state_to_oracle, f64,
                       oracle_forward, rel_l2, run_forward, say)

pytestmark = pytest.mark.gpu

TINY = synth.WORKLOADS["tiny"]
M130 = synth.WORKLOADS["130m"]
B14 = synth.WORKLOADS["1.4b"]
LONG = synth.WORKLOADS["long"]
DEC = synth.WORKLOADS["decode"]


# ------------------------------------------------------------------ conv ----
@pytest.mark.parametrize("seqlen", [1, 5, 256])
@pytest.mark.parametrize("with_state", [False, True])
def test_conv_tiny_fp32_all_slices(seqlen, with_state):
    w = TINY
    inp = synth.xbc_inputs(w, seqlen=seqlen, with_state=True)
    for m in w.slices:
        h = w.heads(m)
        say(f"conv tiny fp32 l={seqlen} state={with_state} heads={h}")
        xin = inp["xbc"].to(DEV)
        out = torch.full_like(xin, float("nan"))
        cs = inp["conv_state"].to(DEV) if with_state else None
        mm.conv1d_silu(xin, inp["w"].to(DEV), None, cs, d_inner=w.d_inner, d_head=w.d_head,
                       d_state=w.d_state, n_heads_active=h, out=out)
        torch.cuda.synchronize()
        ref, st = oracle.conv1d_silu(inp["xbc"], inp["w"], None,
                                     conv_state_to_oracle(inp["conv_state"]) if with_state else None,
                                     d_inner=w.d_inner, d_head=w.d_head, heads_active=h)
        act = np.r_[0:h * w.d_head, w.d_inner:w.conv_dim]
        ina = np.r_[h * w.d_head:w.d_inner]
        got = f64(out)
        assert oracle.rel_l2(got[..., act], ref[..., act]) < TOL[torch.float32]
        assert np.isnan(got[..., ina]).all()
        if with_state:
            gs = f64(cs)
            want = conv_state_from_oracle(st)
            np.testing.assert_allclose(gs[:, :, act], want[:, :, act], rtol=0, atol=0)
            np.testing.assert_array_equal(gs[:, :, ina], f64(inp["conv_state"])[:, :, ina])


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("seqlen", [1, 100])
def test_conv_with_bias_and_state(dtype, seqlen):
    """The optional conv bias (MatMamba block paragraph: a conv layer over
    the concatenated x, B, C channels), through the multi-token kernel and the
    single-token decode kernel, with per-sequence widths."""
    w = M130
    b = 5
    inp = synth.xbc_inputs(w, batch=b, seqlen=seqlen, with_state=True, salt=3)
    bias = synth.draw_conv_bias(w)
    hv = [w.heads(m) for m in (96, 768, 384, 192, 768)]
    say(f"conv bias {dtype} l={seqlen} heads={hv}")
    xin = inp["xbc"].to(dtype).to(DEV)
    out = torch.full_like(xin, float("nan"))
    cs0 = inp["conv_state"]
    cs = cs0.to(DEV)
    mm.conv1d_silu(xin, inp["w"].to(DEV), bias.to(DEV), cs, d_inner=w.d_inner, d_head=w.d_head,
                   d_state=w.d_state, n_heads_active=w.n_heads,
                   heads_per_seq=torch.tensor(hv, dtype=torch.int32, device=DEV), out=out)
    torch.cuda.synchronize()
    ref, st = oracle.conv1d_silu(inp["xbc"].to(dtype), inp["w"], bias, conv_state_to_oracle(cs0),
                                 d_inner=w.d_inner, d_head=w.d_head, heads_active=hv)
    got, gs, want_s = f64(out), f64(cs), conv_state_from_oracle(st)
    for bb, h in enumerate(hv):
        act = np.r_[0:h * w.d_head, w.d_inner:w.conv_dim]
        ina = np.r_[h * w.d_head:w.d_inner]
        assert oracle.rel_l2(got[bb][..., act], ref[bb][..., act]) < TOL[dtype]
        assert np.isnan(got[bb][..., ina]).all()
        np.testing.assert_allclose(gs[bb][:, act], want_s[bb][:, act], rtol=0, atol=0)
        np.testing.assert_array_equal(gs[bb][:, ina], f64(cs0)[bb][:, ina])


def test_conv_bf16_per_sequence_slices_and_long_run():
    w = M130
    b, l = 3, 300
    inp = synth.xbc_inputs(w, batch=b, seqlen=l, with_state=True)
    hv = [w.heads(m) for m in (96, 768, 384)]
    say(f"conv bf16 130m b={b} l={l} heads={hv}")
    xin = inp["xbc"].to(DEV)
    out = torch.full_like(xin, float("nan"))
    cs0 = inp["conv_state"]
    cs = cs0.to(DEV)
    mm.conv1d_silu(xin, inp["w"].to(DEV), None, cs, d_inner=w.d_inner, d_head=w.d_head,
                   d_state=w.d_state, n_heads_active=w.n_heads,
                   heads_per_seq=torch.tensor(hv, dtype=torch.int32, device=DEV), out=out)
    torch.cuda.synchronize()
    ref, st = oracle.conv1d_silu(inp["xbc"], inp["w"], None, conv_state_to_oracle(cs0),
                                 d_inner=w.d_inner, d_head=w.d_head, heads_active=hv)
    got, gs, want_s = f64(out), f64(cs), conv_state_from_oracle(st)
    for bb, h in enumerate(hv):
        act = np.r_[0:h * w.d_head, w.d_inner:w.conv_dim]
        ina = np.r_[h * w.d_head:w.d_inner]
        assert oracle.rel_l2(got[bb][..., act], ref[bb][..., act]) < TOL[torch.bfloat16]
        assert np.isnan(got[bb][..., ina]).all()
        # new state = last three inputs (exact copies of bf16 values)
        np.testing.assert_array_equal(gs[bb][:, act], want_s[bb][:, act])
        np.testing.assert_array_equal(gs[bb][:, ina], f64(cs0)[bb][:, ina])


# ------------------------------------------------------------- scan, fp32 ----
@pytest.mark.parametrize("seqlen", [1, 7, 100, 256, 300])
@pytest.mark.parametrize("chunk", [16, 32, 64, 128, 256])
def test_scan_tiny_fp32_all_slices_and_chunks(seqlen, chunk):
    w = TINY
    inp = synth.forward_inputs(w, seqlen=seqlen, with_state=True)
    for m in w.slices:
        h = w.heads(m)
        say(f"scan tiny fp32 l={seqlen} chunk={chunk} heads={h}")
        y, hT = run_forward(inp, h, chunk, y_fill=float("nan"))
        yr, hr = oracle_forward(inp, h)
        assert rel_l2(y[:, :, :h], yr) < TOL[torch.float32]
        assert rel_l2(hT[:, :h], hr) < TOL[torch.float32]
        assert torch.isnan(y[:, :, h:]).all() and torch.isnan(hT[:, h:]).all()


# ------------------------------------------------------------- scan, bf16 ----
@pytest.mark.parametrize("chunk", [64, 256])
def test_scan_130m_bf16_all_slices_ragged(chunk):
    w = M130
    inp = synth.forward_inputs(w, batch=2, seqlen=600, with_state=True)
    for m in w.slices:
        h = w.heads(m)
        say(f"scan 130m bf16 b=2 l=600 chunk={chunk} heads={h}")
        y, hT = run_forward(inp, h, chunk, y_fill=float("nan"))
        yr, hr = oracle_forward(inp, h)
        e_y, e_h = rel_l2(y[:, :, :h], yr), rel_l2(hT[:, :h], hr)
        say(f"  rel_l2 y={e_y:.3e} state={e_h:.3e}")
        assert e_y < TOL[torch.bfloat16] and e_h < TOL[torch.bfloat16]
        assert torch.isnan(y[:, :, h:]).all() and torch.isnan(hT[:, h:]).all()


@pytest.mark.parametrize("seqlen", [2048, 2000])
def test_scan_130m_full_shape_all_slices(seqlen):
    """The 130M-scale call (b=8) at every slice in the benchmark's launch
    configuration: 3 and 6 heads split each sequence into segments (8 of 2
    tiles, 4 of 4), 12 and 24 heads walk it whole; at 2000 tokens the
    last tile is ragged.  The oracle recomputes the first, middle and last
    active head of every sequence."""
    w = M130
    inp = synth.forward_inputs(w, batch=8, seqlen=seqlen, with_state=True, salt=7)
    want = {3: 8, 6: 4, 12: 1, 24: 1}
    for m in w.slices:
        h = w.heads(m)
        assert mm.ssd_forward_segments(8, seqlen, w.n_heads, 64, 128, 1, h, w.chunk, w.dtype) == want[h]
        say(f"scan 130m bf16 b=8 l={seqlen} heads={h}")
        y, hT = run_forward(inp, h, w.chunk, y_fill=float("nan"))
        sample = sorted({0, h // 2, h - 1})
        yr, hr = oracle_forward(inp, h, head_idx=sample)
        e_y, e_h = rel_l2(y[:, :, sample], yr), rel_l2(hT[:, sample], hr)
        say(f"  heads {sample}: rel_l2 y={e_y:.3e} state={e_h:.3e}")
        assert e_y < TOL[torch.bfloat16] and e_h < TOL[torch.bfloat16]
        assert torch.isnan(y[:, :, h:]).all() and torch.isnan(hT[:, h:]).all()


@pytest.mark.parametrize("seqlen", [1, 2, 127, 128, 129, 255, 257, 383])
def test_scan_bf16_tile_boundaries(seqlen):
    """The bf16 d_head 64 / d_state 128 path at lengths around its 128-token
    tiles (one sequence, one unsplit walk per head); one head and all heads;
    chunk 128 and 256; initial and final states; heads beyond the slice
    untouched."""
    w = M130
    inp = synth.forward_inputs(w, batch=1, seqlen=seqlen, with_state=True, salt=5)
    for h in (1, w.n_heads):
        yr, hr = oracle_forward(inp, h)
        for chunk in (128, 256):
            say(f"scan bf16 tile boundaries l={seqlen} heads={h} chunk={chunk}")
            y, hT = run_forward(inp, h, chunk, y_fill=float("nan"))
            e_y, e_h = rel_l2(y[:, :, :h], yr), rel_l2(hT[:, :h], hr)
            assert e_y < TOL[torch.bfloat16] and e_h < TOL[torch.bfloat16], (e_y, e_h)
            assert torch.isnan(y[:, :, h:]).all() and torch.isnan(hT[:, h:]).all()


@pytest.mark.parametrize("m", [256, 2048])
def test_scan_1p4b_full_size_sampled(m):
    """Full 1.4B-scale call (b=4, l=8192) in the benchmark's launch
    configuration; the oracle recomputes sampled heads over all 8192 tokens."""
    w = B14
    h = w.heads(m)
    inp = synth.forward_inputs(w)
    say(f"scan 1.4b bf16 full size heads={h}")
    y, hT = run_forward(inp, h, w.chunk, h0=False)
    sample = sorted({0, h // 2, h - 1})
    yr, hr = oracle_forward(inp, h, h0=False, head_idx=sample)
    e_y = rel_l2(y[:, :, sample], yr)
    e_h = rel_l2(hT[:, sample], hr)
    say(f"  heads {sample}: rel_l2 y={e_y:.3e} state={e_h:.3e}")
    assert e_y < TOL[torch.bfloat16] and e_h < TOL[torch.bfloat16]


@pytest.mark.parametrize("m", [256, 1024])
def test_scan_long_context_segments(m):
    """Long sequence with few (sequence, head) units: the call is split into
    segments chained through the workspace (inter-chunk state passing over
    many chunks).  Shorter than the 131072-token workload so the oracle can
    check every active head."""
    w = LONG
    h = w.heads(m)
    inp = synth.forward_inputs(w, seqlen=32768, with_state=True)
    say(f"scan long bf16 l=32768 heads={h}")
    y, hT = run_forward(inp, h, w.chunk)
    sample = list(range(h)) if h <= 8 else [0, 3, h - 1]
    yr, hr = oracle_forward(inp, h, head_idx=sample)
    e_y, e_h = rel_l2(y[:, :, sample], yr), rel_l2(hT[:, sample], hr)
    say(f"  rel_l2 y={e_y:.3e} state={e_h:.3e}")
    assert e_y < TOL[torch.bfloat16] and e_h < TOL[torch.bfloat16]


def test_scan_more_than_64_heads_segmented():
    """A block wider than the 130M one (96 heads of 64, 80 active): the
    per-tile dt staging runs over the heads in groups of 64, and the few
    (sequence, head) units split a 32-tile sequence (last tile ragged) into
    segments of 11, 11 and 10 tiles."""
    import dataclasses
    w = dataclasses.replace(M130, d_model=3072, d_inner=6144)
    h = 80
    inp = synth.forward_inputs(w, batch=1, seqlen=4000, with_state=True)
    assert mm.ssd_forward_segments(1, 4000, w.n_heads, 64, 128, 1, h, 256, w.dtype) == 3
    say(f"scan bf16 wide block: {w.n_heads} heads, {h} active, l=4000")
    y, hT = run_forward(inp, h, 256)
    sample = [0, 63, 64, 79]
    yr, hr = oracle_forward(inp, h, head_idx=sample)
    e_y, e_h = rel_l2(y[:, :, sample], yr), rel_l2(hT[:, sample], hr)
    say(f"  rel_l2 y={e_y:.3e} state={e_h:.3e}")
    assert e_y < TOL[torch.bfloat16] and e_h < TOL[torch.bfloat16]


def test_scan_long_context_full_length_sampled():
    w = LONG
    h = w.heads(256)
    inp = synth.forward_inputs(w)
    say(f"scan long bf16 full length l={w.seqlen} heads={h}")
    y, hT = run_forward(inp, h, w.chunk, h0=False)
    sample = [0, h - 1]
    yr, hr = oracle_forward(inp, h, h0=False, head_idx=sample)
    e_y, e_h = rel_l2(y[:, :, sample], yr), rel_l2(hT[:, sample], hr)
    say(f"  rel_l2 y={e_y:.3e} state={e_h:.3e}")
    assert e_y < TOL[torch.bfloat16] and e_h < TOL[torch.bfloat16]


# ------------------------------------------------------------- invariants ----
def _plan_is_single_segment(w, batch, seqlen, heads, chunk):
    return mm.ssd_forward_segments(batch, seqlen, w.n_heads, w.d_head, w.d_state, 1, heads,
                                   chunk, w.dtype) == 1


def test_nesting_bitwise_when_plans_match():
    """Sub-block M_i == first h_i heads of M_g, bit for bit, whenever both
    calls cut the sequence the same way: one (ragged) tile for every slice,
    and a multi-tile batch wide enough that neither call splits into
    segments."""
    w = B14
    cases = [(4, 120, [8, 16, 32, 64]), (8, 1000, [32, 64])]
    for b, l, hs in cases:
        inp = synth.forward_inputs(w, batch=b, seqlen=l, with_state=True)
        say(f"nesting 1.4b-shaped bf16 b={b} l={l}")
        yf, hf = run_forward(inp, w.n_heads, 256)
        for h in hs:
            assert _plan_is_single_segment(w, b, l, h, 256)
            ys, hs_ = run_forward(inp, h, 256)
            assert torch.equal(ys[:, :, :h], yf[:, :, :h])
            assert torch.equal(hs_[:, :h], hf[:, :h])


def test_deterministic_runs():
    w = M130
    inp = synth.forward_inputs(w, batch=2, seqlen=1000, with_state=True)
    say("determinism 130m bf16")
    y1, h1 = run_forward(inp, 12, 256)
    y2, h2 = run_forward(inp, 12, 256)
    assert torch.equal(y1, y2) and torch.equal(h1[:, :12], h2[:, :12])


def test_chunk_size_independence_bf16():
    w = M130
    inp = synth.forward_inputs(w, batch=2, seqlen=700, with_state=True)
    ys = {}
    for q in (32, 64, 128, 256):
        say(f"chunk independence q={q}")
        ys[q], _ = run_forward(inp, 6, q)
    ref = f64(ys[256][:, :, :6])
    for q in (32, 64, 128):
        assert oracle.rel_l2(f64(ys[q][:, :, :6]), ref) < TOL[torch.bfloat16]


def test_state_chaining_in_place():
    """forward(l1) -> final state -> forward(l2, initial_state) equals
    forward(l1 + l2); the state buffer is updated in place (aliased)."""
    w = TINY
    inp = synth.forward_inputs(w, seqlen=300, with_state=True)
    say("state chaining tiny fp32")
    dev = {k: v.to(DEV) for k, v in inp.items()}
    yfull, hfull = run_forward(inp, w.n_heads, 64)
    st = dev["h0"].clone()
    parts = []
    for a, b in ((0, 130), (130, 300)):
        sl = slice(a, b)
        parts.append(mm.ssd_forward(dev["x"][:, sl], dev["dt"][:, sl], dev["A"], dev["B"][:, sl],
                                    dev["C"][:, sl], dev["D"], chunk=64, initial_state=st,
                                    final_state=st))
    torch.cuda.synchronize()
    assert oracle.rel_l2(f64(torch.cat(parts, 1)), f64(yfull)) < TOL[torch.float32]
    assert oracle.rel_l2(f64(st), f64(hfull)) < TOL[torch.float32]


def test_conv_then_scan_through_strided_views():
    """The pipeline of the block: conv output [x | B | C] rows are read by the
    scan through row strides (no copies); dt is its own tensor."""
    w = M130
    b, l = 2, 520
    xi = synth.xbc_inputs(w, batch=b, seqlen=l)
    dt = synth.pipeline_dt(w, batch=b, seqlen=l)
    A, D = synth.draw_A(w), synth.draw_D(w)
    for m in (192, 768):
        h = w.heads(m)
        say(f"pipeline 130m bf16 heads={h}")
        xbc = torch.empty((b, l, w.conv_dim), dtype=w.dtype, device=DEV)
        mm.conv1d_silu(xi["xbc"].to(DEV), xi["w"].to(DEV), None, None, d_inner=w.d_inner,
                       d_head=w.d_head, d_state=w.d_state, n_heads_active=h, out=xbc)
        xv = xbc[..., :w.d_inner].view(b, l, w.n_heads, w.d_head)
        Bv = xbc[..., w.d_inner:w.d_inner + w.d_state].unsqueeze(2)
        Cv = xbc[..., w.d_inner + w.d_state:].unsqueeze(2)
        y = mm.ssd_forward(xv, dt.to(DEV), A.to(DEV), Bv, Cv, D.to(DEV), n_heads_active=h, chunk=256)
        torch.cuda.synchronize()
        u, _ = oracle.conv1d_silu(xi["xbc"], xi["w"], None, None, d_inner=w.d_inner,
                                  d_head=w.d_head, heads_active=h)
        xo = u[..., :w.d_inner].reshape(b, l, w.n_heads, w.d_head)[:, :, :h]
        Bo = u[..., w.d_inner:w.d_inner + w.d_state]
        Co = u[..., w.d_inner + w.d_state:]
        yr, _ = oracle.ssd_forward(xo, f64(dt)[:, :, :h], f64(A)[:h], Bo, Co, f64(D)[:h])
        e = rel_l2(y, yr)
        say(f"  rel_l2 y={e:.3e}")
        assert e < TOL[torch.bfloat16]


# ----------------------------------------------------------------- decode ----
def _decode_run(w, steps, dtype, batch=None):
    b = batch or w.batch
    pool = synth.decode_pool(w, pool=steps, batch=b)
    hv = synth.decode_heads(w, batch=b)
    A, D, cw = synth.draw_A(w), synth.draw_D(w), synth.draw_conv_w(w)
    H, P, N, cd = w.n_heads, w.d_head, w.d_state, w.conv_dim
    rng = torch.Generator().manual_seed(4242)
    st0 = torch.randn(b, H, P, N, generator=rng)
    cs0 = torch.randn(b, 3, cd, generator=rng)
    xbc_t = pool["xbc_t"].to(dtype)
    dt_t = pool["dt_t"].to(dtype)
    # HIP path: conv step (state roll) then scan step, per token
    st = st0.clone().to(DEV)
    st_sentinel = st.clone()
    cs = cs0.clone().to(DEV)
    hvd = hv.to(DEV)
    ys = []
    for k in range(steps):
        u = torch.empty((b, 1, cd), dtype=dtype, device=DEV)
        mm.conv1d_silu(xbc_t[k].unsqueeze(1).to(DEV), cw.to(DEV), None, cs, d_inner=w.d_inner,
                       d_head=P, d_state=N, n_heads_active=H, heads_per_seq=hvd, out=u)
        u2 = u[:, 0]
        y = torch.full((b, H, P), float("nan"), dtype=dtype, device=DEV)
        mm.ssd_step(st, u2[:, :w.d_inner].view(b, H, P), dt_t[k].to(DEV), A.to(DEV),
                    u2[:, w.d_inner:w.d_inner + N], u2[:, w.d_inner + N:], D.to(DEV),
                    n_heads_active=H, heads_per_seq=hvd, y=y)
        ys.append(y)
    torch.cuda.synchronize()
    # oracle
    ost = f64(st0)
    ocs = conv_state_to_oracle(cs0)
    yo = []
    for k in range(steps):
        u, ocs = oracle.conv1d_silu(f64(xbc_t[k]).reshape(b, 1, cd), cw, None, ocs,
                                    d_inner=w.d_inner, d_head=P, heads_active=hv.numpy())
        u = u[:, 0]
        yk, ost = oracle.ssd_step(ost, np.nan_to_num(u[:, :w.d_inner]).reshape(b, H, P), f64(dt_t[k]),
                                  A, u[:, w.d_inner:w.d_inner + N], u[:, w.d_inner + N:], D,
                                  heads_active=hv.numpy())
        yo.append(yk)
    return hv, ys, yo, st, ost, cs, ocs, st_sentinel


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_decode_mixed_slices(dtype):
    w = DEC
    steps = 6
    say(f"decode batch={w.batch} steps={steps} dtype={dtype}")
    hv, ys, yo, st, ost, cs, ocs, st0 = _decode_run(w, steps, dtype)
    tol = TOL[dtype]
    gst = f64(st)
    for bb in range(0, w.batch, 17):
        h = int(hv[bb])
        got = np.stack([f64(ys[k][bb, :h]) for k in range(steps)])
        want = np.stack([yo[k][bb, :h] for k in range(steps)])
        assert oracle.rel_l2(got, want) < tol
        assert torch.isnan(ys[0][bb, h:]).all()
        assert oracle.rel_l2(gst[bb, :h], ost[bb, :h]) < tol
        # inactive heads' state untouched
        assert torch.equal(st[bb, h:], st0[bb, h:])
    # overall over every sequence's active heads
    mask = np.zeros((w.batch, w.n_heads), bool)
    for bb in range(w.batch):
        mask[bb, :int(hv[bb])] = True
    assert oracle.rel_l2(gst[mask], ost[mask]) < tol
    act = np.zeros(w.conv_dim, bool)
    gcs = f64(cs)
    ocs_t = conv_state_from_oracle(ocs)
    for bb in range(0, w.batch, 31):
        act[:] = False
        act[:int(hv[bb]) * w.d_head] = True
        act[w.d_inner:] = True
        assert oracle.rel_l2(gcs[bb][:, act], ocs_t[bb][:, act]) < tol


def test_steps_equal_forward():
    """l single-token steps on the GPU == one chunked forward over l tokens."""
    w = TINY
    inp = synth.forward_inputs(w, seqlen=40, with_state=True)
    dev = {k: v.to(DEV) for k, v in inp.items()}
    say("steps == forward tiny fp32")
    yf, hf = run_forward(inp, w.n_heads, 16)
    st = dev["h0"].clone()
    ys = []
    for t in range(40):
        ys.append(mm.ssd_step(st, dev["x"][:, t], dev["dt"][:, t], dev["A"], dev["B"][:, t],
                              dev["C"][:, t], dev["D"]))
    torch.cuda.synchronize()
    assert oracle.rel_l2(f64(torch.stack(ys, 1)), f64(yf)) < TOL[torch.float32]
    assert oracle.rel_l2(f64(st), f64(hf)) < TOL[torch.float32]

"""The allocation-free scan entry point (mm_ssd_forward_noalloc) against the
workspace entry point it wraps (mm_ssd_forward), through the C ABI: same
kernels and the same segment plan, so the outputs and final states must be
identical bit for bit.  Two calls in a row on one GPU, the second smaller
(the shared device array keeps the first call's contents), then a call whose
workspace would exceed the array, which must be refused before anything runs.
"""
import pytest
import torch

import selective_state_space_12_amd as mm
import synth
from gpu_cases import DEV, say

pytestmark = pytest.mark.gpu


def _pair(w, b, l, h, chunk, salt):
    inp = synth.forward_inputs(w, batch=b, seqlen=l, with_state=True, salt=salt)
    d = {k: v.to(DEV) for k, v in inp.items()}
    H, P, N = w.n_heads, w.d_head, w.d_state
    y_ref = torch.full((b, l, H, P), float("nan"), dtype=w.dtype, device=DEV)
    y_na = torch.full_like(y_ref, float("nan"))
    s_ref = torch.full((b, H, P, N), float("nan"), device=DEV)
    s_na = torch.full_like(s_ref, float("nan"))
    mm.ssd_forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], n_heads_active=h, chunk=chunk,
                   initial_state=d["h0"], final_state=s_ref, y=y_ref)
    mm.ssd_forward_noalloc(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], n_heads_active=h,
                           chunk=chunk, initial_state=d["h0"], final_state=s_na, y=y_na)
    torch.cuda.synchronize()
    nan7 = lambda t: torch.nan_to_num(t.float(), nan=7.0)
    assert torch.equal(nan7(y_na), nan7(y_ref))
    assert torch.equal(nan7(s_na), nan7(s_ref))
    assert torch.isnan(y_na[:, :, h:]).all() and torch.isnan(s_na[:, h:]).all()
    assert not torch.isnan(y_na[:, :, :h]).any()


def test_noalloc_matches_workspace_call_twice():
    w = synth.WORKLOADS["1.4b"]
    cases = [(4, 4096, 64, 1), (1, 700, 8, 2)]  # the second smaller, and split into segments
    for b, l, h, salt in cases:
        need = mm.ssd_forward_workspace_size(b, l, w.n_heads, w.d_head, w.d_state, 1, h, w.chunk,
                                             w.dtype)
        nseg = mm.ssd_forward_segments(b, l, w.n_heads, w.d_head, w.d_state, 1, h, w.chunk, w.dtype)
        say(f"noalloc vs workspace call: b={b} l={l} heads={h} workspace={need} segments={nseg}")
        assert 0 < need <= 64 << 20
        _pair(w, b, l, h, w.chunk, salt)


def test_noalloc_general_path_and_refusal():
    w = synth.WORKLOADS["tiny"]
    say("noalloc fp32 tiny, 3 heads")
    _pair(w, 2, 300, 3, 64, 3)
    big = synth.WORKLOADS["long"]
    need = mm.ssd_forward_workspace_size(1, big.seqlen, big.n_heads, big.d_head, big.d_state, 1,
                                         8, big.chunk, big.dtype)
    assert need > 64 << 20
    say(f"noalloc refusal: workspace {need} bytes")
    x = torch.zeros((1, big.seqlen, big.n_heads, big.d_head), dtype=big.dtype, device=DEV)
    dt = torch.zeros((1, big.seqlen, big.n_heads), dtype=big.dtype, device=DEV)
    bc = torch.zeros((1, big.seqlen, 1, big.d_state), dtype=big.dtype, device=DEV)
    A = torch.zeros(big.n_heads, device=DEV)
    y = torch.empty_like(x)
    with pytest.raises(mm.MMError) as ei:
        mm.ssd_forward_noalloc(x, dt, A, bc, bc, None, n_heads_active=8, chunk=big.chunk, y=y)
    assert ei.value.status == -7  # MM_ERR_WORKSPACE

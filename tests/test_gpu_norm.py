"""GPU parity of the gated RMSNorm epilogue (mm_gated_rmsnorm) against the
fp64 oracle: every Matryoshka width of the 1.4B-scale rows, the tiny fp32
rows, rows wider than the kernel's register cache, strided and in-place
operands.  Bars: relative L2 1e-4 (fp32 storage), 2e-2 (bf16)."""
import pytest
import torch

import oracle
import selective_state_space_12_amd as mm
import synth
from gpu_cases import DEV, TOL, f64, rel_l2, say

pytestmark = pytest.mark.gpu
EPS = 1e-5


@pytest.mark.parametrize("name", ["tiny", "1.4b"])
def test_gated_rmsnorm_all_widths(name):
    w = synth.WORKLOADS[name]
    gi = synth.gate_inputs(w, batch=min(w.batch, 2), seqlen=min(w.seqlen, 2048))
    y, z, nw = gi["y"].to(DEV), gi["z"].to(DEV), gi["w"].to(DEV)
    for m in w.slices:
        d = w.heads(m) * w.d_head
        say(f"gated rmsnorm {name} d={d}")
        out = mm.gated_rmsnorm(y, z, nw, EPS, d=d)
        torch.cuda.synchronize()
        ref = oracle.gated_rmsnorm(gi["y"], gi["z"], gi["w"], EPS, d=d)
        e = rel_l2(out, ref)
        say(f"  rel_l2={e:.3e}")
        assert e < TOL[w.dtype]


def test_gated_rmsnorm_full_size_bf16():
    """All 32768 rows of the 1.4B workload at full width, the benchmark's call."""
    w = synth.WORKLOADS["1.4b"]
    gi = synth.gate_inputs(w)
    say("gated rmsnorm 1.4b full size")
    out = mm.gated_rmsnorm(gi["y"].to(DEV), gi["z"].to(DEV), gi["w"].to(DEV), EPS)
    torch.cuda.synchronize()
    ref = oracle.gated_rmsnorm(gi["y"], gi["z"], gi["w"], EPS, d=w.d_inner)
    e = rel_l2(out, ref)
    say(f"  rel_l2={e:.3e}")
    assert e < TOL[torch.bfloat16]


@pytest.mark.parametrize("d", [8, 512, 520, 1024, 1032, 2048, 2056, 4096, 4104, 8192, 8200, 12288])
def test_gated_rmsnorm_widths_and_cache_edge(d):
    """Row widths on both sides of every launch-shape limit: one wave per row
    holding 1 or 2 chunks of 8 values (up to 512, 1024), then four waves per
    row holding 1, 2 or 4 (up to 2048, 4096, 8192; wider rows recompute the
    gate in a second pass).  Five rows leave rows of the last workgroup
    empty for the one-wave shapes."""
    g = torch.Generator().manual_seed(d)
    y = torch.randn(5, d, generator=g).to(torch.bfloat16)
    z = torch.randn(5, d, generator=g).to(torch.bfloat16)
    nw = 1 + 0.1 * torch.randn(d, generator=g)
    say(f"gated rmsnorm d={d}")
    out = mm.gated_rmsnorm(y.to(DEV), z.to(DEV), nw.to(DEV), EPS)
    torch.cuda.synchronize()
    e = rel_l2(out, oracle.gated_rmsnorm(y, z, nw, EPS, d=d))
    assert e < TOL[torch.bfloat16], e


def test_gated_rmsnorm_strided_and_in_place():
    """z as a column range of a wider row (an in-projection view), out
    written over y, and the channels past d left alone."""
    w = synth.WORKLOADS["130m"]
    gi = synth.gate_inputs(w, batch=2, seqlen=300)
    d = w.heads(384) * w.d_head
    wide = torch.randn(2, 300, w.d_inner + 512, generator=torch.Generator().manual_seed(3)).to(w.dtype)
    wide[..., 256:256 + w.d_inner] = gi["z"]
    zv = wide.to(DEV)[..., 256:256 + w.d_inner]
    y = gi["y"].to(DEV)
    say("gated rmsnorm strided z, in place")
    res = mm.gated_rmsnorm(y, zv, gi["w"].to(DEV), EPS, d=d, out=y[..., :d])
    torch.cuda.synchronize()
    ref = oracle.gated_rmsnorm(gi["y"], gi["z"], gi["w"], EPS, d=d)
    assert rel_l2(res, ref) < TOL[torch.bfloat16]
    assert rel_l2(y[..., :d], ref) < TOL[torch.bfloat16]
    assert torch.equal(y[..., d:].cpu(), gi["y"][..., d:])


def test_gated_rmsnorm_rejects():
    y = torch.zeros(4, 20, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(mm.MMError):  # d not a multiple of 8
        mm.gated_rmsnorm(y, y.clone(), torch.ones(20, device=DEV), EPS, d=20)
    y = torch.zeros(4, 64, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(mm.MMError):  # out overlapping z
        mm.gated_rmsnorm(y.clone(), y, torch.ones(64, device=DEV), EPS, out=y)

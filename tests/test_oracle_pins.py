"""Pins for the fp64 oracle against things other than itself.

Each test fixes the oracle to a fact the pages or the mathematics fix:
hand-derived worked examples, brute force on tiny inputs (the dense
semiseparable-matrix form built with explicit loops, no cumsum), the chunked
algorithm written independently in numpy, closed forms (A = 0 -> prefix sums,
constant parameters -> a textbook IIR filter), degenerate cases, textbook
convolution routines, and invariants the pages state (nesting: a sub-block
M_i is the first h_i heads of M_g).  A dropped term, a wrong sign, an index
shifted by one, a transposed state or a reversed filter fails at least one.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.signal
import torch

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden", "scalar_worked_examples.json")


def _rand_case(rng, b=2, l=23, H=3, P=3, N=4, G=1, with_h0=True, with_D=True):
    x = rng.standard_normal((b, l, H, P))
    dt = np.log1p(np.exp(rng.standard_normal((b, l, H)) - 1.0))
    A = -np.exp(rng.uniform(0, math.log(16.0), H))
    B = rng.standard_normal((b, l, G, N)) / 2
    C = rng.standard_normal((b, l, G, N)) / 2
    D = rng.standard_normal(H) if with_D else None
    h0 = rng.standard_normal((b, H, P, N)) if with_h0 else None
    return x, dt, A, B, C, D, h0


def _brute_force(x, dt, A, B, C, D, h0):
    """Dense semiseparable form with explicit loops and no cumsum:
    y[t] = sum_{s<=t} (C_t.B_s) * exp(sum_{r=s+1..t} dt_r A) * dt_s * x_s
           + exp(sum_{r<=t} dt_r A) * (H0 . C_t) + D x_t
    H_final = exp(sum_r dt_r A) H0 + sum_s exp(sum_{r>s} dt_r A) dt_s x_s B_s^T."""
    b, l, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    y = np.zeros_like(x)
    hf = np.zeros((b, H, P, N))
    for bb in range(b):
        for h in range(H):
            g = h // (H // G)
            for t in range(l):
                for s in range(t + 1):
                    logdec = 0.0
                    for r in range(s + 1, t + 1):
                        logdec += dt[bb, r, h] * A[h]
                    cb = sum(C[bb, t, g, n] * B[bb, s, g, n] for n in range(N))
                    y[bb, t, h] += cb * math.exp(logdec) * dt[bb, s, h] * x[bb, s, h]
                if h0 is not None:
                    logdec = sum(dt[bb, r, h] * A[h] for r in range(t + 1))
                    y[bb, t, h] += math.exp(logdec) * (h0[bb, h] @ C[bb, t, g])
                if D is not None:
                    y[bb, t, h] += D[h] * x[bb, t, h]
            for p in range(P):
                for n in range(N):
                    acc = 0.0
                    if h0 is not None:
                        acc = math.exp(sum(dt[bb, r, h] * A[h] for r in range(l))) * h0[bb, h, p, n]
                    for s in range(l):
                        logdec = sum(dt[bb, r, h] * A[h] for r in range(s + 1, l))
                        acc += math.exp(logdec) * dt[bb, s, h] * x[bb, s, h, p] * B[bb, s, g, n]
                    hf[bb, h, p, n] = acc
    return y, hf


def _chunked_numpy(x, dt, A, B, C, D, h0, Q):
    """The chunked (SSD) algorithm in fp64 numpy, written independently of the
    oracle: per chunk, Lambda = inclusive cumsum of dt*A;
      Y_diag[t] = sum_{s<=t in chunk} exp(L_t - L_s) (C_t.B_s) dt_s x_s
      Y_off[t]  = exp(L_t) H_prev . C_t
      H_next    = exp(L_end) H_prev + sum_s exp(L_end - L_s) dt_s x_s B_s^T."""
    b, l, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    y = np.zeros_like(x)
    hf = np.zeros((b, H, P, N))
    for bb in range(b):
        for h in range(H):
            g = h // (H // G)
            Hs = h0[bb, h].copy() if h0 is not None else np.zeros((P, N))
            for c0 in range(0, l, Q):
                c1 = min(c0 + Q, l)
                a = dt[bb, c0:c1, h] * A[h]
                lam = np.cumsum(a)
                Cc, Bc = C[bb, c0:c1, g], B[bb, c0:c1, g]
                xc, dtc = x[bb, c0:c1, h], dt[bb, c0:c1, h]
                G_ = Cc @ Bc.T
                Lm = np.tril(np.exp(lam[:, None] - lam[None, :]))
                ydiag = (G_ * Lm) @ (dtc[:, None] * xc)
                yoff = np.exp(lam)[:, None] * (Cc @ Hs.T)
                y[bb, c0:c1, h] = ydiag + yoff + (D[h] * xc if D is not None else 0.0)
                w = np.exp(lam[-1] - lam) * dtc
                Hs = np.exp(lam[-1]) * Hs + (w[:, None] * xc).T @ Bc
            hf[bb, h] = Hs
    return y, hf


def test_worked_example_scalar():
    gold = json.load(open(GOLD))["ssd_scalar"]
    l = len(gold["x"])
    x = np.array(gold["x"]).reshape(1, l, 1, 1)
    dt = np.array(gold["dt"]).reshape(1, l, 1)
    B = np.array(gold["B"]).reshape(1, l, 1, 1)
    C = np.array(gold["C"]).reshape(1, l, 1, 1)
    y, hf = oracle.ssd_forward(x, dt, [gold["A"]], B, C, [gold["D"]])
    np.testing.assert_allclose(y.ravel(), gold["y"], rtol=1e-14)
    np.testing.assert_allclose(hf.ravel(), [gold["h_final"]], rtol=1e-14)


def test_worked_example_outer_product_layout():
    """P != N pins the state layout (P, N) with N contiguous, the outer
    product x (outer) B and the contraction with C."""
    gold = json.load(open(GOLD))["ssd_outer_product"]
    x = np.array(gold["x"]).reshape(1, 1, 1, 2)
    dt = np.array(gold["dt"]).reshape(1, 1, 1)
    B = np.array(gold["B"]).reshape(1, 1, 1, 3)
    C = np.array(gold["C"]).reshape(1, 1, 1, 3)
    h0 = np.array(gold["h0"]).reshape(1, 1, 2, 3)
    y, hf = oracle.ssd_forward(x, dt, [gold["A"]], B, C, [gold["D"]], h0)
    np.testing.assert_allclose(y.ravel(), np.ravel(gold["y"]), rtol=0, atol=1e-15)
    np.testing.assert_allclose(hf.ravel(), np.ravel(gold["h_final"]), rtol=0, atol=1e-15)


def test_worked_example_conv():
    gold = json.load(open(GOLD))["conv_silu"]
    u = np.array(gold["u"]).reshape(1, 3, 1)
    w = np.array(gold["w"]).reshape(1, 4)
    out, st = oracle.conv1d_silu(u, w, conv_state=np.zeros((1, 1, 3)), d_inner=1, d_head=1)
    np.testing.assert_allclose(out.ravel(), gold["out"], rtol=1e-15)
    np.testing.assert_allclose(st.ravel(), gold["state"], rtol=0)


@pytest.mark.parametrize("G", [1, 3])
@pytest.mark.parametrize("with_h0,with_D", [(True, True), (False, False)])
def test_brute_force_semiseparable(G, with_h0, with_D):
    rng = np.random.default_rng(7 + G)
    x, dt, A, B, C, D, h0 = _rand_case(rng, b=2, l=17, H=3, P=2, N=3, G=G,
                                       with_h0=with_h0, with_D=with_D)
    y, hf = oracle.ssd_forward(x, dt, A, B, C, D, h0)
    yb, hb = _brute_force(x, dt, A, B, C, D, h0)
    assert oracle.rel_l2(y, yb) < 1e-12
    assert oracle.rel_l2(hf, hb) < 1e-12


@pytest.mark.parametrize("Q", [1, 2, 7, 16, 64, 200])
def test_chunked_equals_sequential(Q):
    rng = np.random.default_rng(11)
    x, dt, A, B, C, D, h0 = _rand_case(rng, b=2, l=200, H=2, P=4, N=5)
    y, hf = oracle.ssd_forward(x, dt, A, B, C, D, h0)
    yc, hc = _chunked_numpy(x, dt, A, B, C, D, h0, Q)
    assert oracle.rel_l2(y, yc) < 1e-12
    assert oracle.rel_l2(hf, hc) < 1e-12


def test_decay_free_is_prefix_sum():
    """A = 0: H_t = H0 + sum_{s<=t} dt_s x_s B_s^T -> a cumulative sum."""
    rng = np.random.default_rng(3)
    x, dt, A, B, C, D, h0 = _rand_case(rng, b=1, l=64, H=2, P=3, N=4)
    A = np.zeros_like(A)
    y, hf = oracle.ssd_forward(x, dt, A, B, C, D, h0)
    outer = dt[..., None, None] * x[..., :, None] * B[:, :, 0, None, :][:, :, None]
    Hs = np.cumsum(outer, axis=1) + h0[:, None]
    yr = np.einsum("blhpn,bln->blhp", Hs, C[:, :, 0]) + D[None, None, :, None] * x
    assert oracle.rel_l2(y, yr) < 1e-13
    assert oracle.rel_l2(hf, Hs[:, -1]) < 1e-13


def test_time_invariant_is_iir_filter():
    """Constant dt, B, C: y_p = lfilter([dt (C.B)], [1, -exp(dt A)], x_p) + D x_p."""
    rng = np.random.default_rng(5)
    l, P, N = 300, 3, 6
    x = rng.standard_normal((1, l, 1, P))
    dtv, Av = 0.07, -2.5
    dt = np.full((1, l, 1), dtv)
    Bv = rng.standard_normal(N)
    Cv = rng.standard_normal(N)
    B = np.broadcast_to(Bv, (1, l, 1, N)).copy()
    C = np.broadcast_to(Cv, (1, l, 1, N)).copy()
    D = np.array([0.3])
    y, _ = oracle.ssd_forward(x, dt, [Av], B, C, D)
    alpha = math.exp(dtv * Av)
    for p in range(P):
        ref = scipy.signal.lfilter([dtv * (Cv @ Bv)], [1.0, -alpha], x[0, :, 0, p]) + 0.3 * x[0, :, 0, p]
        np.testing.assert_allclose(y[0, :, 0, p], ref, rtol=1e-11, atol=1e-12)


def test_memoryless_limits():
    rng = np.random.default_rng(9)
    x, dt, A, B, C, D, h0 = _rand_case(rng, b=1, l=40, H=2, P=3, N=4)
    # dt*A -> -inf: exp underflows to exactly 0, only the current token remains
    y, hf = oracle.ssd_forward(x, np.ones_like(dt), np.full(2, -1e4), B, C, D, h0)
    cb = np.einsum("bln,bln->bl", C[:, :, 0], B[:, :, 0])
    yr = cb[:, :, None, None] * x + D[None, None, :, None] * x
    np.testing.assert_allclose(y, yr, rtol=1e-15, atol=1e-15)
    # dt = 0: no input, no decay: y = H0 . C_t + D x_t and the state is unchanged
    y, hf = oracle.ssd_forward(x, np.zeros_like(dt), A, B, C, D, h0)
    yr = np.einsum("bhpn,bln->blhp", h0, C[:, :, 0]) + D[None, None, :, None] * x
    np.testing.assert_allclose(y, yr, rtol=1e-14, atol=1e-14)
    np.testing.assert_array_equal(hf, h0)


def test_linearity_in_x():
    rng = np.random.default_rng(13)
    x1, dt, A, B, C, D, _ = _rand_case(rng, b=1, l=50, H=2, P=3, N=4)
    x2 = rng.standard_normal(x1.shape)
    a, bcoef = 1.7, -0.6
    y1, _ = oracle.ssd_forward(x1, dt, A, B, C, D)
    y2, _ = oracle.ssd_forward(x2, dt, A, B, C, D)
    y12, _ = oracle.ssd_forward(a * x1 + bcoef * x2, dt, A, B, C, D)
    assert oracle.rel_l2(y12, a * y1 + bcoef * y2) < 1e-12


def test_steps_equal_forward_and_split_chaining():
    rng = np.random.default_rng(17)
    x, dt, A, B, C, D, h0 = _rand_case(rng, b=2, l=30, H=3, P=2, N=3)
    y, hf = oracle.ssd_forward(x, dt, A, B, C, D, h0)
    st = h0.copy()
    ys = []
    for t in range(x.shape[1]):
        yt, st = oracle.ssd_step(st, x[:, t], dt[:, t], A, B[:, t], C[:, t], D)
        ys.append(yt)
    assert oracle.rel_l2(np.stack(ys, 1), y) < 1e-13
    assert oracle.rel_l2(st, hf) < 1e-13
    l1 = 11
    ya, ha = oracle.ssd_forward(x[:, :l1], dt[:, :l1], A, B[:, :l1], C[:, :l1], D, h0)
    yb, hb = oracle.ssd_forward(x[:, l1:], dt[:, l1:], A, B[:, l1:], C[:, l1:], D, ha)
    assert oracle.rel_l2(np.concatenate([ya, yb], 1), y) < 1e-13
    assert oracle.rel_l2(hb, hf) < 1e-13


def test_nesting_invariant_bitwise():
    """MatMamba nesting paragraph: M_i's parameters are the prefix of M_g's
    (A[0:h_i], W_x[0:d_i]); the sub-block's scan is the first h_i heads."""
    rng = np.random.default_rng(19)
    x, dt, A, B, C, D, h0 = _rand_case(rng, b=3, l=33, H=4, P=3, N=4)
    yf, hff = oracle.ssd_forward(x, dt, A, B, C, D, h0)
    for hi in (1, 2, 3):
        ys, hs = oracle.ssd_forward(x[:, :, :hi], dt[:, :, :hi], A[:hi], B, C, D[:hi], h0[:, :hi])
        np.testing.assert_array_equal(ys, yf[:, :, :hi])
        np.testing.assert_array_equal(hs, hff[:, :hi])
        # the same slice requested through heads_active on the full tensors
        yp, hp = oracle.ssd_forward(x, dt, A, B, C, D, h0, heads_active=[hi] * 3)
        np.testing.assert_array_equal(yp[:, :, :hi], yf[:, :, :hi])
        assert np.isnan(yp[:, :, hi:]).all() and np.isnan(hp[:, hi:]).all()
    # per-sequence slices (Mix'n'Match across a batch)
    yp, hp = oracle.ssd_forward(x, dt, A, B, C, D, h0, heads_active=[1, 4, 2])
    for bb, hi in enumerate([1, 4, 2]):
        np.testing.assert_array_equal(yp[bb, :, :hi], yf[bb, :, :hi])
        np.testing.assert_array_equal(hp[bb, :hi], hff[bb, :hi])


def _torch_conv_ref(u, w, bias, hist):
    """torch's depthwise conv1d (cross-correlation) on [history | u] in fp64,
    then torch's SiLU: a library routine independent of the oracle."""
    b, l, cd = u.shape
    seq = np.concatenate([hist.transpose(0, 2, 1), u], axis=1)  # (b, 3+l, cd)
    t = torch.from_numpy(seq).permute(0, 2, 1)  # (b, cd, 3+l)
    wt = torch.from_numpy(w).reshape(cd, 1, 4)
    bt = torch.from_numpy(bias) if bias is not None else None
    pre = torch.nn.functional.conv1d(t, wt, bt, groups=cd)  # valid -> l outputs
    return torch.nn.functional.silu(pre).permute(0, 2, 1).numpy()


@pytest.mark.parametrize("l", [1, 2, 3, 5, 64])
def test_conv_matches_torch_and_state(l):
    rng = np.random.default_rng(23 + l)
    b, d_inner, d_head, N = 2, 8, 4, 3
    cd = d_inner + 2 * N
    u = rng.standard_normal((b, l, cd))
    w = rng.standard_normal((cd, 4)) * 0.5
    bias = rng.standard_normal(cd)
    st0 = rng.standard_normal((b, cd, 3))
    out, st = oracle.conv1d_silu(u, w, bias, st0, d_inner=d_inner, d_head=d_head)
    ref = _torch_conv_ref(u, w, bias, st0)
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-14)
    full = np.concatenate([st0, u.transpose(0, 2, 1)], axis=2)
    np.testing.assert_array_equal(st, full[:, :, -3:])
    # zero history == torch conv1d with padding=3, first l outputs
    out0, _ = oracle.conv1d_silu(u, w, None, None, d_inner=d_inner, d_head=d_head)
    t = torch.from_numpy(u).permute(0, 2, 1)
    pre = torch.nn.functional.conv1d(t, torch.from_numpy(w).reshape(cd, 1, 4), None,
                                     padding=3, groups=cd)[..., :l]
    np.testing.assert_allclose(out0, torch.nn.functional.silu(pre).permute(0, 2, 1).numpy(),
                               rtol=1e-13, atol=1e-14)
    # np.convolve with the reversed filter, one channel
    c = 5
    pre_np = np.convolve(u[0, :, c], w[c, ::-1])[:l]
    np.testing.assert_allclose(out0[0, :, c], pre_np / (1 + np.exp(-pre_np)), rtol=1e-13)


def test_conv_slice_leaves_inactive_channels():
    rng = np.random.default_rng(29)
    b, l, d_inner, d_head, N = 3, 6, 8, 2, 2
    cd = d_inner + 2 * N
    u = rng.standard_normal((b, l, cd))
    w = rng.standard_normal((cd, 4))
    st0 = rng.standard_normal((b, cd, 3))
    full, stf = oracle.conv1d_silu(u, w, None, st0, d_inner=d_inner, d_head=d_head)
    hv = [1, 4, 2]
    part, stp = oracle.conv1d_silu(u, w, None, st0, d_inner=d_inner, d_head=d_head,
                                   heads_active=hv)
    for bb, h in enumerate(hv):
        act = np.r_[0:h * d_head, d_inner:cd]
        ina = np.r_[h * d_head:d_inner]
        np.testing.assert_array_equal(part[bb][:, act], full[bb][:, act])
        assert np.isnan(part[bb][:, ina]).all()
        np.testing.assert_array_equal(stp[bb][act], stf[bb][act])
        np.testing.assert_array_equal(stp[bb][ina], st0[bb][ina])


def test_slice_resolution():
    """h_i = e*m_i/d_head with (e*m_i) mod d_head == 0 (MatMamba nesting and
    Mix'n'Match paragraphs)."""
    assert [oracle.heads_for_dim(64, 128, 32, m) for m in (16, 32, 64)] == [1, 2, 4]
    assert [oracle.heads_for_dim(768, 1536, 64, m) for m in (96, 192, 384, 768)] == [3, 6, 12, 24]
    assert [oracle.heads_for_dim(2048, 4096, 64, m) for m in (256, 512, 1024, 2048)] == [8, 16, 32, 64]
    assert oracle.heads_for_dim(1024, 2048, 64, 768) == 24  # an untrained interpolated width
    for bad in (0, -32, 2049, 16, 100):
        with pytest.raises(ValueError):
            oracle.heads_for_dim(2048, 4096, 64, bad)


def test_softplus_closed_forms():
    """softplus(v) = log(1 + e^v): softplus(0) = ln 2, softplus(v) -
    softplus(-v) = v (e^v = (1 + e^v)/(1 + e^-v)), softplus(v) -> v for large v
    and -> e^v for very negative v; agrees with torch's fp64 softplus."""
    assert abs(oracle.softplus(0.0) - math.log(2.0)) < 1e-16
    v = np.linspace(-30.0, 30.0, 241)
    np.testing.assert_allclose(oracle.softplus(v) - oracle.softplus(-v), v, rtol=0, atol=1e-13)
    assert oracle.softplus(60.0) == 60.0
    assert abs(oracle.softplus(-40.0) / math.exp(-40.0) - 1.0) < 1e-12
    ref = torch.nn.functional.softplus(torch.from_numpy(v), beta=1.0, threshold=1000.0).numpy()
    np.testing.assert_allclose(oracle.softplus(v), ref, rtol=1e-14, atol=1e-300)


@pytest.mark.parametrize("softplus_on", [False, True])
def test_fused_composition_columns_and_dt(softplus_on):
    """The fused prefill composition takes x, B and C from the d_inner, d_state
    and d_state column ranges of the conv output and feeds dt + dt_bias
    (through softplus) to the scan.  With a current-token-only conv filter the
    conv output is SiLU(u) = u * expit(u) (scipy's logistic function), so the
    expected result is the scan on independently sliced columns; the returned
    conv state is the last three raw inputs."""
    import scipy.special
    rng = np.random.default_rng(41)
    b, l, H, P, N = 2, 9, 3, 2, 3
    d_inner = H * P
    cd = d_inner + 2 * N
    u = rng.standard_normal((b, l, cd))
    w = np.zeros((cd, 4))
    w[:, 3] = 1.0
    dt = rng.standard_normal((b, l, H)) - 1.0
    dtb = rng.standard_normal(H) * 0.3
    A = -np.exp(rng.uniform(0, math.log(16.0), H))
    D = rng.standard_normal(H)
    h0 = rng.standard_normal((b, H, P, N))
    st0 = rng.standard_normal((b, cd, 3))
    for h in (1, H):
        y, hf, st = oracle.ssd_forward_fused(u, w, dt, A, D, d_inner=d_inner, d_head=P,
                                             conv_state=st0, dt_bias=dtb, dt_softplus=softplus_on,
                                             h0=h0, heads_active=h)
        s = u * scipy.special.expit(u)
        x = np.stack([s[:, :, k * P:(k + 1) * P] for k in range(H)], axis=2)
        Bm = s[:, :, d_inner:d_inner + N][:, :, None, :]
        Cm = s[:, :, d_inner + N:][:, :, None, :]
        de = dt + dtb[None, None, :]
        if softplus_on:
            de = np.log1p(np.exp(de))
        yr, hr = oracle.ssd_forward(x, de, A, Bm, Cm, D, h0, heads_active=h)
        np.testing.assert_allclose(y[:, :, :h], yr[:, :, :h], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(hf[:, :h], hr[:, :h], rtol=1e-12, atol=1e-13)
        act = np.r_[0:h * P, d_inner:cd]
        np.testing.assert_array_equal(st[:, act], u[:, -3:, :].transpose(0, 2, 1)[:, act])


def test_gated_rmsnorm_against_torch_and_order():
    """Gated RMSNorm over the first d channels: against torch's rms_norm of
    y * silu(z) (fp64); the gate comes before the norm, so with w = 1 and
    eps = 0 every output row has mean square exactly 1 (a norm applied before
    the gate would not); z large makes the gate the identity times z, so the
    result is the plain RMSNorm of y; channels past d never matter."""
    rng = np.random.default_rng(51)
    rows, width, d = 7, 24, 16
    y = rng.standard_normal((rows, width))
    z = rng.standard_normal((rows, width)) * 2
    w = rng.standard_normal(width)
    eps = 1e-5
    out = oracle.gated_rmsnorm(y, z, w, eps, d=d)
    g = torch.from_numpy(y[:, :d]) * torch.nn.functional.silu(torch.from_numpy(z[:, :d]))
    ref = torch.nn.functional.rms_norm(g, (d,), weight=torch.from_numpy(w[:d]), eps=eps).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-14)
    unit = oracle.gated_rmsnorm(y, z, np.ones(width), 0.0, d=d)
    np.testing.assert_allclose((unit ** 2).mean(axis=1), 1.0, rtol=1e-13)
    big = oracle.gated_rmsnorm(y, np.full_like(z, 40.0), np.ones(width), 0.0, d=d)
    plain = y[:, :d] / np.sqrt((y[:, :d] ** 2).mean(axis=1, keepdims=True))
    np.testing.assert_allclose(big, plain, rtol=1e-13)
    y2, z2 = y.copy(), z.copy()
    y2[:, d:] = 1e9
    z2[:, d:] = -1e9
    np.testing.assert_array_equal(oracle.gated_rmsnorm(y2, z2, w, eps, d=d), out)

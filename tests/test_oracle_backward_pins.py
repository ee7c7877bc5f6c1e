"""Pins for the oracle's backward functions (CPU only).

The gradients are checked against central finite differences of the oracle's
own forward functions, which are pinned separately (test_oracle_pins.py):
the backward code shares nothing with the forward code it differentiates, so
a dropped term, a wrong sign or a transposed operand in the chain rule shows
up as a mismatch with the difference quotient.  fp64 with a step of 1e-6 is
accurate to about 1e-9 relative here.  A one-token closed form pins the
same quantities once more without any differencing."""
import numpy as np
import pytest

import oracle

EPS = 1e-6


def _fd(loss, arr):
    """Central differences of loss() with respect to every entry of arr
    (arr is modified in place and restored)."""
    g = np.zeros_like(arr)
    flat, gf = arr.reshape(-1), g.reshape(-1)
    for i in range(flat.size):
        v = flat[i]
        flat[i] = v + EPS
        lp = loss()
        flat[i] = v - EPS
        lm = loss()
        flat[i] = v
        gf[i] = (lp - lm) / (2 * EPS)
    return g


def _ssd_case(seed, b, l, h, P, N, ng):
    r = np.random.default_rng(seed)
    return {
        "x": r.standard_normal((b, l, h, P)),
        "dt": np.exp(r.uniform(-3.0, 0.0, (b, l, h))),
        "A": -np.exp(r.uniform(0.0, 2.0, h)),
        "B": r.standard_normal((b, l, ng, N)),
        "C": r.standard_normal((b, l, ng, N)),
        "D": r.standard_normal(h),
        "h0": r.standard_normal((b, h, P, N)),
        "dy": r.standard_normal((b, l, h, P)),
        "dhT": r.standard_normal((b, h, P, N)),
    }


@pytest.mark.parametrize("ng,heads", [(1, [2, 3]), (2, [4, 2]), (1, [3, 3])])
def test_ssd_backward_matches_finite_differences(ng, heads):
    """Every gradient of L = sum(dy*y) + sum(dhT*h_final), with per-sequence
    widths: inactive heads contribute nothing (their x, dt perturbations do
    not move L) and their gradient entries stay NaN."""
    h = 4 if ng == 2 else 3
    c = _ssd_case(11 + ng, 2, 6, h, 3, 4, ng)
    g = oracle.ssd_backward(c["x"], c["dt"], c["A"], c["B"], c["C"], c["D"], c["h0"], c["dy"],
                            c["dhT"], heads_active=heads)

    def loss():
        y, hf = oracle.ssd_forward(c["x"], c["dt"], c["A"], c["B"], c["C"], c["D"], c["h0"],
                                   heads_active=heads)
        return float(np.nansum(y * c["dy"]) + np.nansum(hf * c["dhT"]))

    act = np.zeros((2, h), bool)
    for bi, hb in enumerate(heads):
        act[bi, :hb] = True
    any_act = act.any(0)
    for name, key in [("x", "dx"), ("dt", "ddt"), ("A", "dA"), ("B", "dB"), ("C", "dC"),
                      ("D", "dD"), ("h0", "dh0")]:
        fd = _fd(loss, c[name])
        got = g[key]
        if key in ("dx", "ddt", "dh0"):
            mask = act.reshape(2, 1, h) if key != "dh0" else act
            if key == "dx":
                mask = act.reshape(2, 1, h, 1)
            elif key == "dh0":
                mask = act.reshape(2, h, 1, 1)
            mask = np.broadcast_to(mask, got.shape)
            assert np.isnan(got[~mask]).all(), key
            np.testing.assert_array_equal(fd[~mask], 0.0)
            np.testing.assert_allclose(got[mask], fd[mask], rtol=1e-6, atol=1e-7, err_msg=key)
        elif key in ("dA", "dD"):
            assert np.isnan(got[~any_act]).all()
            np.testing.assert_allclose(got[any_act], fd[any_act], rtol=1e-6, atol=1e-7,
                                       err_msg=key)
        else:
            np.testing.assert_allclose(got, fd, rtol=1e-6, atol=1e-7, err_msg=key)


def test_ssd_backward_without_optional_inputs():
    """No D, no initial state, no final-state cotangent: D and h0 act as zero
    and the recurrence starts from H = 0."""
    c = _ssd_case(5, 1, 5, 2, 2, 3, 1)
    g = oracle.ssd_backward(c["x"], c["dt"], c["A"], c["B"], c["C"], None, None, c["dy"], None)

    def loss():
        y, _ = oracle.ssd_forward(c["x"], c["dt"], c["A"], c["B"], c["C"])
        return float((y * c["dy"]).sum())

    for name, key in [("x", "dx"), ("dt", "ddt"), ("A", "dA"), ("B", "dB"), ("C", "dC")]:
        np.testing.assert_allclose(g[key], _fd(loss, c[name]), rtol=1e-6, atol=1e-7, err_msg=key)
    # dh0 is the gradient with respect to the (zero) state before the first token
    h0 = np.zeros((1, 2, 2, 3))

    def loss_h0():
        y, _ = oracle.ssd_forward(c["x"], c["dt"], c["A"], c["B"], c["C"], None, h0)
        return float((y * c["dy"]).sum())

    np.testing.assert_allclose(g["dh0"], _fd(loss_h0, h0), rtol=1e-6, atol=1e-7)


def test_ssd_backward_one_token_closed_form():
    """One token from H0: h = a H0 + dt x B^T, y = h C + D x, a = exp(dt A).
    Then dx = dt (B.C) dy + D dy, dB = dt (dy.x) C, dC = h^T dy,
    ddt = A a <dy C^T, H0> + (dy.x)(B.C), dA = dt a <dy C^T, H0>,
    dD = dy.x, dh0 = a dy C^T (no final-state cotangent)."""
    r = np.random.default_rng(3)
    P, N = 3, 4
    x, dy = r.standard_normal(P), r.standard_normal(P)
    B, C, H0 = r.standard_normal(N), r.standard_normal(N), r.standard_normal((P, N))
    dt, A, D = 0.3, -1.7, 0.9
    a = np.exp(dt * A)
    h = a * H0 + dt * np.outer(x, B)
    g = oracle.ssd_backward(x.reshape(1, 1, 1, P), np.array(dt).reshape(1, 1, 1), [A],
                            B.reshape(1, 1, 1, N), C.reshape(1, 1, 1, N), [D],
                            H0.reshape(1, 1, P, N), dy.reshape(1, 1, 1, P))
    gc = np.outer(dy, C)
    np.testing.assert_allclose(g["dx"].ravel(), dt * (B @ C) * dy + D * dy, rtol=1e-13)
    np.testing.assert_allclose(g["dB"].ravel(), dt * (dy @ x) * C, rtol=1e-13)
    np.testing.assert_allclose(g["dC"].ravel(), h.T @ dy, rtol=1e-13)
    np.testing.assert_allclose(g["ddt"].ravel(), [A * a * (gc * H0).sum() + (dy @ x) * (B @ C)],
                               rtol=1e-13)
    np.testing.assert_allclose(g["dA"], [dt * a * (gc * H0).sum()], rtol=1e-13)
    np.testing.assert_allclose(g["dD"], [dy @ x], rtol=1e-13)
    np.testing.assert_allclose(g["dh0"].reshape(P, N), a * gc, rtol=1e-13)


@pytest.mark.parametrize("with_state,with_bias,heads", [(True, True, [1, 2]), (False, False, [2, 2]),
                                                         (True, False, [2, 1])])
def test_conv_backward_matches_finite_differences(with_state, with_bias, heads):
    """Gradients of sum(dout * conv1d_silu(u)) with respect to the input, the
    taps, the bias and the initial conv state; a sequence of 2 tokens (shorter
    than the window) and one of 5 are both covered by the two seeds' shapes."""
    for seqlen in (2, 5):
        r = np.random.default_rng(20 + seqlen)
        b, d_head, N = 2, 2, 2
        d_inner = 4
        conv_dim = d_inner + 2 * N
        u = r.standard_normal((b, seqlen, conv_dim))
        w = 0.7 * r.standard_normal((conv_dim, 4))
        bias = r.standard_normal(conv_dim) if with_bias else None
        st = r.standard_normal((b, conv_dim, 3)) if with_state else None
        dout = r.standard_normal((b, seqlen, conv_dim))
        g = oracle.conv1d_silu_backward(u, w, dout, bias, st, d_inner=d_inner, d_head=d_head,
                                        heads_active=heads)

        def loss():
            out, _ = oracle.conv1d_silu(u, w, bias, st, d_inner=d_inner, d_head=d_head,
                                        heads_active=heads)
            return float(np.nansum(out * dout))

        act = np.ones((b, conv_dim), bool)
        for bi, hb in enumerate(heads):
            act[bi, hb * d_head:d_inner] = False
        any_act = act.any(0)
        m = np.broadcast_to(act[:, None, :], u.shape)
        fd = _fd(loss, u)
        assert np.isnan(g["du"][~m]).all()
        np.testing.assert_allclose(g["du"][m], fd[m], rtol=1e-6, atol=1e-8)
        fd = _fd(loss, w)
        assert np.isnan(g["dw"][~any_act]).all()
        np.testing.assert_allclose(g["dw"][any_act], fd[any_act], rtol=1e-6, atol=1e-8)
        if with_bias:
            fd = _fd(loss, bias)
            np.testing.assert_allclose(g["dbias"][any_act], fd[any_act], rtol=1e-6, atol=1e-8)
        if with_state:
            fd = _fd(loss, st)
            ms = np.broadcast_to(act[:, :, None], st.shape)
            assert np.isnan(g["dstate"][~ms]).all()
            np.testing.assert_allclose(g["dstate"][ms], fd[ms], rtol=1e-6, atol=1e-8)

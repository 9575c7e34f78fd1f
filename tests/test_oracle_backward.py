"""Pins of the oracle's backward pass.

The gradient of the scalar L = sum(dy*y) + sum(dh_n*h_n) + sum(dc_n*c_n) with
respect to every input, initial state and parameter element is checked
against central finite differences of the forward oracle (itself pinned in
test_oracle_pins.py), on shapes small enough to perturb every element; a
planted mistake in the backward's chain rule breaks these checks
(test_oracle_mutations.py).  torch.autograd in float64 is a secondary
cross-check of the same gradients on a larger shape.
"""
import numpy as np
import pytest

import oracle
from layer_lstm_forward_amd.synth import Spec, make_inputs


def _loss(inp, x, params, h0, c0, wy, whn, wcn):
    s = inp.spec
    y, hn, cn = oracle.lstm_forward(x, params, s.hidden_size, s.num_layers, s.bidirectional, h0=h0, c0=c0,
                                    has_bias=s.has_bias)
    return float(np.sum(wy * y) + np.sum(whn * hn) + np.sum(wcn * cn))


def _weights(spec, seed):
    rng = np.random.default_rng(seed)
    D, H, L = spec.D, spec.hidden_size, spec.num_layers
    return (rng.standard_normal((spec.T, spec.B, D * H)), rng.standard_normal((L * D, spec.B, H)),
            rng.standard_normal((L * D, spec.B, H)))


@pytest.mark.parametrize("I,H,L,bidir,T,B,bias", [(2, 2, 1, False, 3, 2, True), (3, 2, 2, True, 3, 2, True),
                                                  (2, 3, 2, False, 4, 1, False), (1, 2, 1, True, 2, 3, True)])
def test_backward_matches_finite_differences(I, H, L, bidir, T, B, bias):
    spec = Spec(I, H, L, bidir, T, B, "f32", 4000 + I + 10 * H + 100 * L + T, "normal0.1", has_bias=bias)
    inp = make_inputs(spec)
    params = [p.astype(np.float64) * 3.0 for p in inp.params]  # every gate in its non-linear range
    x, h0, c0 = (a.astype(np.float64) for a in (inp.x, inp.h0, inp.c0))
    wy, whn, wcn = _weights(spec, 17)
    dx, dh0, dc0, dps = oracle.lstm_backward(x, params, H, L, bidir, wy, h0=h0, c0=c0, dh_n=whn, dc_n=wcn,
                                             has_bias=bias)
    eps = 1e-6

    def fd(arr, setter):
        g = np.empty_like(arr)
        for idx in np.ndindex(arr.shape):
            v = arr[idx]
            arr[idx] = v + eps
            lp = setter()
            arr[idx] = v - eps
            lm = setter()
            arr[idx] = v
            g[idx] = (lp - lm) / (2 * eps)
        return g

    run = lambda: _loss(inp, x, params, h0, c0, wy, whn, wcn)  # noqa: E731
    np.testing.assert_allclose(dx, fd(x, run), rtol=0, atol=2e-7)
    np.testing.assert_allclose(dh0, fd(h0, run), rtol=0, atol=2e-7)
    np.testing.assert_allclose(dc0, fd(c0, run), rtol=0, atol=2e-7)
    for k, p in enumerate(params):
        np.testing.assert_allclose(dps[k], fd(p, run), rtol=0, atol=2e-7, err_msg=f"param {k}")


def test_backward_zero_output_gradient_is_zero():
    spec = Spec(3, 4, 2, True, 3, 2, "f32", 4100, "normal0.1")
    inp = make_inputs(spec)
    dx, dh0, dc0, dps = oracle.lstm_backward(inp.x, inp.params, 4, 2, True, np.zeros((3, 2, 8)), h0=inp.h0,
                                             c0=inp.c0)
    for a in [dx, dh0, dc0] + dps:
        assert np.all(a == 0.0)


def test_backward_matches_torch_autograd_fp64():
    torch = pytest.importorskip("torch")
    spec = Spec(5, 6, 2, True, 5, 3, "f32", 4200, "normal0.1")
    inp = make_inputs(spec)
    H, L = 6, 2
    wy, whn, wcn = _weights(spec, 19)
    m = torch.nn.LSTM(5, H, L, bidirectional=True).double()
    flat = [p.astype(np.float64) for p in inp.params]
    with torch.no_grad():
        for p, v in zip(m._flat_weights, flat):
            p.copy_(torch.from_numpy(v))
    xt = torch.from_numpy(inp.x.astype(np.float64)).requires_grad_()
    h0t = torch.from_numpy(inp.h0.astype(np.float64)).requires_grad_()
    c0t = torch.from_numpy(inp.c0.astype(np.float64)).requires_grad_()
    y, (hn, cn) = m(xt, (h0t, c0t))
    loss = (y * torch.from_numpy(wy)).sum() + (hn * torch.from_numpy(whn)).sum() + (cn * torch.from_numpy(wcn)).sum()
    loss.backward()
    dx, dh0, dc0, dps = oracle.lstm_backward(inp.x, inp.params, H, L, True, wy, h0=inp.h0, c0=inp.c0, dh_n=whn,
                                             dc_n=wcn)
    np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dh0, h0t.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dc0, c0t.grad.numpy(), rtol=0, atol=1e-11)
    for k, p in enumerate(m._flat_weights):
        np.testing.assert_allclose(dps[k], p.grad.numpy(), rtol=0, atol=1e-11)


@pytest.mark.parametrize("L,bidir,lens", [(1, False, [3, 1, 4]), (2, True, [2, 4, 1]), (2, False, [4, 4, 2])])
def test_backward_with_lengths_matches_finite_differences(L, bidir, lens):
    # per-row lengths: padded steps leave the state alone and output 0, so the
    # gradients must flow around them; checked against finite differences of
    # the lengths forward (itself pinned by the brute force)
    spec = Spec(2, 2, L, bidir, 4, 3, "f32", 4500 + L, "normal0.1")
    inp = make_inputs(spec)
    H = spec.hidden_size
    params = [p.astype(np.float64) * 3.0 for p in inp.params]
    x, h0, c0 = (a.astype(np.float64) for a in (inp.x, inp.h0, inp.c0))
    wy, whn, wcn = _weights(spec, 23)
    lengths = np.array(lens, np.int32)
    dx, dh0, dc0, dps = oracle.lstm_backward(x, params, H, L, bidir, wy, h0=h0, c0=c0, dh_n=whn, dc_n=wcn,
                                             lengths=lengths)

    def loss():
        y, hn, cn = oracle.lstm_forward(x, params, H, L, bidir, h0=h0, c0=c0, lengths=lengths)
        return float(np.sum(wy * y) + np.sum(whn * hn) + np.sum(wcn * cn))

    eps = 1e-6

    def fd(arr):
        g = np.empty_like(arr)
        for idx in np.ndindex(arr.shape):
            v = arr[idx]
            arr[idx] = v + eps
            lp = loss()
            arr[idx] = v - eps
            lm = loss()
            arr[idx] = v
            g[idx] = (lp - lm) / (2 * eps)
        return g

    np.testing.assert_allclose(dx, fd(x), rtol=0, atol=2e-7)
    np.testing.assert_allclose(dh0, fd(h0), rtol=0, atol=2e-7)
    np.testing.assert_allclose(dc0, fd(c0), rtol=0, atol=2e-7)
    for k, q in enumerate(params):
        np.testing.assert_allclose(dps[k], fd(q), rtol=0, atol=2e-7, err_msg=f"param {k}")


def test_backward_with_full_lengths_is_the_plain_backward():
    spec = Spec(3, 4, 2, True, 5, 3, "f32", 4600, "normal0.1")
    inp = make_inputs(spec)
    dy = np.random.default_rng(3).standard_normal((5, 3, 8))
    a = oracle.lstm_backward(inp.x, inp.params, 4, 2, True, dy, h0=inp.h0, c0=inp.c0)
    b = oracle.lstm_backward(inp.x, inp.params, 4, 2, True, dy, h0=inp.h0, c0=inp.c0, lengths=[5, 5, 5])
    for u, v in zip(a[:3], b[:3]):
        np.testing.assert_array_equal(u, v)
    for u, v in zip(a[3], b[3]):
        np.testing.assert_array_equal(u, v)

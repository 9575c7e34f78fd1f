"""Pins of the fp64 oracle against what the pages and the mathematics fix.

None of these compares the oracle with itself re-typed: each check comes from a
closed form, an invariant, a symmetry of the definition, a library routine the
pages themselves compare against (torch.nn.LSTMCell / torch.nn.LSTM), or an
independent per-gate brute force.  Together they are chosen so that a dropped
bias, a permuted gate block, a wrong layer/direction index, a reverse output
stored at the step index instead of the time index, or a transposed weight
fails at least one of them.
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle
from layer_lstm_forward_amd.synth import Spec, make_inputs
from tests import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def run(inp, **kw):
    s = inp.spec
    return oracle.lstm_forward(inp.x, inp.params, s.hidden_size, s.num_layers, s.bidirectional,
                               h0=inp.h0, c0=inp.c0, has_bias=s.has_bias, bf16=inp.bf16, **kw)


def sig(z):
    return 1.0 / (1.0 + np.exp(-z))


# --------------------------------------------------------------------------- Z
@pytest.mark.parametrize("L,bidir,T,B,H", [(1, False, 6, 2, 3), (2, True, 5, 3, 4), (3, False, 4, 1, 5),
                                            (3, True, 7, 2, 2)])
def test_zero_weight_closed_form(L, bidir, T, B, H):
    """All weights zero: gates are constants and c follows a geometric series.

    With W = 0 each gate is sigma/tanh of b_ih + b_hh alone, so after n steps
    c_n = f^n c_0 + i g (1 - f^n) / (1 - f) and h_n = o tanh(c_n) (warp-nn
    equation block).  The forward direction has taken t+1 steps at time t, the
    reverse one T-t steps.  Distinct per-gate biases make any gate permutation,
    a dropped bias vector or a wrong state index visible.
    """
    D = 2 if bidir else 1
    rng = np.random.default_rng(7 + L * 10 + T)
    I = 3
    params = []
    for l in range(L):
        for d in range(D):
            in_l = I if l == 0 else D * H
            params += [np.zeros((4 * H, in_l)), np.zeros((4 * H, H)),
                       rng.uniform(-1.5, 1.5, 4 * H), rng.uniform(-1.5, 1.5, 4 * H)]
    x = rng.standard_normal((T, B, I))
    h0 = rng.standard_normal((L * D, B, H))
    c0 = rng.standard_normal((L * D, B, H))
    y, hn, cn = oracle.lstm_forward(x, params, H, L, bidir, h0=h0, c0=c0)

    def closed(l, d, n):
        b = params[(l * D + d) * 4 + 2] + params[(l * D + d) * 4 + 3]
        i, f, g, o = sig(b[:H]), sig(b[H:2 * H]), np.tanh(b[2 * H:3 * H]), sig(b[3 * H:])
        cc = f ** n * c0[l * D + d] + i * g * (1 - f ** n) / (1 - f)
        return o * np.tanh(cc), cc

    for l in range(L):
        for d in range(D):
            h_T, c_T = closed(l, d, T)
            np.testing.assert_allclose(hn[l * D + d], h_T, rtol=0, atol=1e-13)
            np.testing.assert_allclose(cn[l * D + d], c_T, rtol=0, atol=1e-13)
    for t in range(T):
        for d in range(D):
            n = t + 1 if d == 0 else T - t
            h_t, _ = closed(L - 1, d, n)
            np.testing.assert_allclose(y[t, :, d * H:(d + 1) * H], h_t, rtol=0, atol=1e-13)


def test_zero_weight_gate_order_has_power():
    """Negative control: the closed form with gates permuted disagrees."""
    H, T = 4, 5
    rng = np.random.default_rng(3)
    params = [np.zeros((4 * H, 2)), np.zeros((4 * H, H)),
              rng.uniform(-1.5, 1.5, 4 * H), rng.uniform(-1.5, 1.5, 4 * H)]
    y, _, _ = oracle.lstm_forward(np.ones((T, 1, 2)), params, H, 1, False)
    b = params[2] + params[3]
    blocks = [b[q * H:(q + 1) * H] for q in range(4)]
    for perm in itertools.permutations(range(4)):
        i, f, g, o = (blocks[p] for p in perm)
        i, f, g, o = sig(i), sig(f), np.tanh(g), sig(o)
        cc = i * g * (1 - f ** T) / (1 - f)
        close = np.allclose(y[-1, 0], o * np.tanh(cc), atol=1e-12)
        assert close == (perm == (0, 1, 2, 3))


# --------------------------------------------------------------------------- I
@pytest.mark.parametrize("bidir", [False, True])
def test_invariants(bidir):
    """|h| <= |tanh(c)| <= 1 and |c_T| <= |c_0| + T (0 < f < 1, |i g| < 1)."""
    spec = Spec(5, 6, 2, bidir, 9, 3, "f32", 11, "normal0.1")
    inp = make_inputs(spec)
    # large weights push the gates into saturation
    inp.params = [p * 40.0 for p in inp.params]
    y, hn, cn = run(inp)
    for a in (y, hn, cn):
        assert np.all(np.isfinite(a))
    assert np.all(np.abs(y) <= 1.0)
    assert np.all(np.abs(hn) <= np.abs(np.tanh(cn)) + 1e-15)
    assert np.all(np.abs(cn) <= np.abs(inp.c0.astype(np.float64)) + spec.T + 1e-12)


# --------------------------------------------------------------------------- F
@pytest.mark.parametrize("state", ["zeros", "normal0.1"])
def test_time_flip(state):
    """The reverse direction equals a forward run on the time-flipped input.

    warp-nn: the reverse pass reads the sequence from the last element to the
    first with its own parameters; its output at time t has consumed x_{T-1}..x_t
    and its final state is the one after consuming x_0.
    """
    spec = Spec(4, 5, 1, True, 7, 3, "f32", 21, state)
    inp = make_inputs(spec)
    y, hn, cn = run(inp)
    H = spec.hidden_size
    pf, pr = inp.params[:4], inp.params[4:]
    h0f = None if inp.h0 is None else inp.h0[0:1]
    c0f = None if inp.c0 is None else inp.c0[0:1]
    h0r = None if inp.h0 is None else inp.h0[1:2]
    c0r = None if inp.c0 is None else inp.c0[1:2]
    yf, hnf, cnf = oracle.lstm_forward(inp.x, pf, H, 1, False, h0=h0f, c0=c0f)
    yr, hnr, cnr = oracle.lstm_forward(inp.x[::-1].copy(), pr, H, 1, False, h0=h0r, c0=c0r)
    np.testing.assert_array_equal(y[:, :, :H], yf)
    np.testing.assert_array_equal(y[:, :, H:], yr[::-1])
    np.testing.assert_array_equal(hn, np.concatenate([hnf, hnr]))
    np.testing.assert_array_equal(cn, np.concatenate([cnf, cnr]))
    # the reverse final state is the output at time 0
    np.testing.assert_array_equal(hn[1], y[0, :, H:])


# --------------------------------------------------------------------------- S
@pytest.mark.parametrize("bidir", [False, True])
def test_stacking(bidir):
    """An L-layer run is L chained one-layer runs; finals are collected per layer.

    MXNet blog, "Stack Multiple RNN Cells": only the output sequence feeds the
    next layer, each layer's final state is kept.  warp-nn: layer k > 0 reads
    the previous layer's D*H-wide output.
    """
    spec = Spec(3, 4, 3, bidir, 6, 2, "f32", 31, "normal0.1")
    inp = make_inputs(spec)
    y, hn, cn = run(inp)
    D, H = spec.D, spec.hidden_size
    seq = inp.x
    hns, cns = [], []
    for l in range(spec.num_layers):
        p = inp.params[l * D * 4:(l + 1) * D * 4]
        seq, a, b = oracle.lstm_forward(seq, p, H, 1, bidir, h0=inp.h0[l * D:(l + 1) * D],
                                        c0=inp.c0[l * D:(l + 1) * D])
        hns.append(a)
        cns.append(b)
    np.testing.assert_array_equal(y, seq)
    np.testing.assert_array_equal(hn, np.concatenate(hns))
    np.testing.assert_array_equal(cn, np.concatenate(cns))


# -------------------------------------------------------------------------- Bt
def test_batch_rows_independent():
    """No term couples batch rows: permuting rows permutes outputs, subsets match."""
    spec = Spec(5, 4, 2, True, 5, 6, "f32", 41, "normal0.1")
    inp = make_inputs(spec)
    y, hn, cn = run(inp)
    perm = np.array([3, 0, 5, 1, 4, 2])
    yp, hnp_, cnp = run(inp.rows(perm))
    np.testing.assert_array_equal(yp, y[:, perm])
    np.testing.assert_array_equal(hnp_, hn[:, perm])
    np.testing.assert_array_equal(cnp, cn[:, perm])
    ys, hs, cs = run(inp.rows([4]))
    np.testing.assert_array_equal(ys, y[:, [4]])
    np.testing.assert_array_equal(hs, hn[:, [4]])


def test_threads_do_not_change_results():
    spec = Spec(7, 9, 2, True, 4, 5, "f32", 42, "normal0.1")
    inp = make_inputs(spec)
    a = run(inp, nthreads=1)
    b = run(inp, nthreads=4)
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)


# -------------------------------------------------------------------------- Br
CASES = [(I, H, T, B, L, D) for I in (1, 3) for H in (1, 2, 3) for T in (1, 4) for B in (1, 2)
         for L in (1, 2) for D in (1, 2)]


@pytest.mark.parametrize("I,H,T,B,L,D", CASES)
def test_brute_force_per_gate(I, H, T, B, L, D):
    """Tiny shapes against the per-gate scalar evaluator in tests/brute.py."""
    spec = Spec(I, H, L, D == 2, T, B, "f32", 1000 + I * 100 + H * 10 + T + B + L + D, "normal0.1")
    inp = make_inputs(spec)
    # widen the value range so that every gate matters
    inp.params = [p * 3.0 for p in inp.params]
    y, hn, cn = run(inp)
    yb, hb, cb = brute.lstm(inp.x.astype(np.float64).tolist(),
                            [p.astype(np.float64).tolist() for p in inp.params], H, L, D,
                            h0=inp.h0.astype(np.float64).tolist(), c0=inp.c0.astype(np.float64).tolist())
    np.testing.assert_allclose(y, np.array(yb), rtol=0, atol=1e-14)
    np.testing.assert_allclose(hn, np.array(hb), rtol=0, atol=1e-14)
    np.testing.assert_allclose(cn, np.array(cb), rtol=0, atol=1e-14)


@pytest.mark.parametrize("I,H,T,B,L,D", [(2, 3, 4, 3, 1, 1), (3, 2, 5, 3, 2, 2), (1, 3, 4, 2, 2, 1),
                                          (3, 1, 3, 2, 1, 2)])
def test_brute_force_lengths(I, H, T, B, L, D):
    """Variable-length rows against the per-gate evaluator, which walks each
    row's own sequence (forward from its start, reverse from its last valid
    step) and leaves padded outputs at zero."""
    spec = Spec(I, H, L, D == 2, T, B, "f32", 2000 + I * 100 + H * 10 + T + B + L + D, "normal0.1")
    inp = make_inputs(spec)
    inp.params = [p * 3.0 for p in inp.params]
    lengths = [T] + [1 + (b * 2) % T for b in range(1, B)]
    y, hn, cn = run(inp, lengths=lengths)
    yb, hb, cb = brute.lstm(inp.x.astype(np.float64).tolist(),
                            [p.astype(np.float64).tolist() for p in inp.params], H, L, D,
                            h0=inp.h0.astype(np.float64).tolist(), c0=inp.c0.astype(np.float64).tolist(),
                            lengths=lengths)
    np.testing.assert_allclose(y, np.array(yb), rtol=0, atol=1e-14)
    np.testing.assert_allclose(hn, np.array(hb), rtol=0, atol=1e-14)
    np.testing.assert_allclose(cn, np.array(cb), rtol=0, atol=1e-14)


@pytest.mark.parametrize("L,bidir", [(1, False), (2, True), (3, False)])
def test_lengths_equal_truncated_rows(L, bidir):
    """A row with n valid steps gives exactly what the fixed-length forward
    gives for that row's first n steps alone; padded outputs are zero."""
    spec = Spec(5, 6, L, bidir, 7, 5, "f32", 3100 + L, "normal0.1")
    inp = make_inputs(spec)
    lengths = np.array([7, 1, 4, 6, 3], np.int32)
    y, hn, cn = run(inp, lengths=lengths)
    for b, n in enumerate(lengths):
        sub = inp.rows([b])
        yt, ht, ct = oracle.lstm_forward(sub.x[:n], sub.params, 6, L, bidir, h0=sub.h0, c0=sub.c0)
        np.testing.assert_array_equal(y[:n, b], yt[:, 0])
        np.testing.assert_array_equal(hn[:, b], ht[:, 0])
        np.testing.assert_array_equal(cn[:, b], ct[:, 0])
        assert np.all(y[n:, b] == 0.0)
    full, _, _ = run(inp, lengths=np.full(5, 7, np.int32))
    plain, _, _ = run(inp)
    np.testing.assert_array_equal(full, plain)


def test_lengths_out_of_range_rejected():
    inp = make_inputs(Spec(3, 4, 1, False, 5, 2, "f32", 3200, "zeros"))
    for bad in ([0, 3], [6, 5]):
        with pytest.raises(RuntimeError):
            run(inp, lengths=bad)


def test_brute_force_without_bias():
    spec = Spec(3, 3, 2, True, 3, 2, "f32", 77, "zeros", has_bias=False)
    inp = make_inputs(spec)
    y, hn, cn = run(inp)
    yb, hb, cb = brute.lstm(inp.x.astype(np.float64).tolist(),
                            [p.astype(np.float64).tolist() for p in inp.params], 3, 2, 2,
                            has_bias=False)
    np.testing.assert_allclose(y, np.array(yb), rtol=0, atol=1e-14)
    np.testing.assert_allclose(cn, np.array(cb), rtol=0, atol=1e-14)


# --------------------------------------------------------------------------- G
@pytest.mark.parametrize("L,bidir", [(1, False), (2, True), (3, False)])
def test_no_recurrence_is_a_dense_product(L, bidir):
    """W_hh = 0 and a forget bias of -40 (sigma = 4e-18) remove the recurrence.

    Then h_t = o * tanh(i * g) with the four gates read off one dense product
    x_t W_ih^T + b_ih + b_hh (the concatenated-weights view of the MXNet blog's
    "Basic Operators"), computed here with numpy's matmul, layer by layer.
    """
    D = 2 if bidir else 1
    spec = Spec(6, 5, L, bidir, 7, 4, "f32", 51)
    inp = make_inputs(spec)
    H = spec.hidden_size
    params = []
    for idx in range(L * D):
        W_ih, _W_hh, b_ih, b_hh = inp.params[idx * 4:(idx + 1) * 4]
        b_ih = b_ih.astype(np.float64).copy()
        b_hh = b_hh.astype(np.float64)
        b_ih[H:2 * H] = -40.0
        params += [W_ih.astype(np.float64), np.zeros((4 * H, H)), b_ih, b_hh]
    y, _, _ = oracle.lstm_forward(inp.x, params, H, L, bidir)
    seq = inp.x.astype(np.float64)
    for l in range(L):
        outs = []
        for d in range(D):
            W_ih, _, b_ih, b_hh = params[(l * D + d) * 4:(l * D + d + 1) * 4]
            pre = seq @ W_ih.T + b_ih + b_hh
            i, g, o = sig(pre[..., :H]), np.tanh(pre[..., 2 * H:3 * H]), sig(pre[..., 3 * H:])
            outs.append(o * np.tanh(i * g))
        seq = np.concatenate(outs, axis=-1)
    np.testing.assert_allclose(y, seq, rtol=0, atol=1e-12)


# ------------------------------------------------------------------- C and Tch
torch = pytest.importorskip("torch")


def test_single_cell_matches_torch_lstmcell():
    """T = L = D = 1 is one LSTMCell step, the check the Brenndoerfer page runs."""
    spec = Spec(8, 16, 1, False, 1, 3, "f32", 61, "normal0.1")
    inp = make_inputs(spec)
    y, hn, cn = run(inp)
    cell = torch.nn.LSTMCell(8, 16, dtype=torch.float64)
    with torch.no_grad():
        for name, p in zip(["weight_ih", "weight_hh", "bias_ih", "bias_hh"], inp.params):
            getattr(cell, name).copy_(torch.from_numpy(p.astype(np.float64)))
        h, c = cell(torch.from_numpy(inp.x[0].astype(np.float64)),
                    (torch.from_numpy(inp.h0[0].astype(np.float64)),
                     torch.from_numpy(inp.c0[0].astype(np.float64))))
    np.testing.assert_allclose(y[0], h.numpy(), rtol=0, atol=1e-13)
    np.testing.assert_allclose(cn[0], c.numpy(), rtol=0, atol=1e-13)


def test_fp32_agreement_is_within_the_pages_bound():
    """The Brenndoerfer page's own check: an fp32 LSTMCell step (input 8,
    hidden 16, zero state) agrees with a second implementation to a few 1e-8.
    Here the second implementation is the fp64 oracle; the fixture records the
    page's printed figures and the bound derived from them."""
    with open(os.path.join(GOLDEN, "fp32_lstmcell_agreement.json")) as f:
        gold = json.load(f)
    spec = Spec(8, 16, 1, False, 1, 1, "f32", 42)
    inp = make_inputs(spec)
    y, hn, cn = run(inp)
    cell = torch.nn.LSTMCell(8, 16, dtype=torch.float32)
    with torch.no_grad():
        for name, p in zip(["weight_ih", "weight_hh", "bias_ih", "bias_hh"], inp.params):
            getattr(cell, name).copy_(torch.from_numpy(p))
        h, c = cell(torch.from_numpy(inp.x[0]))
    dh = np.max(np.abs(h.double().numpy() - y[0]))
    dc = np.max(np.abs(c.double().numpy() - cn[0]))
    assert dh <= gold["bound"] and dc <= gold["bound"], (dh, dc)


@pytest.mark.parametrize("L,bidir,state", [(1, False, "normal0.1"), (2, True, "normal0.1"),
                                           (3, True, "zeros"), (2, False, "normal0.1")])
def test_matches_torch_lstm_fp64(L, bidir, state):
    """Library cross-check of the conventions the pages leave open (reverse
    alignment, final reverse state, l*D+d state order) against torch.nn.LSTM,
    the module traced on the "Complete Trace: nn.LSTM" page, run in float64."""
    spec = Spec(5, 7, L, bidir, 6, 3, "f32", 71 + L, state)
    inp = make_inputs(spec)
    y, hn, cn = run(inp)
    m = torch.nn.LSTM(5, 7, num_layers=L, bidirectional=bidir, dtype=torch.float64)
    names = []
    for l in range(L):
        for d in range(spec.D):
            sfx = f"_l{l}" + ("_reverse" if d else "")
            names += ["weight_ih" + sfx, "weight_hh" + sfx, "bias_ih" + sfx, "bias_hh" + sfx]
    with torch.no_grad():
        for name, p in zip(names, inp.params):
            getattr(m, name).copy_(torch.from_numpy(p.astype(np.float64)))
        hx = None
        if inp.h0 is not None:
            hx = (torch.from_numpy(inp.h0.astype(np.float64)), torch.from_numpy(inp.c0.astype(np.float64)))
        yt, (ht, ct) = m(torch.from_numpy(inp.x.astype(np.float64)), hx)
    np.testing.assert_allclose(y, yt.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(hn, ht.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(cn, ct.numpy(), rtol=0, atol=1e-12)


def test_bf16_inputs_widen_exactly():
    """bf16 bit patterns reach the oracle without rounding (x * 1 path)."""
    spec = Spec(4, 3, 1, False, 2, 2, "bf16", 81)
    inp = make_inputs(spec)
    x64 = oracle.as_f64(inp.x, bf16=True)
    back = (x64.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    np.testing.assert_array_equal(back, inp.x)
    y, _, _ = run(inp)
    assert np.all(np.isfinite(y))

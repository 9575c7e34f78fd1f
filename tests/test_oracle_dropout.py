"""Pins of the oracle's training dropout (between layers) and of its
counter-based generator.

- The oracle's Philox4x64-10 block function equals numpy's independent
  implementation of the same published generator (numpy.random.Philox, which
  advances its 256-bit counter by one before each block it returns).
- The training forward equals the per-gate brute force of tests/brute.py fed
  with masks drawn from numpy's Philox under the stated indexing: so the
  counter layout, the word choice, the keep rule, the 1/(1-p) scale and the
  layer the mask applies to are all pinned from outside the oracle.
- p = 0 is the plain forward, bit for bit; p = 1 cuts every layer above the
  first off from its input (closed form: the top layer alone on zero input).
- The backward with dropout matches central finite differences of the
  training forward (the draw is fixed by seed and call).
"""
import numpy as np
import pytest

import oracle
from layer_lstm_forward_amd.synth import Spec, make_inputs
from tests import brute

M64 = (1 << 64) - 1


def numpy_philox_block(counter, key):
    """numpy's Philox block for `counter` (numpy returns the block of its counter + 1)."""
    c = sum(int(v) << (64 * i) for i, v in enumerate(counter))
    c = (c - 1) % (1 << 256)
    g = np.random.Philox(counter=np.array([(c >> (64 * i)) & M64 for i in range(4)], dtype=np.uint64),
                         key=np.array([int(k) for k in key], dtype=np.uint64))
    return [int(v) for v in g.random_raw(4)]


def numpy_keep_mask(p, seed, call, layer, n):
    """Keep decisions of elements 0..n-1 of layer `layer`'s output: block
    counter (e // 4, layer, call, 0), key (seed, 0), word e % 4, kept when
    (word >> 11) * 2^-53 >= p."""
    nblk = (n + 3) // 4
    c = ((int(call) << 128) | (int(layer) << 64)) - 1
    c %= 1 << 256
    g = np.random.Philox(counter=np.array([(c >> (64 * i)) & M64 for i in range(4)], dtype=np.uint64),
                         key=np.array([int(seed), 0], dtype=np.uint64))
    w = g.random_raw(4 * nblk)[:n]
    u = (w >> np.uint64(11)).astype(np.float64) * 2.0 ** -53
    return u >= p


@pytest.mark.parametrize("counter,key", [((0, 0, 0, 0), (0, 0)), ((5, 7, 9, 11), (123, 456)),
                                         ((M64, 0, 3, 0), (1, 2)), ((M64, M64, 7, 1), (M64, 99)),
                                         ((12345, 2, 1 << 40, 0), (0xDEADBEEF, 0))])
def test_philox_matches_numpy(counter, key):
    assert oracle.philox4x64_10(counter, key) == numpy_philox_block(counter, key)


@pytest.mark.parametrize("p,seed,call,layer,n", [(0.3, 7, 0, 0, 1001), (0.5, 1 << 60, 9, 2, 4096),
                                                  (0.999, 3, 1, 1, 777), (1.0, 5, 0, 0, 64), (0.0, 5, 0, 0, 64)])
def test_oracle_keep_decisions_match_numpy(p, seed, call, layer, n):
    want = numpy_keep_mask(p, seed, call, layer, n).astype(np.uint8)
    np.testing.assert_array_equal(oracle.dropout_keep(p, seed, call, layer, n), want)


def test_numpy_mask_keep_fraction():
    # the test's own mask helper: keeps about 1 - p (binomial, 6 sigma)
    n, p = 200000, 0.3
    k = int(np.sum(numpy_keep_mask(p, 42, 3, 1, n)))
    assert abs(k - n * (1 - p)) < 6 * np.sqrt(n * p * (1 - p))


def _spec(L=3, bidir=True, T=4, B=3, H=3, I=2, bias=True, seed=6100):
    return Spec(I, H, L, bidir, T, B, "f32", seed, "normal0.1", has_bias=bias)


@pytest.mark.parametrize("p,seed,call", [(0.3, 7, 0), (0.5, 123456789, 5), (0.9, 1, 1 << 33)])
@pytest.mark.parametrize("L,bidir", [(2, False), (3, True)])
def test_forward_dropout_matches_brute_force_with_numpy_masks(p, seed, call, L, bidir):
    spec = _spec(L=L, bidir=bidir)
    inp = make_inputs(spec)
    H, D, T, B = spec.hidden_size, spec.D, spec.T, spec.B
    between = []
    for l in range(L - 1):
        keep = numpy_keep_mask(p, seed, call, l, T * B * D * H).reshape(T, B, D * H)
        between.append((keep / (1.0 - p)).tolist())
    ref_y, ref_hn, ref_cn = brute.lstm(inp.x.tolist(), [q.tolist() for q in inp.params], H, L, D,
                                       h0=inp.h0.tolist(), c0=inp.c0.tolist(), between=between)
    y, hn, cn = oracle.lstm_forward(inp.x, inp.params, H, L, bidir, h0=inp.h0, c0=inp.c0, dropout=(p, seed, call))
    np.testing.assert_allclose(y, np.array(ref_y), rtol=0, atol=1e-13)
    np.testing.assert_allclose(hn, np.array(ref_hn), rtol=0, atol=1e-13)
    np.testing.assert_allclose(cn, np.array(ref_cn), rtol=0, atol=1e-13)
    # the draw matters: another call index gives another output
    y2, _, _ = oracle.lstm_forward(inp.x, inp.params, H, L, bidir, h0=inp.h0, c0=inp.c0,
                                   dropout=(p, seed, call + 1))
    assert np.max(np.abs(y2 - y)) > 1e-6


def test_dropout_zero_is_plain_forward():
    spec = _spec()
    inp = make_inputs(spec)
    args = (inp.x, inp.params, spec.hidden_size, spec.num_layers, spec.bidirectional)
    a = oracle.lstm_forward(*args, h0=inp.h0, c0=inp.c0, dropout=(0.0, 5, 5))
    b = oracle.lstm_forward(*args, h0=inp.h0, c0=inp.c0)
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)


def test_dropout_one_cuts_upper_layers_off():
    # p = 1: layer 1 sees zero input, so it equals a one-layer LSTM with
    # layer 1's parameters and initial state running on zeros
    spec = _spec(L=2, bidir=True)
    inp = make_inputs(spec)
    H, D = spec.hidden_size, spec.D
    y, hn, cn = oracle.lstm_forward(inp.x, inp.params, H, 2, True, h0=inp.h0, c0=inp.c0, dropout=(1.0, 3, 0))
    per = 4
    top = inp.params[D * per:]
    z = np.zeros((spec.T, spec.B, D * H))
    y1, hn1, cn1 = oracle.lstm_forward(z, top, H, 1, True, h0=inp.h0[D:], c0=inp.c0[D:])
    np.testing.assert_allclose(y, y1, rtol=0, atol=1e-15)
    np.testing.assert_allclose(hn[D:], hn1, rtol=0, atol=1e-15)
    np.testing.assert_allclose(cn[D:], cn1, rtol=0, atol=1e-15)


@pytest.mark.parametrize("L,bidir,p", [(2, False, 0.4), (3, True, 0.25)])
def test_backward_with_dropout_matches_finite_differences(L, bidir, p):
    spec = _spec(L=L, bidir=bidir, T=3, B=2, H=2, I=2, seed=6200 + L)
    inp = make_inputs(spec)
    H = spec.hidden_size
    drop = (p, 77, 4)
    params = [q.astype(np.float64) * 3.0 for q in inp.params]
    x, h0, c0 = (a.astype(np.float64) for a in (inp.x, inp.h0, inp.c0))
    rng = np.random.default_rng(9)
    wy = rng.standard_normal((spec.T, spec.B, spec.D * H))
    whn = rng.standard_normal((L * spec.D, spec.B, H))
    wcn = rng.standard_normal((L * spec.D, spec.B, H))
    dx, dh0, dc0, dps = oracle.lstm_backward(x, params, H, L, bidir, wy, h0=h0, c0=c0, dh_n=whn, dc_n=wcn,
                                             dropout=drop)

    def loss():
        y, hn, cn = oracle.lstm_forward(x, params, H, L, bidir, h0=h0, c0=c0, dropout=drop)
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


@pytest.mark.parametrize("L,bidir", [(2, False), (3, True)])
def test_dropout_with_lengths_matches_brute_force(L, bidir):
    # per-row lengths and dropout together: padded outputs are 0 before and after the mask
    spec = _spec(L=L, bidir=bidir, T=5, B=3)
    inp = make_inputs(spec)
    H, D, T, B = spec.hidden_size, spec.D, spec.T, spec.B
    p, seed, call = 0.4, 99, 7
    lengths = [5, 2, 3]
    between = []
    for l in range(L - 1):
        keep = numpy_keep_mask(p, seed, call, l, T * B * D * H).reshape(T, B, D * H)
        between.append((keep / (1.0 - p)).tolist())
    ref_y, ref_hn, ref_cn = brute.lstm(inp.x.tolist(), [q.tolist() for q in inp.params], H, L, D,
                                       h0=inp.h0.tolist(), c0=inp.c0.tolist(), lengths=lengths, between=between)
    y, hn, cn = oracle.lstm_forward(inp.x, inp.params, H, L, bidir, h0=inp.h0, c0=inp.c0, dropout=(p, seed, call),
                                    lengths=lengths)
    np.testing.assert_allclose(y, np.array(ref_y), rtol=0, atol=1e-13)
    np.testing.assert_allclose(hn, np.array(ref_hn), rtol=0, atol=1e-13)
    np.testing.assert_allclose(cn, np.array(ref_cn), rtol=0, atol=1e-13)

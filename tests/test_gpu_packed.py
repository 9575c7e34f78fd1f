"""Packed sequences (lstm_forward_packed, through the C ABI) against the fp64
oracle's per-row-lengths forward on the same problem: the rows of step t in
the packed data are the sequences still running at t, in order of
non-increasing length, so the packed result is the padded one's valid rows
taken step by step.

Max-abs error relative to max(1, max|ref|): 1e-4 for fp32, 2e-2 for bf16.
"""
import numpy as np
import pytest

import layer_lstm_forward_amd as pkg
import oracle
from layer_lstm_forward_amd.synth import Spec, make_inputs, make_lengths
from tests.gpu_util import oracle_threads, to_dev

pytestmark = pytest.mark.gpu
TOL = {"f32": 1e-4, "bf16": 2e-2}

CASES = [  # spec, length mix
    (Spec(24, 32, 1, False, 9, 11, "f32", 1201, "normal0.1"), "ragged"),
    (Spec(40, 64, 2, True, 13, 70, "f32", 1202, "normal0.1"), "ragged"),     # two layers, both directions
    (Spec(64, 96, 2, False, 7, 20, "bf16", 1203, "zeros"), "mix"),
    (Spec(16, 40, 3, True, 5, 3, "f32", 1204, "normal0.1", has_bias=False), "ragged"),
    (Spec(24, 64, 2, False, 8, 21, "f32", 1205, "normal0.1", mode="gru"), "ragged"),
    (Spec(256, 512, 2, False, 128, 64, "f32", 1206, "normal0.1"), "mix"),    # the benchmark shape
]


def _check(got, ref, dtype, what):
    scale = max(1.0, float(np.max(np.abs(ref))))
    err = float(np.max(np.abs(got - ref)))
    assert err <= TOL[dtype] * scale, f"{what}: max-abs error {err:.3g} > {TOL[dtype]} x {scale:.3g}"


def _pack(a, batch_sizes):
    """[T, B, W] -> [sum(batch_sizes), W]: the first batch_sizes[t] rows of each step."""
    return np.concatenate([a[t, :n] for t, n in enumerate(batch_sizes)], axis=0)


@pytest.mark.parametrize("spec,mix", CASES,
                         ids=lambda v: f"{v.mode}-{v.dtype}-H{v.hidden_size}-L{v.num_layers}-D{v.D}-T{v.T}-B{v.B}"
                         if isinstance(v, Spec) else v)
def test_packed_matches_oracle(spec, mix):
    import torch
    print(f"case packed {spec} {mix}", flush=True)
    bf = spec.dtype == "bf16"
    lengths = make_lengths(spec, mix)
    order = np.argsort(-lengths, kind="stable")          # sequences by non-increasing length
    inp = make_inputs(spec).rows(order)
    lens = lengths[order]
    T = int(lens[0])
    batch_sizes = [int(np.sum(lens > t)) for t in range(T)]
    x_pad = inp.x[:T]
    m = pkg.LSTM(spec.input_size, spec.hidden_size, spec.num_layers, spec.bidirectional, bias=spec.has_bias,
                 dtype=spec.dtype, mode=spec.mode)
    x = to_dev(np.ascontiguousarray(_pack(x_pad, batch_sizes)), bf, "cuda:0")
    w = [to_dev(p, bf, "cuda:0") for p in inp.params]
    h0 = None if inp.h0 is None else to_dev(inp.h0, bf, "cuda:0")
    c0 = None if inp.c0 is None or spec.mode != "lstm" else torch.from_numpy(inp.c0).to("cuda:0")
    y, hn, cn = m.forward_packed(x, batch_sizes, w, h0, c0)
    torch.cuda.synchronize()
    cpu = lambda t: t.float().cpu().numpy().astype(np.float64)  # noqa: E731
    H, L, D = spec.hidden_size, spec.num_layers, spec.bidirectional
    if spec.mode == "lstm":
        ry, rhn, rcn = oracle.lstm_forward(x_pad, inp.params, H, L, D, h0=inp.h0, c0=inp.c0, has_bias=spec.has_bias,
                                           bf16=bf, nthreads=oracle_threads(), lengths=lens)
        _check(cpu(cn), rcn, spec.dtype, "c_n")
    else:
        ry, rhn = oracle.rnn_forward(spec.mode, x_pad, inp.params, H, L, D, h0=inp.h0, has_bias=spec.has_bias,
                                     bf16=bf, nthreads=oracle_threads(), lengths=lens)
        assert cn is None
    assert y.shape[0] == sum(batch_sizes)
    _check(cpu(y), _pack(ry, batch_sizes), spec.dtype, "y")
    _check(cpu(hn), rhn, spec.dtype, "h_n")

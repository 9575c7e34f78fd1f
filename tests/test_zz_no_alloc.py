"""lstm_forward_static (the forward on the library's own device array, for
callers that cannot allocate) through the C ABI, against lstm_forward on a
caller workspace: identical outputs (the same kernels on the same inputs),
and both within the oracle's tolerance, on two calls in a row with the second
smaller, for several plans; a (T, B) beyond the array's size is refused with
nothing written."""
import numpy as np
import pytest

import layer_lstm_forward_amd as pkg
from layer_lstm_forward_amd.synth import WORKLOADS, Spec, make_inputs
from tests.gpu_util import assert_parity, run_oracle, to_dev

pytestmark = pytest.mark.gpu


def _outputs(spec, dev):
    import torch
    tdt = torch.bfloat16 if spec.dtype == "bf16" else torch.float32
    H, L, D = spec.hidden_size, spec.num_layers, spec.D
    return (torch.full((spec.T, spec.B, D * H), 7.0, dtype=tdt, device=dev),
            torch.full((L * D, spec.B, H), 7.0, dtype=tdt, device=dev),
            torch.full((L * D, spec.B, H), 7.0, dtype=torch.float32, device=dev))


def _call(m, spec, inp, static):
    """One forward of plan m on inp; returns the outputs as float64 numpy."""
    import torch
    dev = "cuda:0"
    bf = spec.dtype == "bf16"
    x = to_dev(inp.x, bf, dev)
    w = [to_dev(p, bf, dev) for p in inp.params]
    h0, c0 = to_dev(inp.h0, bf, dev), to_dev(inp.c0, False, dev)
    y, hn, cn = _outputs(spec, dev)
    stream = torch.cuda.current_stream().cuda_stream
    args = (h0.data_ptr() if h0 is not None else 0, c0.data_ptr() if c0 is not None else 0,
            [t.data_ptr() for t in w], spec.T, spec.B, spec.num_layers, spec.bidirectional,
            y.data_ptr(), hn.data_ptr(), cn.data_ptr())
    if static:
        status = torch.full((1,), 12345, dtype=torch.int32, device=dev)
        rc = pkg.lstm_forward_static(m.plan, x.data_ptr(), *args, status.data_ptr(), stream)
        assert rc == 0, pkg.lstm_strerror(rc)
        torch.cuda.synchronize()
        assert int(status.item()) == 0, "a step barrier gave up"
    else:
        ws, nbytes = m.workspace(spec.T, spec.B, x.device)
        rc = pkg.lstm_forward(m.plan, x.data_ptr(), *args, ws.data_ptr(), nbytes, stream)
        assert rc == 0, pkg.lstm_strerror(rc)
        torch.cuda.synchronize()
        assert m.device_status() == (0, 0)
    return tuple(t.float().cpu().numpy().astype(np.float64) for t in (y, hn, cn))


PAIRS = [  # (first call, second smaller call) on one plan: same sizes and layers, smaller T and B
    (Spec(37, 52, 2, True, 9, 19, "f32", 801, "normal0.1"), Spec(37, 52, 2, True, 4, 6, "f32", 802, "normal0.1")),
    (Spec(64, 96, 3, False, 11, 40, "bf16", 803, "normal0.1"), Spec(64, 96, 3, False, 7, 3, "bf16", 804, "zeros")),
    (WORKLOADS["l2_in256_h512_t128_b64_f32"], Spec(256, 512, 2, False, 50, 17, "f32", 805, "normal0.1")),
    (WORKLOADS["l1_in1024_h1024_t1024_b1_bf16"], Spec(1024, 1024, 1, False, 100, 1, "bf16", 806, "zeros")),
]


@pytest.mark.parametrize("pair", PAIRS, ids=lambda p: f"{p[0].dtype}-H{p[0].hidden_size}-L{p[0].num_layers}"
                                                      f"-T{p[0].T}xB{p[0].B}-then-T{p[1].T}xB{p[1].B}")
def test_static_equals_workspace_forward(pair):
    first, second = pair
    m = pkg.LSTM(first.input_size, first.hidden_size, first.num_layers, first.bidirectional, dtype=first.dtype)
    assert pkg.lstm_workspace_size(m.plan, first.T, first.B) <= pkg.LSTM_STATIC_WORKSPACE_BYTES
    for spec in (first, second):
        print(f"case static {spec}", flush=True)
        inp = make_inputs(spec)
        got = _call(m, spec, inp, static=True)
        want = _call(m, spec, inp, static=False)
        for g, w in zip(got, want):
            np.testing.assert_array_equal(g, w)
        rows = None if spec.B <= 20 else [0, spec.B // 2, spec.B - 1]
        if rows is None:
            assert_parity(got, run_oracle(inp), spec.dtype, "static")
        else:
            # rows are independent: a row subset run alone is the reference
            assert_parity(tuple(a[:, rows] for a in got), run_oracle(inp.rows(rows)), spec.dtype, "static rows")


def test_static_refuses_beyond_its_size():
    import torch
    spec = Spec(512, 1024, 2, True, 256, 32, "bf16", 807, "zeros")  # about 293 MiB of workspace
    m = pkg.LSTM(spec.input_size, spec.hidden_size, spec.num_layers, spec.bidirectional, dtype="bf16")
    assert pkg.lstm_workspace_size(m.plan, spec.T, spec.B) > pkg.LSTM_STATIC_WORKSPACE_BYTES
    inp = make_inputs(spec)
    dev = "cuda:0"
    x = to_dev(inp.x, True, dev)
    w = [to_dev(p, True, dev) for p in inp.params]
    y, hn, cn = _outputs(spec, dev)
    rc = pkg.lstm_forward_static(m.plan, x.data_ptr(), 0, 0, [t.data_ptr() for t in w], spec.T, spec.B,
                                 spec.num_layers, spec.bidirectional, y.data_ptr(), hn.data_ptr(), cn.data_ptr(),
                                 0, torch.cuda.current_stream().cuda_stream)
    assert rc == -5  # LSTM_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool(torch.all(y.float() == 7.0)) and bool(torch.all(cn == 7.0))

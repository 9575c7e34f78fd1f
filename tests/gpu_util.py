"""Helpers for the GPU tests: move seeded inputs to the device, run the HIP
path through the C ABI, and compare with the fp64 oracle."""
import os

import numpy as np

import oracle

TOL = {"f32": 1e-4, "bf16": 2e-2}


def oracle_threads():
    return max(1, min(16, os.cpu_count() or 1))


def to_dev(a, bf16, device):
    import torch
    if a is None:
        return None
    if bf16 and a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def run_gpu(inp, recurrence=0, rec_tile=0, model=None, device="cuda:0", repeat=1, options=None, lengths=None,
            batch_first=False):
    """batch_first: run a batch-first plan on x transposed to [B, T, I] and
    return y transposed back to [T, B, D*H] (h_n, c_n have one layout)."""
    """Returns (y, h_n, c_n) as float64 numpy arrays and the model used."""
    import torch
    import layer_lstm_forward_amd as pkg
    s = inp.spec
    bf = s.dtype == "bf16"
    if model is None:
        model = pkg.LSTM(s.input_size, s.hidden_size, s.num_layers, s.bidirectional, bias=s.has_bias,
                         dtype=s.dtype, recurrence=recurrence, rec_tile=rec_tile, options=options,
                         batch_first=batch_first)
    x = to_dev(np.ascontiguousarray(inp.x.transpose(1, 0, 2)) if batch_first else inp.x, bf, device)
    w = [to_dev(p, bf, device) for p in inp.params]
    h0 = to_dev(inp.h0, bf, device)
    c0 = to_dev(inp.c0, False, device)
    for _ in range(repeat):
        y, hn, cn = model.forward(x, w, h0, c0, lengths=lengths)
    torch.cuda.synchronize()
    rc, flags = model.device_status()
    assert rc == 0 and flags == 0, f"device status {rc} flags {flags}"
    out = tuple(t.float().cpu().numpy().astype(np.float64) for t in (y, hn, cn))
    if batch_first:
        out = (np.ascontiguousarray(out[0].transpose(1, 0, 2)),) + out[1:]
    return out, model


def run_oracle(inp, lengths=None):
    s = inp.spec
    return oracle.lstm_forward(inp.x, inp.params, s.hidden_size, s.num_layers, s.bidirectional,
                               h0=inp.h0, c0=inp.c0, has_bias=s.has_bias, bf16=s.dtype == "bf16",
                               nthreads=oracle_threads(), lengths=lengths)


def max_errs(got, ref):
    return [float(np.max(np.abs(g - r))) if g.size else 0.0 for g, r in zip(got, ref)]


def assert_parity(got, ref, dtype, what=""):
    tol = TOL[dtype]
    errs = max_errs(got, ref)
    names = ("y", "h_n", "c_n")
    bad = [f"{n}={e:.3g}" for n, e in zip(names, errs) if not (e <= tol)]
    assert not bad, f"{what} max-abs error above {tol}: {', '.join(bad)} (all: {errs})"
    return errs

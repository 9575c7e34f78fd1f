"""The HIP backward pass (lstm_forward_train + lstm_backward, through the C
ABI) against the fp64 oracle's backward on the same seeded inputs.

Gradients are compared by max-abs error relative to the gradient's own scale,
max(1, max|reference|): 1e-4 for fp32, 3e-2 for bf16 (the bf16 forward rounds h
to bf16 where it is stored, and the backward reuses those stored outputs; with
an even H it also keeps dz in bf16 for its products, fp32 accumulation).
"""
import numpy as np
import pytest

import layer_lstm_forward_amd as pkg
import oracle
from layer_lstm_forward_amd.synth import Spec, make_inputs
from tests.gpu_util import run_gpu, to_dev

pytestmark = pytest.mark.gpu
TOL = {"f32": 1e-4, "bf16": 3e-2}

SPECS = [
    Spec(24, 32, 1, False, 6, 5, "f32", 801, "normal0.1"),
    Spec(37, 52, 2, True, 7, 19, "f32", 802, "normal0.1"),      # ragged sizes, both directions
    Spec(40, 48, 3, False, 5, 33, "f32", 803, "zeros"),          # three layers, no initial state
    Spec(16, 40, 2, True, 4, 3, "f32", 804, "normal0.1", has_bias=False),
    Spec(64, 96, 2, True, 6, 20, "bf16", 805, "normal0.1"),
    Spec(32, 64, 1, False, 9, 40, "bf16", 806, "zeros"),
    # weight- and input-gradient products split over K (T*B or D*4H) into slabs:
    Spec(96, 128, 2, False, 64, 16, "f32", 807, "normal0.1"),   # 128x128 tiles, 4 splits
    Spec(20, 24, 1, True, 35, 20, "f32", 808, "normal0.1"),     # a ragged last split (384 + 316)
    Spec(64, 128, 2, True, 48, 24, "bf16", 810, "normal0.1"),   # bf16 weights, 320-deep splits
    Spec(32, 64, 1, False, 256, 256, "f32", 809, "normal0.1"),  # 256x256 direct-to-LDS tiles, 256 splits
    # bf16 parameters with an odd H: dz and the backward products stay fp32
    Spec(30, 37, 2, True, 6, 9, "bf16", 811, "normal0.1"),
    # 256 recurrent 16x16 tiles fill the CUs: K stays whole in one workgroup
    # (every case above has at most 128 and splits K between two)
    Spec(64, 1024, 1, True, 4, 32, "f32", 812, "normal0.1"),
    Spec(32, 1024, 1, True, 3, 32, "bf16", 813, "zeros"),
]


def _id(s):
    return f"{s.dtype}-I{s.input_size}-H{s.hidden_size}-L{s.num_layers}-D{s.D}-T{s.T}-B{s.B}"


def _grads(spec, seed):
    rng = np.random.default_rng(seed)
    D, H, L = spec.D, spec.hidden_size, spec.num_layers
    return (rng.standard_normal((spec.T, spec.B, D * H)).astype(np.float32),
            rng.standard_normal((L * D, spec.B, H)).astype(np.float32),
            rng.standard_normal((L * D, spec.B, H)).astype(np.float32))


def _check(got, ref, dtype, what):
    g = np.asarray(got, np.float64)
    scale = max(1.0, float(np.max(np.abs(ref))) if ref.size else 1.0)
    err = float(np.max(np.abs(g - ref))) if ref.size else 0.0
    assert err <= TOL[dtype] * scale, f"{what}: max-abs error {err:.3g} > {TOL[dtype]} x {scale:.3g}"


@pytest.mark.parametrize("spec", SPECS, ids=_id)
def test_backward_matches_oracle(spec):
    import torch
    print(f"case {_id(spec)} backward", flush=True)
    inp = make_inputs(spec)
    bf = spec.dtype == "bf16"
    dev = "cuda:0"
    dy, dhn, dcn = _grads(spec, spec.seed + 5)
    if bf:
        from layer_lstm_forward_amd.synth import bf16_bits_to_f32, f32_to_bf16_bits
        dy_b, dhn_b = f32_to_bf16_bits(dy), f32_to_bf16_bits(dhn)
        dy, dhn = bf16_bits_to_f32(dy_b), bf16_bits_to_f32(dhn_b)  # what the GPU sees
    m = pkg.LSTM(spec.input_size, spec.hidden_size, spec.num_layers, spec.bidirectional, bias=spec.has_bias,
                 dtype=spec.dtype)
    x = to_dev(inp.x, bf, dev)
    w = [to_dev(p, bf, dev) for p in inp.params]
    h0 = to_dev(inp.h0, bf, dev)
    c0 = None if inp.c0 is None else torch.from_numpy(inp.c0).to(dev)
    y, hn, cn, reserve = m.forward_train(x, w, h0, c0)
    # saving activations changes nothing: the training forward equals the
    # layer-by-layer inference forward of the per-layer kernels bit for bit
    # (the layer wavefront, the one-XCD small-batch kernel and the resident
    # large-batch kernel, inference defaults where they apply, sum in other
    # orders)
    plain, _ = run_gpu(inp, options={pkg.LSTM_OPT_LAYER_PIPE: 0, pkg.LSTM_OPT_SMALL_BATCH: 0,
                                     pkg.LSTM_OPT_RESIDENT: 0})
    np.testing.assert_array_equal(y.float().cpu().numpy(), plain[0])
    dy_d = to_dev(dy_b if bf else dy, bf, dev)
    dhn_d = to_dev(dhn_b if bf else dhn, bf, dev)
    dcn_d = torch.from_numpy(dcn).to(dev)
    dx, dh0, dc0, dws = m.backward(x, w, y, reserve, dy_d, h0=h0, c0=c0, dh_n=dhn_d, dc_n=dcn_d)
    torch.cuda.synchronize()
    assert m.backward_status() == (0, 0)  # no hand-over wait gave up
    rdx, rdh0, rdc0, rdps = oracle.lstm_backward(inp.x, inp.params, spec.hidden_size, spec.num_layers,
                                                 spec.bidirectional, dy, h0=inp.h0, c0=inp.c0, dh_n=dhn, dc_n=dcn,
                                                 has_bias=spec.has_bias, bf16=bf)
    cpu = lambda t: t.float().cpu().numpy()  # noqa: E731
    _check(cpu(dx), rdx, spec.dtype, "dx")
    if inp.h0 is not None:
        _check(cpu(dh0), rdh0, spec.dtype, "dh0")
        _check(cpu(dc0), rdc0, spec.dtype, "dc0")
    for k, (g, r) in enumerate(zip(dws, rdps)):
        _check(cpu(g), r, spec.dtype, f"dweights[{k}]")


def test_backward_host_validation():
    m = pkg.LSTM(8, 16, 1, False, dtype="f32")
    FAKE = 0x10000
    args = dict(x=FAKE, h0=0, c0=0, weights=[FAKE] * 4, y=FAKE, dy=FAKE, dh_n=0, dc_n=0, reserve=FAKE,
                reserve_bytes=1 << 40, T=5, B=2, layers=1, bidir=False, dx=0, dh0=0, dc0=0, dweights=[FAKE] * 4,
                workspace=FAKE, workspace_bytes=1 << 40, stream=0)

    def call(**kw):
        a = dict(args, **kw)
        return pkg.lstm_backward(m.plan, *a.values())
    assert call(layers=2) == -2
    assert call(reserve=0) == -1
    assert call(reserve_bytes=16) == -5
    assert call(workspace_bytes=16) == -5
    assert call(dweights=[FAKE, 0, FAKE, FAKE]) == -1


# training dropout between layers: (spec, probability, seed, first call index)
DROP_SPECS = [
    (Spec(24, 32, 2, False, 9, 11, "f32", 821, "normal0.1"), 0.3, 17, 2),
    (Spec(20, 48, 3, True, 7, 19, "f32", 822, "normal0.1"), 0.5, 1 << 40, 0),
    (Spec(64, 64, 2, True, 6, 20, "bf16", 823, "normal0.1"), 0.2, 5, 3),
    (Spec(16, 24, 2, False, 5, 3, "f32", 824, "zeros"), 1.0, 9, 0),
]
FWD_TOL = {"f32": 1e-4, "bf16": 2e-2}


def _keep_bytes(reserve, spec, l):
    """Layer l's keep bytes in the reserve: after every layer's activations
    ([T,B,D,5,H] fp32) and the outputs of the layers below the top one, each
    dropped layer holds its dropped output then its keep bytes (regions
    256-byte aligned)."""
    up = lambda v: (v + 255) // 256 * 256  # noqa: E731
    T, B, D, H, L = spec.T, spec.B, spec.D, spec.hidden_size, spec.num_layers
    es = 2 if spec.dtype == "bf16" else 4
    n = T * B * D * H
    acts, ylay, keep = up(n * 5 * 4), up(n * es), up(n)
    off = acts * L + ylay * (L - 1) + (ylay + keep) * l + ylay
    return reserve[off:off + n].cpu().numpy()


@pytest.mark.parametrize("spec,p,seed,call", DROP_SPECS, ids=lambda v: _id(v) if isinstance(v, Spec) else str(v))
def test_dropout_training_matches_oracle(spec, p, seed, call):
    import torch
    print(f"case {_id(spec)} dropout p={p} seed={seed} call={call}", flush=True)
    inp = make_inputs(spec)
    bf = spec.dtype == "bf16"
    dev = "cuda:0"
    H, L, bidir = spec.hidden_size, spec.num_layers, spec.bidirectional
    m = pkg.LSTM(spec.input_size, H, L, bidir, bias=spec.has_bias, dtype=spec.dtype)
    m.set_dropout(p, seed, call)
    x = to_dev(inp.x, bf, dev)
    w = [to_dev(q, bf, dev) for q in inp.params]
    h0 = to_dev(inp.h0, bf, dev)
    c0 = None if inp.c0 is None else torch.from_numpy(inp.c0).to(dev)
    y, hn, cn, reserve = m.forward_train(x, w, h0, c0)
    torch.cuda.synchronize()
    cpu = lambda t: t.float().cpu().numpy().astype(np.float64)  # noqa: E731
    ry, rhn, rcn = oracle.lstm_forward(inp.x, inp.params, H, L, bidir, h0=inp.h0, c0=inp.c0,
                                       has_bias=spec.has_bias, bf16=bf, dropout=(p, seed, call))
    for got, ref, what in ((y, ry, "y"), (hn, rhn, "h_n"), (cn, rcn, "c_n")):
        err = float(np.max(np.abs(cpu(got) - ref)))
        assert err <= FWD_TOL[spec.dtype], f"{what}: max-abs error {err:.3g}"
    n = spec.T * spec.B * spec.D * H
    for l in range(L - 1):  # the keep decisions are byte work: exact
        np.testing.assert_array_equal(_keep_bytes(reserve, spec, l), oracle.dropout_keep(p, seed, call, l, n),
                                      err_msg=f"keep bytes of layer {l}")

    dy, dhn, dcn = _grads(spec, spec.seed + 5)
    if bf:
        from layer_lstm_forward_amd.synth import bf16_bits_to_f32, f32_to_bf16_bits
        dy_b, dhn_b = f32_to_bf16_bits(dy), f32_to_bf16_bits(dhn)
        dy, dhn = bf16_bits_to_f32(dy_b), bf16_bits_to_f32(dhn_b)
    dy_d = to_dev(dy_b if bf else dy, bf, dev)
    dhn_d = to_dev(dhn_b if bf else dhn, bf, dev)
    dcn_d = torch.from_numpy(dcn).to(dev)
    dx, dh0, dc0, dws = m.backward(x, w, y, reserve, dy_d, h0=h0, c0=c0, dh_n=dhn_d, dc_n=dcn_d)
    torch.cuda.synchronize()
    assert m.backward_status() == (0, 0)  # no hand-over wait gave up
    rdx, rdh0, rdc0, rdps = oracle.lstm_backward(inp.x, inp.params, H, L, bidir, dy, h0=inp.h0, c0=inp.c0,
                                                 dh_n=dhn, dc_n=dcn, has_bias=spec.has_bias, bf16=bf,
                                                 dropout=(p, seed, call))
    _check(cpu(dx), rdx, spec.dtype, "dx")
    if inp.h0 is not None:
        _check(cpu(dh0), rdh0, spec.dtype, "dh0")
        _check(cpu(dc0), rdc0, spec.dtype, "dc0")
    for k, (g, r) in enumerate(zip(dws, rdps)):
        _check(cpu(g), r, spec.dtype, f"dweights[{k}]")

    # the next training forward draws the next mask
    y2, _, _, _ = m.forward_train(x, w, h0, c0)
    torch.cuda.synchronize()
    ry2, _, _ = oracle.lstm_forward(inp.x, inp.params, H, L, bidir, h0=inp.h0, c0=inp.c0,
                                    has_bias=spec.has_bias, bf16=bf, dropout=(p, seed, call + 1))
    err = float(np.max(np.abs(cpu(y2) - ry2)))
    assert err <= FWD_TOL[spec.dtype], f"second call y: max-abs error {err:.3g}"


# per-row lengths (lstm_forward_train_lengths + lstm_backward_lengths):
# (spec, length mix, recurrence option)
LEN_SPECS = [
    (Spec(24, 32, 1, False, 9, 11, "f32", 831, "normal0.1"), "ragged", None),
    (Spec(37, 52, 2, True, 7, 19, "f32", 832, "normal0.1"), "ragged", None),
    (Spec(40, 48, 3, False, 5, 33, "f32", 833, "zeros"), "mix", None),
    (Spec(64, 96, 2, True, 6, 20, "bf16", 834, "normal0.1"), "mix", None),
    (Spec(32, 64, 2, True, 6, 21, "f32", 835, "normal0.1"), "ragged", "gemm"),  # one GEMM-step launch per step
]


@pytest.mark.parametrize("spec,mode,rec", LEN_SPECS, ids=lambda v: _id(v) if isinstance(v, Spec) else str(v))
def test_backward_with_lengths_matches_oracle(spec, mode, rec):
    import torch
    from layer_lstm_forward_amd.synth import make_lengths
    print(f"case {_id(spec)} lengths {mode} rec {rec}", flush=True)
    inp = make_inputs(spec)
    lens = make_lengths(spec, mode)
    bf = spec.dtype == "bf16"
    dev = "cuda:0"
    dy, dhn, dcn = _grads(spec, spec.seed + 5)
    if bf:
        from layer_lstm_forward_amd.synth import bf16_bits_to_f32, f32_to_bf16_bits
        dy_b, dhn_b = f32_to_bf16_bits(dy), f32_to_bf16_bits(dhn)
        dy, dhn = bf16_bits_to_f32(dy_b), bf16_bits_to_f32(dhn_b)
    m = pkg.LSTM(spec.input_size, spec.hidden_size, spec.num_layers, spec.bidirectional, bias=spec.has_bias,
                 dtype=spec.dtype, recurrence=pkg.LSTM_REC_GEMM if rec == "gemm" else pkg.LSTM_REC_AUTO,
                 options={pkg.LSTM_OPT_LAYER_PIPE: 0})  # the training forward runs layer by layer
    x = to_dev(inp.x, bf, dev)
    w = [to_dev(p, bf, dev) for p in inp.params]
    h0 = to_dev(inp.h0, bf, dev)
    c0 = None if inp.c0 is None else torch.from_numpy(inp.c0).to(dev)
    y, hn, cn, reserve = m.forward_train(x, w, h0, c0, lengths=lens)
    y_plain, hn_plain, cn_plain = m.forward(x, w, h0, c0, lengths=lens)
    torch.cuda.synchronize()
    # keeping the activations changes nothing
    np.testing.assert_array_equal(y.float().cpu().numpy(), y_plain.float().cpu().numpy())
    np.testing.assert_array_equal(cn.cpu().numpy(), cn_plain.cpu().numpy())
    dy_d = to_dev(dy_b if bf else dy, bf, dev)
    dhn_d = to_dev(dhn_b if bf else dhn, bf, dev)
    dcn_d = torch.from_numpy(dcn).to(dev)
    dx, dh0, dc0, dws = m.backward(x, w, y, reserve, dy_d, h0=h0, c0=c0, dh_n=dhn_d, dc_n=dcn_d, lengths=lens)
    torch.cuda.synchronize()
    assert m.backward_status() == (0, 0)  # no hand-over wait gave up
    rdx, rdh0, rdc0, rdps = oracle.lstm_backward(inp.x, inp.params, spec.hidden_size, spec.num_layers,
                                                 spec.bidirectional, dy, h0=inp.h0, c0=inp.c0, dh_n=dhn, dc_n=dcn,
                                                 has_bias=spec.has_bias, bf16=bf, lengths=lens)
    cpu = lambda t: t.float().cpu().numpy()  # noqa: E731
    _check(cpu(dx), rdx, spec.dtype, "dx")
    if inp.h0 is not None:
        _check(cpu(dh0), rdh0, spec.dtype, "dh0")
        _check(cpu(dc0), rdc0, spec.dtype, "dc0")
    for k, (g, r) in enumerate(zip(dws, rdps)):
        _check(cpu(g), r, spec.dtype, f"dweights[{k}]")


def test_dropout_with_lengths_matches_oracle():
    import torch
    from layer_lstm_forward_amd.synth import make_lengths
    spec = Spec(20, 48, 3, True, 7, 19, "f32", 841, "normal0.1")
    p, seed, call = 0.35, 12345, 4
    print(f"case {_id(spec)} dropout {p} with ragged lengths", flush=True)
    inp = make_inputs(spec)
    lens = make_lengths(spec, "ragged")
    H, L, bidir, dev = spec.hidden_size, spec.num_layers, spec.bidirectional, "cuda:0"
    m = pkg.LSTM(spec.input_size, H, L, bidir)
    m.set_dropout(p, seed, call)
    x = to_dev(inp.x, False, dev)
    w = [to_dev(q, False, dev) for q in inp.params]
    h0 = to_dev(inp.h0, False, dev)
    c0 = torch.from_numpy(inp.c0).to(dev)
    y, hn, cn, reserve = m.forward_train(x, w, h0, c0, lengths=lens)
    torch.cuda.synchronize()
    ry, rhn, rcn = oracle.lstm_forward(inp.x, inp.params, H, L, bidir, h0=inp.h0, c0=inp.c0, dropout=(p, seed, call),
                                       lengths=lens)
    cpu = lambda t: t.float().cpu().numpy().astype(np.float64)  # noqa: E731
    for got, ref, what in ((y, ry, "y"), (hn, rhn, "h_n"), (cn, rcn, "c_n")):
        err = float(np.max(np.abs(cpu(got) - ref)))
        assert err <= FWD_TOL["f32"], f"{what}: max-abs error {err:.3g}"
    dy, dhn, dcn = _grads(spec, spec.seed + 5)
    dx, dh0, dc0, dws = m.backward(x, w, y, reserve, torch.from_numpy(dy).to(dev), h0=h0, c0=c0,
                                   dh_n=torch.from_numpy(dhn).to(dev), dc_n=torch.from_numpy(dcn).to(dev), lengths=lens)
    torch.cuda.synchronize()
    assert m.backward_status() == (0, 0)  # no hand-over wait gave up
    rdx, rdh0, rdc0, rdps = oracle.lstm_backward(inp.x, inp.params, H, L, bidir, dy, h0=inp.h0, c0=inp.c0, dh_n=dhn,
                                                 dc_n=dcn, dropout=(p, seed, call), lengths=lens)
    _check(cpu(dx), rdx, "f32", "dx")
    _check(cpu(dh0), rdh0, "f32", "dh0")
    _check(cpu(dc0), rdc0, "f32", "dc0")
    for k, (g, r) in enumerate(zip(dws, rdps)):
        _check(cpu(g), r, "f32", f"dweights[{k}]")


# batch-first training: the plan runs on x transposed to [B, T, I] and dy to
# [B, T, D*H]; y and dx come back transposed and are compared with the
# (time-major) oracle.  (spec, lengths mix or None, dropout probability)
BF_SPECS = [
    (Spec(24, 32, 2, True, 9, 11, "f32", 851, "normal0.1"), None, 0.0),
    (Spec(37, 52, 2, False, 7, 19, "f32", 852, "zeros"), "ragged", 0.0),
    (Spec(40, 48, 3, True, 6, 13, "f32", 853, "normal0.1"), "ragged", 0.3),
    (Spec(64, 96, 2, True, 6, 20, "bf16", 854, "normal0.1"), "mix", 0.2),
]


@pytest.mark.parametrize("spec,mode,p", BF_SPECS, ids=lambda v: _id(v) if isinstance(v, Spec) else str(v))
def test_batch_first_training_matches_oracle(spec, mode, p):
    import torch
    from layer_lstm_forward_amd.synth import make_lengths
    print(f"case {_id(spec)} batch-first lengths {mode} dropout {p}", flush=True)
    inp = make_inputs(spec)
    lens = None if mode is None else make_lengths(spec, mode)
    bf = spec.dtype == "bf16"
    dev = "cuda:0"
    H, L, bidir = spec.hidden_size, spec.num_layers, spec.bidirectional
    seed, call = 77, 5
    dy, dhn, dcn = _grads(spec, spec.seed + 5)
    if bf:
        from layer_lstm_forward_amd.synth import bf16_bits_to_f32, f32_to_bf16_bits
        dy_b, dhn_b = f32_to_bf16_bits(dy), f32_to_bf16_bits(dhn)
        dy, dhn = bf16_bits_to_f32(dy_b), bf16_bits_to_f32(dhn_b)
    m = pkg.LSTM(spec.input_size, H, L, bidir, bias=spec.has_bias, dtype=spec.dtype, batch_first=True)
    if p:
        m.set_dropout(p, seed, call)
    tb = lambda a: np.ascontiguousarray(a.transpose(1, 0, 2))  # noqa: E731
    x = to_dev(tb(inp.x), bf, dev)
    w = [to_dev(q, bf, dev) for q in inp.params]
    h0 = to_dev(inp.h0, bf, dev)
    c0 = None if inp.c0 is None else torch.from_numpy(inp.c0).to(dev)
    y, hn, cn, reserve = m.forward_train(x, w, h0, c0, lengths=lens)
    torch.cuda.synchronize()
    drop = (p, seed, call) if p else None
    ry, rhn, rcn = oracle.lstm_forward(inp.x, inp.params, H, L, bidir, h0=inp.h0, c0=inp.c0, has_bias=spec.has_bias,
                                       bf16=bf, dropout=drop, lengths=lens)
    cpu = lambda t: t.float().cpu().numpy().astype(np.float64)  # noqa: E731
    for got, ref, what in ((tb(cpu(y)), ry, "y"), (cpu(hn), rhn, "h_n"), (cpu(cn), rcn, "c_n")):
        err = float(np.max(np.abs(got - ref)))
        assert err <= FWD_TOL[spec.dtype], f"{what}: max-abs error {err:.3g}"
    dy_d = to_dev(tb(dy_b if bf else dy), bf, dev)
    dhn_d = to_dev(dhn_b if bf else dhn, bf, dev)
    dx, dh0, dc0, dws = m.backward(x, w, y, reserve, dy_d, h0=h0, c0=c0, dh_n=dhn_d,
                                   dc_n=torch.from_numpy(dcn).to(dev), lengths=lens)
    torch.cuda.synchronize()
    assert m.backward_status() == (0, 0)  # no hand-over wait gave up
    rdx, rdh0, rdc0, rdps = oracle.lstm_backward(inp.x, inp.params, H, L, bidir, dy, h0=inp.h0, c0=inp.c0, dh_n=dhn,
                                                 dc_n=dcn, has_bias=spec.has_bias, bf16=bf, dropout=drop,
                                                 lengths=lens)
    _check(tb(cpu(dx)), rdx, spec.dtype, "dx")
    if inp.h0 is not None:
        _check(cpu(dh0), rdh0, spec.dtype, "dh0")
        _check(cpu(dc0), rdc0, spec.dtype, "dc0")
    for k, (g, r) in enumerate(zip(dws, rdps)):
        _check(cpu(g), r, spec.dtype, f"dweights[{k}]")


FULL_TRAIN = [
    # the training benchmark's workload: (spec, sampled batch rows); its 128
    # recurrent 16x16 tiles leave half the CUs idle, so K is split between
    # two workgroups.  (The bidirectional bf16 workload would take the oracle
    # about 100 s per row; its 256-tile schedule is checked at a smaller T.)
    (Spec(256, 512, 2, False, 128, 64, "f32", 1101, "normal0.1"), [0, 29, 63]),
]


@pytest.mark.parametrize("spec,rows", FULL_TRAIN, ids=lambda v: _id(v) if isinstance(v, Spec) else "")
def test_full_size_training_sampled_rows(spec, rows):
    # Rows are independent given their own dy, dh_n and dc_n, so dx, dh0 and
    # dc0 of a few rows of the full-size launch are checked against the
    # oracle run on those rows alone.  (The weight gradients sum over every
    # row; the smaller cases above check them element by element.)
    import torch
    print(f"case {_id(spec)} full-size training, rows {rows}", flush=True)
    inp = make_inputs(spec)
    bf = spec.dtype == "bf16"
    dev = "cuda:0"
    dy, dhn, dcn = _grads(spec, spec.seed + 5)
    if bf:
        from layer_lstm_forward_amd.synth import bf16_bits_to_f32, f32_to_bf16_bits
        dy_b, dhn_b = f32_to_bf16_bits(dy), f32_to_bf16_bits(dhn)
        dy, dhn = bf16_bits_to_f32(dy_b), bf16_bits_to_f32(dhn_b)
    m = pkg.LSTM(spec.input_size, spec.hidden_size, spec.num_layers, spec.bidirectional, dtype=spec.dtype)
    x = to_dev(inp.x, bf, dev)
    w = [to_dev(p, bf, dev) for p in inp.params]
    h0 = None if inp.h0 is None else to_dev(inp.h0, bf, dev)
    c0 = None if inp.c0 is None else torch.from_numpy(inp.c0).to(dev)
    y, hn, cn, reserve = m.forward_train(x, w, h0, c0)
    dx, dh0, dc0, dws = m.backward(x, w, y, reserve, to_dev(dy_b if bf else dy, bf, dev), h0=h0, c0=c0,
                                   dh_n=to_dev(dhn_b if bf else dhn, bf, dev), dc_n=torch.from_numpy(dcn).to(dev))
    torch.cuda.synchronize()
    assert m.backward_status() == (0, 0)
    sub = inp.rows(rows)
    rdx, rdh0, rdc0, _ = oracle.lstm_backward(sub.x, sub.params, spec.hidden_size, spec.num_layers,
                                              spec.bidirectional, np.ascontiguousarray(dy[:, rows]), h0=sub.h0,
                                              c0=sub.c0, dh_n=np.ascontiguousarray(dhn[:, rows]),
                                              dc_n=np.ascontiguousarray(dcn[:, rows]), bf16=bf)
    cpu = lambda t: t.float().cpu().numpy()  # noqa: E731
    _check(cpu(dx)[:, rows], rdx, spec.dtype, "dx")
    _check(cpu(dh0)[:, rows], rdh0, spec.dtype, "dh0")
    _check(cpu(dc0)[:, rows], rdc0, spec.dtype, "dc0")


@pytest.mark.parametrize("spec,rows", FULL_TRAIN, ids=lambda v: _id(v) if isinstance(v, Spec) else "")
def test_full_size_weight_gradients_of_sampled_rows(spec, rows):
    # The weight and bias gradients sum over every row, so at full size they
    # are checked through the rows' independence: every row outside `rows`
    # gets zero dy, dh_n and dc_n, hence zero gradient at every step, and the
    # full-size launch's weight gradients must then equal the oracle's for
    # the sampled rows alone.  dx of the zeroed rows must be exactly zero.
    import torch
    print(f"case {_id(spec)} full-size weight gradients, rows {rows}", flush=True)
    inp = make_inputs(spec)
    assert spec.dtype == "f32"
    dev = "cuda:0"
    dy, dhn, dcn = _grads(spec, spec.seed + 7)
    others = np.setdiff1d(np.arange(spec.B), rows)
    dy[:, others] = 0.0
    dhn[:, others] = 0.0
    dcn[:, others] = 0.0
    m = pkg.LSTM(spec.input_size, spec.hidden_size, spec.num_layers, spec.bidirectional, dtype=spec.dtype)
    x = to_dev(inp.x, False, dev)
    w = [to_dev(p, False, dev) for p in inp.params]
    h0 = None if inp.h0 is None else to_dev(inp.h0, False, dev)
    c0 = None if inp.c0 is None else torch.from_numpy(inp.c0).to(dev)
    y, hn, cn, reserve = m.forward_train(x, w, h0, c0)
    dx, dh0, dc0, dws = m.backward(x, w, y, reserve, to_dev(dy, False, dev), h0=h0, c0=c0,
                                   dh_n=to_dev(dhn, False, dev), dc_n=torch.from_numpy(dcn).to(dev))
    torch.cuda.synchronize()
    assert m.backward_status() == (0, 0)
    sub = inp.rows(rows)
    rdx, _, _, rdws = oracle.lstm_backward(sub.x, sub.params, spec.hidden_size, spec.num_layers,
                                           spec.bidirectional, np.ascontiguousarray(dy[:, rows]), h0=sub.h0,
                                           c0=sub.c0, dh_n=np.ascontiguousarray(dhn[:, rows]),
                                           dc_n=np.ascontiguousarray(dcn[:, rows]), bf16=False)
    cpu = lambda t: t.float().cpu().numpy()  # noqa: E731
    _check(cpu(dx)[:, rows], rdx, spec.dtype, "dx")
    assert np.all(cpu(dx)[:, others] == 0.0)
    assert len(dws) == len(rdws)
    for k, (g, r) in enumerate(zip(dws, rdws)):
        _check(cpu(g), r, spec.dtype, f"dweights[{k}]")

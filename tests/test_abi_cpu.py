"""The C ABI without a GPU: the library loads, exports every function declared
in include/lstm.h, and its host-side checks return the documented status codes
before anything touches a device."""
import ctypes
import os
import re

import pytest

import layer_lstm_forward_amd as pkg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lstm.h")

pytestmark = pytest.mark.skipif(not os.path.exists(pkg.LIB_PATH), reason="liblstm_amd.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lstm_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_function():
    names = declared_functions()
    assert {"lstm_create", "lstm_forward", "lstm_destroy", "lstm_workspace_size"} <= set(names)
    lib = ctypes.CDLL(pkg.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in lstm.h but not exported"


def test_version_and_strerror():
    assert pkg.lstm_version() == 110
    for code in pkg.STATUS:
        assert pkg.lstm_strerror(code) and pkg.lstm_strerror(code) != "unknown status"
    assert pkg.lstm_strerror(12345) == "unknown status"


@pytest.mark.parametrize("args,code", [
    ((8, 16, 0, 0, 1, 0), -1),    # fewer than one layer
    ((0, 16, 1, 0, 1, 0), -1),
    ((8, 0, 1, 0, 1, 0), -1),
    ((8, 16, 1, 2, 1, 0), -1),    # bidirectional not 0/1
    ((8, 16, 1, 0, 3, 0), -1),
    ((8, 16, 1, 0, 1, 7), -3),    # dtype
])
def test_create_errors(args, code):
    lib = pkg.load_library()
    h = ctypes.c_void_p(1)
    assert lib.lstm_create(ctypes.byref(h), *args) == code
    assert h.value is None
    assert lib.lstm_create(None, 8, 16, 1, 0, 1, 0) == -1


def test_workspace_size_layout():
    p1 = pkg.lstm_create(8, 16, 1, False, True, pkg.LSTM_F32)
    p3 = pkg.lstm_create(8, 16, 3, True, True, pkg.LSTM_BF16)
    try:
        a = pkg.lstm_workspace_size(p1, 5, 1)
        b = pkg.lstm_workspace_size(p1, 10, 1)
        assert 0 < a < b
        # G holds T*B*D*4H fp32 values
        assert b - a >= 5 * 4 * 16 * 4
        c = pkg.lstm_workspace_size(p3, 5, 2)
        assert c > 2 * 5 * 2 * 2 * 16 * 2  # two intermediate outputs of [T,B,D*H] bf16
        with pytest.raises(pkg.LSTMError) as e:
            pkg.lstm_workspace_size(p1, 0, 1)
        assert e.value.status == -2
    finally:
        pkg.lstm_destroy(p1)
        pkg.lstm_destroy(p3)


def test_set_option():
    p = pkg.lstm_create(8, 16, 1, False, True, pkg.LSTM_F32)
    try:
        pkg.lstm_set_option(p, pkg.LSTM_OPT_RECURRENCE, pkg.LSTM_REC_GEMM)
        pkg.lstm_set_option(p, pkg.LSTM_OPT_RECURRENCE, pkg.LSTM_REC_STEP)
        pkg.lstm_set_option(p, pkg.LSTM_OPT_REC_TILE, 412)
        for v in (0, 1000, 100000):
            pkg.lstm_set_option(p, pkg.LSTM_OPT_READ_PACE, v)
        for v in (0, 1):
            pkg.lstm_set_option(p, pkg.LSTM_OPT_FUSE_INPUT, v)
            pkg.lstm_set_option(p, pkg.LSTM_OPT_BATCH_FIRST, v)
        for opt, val in ((pkg.LSTM_OPT_RECURRENCE, 4), (pkg.LSTM_OPT_REC_TILE, 333), (6, 0),
                         (pkg.LSTM_OPT_READ_PACE, -1), (pkg.LSTM_OPT_READ_PACE, 100001),
                         (pkg.LSTM_OPT_FUSE_INPUT, 2), (pkg.LSTM_OPT_BATCH_FIRST, -1), (99, 0)):
            with pytest.raises(pkg.LSTMError) as e:
                pkg.lstm_set_option(p, opt, val)
            assert e.value.status == -7
    finally:
        pkg.lstm_destroy(p)


FAKE = 0x10000  # never dereferenced: every case below fails host validation first


def _fwd(plan, **kw):
    a = dict(x=FAKE, h0=0, c0=0, weights=[FAKE] * 4, T=5, B=1, layers=1, bidir=False, y=FAKE, h_n=0, c_n=0,
             workspace=FAKE, workspace_bytes=1 << 40, stream=0)
    a.update(kw)
    return pkg.lstm_forward(plan, a["x"], a["h0"], a["c0"], a["weights"], a["T"], a["B"], a["layers"],
                            a["bidir"], a["y"], a["h_n"], a["c_n"], a["workspace"], a["workspace_bytes"],
                            a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(layers=2), -2),
    (dict(bidir=True), -2),
    (dict(T=0), -2),
    (dict(B=0), -2),
    (dict(B=-3), -2),
    (dict(x=0), -1),
    (dict(y=0), -1),
    (dict(h0=FAKE), -1),             # h0 without c0
    (dict(c0=FAKE), -1),             # c0 without h0
    (dict(weights=[FAKE, 0, FAKE, FAKE]), -1),
    (dict(workspace=0), -5),
    (dict(workspace_bytes=64), -5),
])
def test_forward_host_validation(kw, code):
    p = pkg.lstm_create(8, 16, 1, False, True, pkg.LSTM_F32)
    try:
        assert _fwd(p, **kw) == code
    finally:
        pkg.lstm_destroy(p)


def test_forward_null_plan():
    assert _fwd(None) == -1


def _fwd_len(plan, lengths, **kw):
    a = dict(x=FAKE, h0=0, c0=0, weights=[FAKE] * 4, T=5, B=2, layers=1, bidir=False, y=FAKE, h_n=0, c_n=0,
             workspace=FAKE, workspace_bytes=1 << 40, stream=0)
    a.update(kw)
    return pkg.lstm_forward_lengths(plan, a["x"], lengths, a["h0"], a["c0"], a["weights"], a["T"], a["B"],
                                    a["layers"], a["bidir"], a["y"], a["h_n"], a["c_n"], a["workspace"],
                                    a["workspace_bytes"], a["stream"])


@pytest.mark.parametrize("lengths,kw,code", [
    (None, {}, -1),                   # no lengths
    ([0, 5], {}, -1),                 # a row without steps
    ([5, 6], {}, -1),                 # longer than T
    ([5, -1], {}, -1),
    ([5, 5], dict(T=0), -2),
    ([5, 5], dict(layers=3), -2),     # the rest is checked as lstm_forward does
    ([5, 5], dict(workspace_bytes=64), -5),
])
def test_forward_lengths_host_validation(lengths, kw, code):
    p = pkg.lstm_create(8, 16, 1, False, True, pkg.LSTM_F32)
    try:
        assert _fwd_len(p, lengths, **kw) == code
    finally:
        pkg.lstm_destroy(p)


def test_forward_weights_count_follows_bias_flag():
    p = pkg.lstm_create(8, 16, 1, False, False, pkg.LSTM_F32)
    try:
        # without biases only W_ih and W_hh are read: two entries pass the
        # NULL check and reach the device check; a NULL second entry does not
        assert _fwd(p, weights=[FAKE, FAKE]) == -4
        assert _fwd(p, weights=[FAKE, 0]) == -1
    finally:
        pkg.lstm_destroy(p)


def test_forward_rejects_non_device_pointers():
    """Valid shapes but pointers that are not device memory (or no device at
    all): LSTM_ERR_DEVICE, before any launch."""
    p = pkg.lstm_create(8, 16, 1, False, True, pkg.LSTM_F32)
    try:
        host = (ctypes.c_float * 64)()
        addr = ctypes.addressof(host)
        assert _fwd(p, x=addr, y=addr, workspace=addr, weights=[addr] * 4) == -4
    finally:
        pkg.lstm_destroy(p)


def test_dropout_settings_and_reserve_size():
    # prob in [0, 1]; the reserve grows by each dropped layer input and its keep bytes
    for dtype, es in (("f32", 4), ("bf16", 2)):
        p = pkg.lstm_create(24, 32, 3, True, True, pkg.LSTM_BF16 if dtype == "bf16" else pkg.LSTM_F32)
        try:
            T, B, D, H = 7, 5, 2, 32
            base = pkg.lstm_reserve_size(p, T, B)
            for bad in (-0.1, 1.5, float("nan")):
                with pytest.raises(pkg.LSTMError):
                    pkg.lstm_set_dropout(p, bad, 1, 0)
            assert pkg.lstm_reserve_size(p, T, B) == base
            pkg.lstm_set_dropout(p, 0.25, 99, 3)
            n = T * B * D * H
            up = lambda v: (v + 255) // 256 * 256  # noqa: E731
            assert pkg.lstm_reserve_size(p, T, B) == base + 2 * (up(n * es) + up(n))
            pkg.lstm_set_dropout(p, 0.0, 99, 3)
            assert pkg.lstm_reserve_size(p, T, B) == base
        finally:
            pkg.lstm_destroy(p)
    # one layer: nothing to drop
    p = pkg.lstm_create(8, 16, 1, False, True, pkg.LSTM_F32)
    try:
        base = pkg.lstm_reserve_size(p, 4, 2)
        pkg.lstm_set_dropout(p, 0.5, 1, 0)
        assert pkg.lstm_reserve_size(p, 4, 2) == base
    finally:
        pkg.lstm_destroy(p)


def test_modes_create_and_validate():
    # mode outside the enum; the GRU's projection is 3H wide, the RNNs' H
    h = ctypes.c_void_p()
    lib = ctypes.CDLL(pkg.LIB_PATH)
    assert lib.lstm_create_mode(ctypes.byref(h), 4, 8, 16, 1, 0, 1, 0) == -1
    assert lib.lstm_create_mode(ctypes.byref(h), -1, 8, 16, 1, 0, 1, 0) == -1
    sizes = {}
    for name, mode in pkg.MODES.items():
        p = pkg.lstm_create_mode(mode, 24, 32, 2, True, True, pkg.LSTM_F32)
        try:
            sizes[name] = pkg.lstm_workspace_size(p, 10, 8)
            if mode != pkg.LSTM_MODE_LSTM:
                FAKE = 0x10000
                # c0 (and c_n) belong to the LSTM only; validation precedes any device access
                rc = pkg.lstm_forward(p, FAKE, FAKE, FAKE, [FAKE] * 8, 10, 8, 2, True, FAKE, 0, 0, FAKE, 1 << 40, 0)
                assert rc == -1
                rc = pkg.lstm_forward_lengths(p, FAKE, [3] * 8, 0, FAKE, [FAKE] * 8, 10, 8, 2, True, FAKE, 0, 0,
                                              FAKE, 1 << 40, 0)
                assert rc == -1
                rc = pkg.lstm_forward_lengths(p, FAKE, [3] * 7 + [11], 0, 0, [FAKE] * 8, 10, 8, 2, True, FAKE, 0, 0,
                                              FAKE, 1 << 40, 0)
                assert rc == -1
                with pytest.raises(pkg.LSTMError):
                    pkg.lstm_reserve_size(p, 10, 8)
                with pytest.raises(pkg.LSTMError):
                    pkg.lstm_backward_workspace_size(p, 10, 8)
        finally:
            pkg.lstm_destroy(p)
    # the other modes add their parameters padded to four gate blocks (W_ih,
    # W_hh, b_ih, b_hh per layer and direction, 256-byte aligned)
    up = lambda v: (v + 255) // 256 * 256  # noqa: E731
    pad = sum(2 * (up(128 * in_l * 4) + up(128 * 32 * 4) + 2 * up(128 * 4)) for in_l in (24, 64))
    for name in ("gru", "rnn_tanh", "rnn_relu"):
        assert sizes[name] - sizes["lstm"] == pad


def test_training_lengths_validated_on_the_host():
    # NULL lengths and lengths outside 1..T are argument errors, before any device access
    FAKE = 0x10000
    p = pkg.lstm_create(8, 16, 1, False, True, pkg.LSTM_F32)
    lib = ctypes.CDLL(pkg.LIB_PATH)
    try:
        common = dict(h0=0, c0=0, weights=[FAKE] * 4, T=5, B=2, layers=1, bidir=False, y=FAKE, h_n=0, c_n=0,
                      reserve=FAKE, reserve_bytes=1 << 40, workspace=FAKE, workspace_bytes=1 << 40, stream=0)
        for bad in ([0, 3], [6, 1]):
            assert pkg.lstm_forward_train(p, FAKE, lengths=bad, **common) == -1
        v = ctypes.c_void_p
        assert lib.lstm_forward_train_lengths(v(p), v(FAKE), None, None, None, pkg._ptrs([FAKE] * 4), 5, 2, 1, 0,
                                              v(FAKE), None, None, v(FAKE), ctypes.c_size_t(1 << 40), v(FAKE),
                                              ctypes.c_size_t(1 << 40), None) == -1
        bargs = dict(h0=0, c0=0, weights=[FAKE] * 4, y=FAKE, dy=FAKE, dh_n=0, dc_n=0, reserve=FAKE,
                     reserve_bytes=1 << 40, T=5, B=2, layers=1, bidir=False, dx=0, dh0=0, dc0=0,
                     dweights=[FAKE] * 4, workspace=FAKE, workspace_bytes=1 << 40, stream=0)
        for bad in ([0, 3], [6, 1]):
            assert pkg.lstm_backward(p, FAKE, lengths=bad, **bargs) == -1
    finally:
        pkg.lstm_destroy(p)


def test_backward_rejects_steps_past_32_bit_offsets():
    # one step's saved activations (B * D * 5H floats) must stay under 2^31
    # bytes: the backward cell reads them with 32-bit offsets; checked on the
    # host before any device access
    FAKE = 0x10000
    p = pkg.lstm_create(8, 2048, 1, True, True, pkg.LSTM_F32)
    try:
        bargs = dict(h0=0, c0=0, weights=[FAKE] * 8, y=FAKE, dy=FAKE, dh_n=0, dc_n=0, reserve=FAKE,
                     reserve_bytes=1 << 60, T=1, B=32768, layers=1, bidir=True, dx=0, dh0=0, dc0=0,
                     dweights=[FAKE] * 8, workspace=FAKE, workspace_bytes=1 << 60, stream=0)
        assert pkg.lstm_backward(p, FAKE, **bargs) == -7          # 32768 * 2 * 5 * 2048 * 4 = 2^31 bytes
        assert pkg.lstm_backward(p, FAKE, **dict(bargs, B=0)) == -2
    finally:
        pkg.lstm_destroy(p)


def test_packed_batch_sizes_validated_on_the_host():
    # batch_sizes must be non-increasing and positive (B = batch_sizes[0]);
    # checked before any device access
    FAKE = 0x10000
    p = pkg.lstm_create(8, 16, 1, False, True, pkg.LSTM_F32)
    try:
        n = pkg.lstm_packed_workspace_size(p, [3, 2, 2, 1])
        assert n >= pkg.lstm_workspace_size(p, 4, 3)
        for bad in ([2, 3], [3, 0], [0], [3, -1, 1]):
            with pytest.raises(pkg.LSTMError):
                pkg.lstm_packed_workspace_size(p, bad)
            assert pkg.lstm_forward_packed(p, FAKE, bad, 0, 0, [FAKE] * 4, 1, False, FAKE, 0, 0, FAKE, 1 << 40,
                                           0) == -1
        assert pkg.lstm_forward_packed(p, FAKE, None, 0, 0, [FAKE] * 4, 1, False, FAKE, 0, 0, FAKE, 1 << 40, 0,
                                       T=2) == -1
        assert pkg.lstm_forward_packed(p, FAKE, [3, 2], 0, 0, [FAKE] * 4, 1, False, FAKE, 0, 0, FAKE, 16, 0) == -5
    finally:
        pkg.lstm_destroy(p)
    q = pkg.lstm_create(8, 16, 1, False, True, pkg.LSTM_F32)
    try:
        pkg.lstm_set_option(q, pkg.LSTM_OPT_BATCH_FIRST, 1)  # raises on failure
        assert pkg.lstm_forward_packed(q, FAKE, [2, 1], 0, 0, [FAKE] * 4, 1, False, FAKE, 0, 0, FAKE, 1 << 40,
                                       0) == -7
    finally:
        pkg.lstm_destroy(q)

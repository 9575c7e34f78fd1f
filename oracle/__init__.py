"""fp64 CPU oracle of the multi-layer, optionally bidirectional LSTM forward.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The product (``layer_lstm_forward_amd``)
never imports this package, and this package imports nothing from it.

The arithmetic lives in ``lstm_oracle.c`` (plain loops, fp64, built with
``-O2`` and without fast-math); this module only builds it, converts inputs to
float64 exactly and calls it.  Which passage of the source pages each step
follows is stated at the top of the C file.

Inputs may be float32/float64 arrays, or bfloat16 bit patterns held in uint16
arrays (``bf16=True``); both convert to float64 without rounding.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_DIR = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_DIR, "lstm_oracle.c")
_LIB = os.path.join(_DIR, "liblstm_oracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, no fast-math, OpenMP) into a .so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
             "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        # LSTM_ORACLE_LIB lets the mutation test point the pins at a copy of
        # the oracle built with a planted mistake.
        path = os.environ.get("LSTM_ORACLE_LIB") or build()
        lib = ctypes.CDLL(path)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.oracle_lstm_forward.restype = ctypes.c_int
        lib.oracle_lstm_forward.argtypes = [
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            dp, dp, dp, ctypes.POINTER(dp), ctypes.c_int, dp, dp, dp, ctypes.c_int]
        lib.oracle_lstm_forward_lengths.restype = ctypes.c_int
        lib.oracle_lstm_forward_lengths.argtypes = [
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            dp, ctypes.POINTER(ctypes.c_int), dp, dp, ctypes.POINTER(dp), ctypes.c_int, dp, dp, dp,
            ctypes.c_int]
        u64 = ctypes.c_uint64
        lib.oracle_lstm_forward_dropout.restype = ctypes.c_int
        lib.oracle_lstm_forward_dropout.argtypes = [
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            dp, ctypes.POINTER(ctypes.c_int), dp, dp, ctypes.POINTER(dp), ctypes.c_int, ctypes.c_double, u64, u64,
            dp, dp, dp, ctypes.c_int]
        lib.oracle_lstm_backward.restype = ctypes.c_int
        lib.oracle_lstm_backward.argtypes = [
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            dp, ctypes.POINTER(ctypes.c_int), dp, dp, ctypes.POINTER(dp), ctypes.c_int, ctypes.c_double, u64, u64,
            dp, dp, dp, dp, dp, dp, ctypes.POINTER(dp)]
        lib.oracle_rnn_forward.restype = ctypes.c_int
        lib.oracle_rnn_forward.argtypes = [
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            dp, ctypes.POINTER(ctypes.c_int), dp, ctypes.POINTER(dp), ctypes.c_int, dp, dp, ctypes.c_int]
        lib.oracle_dropout_keep.restype = None
        lib.oracle_dropout_keep.argtypes = [ctypes.c_double, u64, u64, ctypes.c_int, ctypes.c_size_t,
                                            ctypes.POINTER(ctypes.c_ubyte)]
        lib.oracle_philox4x64_10.restype = None
        lib.oracle_philox4x64_10.argtypes = [ctypes.POINTER(u64), ctypes.POINTER(u64), ctypes.POINTER(u64)]
        lib.oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def as_f64(a, bf16: bool = False) -> np.ndarray:
    """Exact conversion to float64 (bf16 bit patterns widen by a 16-bit shift)."""
    a = np.asarray(a)
    if bf16:
        assert a.dtype == np.uint16, "bf16 inputs are passed as uint16 bit patterns"
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def _ptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def lstm_forward(x, params, hidden_size: int, num_layers: int, bidirectional: bool,
                 h0=None, c0=None, has_bias: bool = True, bf16: bool = False,
                 c_state_bf16: bool = False, nthreads: int = 1, lengths=None, dropout=None):
    """Run the oracle.

    x       [T, B, I]
    params  flat list in (layer, direction, W_ih, W_hh[, b_ih, b_hh]) order
    h0, c0  [L*D, B, H] or None (zeros); c0 is never bf16 unless c_state_bf16
    lengths None (every row has T steps) or B ints in 1..T: row b takes part
            only in steps t < lengths[b] (see the C file)
    dropout None, or (p, seed, call): the training forward's dropout between
            layers (see the C file)
    Returns (y [T, B, D*H], h_n [L*D, B, H], c_n [L*D, B, H]) as float64.
    """
    lib = _load()
    x64 = np.ascontiguousarray(as_f64(x, bf16))
    T, B, I = x64.shape
    H, L, D = int(hidden_size), int(num_layers), 2 if bidirectional else 1
    per = 4 if has_bias else 2
    if len(params) != L * D * per:
        raise ValueError(f"expected {L * D * per} parameter arrays, got {len(params)}")
    p64 = [np.ascontiguousarray(as_f64(p, bf16)) for p in params]
    for idx, p in enumerate(p64):
        l, rem = divmod(idx, D * per)
        kind = rem % per
        in_l = I if l == 0 else D * H
        want = [(4 * H, in_l), (4 * H, H), (4 * H,), (4 * H,)][kind]
        if p.shape != want:
            raise ValueError(f"param {idx} has shape {p.shape}, expected {want}")
    arr = (ctypes.POINTER(ctypes.c_double) * len(p64))(*[_ptr(p) for p in p64])
    h064 = None if h0 is None else np.ascontiguousarray(as_f64(h0, bf16))
    c064 = None if c0 is None else np.ascontiguousarray(as_f64(c0, c_state_bf16))
    for s in (h064, c064):
        if s is not None and s.shape != (L * D, B, H):
            raise ValueError(f"state shape {s.shape} != {(L * D, B, H)}")
    len32 = None
    if lengths is not None:
        len32 = np.ascontiguousarray(np.asarray(lengths, np.int32))
        if len32.shape != (B,):
            raise ValueError(f"lengths shape {len32.shape} != {(B,)}")
    y = np.empty((T, B, D * H), np.float64)
    hn = np.empty((L * D, B, H), np.float64)
    cn = np.empty((L * D, B, H), np.float64)
    if dropout is not None:
        dp_, seed, call = dropout
        rc = lib.oracle_lstm_forward_dropout(
            T, B, I, H, L, D, _ptr(x64),
            len32.ctypes.data_as(ctypes.POINTER(ctypes.c_int)) if len32 is not None else None,
            _ptr(h064) if h064 is not None else None,
            _ptr(c064) if c064 is not None else None, arr, 1 if has_bias else 0, float(dp_), int(seed), int(call),
            _ptr(y), _ptr(hn), _ptr(cn), int(nthreads))
        if rc != 0:
            raise RuntimeError(f"oracle_lstm_forward_dropout failed with {rc}")
        return y, hn, cn
    rc = lib.oracle_lstm_forward_lengths(
        T, B, I, H, L, D, _ptr(x64),
        len32.ctypes.data_as(ctypes.POINTER(ctypes.c_int)) if len32 is not None else None,
        _ptr(h064) if h064 is not None else None,
        _ptr(c064) if c064 is not None else None,
        arr, 1 if has_bias else 0, _ptr(y), _ptr(hn), _ptr(cn), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_lstm_forward failed with {rc}")
    return y, hn, cn


def lstm_backward(x, params, hidden_size: int, num_layers: int, bidirectional: bool, dy,
                  h0=None, c0=None, dh_n=None, dc_n=None, has_bias: bool = True, bf16: bool = False,
                  dropout=None, lengths=None):
    """Gradients of the forward pass (see the C file).

    dy [T, B, D*H]; dh_n, dc_n [L*D, B, H] or None (zeros).
    Returns (dx [T, B, I], dh0 [L*D, B, H], dc0 [L*D, B, H], dparams) as
    float64, dparams in the order and shapes of params.
    """
    lib = _load()
    x64 = np.ascontiguousarray(as_f64(x, bf16))
    T, B, I = x64.shape
    H, L, D = int(hidden_size), int(num_layers), 2 if bidirectional else 1
    per = 4 if has_bias else 2
    if len(params) != L * D * per:
        raise ValueError(f"expected {L * D * per} parameter arrays, got {len(params)}")
    p64 = [np.ascontiguousarray(as_f64(p, bf16)) for p in params]
    arr = (ctypes.POINTER(ctypes.c_double) * len(p64))(*[_ptr(p) for p in p64])
    dps = [np.empty_like(p) for p in p64]
    darr = (ctypes.POINTER(ctypes.c_double) * len(dps))(*[_ptr(p) for p in dps])
    h064 = None if h0 is None else np.ascontiguousarray(as_f64(h0, bf16))
    c064 = None if c0 is None else np.ascontiguousarray(as_f64(c0))
    dy64 = np.ascontiguousarray(np.asarray(dy, np.float64))
    if dy64.shape != (T, B, D * H):
        raise ValueError(f"dy shape {dy64.shape} != {(T, B, D * H)}")
    dhn = None if dh_n is None else np.ascontiguousarray(np.asarray(dh_n, np.float64))
    dcn = None if dc_n is None else np.ascontiguousarray(np.asarray(dc_n, np.float64))
    dx = np.empty((T, B, I), np.float64)
    dh0 = np.empty((L * D, B, H), np.float64)
    dc0 = np.empty((L * D, B, H), np.float64)
    opt = lambda a: _ptr(a) if a is not None else None  # noqa: E731
    dp_, seed, call = (0.0, 0, 0) if dropout is None else dropout
    len32 = None
    if lengths is not None:
        len32 = np.ascontiguousarray(np.asarray(lengths, np.int32))
        if len32.shape != (B,):
            raise ValueError(f"lengths shape {len32.shape} != {(B,)}")
    lenp = len32.ctypes.data_as(ctypes.POINTER(ctypes.c_int)) if len32 is not None else None
    rc = lib.oracle_lstm_backward(T, B, I, H, L, D, _ptr(x64), lenp, opt(h064), opt(c064), arr, 1 if has_bias else 0,
                                  float(dp_), int(seed), int(call), _ptr(dy64), opt(dhn), opt(dcn), _ptr(dx), _ptr(dh0), _ptr(dc0), darr)
    if rc != 0:
        raise RuntimeError(f"oracle_lstm_backward failed with {rc}")
    return dx, dh0, dc0, dps


def philox4x64_10(counter, key):
    """One Philox4x64-10 block (four uint64 words) of the oracle's generator."""
    lib = _load()
    c = (ctypes.c_uint64 * 4)(*[int(v) for v in counter])
    k = (ctypes.c_uint64 * 2)(*[int(v) for v in key])
    out = (ctypes.c_uint64 * 4)()
    lib.oracle_philox4x64_10(c, k, out)
    return [int(v) for v in out]


def dropout_keep(p, seed, call, layer, n):
    """The training dropout's keep decisions (uint8, 1 = kept) of elements
    0..n-1 of layer `layer`'s output for draw (seed, call)."""
    lib = _load()
    out = np.zeros(int(n), np.uint8)
    lib.oracle_dropout_keep(float(p), int(seed), int(call), int(layer), int(n),
                            out.ctypes.data_as(ctypes.POINTER(ctypes.c_ubyte)))
    return out


MODES = {"gru": 1, "rnn_tanh": 2, "rnn_relu": 3}


def rnn_forward(mode, x, params, hidden_size: int, num_layers: int, bidirectional: bool, h0=None,
                has_bias: bool = True, bf16: bool = False, nthreads: int = 1, lengths=None):
    """The other recurrent modes ("gru", "rnn_tanh", "rnn_relu"; see the C
    file).  params in (layer, direction, W_ih, W_hh[, b_ih, b_hh]) order with
    3H (GRU) or H gate rows.  Returns (y [T, B, D*H], h_n [L*D, B, H]) as
    float64."""
    lib = _load()
    m = MODES[mode]
    x64 = np.ascontiguousarray(as_f64(x, bf16))
    T, B, I = x64.shape
    H, L, D = int(hidden_size), int(num_layers), 2 if bidirectional else 1
    per = 4 if has_bias else 2
    ng = 3 if m == 1 else 1
    if len(params) != L * D * per:
        raise ValueError(f"expected {L * D * per} parameter arrays, got {len(params)}")
    p64 = [np.ascontiguousarray(as_f64(p, bf16)) for p in params]
    for idx, p in enumerate(p64):
        l, rem = divmod(idx, D * per)
        in_l = I if l == 0 else D * H
        want = [(ng * H, in_l), (ng * H, H), (ng * H,), (ng * H,)][rem % per]
        if p.shape != want:
            raise ValueError(f"param {idx} has shape {p.shape}, expected {want}")
    arr = (ctypes.POINTER(ctypes.c_double) * len(p64))(*[_ptr(p) for p in p64])
    h064 = None if h0 is None else np.ascontiguousarray(as_f64(h0, bf16))
    if h064 is not None and h064.shape != (L * D, B, H):
        raise ValueError(f"h0 shape {h064.shape} != {(L * D, B, H)}")
    y = np.empty((T, B, D * H), np.float64)
    hn = np.empty((L * D, B, H), np.float64)
    len32 = None if lengths is None else np.ascontiguousarray(np.asarray(lengths, np.int32))
    if len32 is not None and len32.shape != (B,):
        raise ValueError(f"lengths shape {len32.shape} != {(B,)}")
    rc = lib.oracle_rnn_forward(m, T, B, I, H, L, D, _ptr(x64),
                                len32.ctypes.data_as(ctypes.POINTER(ctypes.c_int)) if len32 is not None else None,
                                _ptr(h064) if h064 is not None else None, arr,
                                1 if has_bias else 0, _ptr(y), _ptr(hn), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_rnn_forward failed with {rc}")
    return y, hn

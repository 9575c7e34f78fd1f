"""The exchange word formats of the persistent recurrence, checked on the CPU.

Workgroups of the persistent recurrence hand h_t to each other as 32-bit words
that carry the value and a one-bit step tag (device.h).  These tests compile
the word functions for the host (hipcc --offload-host-only, tests/xword_host.cpp)
and check, over every bf16 bit pattern:
  - the bf16 pair word keeps its tag in bit 30, the top exponent bit of the
    upper value, so it is sound only for |h| < 2: at h = 2.0 the tag reads
    wrong and removing it destroys the value (why the relu RNN, the GRU from a
    caller's h0, and padded steps that republish h0 take the wide words);
  - the wide word (one bf16 value per word, tag in bit 0) round-trips every
    bf16 value, infinities and NaNs included, with either tag;
  - the fp32 word keeps the value within one ulp;
  - the tag sequence the host and kernels agree on alternates on every buffer
    across the layers of one call, starting from the zeroed buffer's tag 0.
"""
import ctypes
import os
import shutil
import subprocess

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
F32, PAIR, WIDE = 0, 1, 2


@pytest.fixture(scope="module")
def xw(tmp_path_factory):
    if not (os.path.exists(HIPCC) or shutil.which(HIPCC)):
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("xword") / "libxword_host.so")
    subprocess.run([HIPCC, "-x", "hip", "--offload-host-only", "-O1", "-std=c++17", "-shared", "-fPIC",
                    os.path.join(HERE, "xword_host.cpp"), "-o", out], check=True,
                   stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    lib = ctypes.CDLL(out)
    u32, u16, uint = ctypes.c_uint32, ctypes.c_uint16, ctypes.c_uint
    for name, res, args in (("xw_word_f32", u32, [u32, uint]), ("xw_word_pair", u32, [u16, u16, uint]),
                            ("xw_word_wide", u32, [u16, uint]), ("xw_word_tag", uint, [u32, ctypes.c_int]),
                            ("xw_pair_value", u32, [u32]), ("xw_wide_pair", u32, [u32, u32]),
                            ("xw_tag", uint, [uint, ctypes.c_int]),
                            ("xw_ok4", ctypes.c_int, [ctypes.POINTER(u32), uint, ctypes.c_int])):
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    return lib


def bf16_value(bits):
    return float(np.array([bits << 16], dtype=np.uint32).view(np.float32)[0])


def ok4(xw, words, tb, fmt):
    arr = (ctypes.c_uint32 * 4)(*words)
    return bool(xw.xw_ok4(arr, tb, fmt))


def test_pair_word_breaks_at_two(xw):
    """bf16(2.0) = 0x4000 in the upper half sets bit 30: the word reads as tag
    1 whatever tag was written, and removing the tag bit turns 2.0 into 0."""
    two = 0x4000
    assert bf16_value(two) == 2.0
    w = xw.xw_word_pair(0x3F80, two, 0)  # lower 1.0, upper 2.0, written with tag 0
    assert xw.xw_word_tag(w, PAIR) == 1  # the consumer sees the other tag
    assert not ok4(xw, [w] * 4, 0, PAIR)  # so it waits for a tag that never comes ...
    assert ok4(xw, [w] * 4, 1, PAIR)  # ... or accepts the word as the next step's
    assert xw.xw_pair_value(w) >> 16 == 0  # and the value 2.0 loses its top exponent bit: 0.0
    # -2.0 and larger magnitudes alike
    for hi in (0xC000, 0x4040, 0x7F7F):
        assert xw.xw_word_tag(xw.xw_word_pair(0, hi, 0), PAIR) == 1


def test_pair_word_sound_below_two(xw):
    """Every finite bf16 with |h| < 2 in either half keeps its tag and value."""
    bits = np.arange(0x10000, dtype=np.uint32)
    mag = bits & 0x7FFF
    small = bits[mag < 0x4000]  # biased exponent <= 127: |h| < 2
    rng = np.random.default_rng(5)
    for tb in (0, 1):
        for hi in small:
            lo = int(rng.choice(small))
            w = xw.xw_word_pair(lo, int(hi), tb)
            assert xw.xw_word_tag(w, PAIR) == tb
            v = xw.xw_pair_value(w)
            assert v & 0xFFFF == lo and v >> 16 == int(hi)


def test_wide_word_every_bf16(xw):
    """The wide word carries any bf16 (including inf and NaN) with either tag,
    and two wide words repack into the bf16 pair the matrix cores take."""
    for tb in (0, 1):
        prev = None
        for h in range(0x10000):
            w = xw.xw_word_wide(h, tb)
            assert xw.xw_word_tag(w, WIDE) == tb
            assert w >> 16 == h
            if prev is not None:
                pair = xw.xw_wide_pair(prev[1], w)
                assert pair & 0xFFFF == prev[0] and pair >> 16 == h
            prev = (h, w)
    big = [xw.xw_word_wide(b, 0) for b in (0x4000, 0xC000, 0x7F80, 0xFF80)]  # 2, -2, inf, -inf
    assert ok4(xw, big, 0, WIDE) and not ok4(xw, big, 1, WIDE)


def test_f32_word_within_one_ulp(xw):
    rng = np.random.default_rng(6)
    vals = np.concatenate([rng.standard_normal(2000).astype(np.float32) * 10.0 ** rng.integers(-3, 4, 2000),
                           np.array([2.0, -2.0, 1e30, -1e-30, 0.0], np.float32)])
    for tb in (0, 1):
        for v in vals.view(np.uint32):
            w = xw.xw_word_f32(int(v), tb)
            assert xw.xw_word_tag(w, F32) == tb
            assert abs(int(w) - int(v)) <= 1


def test_ok4_needs_all_four(xw):
    good = [xw.xw_word_wide(0x3F80, 1)] * 4
    for k in range(4):
        mixed = list(good)
        mixed[k] = xw.xw_word_wide(0x3F80, 0)
        assert not ok4(xw, mixed, 1, WIDE)
    assert ok4(xw, good, 1, WIDE)


@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 8, 127, 128])
def test_tag_sequence_alternates_across_layers(xw, T):
    """The host's per-layer update of the write parities (lstm_api.cpp) and the
    kernels' tag rule: each buffer's writes carry tags 1, 0, 1, ... over the
    whole call (the zeroed buffer holds tag 0), and a reader at step s expects
    the tag of the write at step s - 1."""
    layer_writes = ((T // 2) & 1) | ((((T - 1) // 2) & 1) << 1)
    xpar = 0
    last = {0: 0, 1: 0}
    for _layer in range(4):
        for s in range(T - 1):  # a layer publishes at every step but its last
            tag = xw.xw_tag(xpar, s)
            assert tag == 1 - last[s & 1], (T, s)
            last[s & 1] = tag
            if s >= 1:  # the reader of step s + 1 expects exactly this write
                assert xw.xw_tag(xpar, s) == tag
        xpar ^= layer_writes

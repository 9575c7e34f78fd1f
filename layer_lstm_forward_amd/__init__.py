"""MI355X (gfx950) LSTM forward: thin Python binding of liblstm_amd.so.

The functions below carry the names of the C ABI in include/lstm.h and only
marshal arguments; every step of the forward pass runs in the HIP kernels of
the shared library.  There is no fallback: if the library is not built or no
GPU is present, calls raise.

``LSTM`` is a convenience wrapper that owns a plan and a cached workspace and
takes/returns torch tensors (torch provides device memory and streams only).
"""
from __future__ import annotations

import ctypes
import os
import sys

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblstm_amd.so")

LSTM_F32, LSTM_BF16 = 0, 1
LSTM_REC_AUTO, LSTM_REC_STEP, LSTM_REC_PERSISTENT, LSTM_REC_GEMM = 0, 1, 2, 3
LSTM_OPT_RECURRENCE, LSTM_OPT_REC_TILE, LSTM_OPT_TIMING = 1, 2, 3
LSTM_OPT_PARTIAL_BUFFERS, LSTM_OPT_POLL_SLEEP, LSTM_OPT_TEAM_ROWS = 4, 5, 7
LSTM_OPT_PROJ_TILE = 8
LSTM_OPT_READ_PACE = 9
LSTM_OPT_LAYER_PIPE = 10
LSTM_OPT_FUSE_INPUT = 11
LSTM_OPT_BATCH_FIRST = 12
LSTM_OPT_SMALL_BATCH = 13
LSTM_OPT_RESIDENT = 14
STATUS = {0: "LSTM_OK", -1: "LSTM_ERR_ARG", -2: "LSTM_ERR_SHAPE", -3: "LSTM_ERR_DTYPE",
          -4: "LSTM_ERR_DEVICE", -5: "LSTM_ERR_WORKSPACE", -6: "LSTM_ERR_LAUNCH",
          -7: "LSTM_ERR_UNSUPPORTED", -8: "LSTM_ERR_DEVICE_TIMEOUT"}

_lib = None


class lstm_timing(ctypes.Structure):
    _fields_ = [("proj_ms", ctypes.c_double), ("rec_ms", ctypes.c_double), ("calls", ctypes.c_int),
                ("proj_launches", ctypes.c_int), ("rec_launches", ctypes.c_int),
                ("bwd_rec_ms", ctypes.c_double), ("bwd_gemm_ms", ctypes.c_double), ("bwd_calls", ctypes.c_int),
                ("bwd_rec_launches", ctypes.c_int), ("bwd_gemm_launches", ctypes.c_int)]


class LSTMError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({lstm_strerror(status)})")


def load_library():
    """Load liblstm_amd.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing; build it with __graft_entry__.build() "
                          "or python -m layer_lstm_forward_amd.build")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.lstm_create.restype = i
    lib.lstm_create.argtypes = [ctypes.POINTER(vp), i, i, i, i, i, i]
    lib.lstm_create_mode.restype = i
    lib.lstm_create_mode.argtypes = [ctypes.POINTER(vp), i, i, i, i, i, i, i]
    lib.lstm_destroy.restype = None
    lib.lstm_destroy.argtypes = [vp]
    lib.lstm_set_option.restype = i
    lib.lstm_set_option.argtypes = [vp, i, i]
    lib.lstm_set_dropout.restype = i
    lib.lstm_set_dropout.argtypes = [vp, ctypes.c_double, ctypes.c_ulonglong, ctypes.c_ulonglong]
    lib.lstm_workspace_size.restype = i
    lib.lstm_workspace_size.argtypes = [vp, i, i, ctypes.POINTER(sz)]
    lib.lstm_forward.restype = i
    lib.lstm_forward.argtypes = [vp, vp, vp, vp, ctypes.POINTER(vp), i, i, i, i, vp, vp, vp, vp, sz, vp]
    lib.lstm_forward_static.restype = i
    lib.lstm_forward_static.argtypes = [vp, vp, vp, vp, ctypes.POINTER(vp), i, i, i, i, vp, vp, vp, vp, vp]
    lib.lstm_forward_lengths.restype = i
    lib.lstm_forward_lengths.argtypes = [vp, vp, ctypes.POINTER(ctypes.c_int), vp, vp, ctypes.POINTER(vp),
                                         i, i, i, i, vp, vp, vp, vp, sz, vp]
    lib.lstm_packed_workspace_size.restype = i
    lib.lstm_packed_workspace_size.argtypes = [vp, ctypes.POINTER(ctypes.c_int), i, ctypes.POINTER(ctypes.c_size_t)]
    lib.lstm_forward_packed.restype = i
    lib.lstm_forward_packed.argtypes = [vp, vp, ctypes.POINTER(ctypes.c_int), i, vp, vp, ctypes.POINTER(vp), i, i,
                                        vp, vp, vp, vp, sz, vp]
    for fn in ("lstm_reserve_size", "lstm_backward_workspace_size"):
        getattr(lib, fn).restype = i
        getattr(lib, fn).argtypes = [vp, i, i, ctypes.POINTER(sz)]
    lib.lstm_forward_train.restype = i
    lib.lstm_forward_train.argtypes = [vp, vp, vp, vp, ctypes.POINTER(vp), i, i, i, i, vp, vp, vp, vp, sz, vp, sz,
                                       vp]
    lib.lstm_backward.restype = i
    lib.lstm_backward.argtypes = [vp, vp, vp, vp, ctypes.POINTER(vp), vp, vp, vp, vp, vp, sz, i, i, i, i, vp, vp,
                                  vp, ctypes.POINTER(vp), vp, sz, vp]
    ip = ctypes.POINTER(ctypes.c_int)
    lib.lstm_forward_train_lengths.restype = i
    lib.lstm_forward_train_lengths.argtypes = [vp, vp, ip, vp, vp, ctypes.POINTER(vp), i, i, i, i, vp, vp, vp, vp,
                                               sz, vp, sz, vp]
    lib.lstm_backward_lengths.restype = i
    lib.lstm_backward_lengths.argtypes = [vp, vp, ip, vp, vp, ctypes.POINTER(vp), vp, vp, vp, vp, vp, sz, i, i, i,
                                          i, vp, vp, vp, ctypes.POINTER(vp), vp, sz, vp]
    lib.lstm_device_status.restype = i
    lib.lstm_device_status.argtypes = [vp, sz, vp, ctypes.POINTER(ctypes.c_uint)]
    lib.lstm_describe.restype = i
    lib.lstm_describe.argtypes = [vp, i, i, ctypes.c_char_p, sz]
    lib.lstm_read_timing.restype = i
    lib.lstm_read_timing.argtypes = [vp, ctypes.POINTER(lstm_timing), i]
    lib.lstm_strerror.restype = ctypes.c_char_p
    lib.lstm_strerror.argtypes = [i]
    lib.lstm_version.restype = i
    lib.lstm_version.argtypes = []
    _lib = lib
    return lib


# ------------------------------------------------------------- C-ABI mirror
def lstm_strerror(status: int) -> str:
    return load_library().lstm_strerror(int(status)).decode()


def lstm_version() -> int:
    return int(load_library().lstm_version())


def lstm_create(input_size, hidden_size, num_layers, bidirectional, has_bias, dtype):
    """Returns an opaque plan handle (int)."""
    h = ctypes.c_void_p()
    rc = load_library().lstm_create(ctypes.byref(h), int(input_size), int(hidden_size), int(num_layers),
                                    int(bool(bidirectional)), int(bool(has_bias)), int(dtype))
    if rc:
        raise LSTMError(rc, "lstm_create")
    return h.value


LSTM_MODE_LSTM, LSTM_MODE_GRU, LSTM_MODE_RNN_TANH, LSTM_MODE_RNN_RELU = 0, 1, 2, 3
MODES = {"lstm": LSTM_MODE_LSTM, "gru": LSTM_MODE_GRU, "rnn_tanh": LSTM_MODE_RNN_TANH, "rnn_relu": LSTM_MODE_RNN_RELU}


def lstm_create_mode(mode, input_size, hidden_size, num_layers, bidirectional, has_bias, dtype):
    """lstm_create for a recurrent mode (LSTM_MODE_*); returns the plan handle."""
    h = ctypes.c_void_p()
    rc = load_library().lstm_create_mode(ctypes.byref(h), int(mode), int(input_size), int(hidden_size),
                                         int(num_layers), int(bool(bidirectional)), int(bool(has_bias)), int(dtype))
    if rc:
        raise LSTMError(rc, "lstm_create_mode")
    return h.value


def lstm_destroy(plan) -> None:
    if plan:
        load_library().lstm_destroy(ctypes.c_void_p(plan))


def lstm_set_option(plan, option: int, value: int) -> None:
    rc = load_library().lstm_set_option(ctypes.c_void_p(plan), int(option), int(value))
    if rc:
        raise LSTMError(rc, "lstm_set_option")


def lstm_set_dropout(plan, prob: float, seed: int = 0, call: int = 0) -> None:
    rc = load_library().lstm_set_dropout(ctypes.c_void_p(plan), float(prob), int(seed), int(call))
    if rc:
        raise LSTMError(rc, "lstm_set_dropout")


def lstm_workspace_size(plan, T: int, B: int) -> int:
    n = ctypes.c_size_t()
    rc = load_library().lstm_workspace_size(ctypes.c_void_p(plan), int(T), int(B), ctypes.byref(n))
    if rc:
        raise LSTMError(rc, "lstm_workspace_size")
    return int(n.value)


def lstm_forward(plan, x, h0, c0, weights, T, B, layers, bidir, y, h_n, c_n, workspace,
                 workspace_bytes, stream) -> int:
    """Raw call with integer device addresses (0 = NULL); returns the status."""
    arr = (ctypes.c_void_p * len(weights))(*[int(w) for w in weights])
    return int(load_library().lstm_forward(
        ctypes.c_void_p(plan), ctypes.c_void_p(x), ctypes.c_void_p(h0 or None), ctypes.c_void_p(c0 or None),
        arr, int(T), int(B), int(layers), int(bool(bidir)), ctypes.c_void_p(y),
        ctypes.c_void_p(h_n or None), ctypes.c_void_p(c_n or None), ctypes.c_void_p(workspace),
        int(workspace_bytes), ctypes.c_void_p(stream or None)))


LSTM_STATIC_WORKSPACE_BYTES = 96 << 20


def lstm_forward_static(plan, x, h0, c0, weights, T, B, layers, bidir, y, h_n, c_n, device_status, stream) -> int:
    """Raw call of the forward on the library's own workspace (integer device
    addresses, 0 = NULL; device_status: device address of one unsigned, or 0);
    returns the status."""
    arr = (ctypes.c_void_p * len(weights))(*[int(w) for w in weights])
    return int(load_library().lstm_forward_static(
        ctypes.c_void_p(plan), ctypes.c_void_p(x), ctypes.c_void_p(h0 or None), ctypes.c_void_p(c0 or None),
        arr, int(T), int(B), int(layers), int(bool(bidir)), ctypes.c_void_p(y),
        ctypes.c_void_p(h_n or None), ctypes.c_void_p(c_n or None), ctypes.c_void_p(device_status or None),
        ctypes.c_void_p(stream or None)))


def lstm_forward_lengths(plan, x, lengths, h0, c0, weights, T, B, layers, bidir, y, h_n, c_n, workspace,
                         workspace_bytes, stream) -> int:
    """Raw call with per-row lengths (a host sequence of B ints); returns the status."""
    arr = (ctypes.c_void_p * len(weights))(*[int(w) for w in weights])
    lens = None if lengths is None else (ctypes.c_int * len(lengths))(*[int(v) for v in lengths])
    return int(load_library().lstm_forward_lengths(
        ctypes.c_void_p(plan), ctypes.c_void_p(x), lens, ctypes.c_void_p(h0 or None), ctypes.c_void_p(c0 or None),
        arr, int(T), int(B), int(layers), int(bool(bidir)), ctypes.c_void_p(y),
        ctypes.c_void_p(h_n or None), ctypes.c_void_p(c_n or None), ctypes.c_void_p(workspace),
        int(workspace_bytes), ctypes.c_void_p(stream or None)))


def _int_array(values):
    return None if values is None else (ctypes.c_int * len(values))(*[int(v) for v in values])


def lstm_packed_workspace_size(plan, batch_sizes) -> int:
    """Workspace bytes of lstm_forward_packed for these batch_sizes (host ints)."""
    n = ctypes.c_size_t()
    rc = load_library().lstm_packed_workspace_size(ctypes.c_void_p(plan), _int_array(batch_sizes),
                                                   len(batch_sizes) if batch_sizes is not None else 0,
                                                   ctypes.byref(n))
    if rc:
        raise LSTMError(rc, "lstm_packed_workspace_size")
    return int(n.value)


def lstm_forward_packed(plan, x, batch_sizes, h0, c0, weights, layers, bidir, y, h_n, c_n, workspace,
                        workspace_bytes, stream, T=None) -> int:
    """Raw call on packed rows (batch_sizes: a host sequence of T ints); returns the status."""
    arr = (ctypes.c_void_p * len(weights))(*[int(w) for w in weights])
    T = len(batch_sizes) if T is None else T
    return int(load_library().lstm_forward_packed(
        ctypes.c_void_p(plan), ctypes.c_void_p(x), _int_array(batch_sizes), int(T), ctypes.c_void_p(h0 or None),
        ctypes.c_void_p(c0 or None), arr, int(layers), int(bool(bidir)), ctypes.c_void_p(y),
        ctypes.c_void_p(h_n or None), ctypes.c_void_p(c_n or None), ctypes.c_void_p(workspace),
        int(workspace_bytes), ctypes.c_void_p(stream or None)))


def _size_query(fn, plan, T, B) -> int:
    n = ctypes.c_size_t()
    rc = getattr(load_library(), fn)(ctypes.c_void_p(plan), int(T), int(B), ctypes.byref(n))
    if rc:
        raise LSTMError(rc, fn)
    return int(n.value)


def lstm_reserve_size(plan, T: int, B: int) -> int:
    return _size_query("lstm_reserve_size", plan, T, B)


def lstm_backward_workspace_size(plan, T: int, B: int) -> int:
    return _size_query("lstm_backward_workspace_size", plan, T, B)


def _ptrs(addrs):
    return (ctypes.c_void_p * len(addrs))(*[int(a) for a in addrs])


def _lens(lengths):
    return None if lengths is None else (ctypes.c_int * len(lengths))(*[int(v) for v in lengths])


def lstm_forward_train(plan, x, h0, c0, weights, T, B, layers, bidir, y, h_n, c_n, reserve, reserve_bytes,
                       workspace, workspace_bytes, stream, lengths=None) -> int:
    """lengths: None, or B host ints (lstm_forward_train_lengths)."""
    v = ctypes.c_void_p
    lib = load_library()
    common = (v(h0 or None), v(c0 or None), _ptrs(weights), int(T), int(B), int(layers), int(bool(bidir)), v(y),
              v(h_n or None), v(c_n or None), v(reserve), int(reserve_bytes), v(workspace), int(workspace_bytes),
              v(stream or None))
    if lengths is None:
        return int(lib.lstm_forward_train(v(plan), v(x), *common))
    return int(lib.lstm_forward_train_lengths(v(plan), v(x), _lens(lengths), *common))


def lstm_backward(plan, x, h0, c0, weights, y, dy, dh_n, dc_n, reserve, reserve_bytes, T, B, layers, bidir, dx,
                  dh0, dc0, dweights, workspace, workspace_bytes, stream, lengths=None) -> int:
    """lengths: None, or B host ints (lstm_backward_lengths)."""
    v = ctypes.c_void_p
    lib = load_library()
    common = (v(h0 or None), v(c0 or None), _ptrs(weights), v(y), v(dy), v(dh_n or None), v(dc_n or None),
              v(reserve), int(reserve_bytes), int(T), int(B), int(layers), int(bool(bidir)), v(dx or None),
              v(dh0 or None), v(dc0 or None), _ptrs(dweights), v(workspace), int(workspace_bytes), v(stream or None))
    if lengths is None:
        return int(lib.lstm_backward(v(plan), v(x), *common))
    return int(lib.lstm_backward_lengths(v(plan), v(x), _lens(lengths), *common))


def lstm_device_status(workspace, workspace_bytes, stream):
    """Returns (status, flags) after synchronising the stream."""
    flags = ctypes.c_uint()
    rc = load_library().lstm_device_status(ctypes.c_void_p(workspace), int(workspace_bytes),
                                           ctypes.c_void_p(stream or None), ctypes.byref(flags))
    return int(rc), int(flags.value)


def lstm_read_timing(plan, reset: bool = True) -> dict:
    t = lstm_timing()
    rc = load_library().lstm_read_timing(ctypes.c_void_p(plan), ctypes.byref(t), int(bool(reset)))
    if rc:
        raise LSTMError(rc, "lstm_read_timing")
    return {f: getattr(t, f) for f, _ in lstm_timing._fields_}


def lstm_describe(plan, T: int, B: int) -> str:
    buf = ctypes.create_string_buffer(512)
    rc = load_library().lstm_describe(ctypes.c_void_p(plan), int(T), int(B), buf, 512)
    if rc:
        raise LSTMError(rc, "lstm_describe")
    return buf.value.decode()


# ------------------------------------------------------------ torch wrapper
class LSTM:
    """A plan plus a cached workspace, taking and returning torch tensors.

    weights: flat list in (layer, direction, W_ih, W_hh[, b_ih, b_hh]) order,
    contiguous device tensors of the plan's dtype.
    """

    def __init__(self, input_size, hidden_size, num_layers=1, bidirectional=False, bias=True,
                 dtype="f32", recurrence=LSTM_REC_AUTO, rec_tile=0, options=None, batch_first=False, dropout=0.0,
                 dropout_seed=0, mode="lstm"):
        self.input_size, self.hidden_size = int(input_size), int(hidden_size)
        self.num_layers, self.bidirectional, self.bias = int(num_layers), bool(bidirectional), bool(bias)
        self.dtype = dtype
        self.batch_first = bool(batch_first)
        self.D = 2 if self.bidirectional else 1
        self.mode = mode
        self.plan = lstm_create_mode(MODES[mode], input_size, hidden_size, num_layers, bidirectional, bias,
                                     LSTM_BF16 if dtype == "bf16" else LSTM_F32)
        if recurrence != LSTM_REC_AUTO:
            lstm_set_option(self.plan, LSTM_OPT_RECURRENCE, recurrence)
        if rec_tile:
            lstm_set_option(self.plan, LSTM_OPT_REC_TILE, rec_tile)
        if self.batch_first:
            lstm_set_option(self.plan, LSTM_OPT_BATCH_FIRST, 1)
        for opt, val in (options or {}).items():
            lstm_set_option(self.plan, opt, val)
        if dropout:
            lstm_set_dropout(self.plan, dropout, dropout_seed, 0)
        self._ws = None

    def set_dropout(self, prob, seed=0, call=0):
        """Training dropout between layers; `call` is the draw index of the
        next forward_train (each one advances it)."""
        lstm_set_dropout(self.plan, prob, seed, call)

    def __del__(self, _finalizing=sys.is_finalizing):
        # at interpreter shutdown the plan's host memory goes with the process;
        # no runtime call is made from a finaliser then
        if _finalizing():
            return
        try:
            lstm_destroy(self.plan)
        except Exception:
            pass

    def describe(self, T, B) -> str:
        return lstm_describe(self.plan, T, B)

    def workspace(self, T, B, device):
        import torch
        n = lstm_workspace_size(self.plan, T, B)
        if self._ws is None or self._ws.numel() < n or self._ws.device != device:
            self._ws = torch.empty(n, dtype=torch.uint8, device=device)
        return self._ws, n

    def forward(self, x, weights, h0=None, c0=None, stream=None, out=None, lengths=None):
        """lengths: None, or B ints in 1..T (per-row sequence lengths, host side)."""
        import torch
        tdt = torch.bfloat16 if self.dtype == "bf16" else torch.float32
        if not x.is_cuda or x.dtype != tdt or not x.is_contiguous() or x.dim() != 3:
            raise ValueError("x must be a contiguous [T, B, input_size] ([B, T, input_size] with batch_first) "
                             "device tensor of the plan's dtype")
        for w in weights:
            if not w.is_cuda or w.dtype != tdt or not w.is_contiguous():
                raise ValueError("weights must be contiguous device tensors of the plan's dtype")
        T, B, _ = x.shape
        if self.batch_first:
            B, T = T, B
        H, L, D = self.hidden_size, self.num_layers, self.D
        if out is None:
            y = torch.empty(*((B, T) if self.batch_first else (T, B)), D * H, dtype=tdt, device=x.device)
            hn = torch.empty(L * D, B, H, dtype=tdt, device=x.device)
            # the GRU and the RNNs have no cell state
            cn = torch.empty(L * D, B, H, dtype=torch.float32, device=x.device) if self.mode == "lstm" else None
        else:
            y, hn, cn = out
        ws, nbytes = self.workspace(T, B, x.device)
        if stream is None:
            stream = torch.cuda.current_stream(x.device).cuda_stream
        args = (h0.data_ptr() if h0 is not None else 0, c0.data_ptr() if c0 is not None else 0,
                [w.data_ptr() for w in weights], T, B, L, self.bidirectional, y.data_ptr(),
                hn.data_ptr() if hn is not None else 0, cn.data_ptr() if cn is not None else 0,
                ws.data_ptr(), nbytes, stream)
        if lengths is None:
            rc = lstm_forward(self.plan, x.data_ptr(), *args)
        else:
            rc = lstm_forward_lengths(self.plan, x.data_ptr(), [int(v) for v in lengths], *args)
        if rc:
            raise LSTMError(rc, "lstm_forward_lengths" if lengths is not None else "lstm_forward")
        return y, hn, cn

    def forward_packed(self, x, batch_sizes, weights, h0=None, c0=None, stream=None):
        """Packed sequences: x [N, input_size] with the rows of step t after those of
        the earlier steps, batch_sizes the T host ints (non-increasing).  Returns
        (y [N, D*H], h_n, c_n) with h_n, c_n rows in the packed sequence order."""
        import torch
        tdt = torch.bfloat16 if self.dtype == "bf16" else torch.float32
        if not x.is_cuda or x.dtype != tdt or not x.is_contiguous() or x.dim() != 2:
            raise ValueError("x must be a contiguous [N, input_size] device tensor of the plan's dtype")
        bs = [int(v) for v in batch_sizes]
        B, H, L, D = bs[0], self.hidden_size, self.num_layers, self.D
        y = torch.empty(x.shape[0], D * H, dtype=tdt, device=x.device)
        hn = torch.empty(L * D, B, H, dtype=tdt, device=x.device)
        cn = torch.empty(L * D, B, H, dtype=torch.float32, device=x.device) if self.mode == "lstm" else None
        nbytes = lstm_packed_workspace_size(self.plan, bs)
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
        if stream is None:
            stream = torch.cuda.current_stream(x.device).cuda_stream
        rc = lstm_forward_packed(self.plan, x.data_ptr(), bs, h0.data_ptr() if h0 is not None else 0,
                                 c0.data_ptr() if c0 is not None else 0, [w.data_ptr() for w in weights], L,
                                 self.bidirectional, y.data_ptr(), hn.data_ptr(),
                                 cn.data_ptr() if cn is not None else 0, ws.data_ptr(), nbytes, stream)
        if rc:
            raise LSTMError(rc, "lstm_forward_packed")
        self._pws = ws  # kept until the next call: the stream may still be using it
        return y, hn, cn

    def forward_train(self, x, weights, h0=None, c0=None, stream=None, lengths=None):
        """Forward that also keeps the reserve for backward(); returns
        (y, h_n, c_n, reserve).  lengths: None or B per-row lengths (host ints)."""
        import torch
        T, B, _ = x.shape
        if self.batch_first:
            B, T = T, B
        H, L, D = self.hidden_size, self.num_layers, self.D
        tdt = x.dtype
        y = torch.empty(*((B, T) if self.batch_first else (T, B)), D * H, dtype=tdt, device=x.device)
        hn = torch.empty(L * D, B, H, dtype=tdt, device=x.device)
        cn = torch.empty(L * D, B, H, dtype=torch.float32, device=x.device)
        rbytes = lstm_reserve_size(self.plan, T, B)
        reserve = torch.empty(max(rbytes, 1), dtype=torch.uint8, device=x.device)
        ws, nbytes = self.workspace(T, B, x.device)
        if stream is None:
            stream = torch.cuda.current_stream(x.device).cuda_stream
        rc = lstm_forward_train(self.plan, x.data_ptr(), h0.data_ptr() if h0 is not None else 0,
                                c0.data_ptr() if c0 is not None else 0, [w.data_ptr() for w in weights], T, B, L,
                                self.bidirectional, y.data_ptr(), hn.data_ptr(), cn.data_ptr(), reserve.data_ptr(),
                                rbytes, ws.data_ptr(), nbytes, stream, lengths=lengths)
        if rc:
            raise LSTMError(rc, "lstm_forward_train")
        return y, hn, cn, reserve

    def backward(self, x, weights, y, reserve, dy, h0=None, c0=None, dh_n=None, dc_n=None, stream=None,
                 lengths=None):
        """Gradients (dx, dh0, dc0, dweights) of a forward_train() call (with the same lengths)."""
        import torch
        T, B, _ = x.shape
        if self.batch_first:
            B, T = T, B
        H, L, D = self.hidden_size, self.num_layers, self.D
        dx = torch.empty_like(x)
        dh0 = torch.empty(L * D, B, H, dtype=x.dtype, device=x.device)
        dc0 = torch.empty(L * D, B, H, dtype=torch.float32, device=x.device)
        dws = [torch.empty_like(w) for w in weights]
        nbytes = lstm_backward_workspace_size(self.plan, T, B)
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
        if stream is None:
            stream = torch.cuda.current_stream(x.device).cuda_stream
        addr = lambda t: t.data_ptr() if t is not None else 0  # noqa: E731
        rc = lstm_backward(self.plan, x.data_ptr(), addr(h0), addr(c0), [w.data_ptr() for w in weights],
                           y.data_ptr(), dy.data_ptr(), addr(dh_n), addr(dc_n), reserve.data_ptr(), reserve.numel(),
                           T, B, L, self.bidirectional, dx.data_ptr(), dh0.data_ptr(), dc0.data_ptr(),
                           [w.data_ptr() for w in dws], ws.data_ptr(), nbytes, stream, lengths=lengths)
        if rc:
            raise LSTMError(rc, "lstm_backward")
        self._bws = ws
        return dx, dh0, dc0, dws

    def backward_status(self, stream=None):
        """lstm_device_status on the last backward call's workspace (a K-split step's wait gave up: flag 2)."""
        import torch
        if getattr(self, "_bws", None) is None:
            return 0, 0
        if stream is None:
            stream = torch.cuda.current_stream(self._bws.device).cuda_stream
        return lstm_device_status(self._bws.data_ptr(), self._bws.numel(), stream)

    def device_status(self, stream=None):
        import torch
        if self._ws is None:
            return 0, 0
        if stream is None:
            stream = torch.cuda.current_stream(self._ws.device).cuda_stream
        return lstm_device_status(self._ws.data_ptr(), self._ws.numel(), stream)

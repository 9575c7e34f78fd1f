"""Seeded synthetic inputs for the LSTM forward (no LSTM arithmetic here).

Both the HIP path and the fp64 oracle consume the bytes this module writes, so
it holds only random draws and the one-time fp32 -> bf16 rounding of inputs.

Recipe (the same for every workload):
  * ``numpy.random.default_rng(seed)`` (PCG64);
  * draw order: parameters layer by layer, direction by direction, each as
    W_ih, W_hh, b_ih, b_hh; then x; then h0; then c0;
  * parameters ~ U(-k, k) with k = 1/sqrt(hidden_size), the initialisation the
    warp-nn "Long Short-Term Memory (LSTM)" page states under its parameter
    table (biases included);
  * x ~ N(0, 1) drawn as float32;
  * h0, c0 either absent (zeros) or ~ N(0, 0.1) (standard deviation 0.1);
    c0 is drawn for every mode (the GRU and the RNNs do not read it);
  * the gate blocks per parameter are 4 (LSTM), 3 (GRU) or 1 (RNN);
  * bf16 workloads draw in fp32 and round to nearest-even bf16 once, here;
    the cell state c0 stays fp32.
  * per-row sequence lengths (variable-length batches), from their own
    generator ``default_rng(seed + 7919)`` so that the other draws do not
    change: ``ragged`` is uniform on 1..T, ``mix`` has a quarter of the rows
    at T and the rest uniform on T/2..T (a padded bucket whose longest row
    sets T), ``full`` is T for every row.  The pages give no length mix.
"""
from __future__ import annotations

import dataclasses

import numpy as np


@dataclasses.dataclass(frozen=True)
class Spec:
    input_size: int
    hidden_size: int
    num_layers: int
    bidirectional: bool
    T: int
    B: int
    dtype: str = "f32"          # "f32" or "bf16" (x, weights, biases, h0, y, h_n)
    seed: int = 0
    state: str = "zeros"        # "zeros" (h0 = c0 = None) or "normal0.1"
    has_bias: bool = True
    mode: str = "lstm"          # "lstm", "gru", "rnn_tanh" or "rnn_relu"

    @property
    def gates(self) -> int:
        """Gate blocks of H rows in W_ih, W_hh and the biases."""
        return {"lstm": 4, "gru": 3, "rnn_tanh": 1, "rnn_relu": 1}[self.mode]

    @property
    def D(self) -> int:
        return 2 if self.bidirectional else 1

    @property
    def cells(self) -> int:
        """Timestep-cells B*T*H*L*D, the unit of the throughput metric."""
        return self.B * self.T * self.hidden_size * self.num_layers * self.D

    def layer_input(self, l: int) -> int:
        return self.input_size if l == 0 else self.D * self.hidden_size

    def flops(self) -> int:
        """Multiply-add FLOPs of the two products, 2*gates*(in_l + H) per cell per layer."""
        H = self.hidden_size
        return sum(2 * self.gates * (self.layer_input(l) + H) * self.B * self.T * H * self.D
                   for l in range(self.num_layers))


# The benchmark workloads, named by what they are.
WORKLOADS = {
    "l1_in8_h16_t5_b1_f32": Spec(8, 16, 1, False, 5, 1, "f32", 1001),
    "l2_in256_h512_t128_b64_f32": Spec(256, 512, 2, False, 128, 64, "f32", 1002, "normal0.1"),
    "l2bi_in512_h1024_t256_b32_bf16": Spec(512, 1024, 2, True, 256, 32, "bf16", 1003),
    "l1_in1024_h1024_t1024_b1_bf16": Spec(1024, 1024, 1, False, 1024, 1, "bf16", 1004),
    "l1_in1024_h1024_t1024_b4_bf16": Spec(1024, 1024, 1, False, 1024, 4, "bf16", 1005),
    "l4_in2048_h2048_t512_b256_bf16": Spec(2048, 2048, 4, False, 512, 256, "bf16", 1006),
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to the nearest bfloat16 (ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(a: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Inputs:
    spec: Spec
    x: np.ndarray               # [T, B, I]   float32, or uint16 bf16 bits
    params: list                # flat (layer, direction, W_ih, W_hh[, b_ih, b_hh])
    h0: np.ndarray | None       # [L*D, B, H] like x, or None
    c0: np.ndarray | None       # [L*D, B, H] float32, or None

    @property
    def bf16(self) -> bool:
        return self.spec.dtype == "bf16"

    def rows(self, idx) -> "Inputs":
        """The same problem restricted to a subset of batch rows."""
        idx = np.asarray(idx)
        spec = dataclasses.replace(self.spec, B=len(idx))
        return Inputs(spec, np.ascontiguousarray(self.x[:, idx]), self.params,
                      None if self.h0 is None else np.ascontiguousarray(self.h0[:, idx]),
                      None if self.c0 is None else np.ascontiguousarray(self.c0[:, idx]))


def make_inputs(spec: Spec) -> Inputs:
    rng = np.random.default_rng(spec.seed)
    H, D, L = spec.hidden_size, spec.D, spec.num_layers
    k = 1.0 / np.sqrt(H)
    cast = f32_to_bf16_bits if spec.dtype == "bf16" else (lambda a: a)
    params = []
    G = spec.gates * H
    for l in range(L):
        for _d in range(D):
            shapes = [(G, spec.layer_input(l)), (G, H)]
            if spec.has_bias:
                shapes += [(G,), (G,)]
            for shp in shapes:
                params.append(cast(rng.uniform(-k, k, size=shp).astype(np.float32)))
    x = cast(rng.standard_normal(size=(spec.T, spec.B, spec.input_size), dtype=np.float32))
    h0 = c0 = None
    if spec.state == "normal0.1":
        st = (L * D, spec.B, H)
        h0 = cast(rng.normal(0.0, 0.1, size=st).astype(np.float32))
        c0 = rng.normal(0.0, 0.1, size=st).astype(np.float32)
    elif spec.state != "zeros":
        raise ValueError(f"unknown state recipe {spec.state!r}")
    return Inputs(spec, x, params, h0, c0)


def make_lengths(spec: Spec, mode: str = "mix") -> np.ndarray:
    """Seeded per-row lengths in 1..T (int32, one per batch row)."""
    T, B = spec.T, spec.B
    rng = np.random.default_rng(spec.seed + 7919)
    if mode == "full":
        return np.full(B, T, np.int32)
    if mode == "ragged":
        return rng.integers(1, T + 1, size=B).astype(np.int32)
    if mode == "mix":
        n = rng.integers(max(1, T // 2), T + 1, size=B)
        n[rng.permutation(B)[:max(1, B // 4)]] = T
        return n.astype(np.int32)
    raise ValueError(f"unknown length mode {mode!r}")

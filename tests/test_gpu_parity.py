"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Tolerances (max-abs over y, h_n, c_n): 1e-4 for fp32 weights, 2e-2 for bf16
weights with an fp32 cell.  Small shapes span several tiles with ragged tails
and are checked element by element; the benchmark workloads run at full size
in the schedule the benchmark times, and the oracle recomputes a sample of
batch rows (rows are independent, so a row subset run alone is exact).
"""
import numpy as np
import pytest

import layer_lstm_forward_amd as pkg
from layer_lstm_forward_amd.synth import WORKLOADS, Spec, make_inputs
from tests.gpu_util import assert_parity, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

SMALL = [
    Spec(37, 52, 2, True, 9, 19, "f32", 101, "normal0.1"),    # ragged H, I, two batch groups
    Spec(13, 13, 1, False, 7, 3, "f32", 102, "normal0.1"),    # H % 4 != 0: element-wise loads
    Spec(70, 40, 3, False, 6, 33, "bf16", 103, "normal0.1"),  # three layers, partial K chunk
    Spec(64, 96, 2, True, 11, 5, "bf16", 104, "zeros"),
    Spec(5, 7, 1, True, 4, 2, "f32", 105, "zeros", has_bias=False),
    Spec(200, 264, 1, False, 12, 40, "f32", 106),
    Spec(256, 200, 2, True, 8, 70, "bf16", 107, "normal0.1"),
    Spec(1, 1, 1, False, 1, 1, "f32", 108, "normal0.1"),      # degenerate: one unit, one step
]
TILES = [411, 412, 414, 211, 212, 214, 111, 112, 114, 141, 142]


def _id(s):
    return f"{s.dtype}-I{s.input_size}-H{s.hidden_size}-L{s.num_layers}-D{s.D}-T{s.T}-B{s.B}"


@pytest.mark.parametrize("spec", SMALL, ids=_id)
@pytest.mark.parametrize("mode", [pkg.LSTM_REC_STEP, pkg.LSTM_REC_AUTO], ids=["step", "auto"])
def test_small_shapes(spec, mode):
    print(f"case {_id(spec)} mode {mode}", flush=True)
    inp = make_inputs(spec)
    got, m = run_gpu(inp, recurrence=mode)
    ref = run_oracle(inp)
    assert_parity(got, ref, spec.dtype, m.describe(spec.T, spec.B))


def _gemm_step_shape_ok(spec):
    return (spec.hidden_size * (2 if spec.dtype == "bf16" else 4)) % 16 == 0


@pytest.mark.parametrize("spec", SMALL, ids=_id)
def test_small_shapes_gemm_step(spec):
    """The per-step GEMM recurrence (k_rec_step) on the small shapes; shapes
    whose rows are not 16-byte multiples are refused with LSTM_ERR_UNSUPPORTED."""
    print(f"case {_id(spec)} gemm step", flush=True)
    inp = make_inputs(spec)
    if not _gemm_step_shape_ok(spec):
        with pytest.raises(pkg.LSTMError) as e:
            run_gpu(inp, recurrence=pkg.LSTM_REC_GEMM)
        assert e.value.status == -7
        return
    got, m = run_gpu(inp, recurrence=pkg.LSTM_REC_GEMM)
    assert "gemm-step" in m.describe(spec.T, spec.B)
    assert_parity(got, run_oracle(inp), spec.dtype, "gemm step")


@pytest.mark.parametrize("spec", [
    Spec(32, 256, 2, False, 6, 130, "bf16", 401, "normal0.1"),   # 8 unit blocks (XCD-grouped), 3 row blocks, ragged
    Spec(40, 96, 1, True, 5, 70, "f32", 402, "normal0.1"),       # 3 unit blocks, 2 row blocks, both directions
    Spec(24, 520, 1, False, 4, 64, "f32", 403, "zeros"),         # ragged last unit block, K not a stage multiple
    Spec(16, 64, 3, True, 3, 1, "bf16", 404, "normal0.1"),       # one batch row, three layers
    Spec(48, 160, 2, False, 4, 300, "f32", 405, "normal0.1"),    # 128-row blocks, ragged third
], ids=_id)
def test_gemm_step_blocks(spec):
    """k_rec_step (64- and 128-row blocks) over several row and unit blocks with
    ragged edges, against the oracle and against the automatic schedule."""
    print(f"case {_id(spec)} gemm step blocks", flush=True)
    inp = make_inputs(spec)
    ref = run_oracle(inp)
    got, m = run_gpu(inp, recurrence=pkg.LSTM_REC_GEMM)
    assert_parity(got, ref, spec.dtype, "gemm step")
    pers, _ = run_gpu(inp, recurrence=pkg.LSTM_REC_AUTO)
    assert_parity(pers, ref, spec.dtype, "auto")


@pytest.mark.parametrize("spec", [
    Spec(24, 64, 2, False, 9, 40, "f32", 501, "normal0.1"),     # two layers, two batch groups
    Spec(32, 52, 3, False, 7, 19, "f32", 502, "zeros"),         # three layers, ragged H (partial unit slice)
    Spec(40, 96, 4, False, 5, 70, "bf16", 503, "normal0.1"),    # four layers, ragged batch groups
    Spec(16, 40, 2, False, 6, 3, "bf16", 504, "normal0.1", has_bias=False),
    Spec(8, 16, 2, False, 1, 1, "f32", 505, "normal0.1"),       # one step, one row
    # waves whose exchange fragments are all live (they skip the per-word
    # settling) beside partial waves and a ragged last team, in one launch
    Spec(128, 400, 2, False, 6, 40, "f32", 506, "normal0.1"),
    Spec(64, 1024, 2, False, 4, 20, "bf16", 507, "normal0.1"),
], ids=_id)
def test_layer_wavefront(spec):
    """All layers of a unidirectional stack in one launch, layer l consuming
    layer l-1's h_t as it is produced (k_rec_wave), against the oracle and
    against the layer-by-layer path."""
    print(f"case {_id(spec)} layer wavefront", flush=True)
    inp = make_inputs(spec)
    ref = run_oracle(inp)
    got, m = run_gpu(inp, options={pkg.LSTM_OPT_LAYER_PIPE: 1})
    assert "wavefront" in m.describe(spec.T, spec.B)
    assert_parity(got, ref, spec.dtype, "wavefront")
    seq, m2 = run_gpu(inp, options={pkg.LSTM_OPT_LAYER_PIPE: 0})
    assert "wavefront" not in m2.describe(spec.T, spec.B)
    assert_parity(seq, ref, spec.dtype, "layer by layer")
    # a two-layer stack paired in 512-thread workgroups (lockstep slots, layer
    # 1 two steps behind); deeper stacks keep one workgroup per layer
    paired, m3 = run_gpu(inp, options={pkg.LSTM_OPT_LAYER_PIPE: 2})
    desc = m3.describe(spec.T, spec.B)
    assert "wavefront" in desc and ("layers_per_wg=2" in desc) == (spec.num_layers == 2), desc
    assert_parity(paired, ref, spec.dtype, "paired wavefront")


@pytest.mark.parametrize("spec", [
    Spec(24, 64, 2, False, 9, 40, "f32", 601, "normal0.1"),      # layer 0: one input chunk for four waves
    Spec(256, 128, 2, True, 7, 37, "f32", 602, "normal0.1"),    # both directions, ragged batch groups
    Spec(96, 80, 3, False, 5, 16, "bf16", 603, "normal0.1"),    # partial unit slice, three layers
    Spec(512, 96, 1, True, 4, 20, "bf16", 604, "zeros", has_bias=False),
    Spec(64, 256, 2, False, 3, 1, "f32", 605, "normal0.1"),     # one batch row
], ids=_id)
def test_fused_input_projection(spec):
    """x_t W_ih^T computed inside the persistent recurrence (fused) against
    the oracle and against the hoisted projection GEMM."""
    print(f"case {_id(spec)} fused projection", flush=True)
    inp = make_inputs(spec)
    ref = run_oracle(inp)
    got, m = run_gpu(inp, options={pkg.LSTM_OPT_FUSE_INPUT: 1})
    assert "fused" in m.describe(spec.T, spec.B)
    assert_parity(got, ref, spec.dtype, "fused")
    hoisted, m2 = run_gpu(inp, options={pkg.LSTM_OPT_FUSE_INPUT: 0})
    assert "fused" not in m2.describe(spec.T, spec.B)
    assert_parity(hoisted, ref, spec.dtype, "hoisted")


@pytest.mark.parametrize("spec", [
    Spec(64, 1024, 1, False, 9, 1, "bf16", 651, "zeros"),        # the latency-bound workload's shape, short
    Spec(64, 1024, 1, True, 7, 4, "bf16", 652, "normal0.1"),     # both directions: one XCD each
    Spec(40, 40, 2, False, 6, 16, "bf16", 653, "normal0.1"),     # partial unit slice, a full 16-row tile
    Spec(24, 512, 2, True, 5, 3, "f32", 654, "normal0.1"),       # fp32 at its widest K
    Spec(8, 16, 1, False, 5, 1, "f32", 655, "zeros"),            # one workgroup per direction
], ids=_id)
def test_small_batch_one_xcd(spec):
    """Batches of at most 16 rows: each direction's recurrence on the 32 CUs of
    one XCD (k_rec_xcd), against the oracle and against the general path."""
    print(f"case {_id(spec)} small batch", flush=True)
    inp = make_inputs(spec)
    ref = run_oracle(inp)
    lbl = {pkg.LSTM_OPT_LAYER_PIPE: 0}  # a unidirectional stack would otherwise take the layer wavefront
    got, m = run_gpu(inp, options=lbl)
    assert "small-batch" in m.describe(spec.T, spec.B)
    assert_parity(got, ref, spec.dtype, "one XCD")
    gen, m2 = run_gpu(inp, options={**lbl, pkg.LSTM_OPT_SMALL_BATCH: 0})
    assert "small-batch" not in m2.describe(spec.T, spec.B)
    assert_parity(gen, ref, spec.dtype, "general")


RESIDENT_SPECS = [
    Spec(40, 256, 2, False, 6, 130, "bf16", 801, "normal0.1"),   # 2 chunks a wave, ragged second row block, two layers
    Spec(64, 512, 1, True, 5, 200, "bf16", 802, "normal0.1"),    # both directions, 4 row groups of 32 slices
    Spec(32, 1024, 1, False, 4, 20, "bf16", 803, "zeros"),       # one partial row block
    Spec(24, 1536, 1, True, 3, 40, "bf16", 805, "normal0.1"),    # 12 chunks a wave, 192 workgroups
    Spec(16, 2048, 1, False, 3, 130, "bf16", 804, "normal0.1"),  # the H = 2048 shape: every CU, 16 chunks a wave
]


@pytest.mark.parametrize("spec", RESIDENT_SPECS, ids=_id)
def test_resident_recurrence(spec):
    """W_hh held once across the chip and h_{t-1} exchanged through a ring
    of step-tagged words (k_rec_res), forced on shapes that would otherwise run another
    recurrence, against the oracle and against the per-step GEMM."""
    print(f"case {_id(spec)} resident", flush=True)
    inp = make_inputs(spec)
    ref = run_oracle(inp)
    opts = {pkg.LSTM_OPT_LAYER_PIPE: 0, pkg.LSTM_OPT_RESIDENT: 2}
    got, m = run_gpu(inp, options=opts)
    assert "resident" in m.describe(spec.T, spec.B)
    assert_parity(got, ref, spec.dtype, "resident")
    gem, m2 = run_gpu(inp, recurrence=pkg.LSTM_REC_GEMM, options={pkg.LSTM_OPT_RESIDENT: 0})
    assert "resident" not in m2.describe(spec.T, spec.B)
    assert_parity(gem, ref, spec.dtype, "gemm step")


def test_resident_large_h0_and_saturation():
    """The resident recurrence from a caller's h0 of magnitude up to ~10 (read
    directly at the first step) and with every gate saturated (|h| = 1
    exactly in y, the words the next step reads)."""
    from layer_lstm_forward_amd.synth import bf16_bits_to_f32
    spec = Spec(32, 256, 1, True, 12, 150, "bf16", 806, "normal0.1")
    opts = {pkg.LSTM_OPT_LAYER_PIPE: 0, pkg.LSTM_OPT_RESIDENT: 2}
    print("case resident large h0", flush=True)
    inp = make_inputs(spec)
    inp.h0 = _scaled(inp.h0, 40.0, True)
    assert np.max(np.abs(bf16_bits_to_f32(inp.h0))) >= 2.0
    got, m = run_gpu(inp, options=opts)
    assert "resident" in m.describe(spec.T, spec.B)
    assert_parity(got, run_oracle(inp), "bf16", "resident, large h0")
    print("case resident saturated", flush=True)
    inp = _saturating(spec)
    got, m = run_gpu(inp, options=opts)
    assert np.mean(np.abs(got[0]) == 1.0) > 0.1, "the case should drive h to +-1 exactly"
    assert_parity(got, run_oracle(inp), "bf16", "resident, saturated")


LENGTH_SPECS = [
    Spec(24, 64, 2, False, 9, 40, "f32", 701, "normal0.1"),      # fused projection
    Spec(37, 52, 2, True, 9, 19, "f32", 702, "normal0.1"),       # ragged H and I, both directions
    Spec(70, 40, 3, False, 6, 33, "bf16", 703, "normal0.1"),     # three layers
    Spec(64, 96, 2, True, 11, 5, "bf16", 704, "zeros"),
]
LENGTH_MODES = {"auto": (pkg.LSTM_REC_AUTO, {}), "hoisted": (pkg.LSTM_REC_AUTO, {pkg.LSTM_OPT_FUSE_INPUT: 0}),
                "step": (pkg.LSTM_REC_STEP, {}), "gemm": (pkg.LSTM_REC_GEMM, {})}


@pytest.mark.parametrize("spec", LENGTH_SPECS, ids=_id)
@pytest.mark.parametrize("mode", sorted(LENGTH_MODES))
def test_variable_lengths(spec, mode):
    """Per-row lengths (lstm_forward_lengths) against the oracle in every
    recurrence mode; padded outputs are exactly zero."""
    from layer_lstm_forward_amd.synth import make_lengths
    print(f"case {_id(spec)} lengths {mode}", flush=True)
    inp = make_inputs(spec)
    lengths = make_lengths(spec, "ragged")
    lengths[0] = spec.T
    lengths[-1] = 1
    rec, opts = LENGTH_MODES[mode]
    if mode == "gemm" and not _gemm_step_shape_ok(spec):
        pytest.skip("rows are not 16-byte multiples: the per-step GEMM refuses this shape")
    got, m = run_gpu(inp, recurrence=rec, options=opts, lengths=lengths)
    ref = run_oracle(inp, lengths=lengths)
    assert_parity(got, ref, spec.dtype, f"lengths {mode}: {m.describe(spec.T, spec.B)}")
    y = got[0]
    for b, n in enumerate(lengths):
        assert np.all(y[n:, b] == 0.0), f"row {b}: padded outputs not zero"


@pytest.mark.parametrize("spec", LENGTH_SPECS, ids=_id)
@pytest.mark.parametrize("mode", sorted(LENGTH_MODES))
@pytest.mark.parametrize("with_lengths", [False, True], ids=["full", "lengths"])
def test_batch_first(spec, mode, with_lengths):
    """x [B, T, I] and y [B, T, D*H] (batch_first) in every recurrence mode,
    with and without per-row lengths, against the oracle on the same data."""
    from layer_lstm_forward_amd.synth import make_lengths
    print(f"case {_id(spec)} batch_first {mode} {with_lengths}", flush=True)
    rec, opts = LENGTH_MODES[mode]
    if mode == "gemm" and not _gemm_step_shape_ok(spec):
        pytest.skip("rows are not 16-byte multiples: the per-step GEMM refuses this shape")
    inp = make_inputs(spec)
    lengths = make_lengths(spec, "ragged") if with_lengths else None
    got, m = run_gpu(inp, recurrence=rec, options=opts, lengths=lengths, batch_first=True)
    assert "batch-first" in m.describe(spec.T, spec.B) or mode == "gemm"
    ref = run_oracle(inp, lengths=lengths)
    assert_parity(got, ref, spec.dtype, f"batch_first {mode}: {m.describe(spec.T, spec.B)}")


def _scaled(a, factor, bf):
    """a * factor in the same storage type (bf16 bits rounded once, like every input)."""
    from layer_lstm_forward_amd.synth import bf16_bits_to_f32, f32_to_bf16_bits
    if a is None:
        return None
    if bf:
        return f32_to_bf16_bits(bf16_bits_to_f32(a) * np.float32(factor))
    return (a * np.float32(factor)).astype(np.float32)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("mode", sorted(LENGTH_MODES))
def test_lengths_large_h0(dtype, mode):
    """Per-row lengths with a caller's h0 of magnitude up to ~10 (N(0, 0.1) x
    40): the reverse scan republishes h0 on its leading padded steps, so
    values of magnitude 2 and more pass between workgroups (bf16: the wide
    exchange words).  Every wait ends and the outputs match the oracle."""
    from layer_lstm_forward_amd.synth import make_lengths
    spec = Spec(40, 64, 2, True, 9, 20, dtype, 710, "normal0.1")
    print(f"case lengths large h0 {dtype} {mode}", flush=True)
    inp = make_inputs(spec)
    bf = dtype == "bf16"
    inp.h0 = _scaled(inp.h0, 40.0, bf)
    lengths = make_lengths(spec, "ragged")
    lengths[0] = 1
    rec, opts = LENGTH_MODES[mode]
    got, m = run_gpu(inp, recurrence=rec, options=opts, lengths=lengths)
    ref = run_oracle(inp, lengths=lengths)
    # the reverse scan of a row shorter than T republishes h0 on its padded
    # steps and multiplies it at its first valid step: h0 reaches the range
    from layer_lstm_forward_amd.synth import bf16_bits_to_f32
    assert np.max(np.abs(bf16_bits_to_f32(inp.h0) if bf else inp.h0)) >= 2.0 and min(lengths) < spec.T
    assert_parity(got, ref, dtype, f"lengths, large h0, {mode}: {m.describe(spec.T, spec.B)}")


def _saturating(spec):
    """Inputs whose every gate sits at a saturated end: b_ih of i and o +30
    (sigma = 1 exactly in fp32), of g +-30 (tanh = +-1), of f +30 or -100
    (sigma = 0 exactly: exp2 overflows to +inf and its reciprocal is 0);
    b_hh = 0; weights as drawn.  c then moves by exactly +-1 per step where
    f = 1, so h = o tanh(c) reaches +-1 exactly after a few steps, and the
    saturated gates make the recurrence contract instead of amplifying
    rounding differences."""
    from layer_lstm_forward_amd.synth import f32_to_bf16_bits
    inp = make_inputs(spec)
    H, bf = spec.hidden_size, spec.dtype == "bf16"
    rng = np.random.default_rng(spec.seed + 1)
    for k in range(len(inp.params)):
        if k % 4 == 2:
            b = np.empty(4 * H, np.float32)
            b[:H] = 30.0
            b[H:2 * H] = np.where(rng.random(H) < 0.3, -100.0, 30.0)
            b[2 * H:3 * H] = np.where(rng.random(H) < 0.5, 30.0, -30.0)
            b[3 * H:] = 30.0
            inp.params[k] = f32_to_bf16_bits(b) if bf else b
        elif k % 4 == 3:
            inp.params[k] = np.zeros_like(inp.params[k])
    return inp


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("mode", sorted(LENGTH_MODES))
def test_saturated_gates(dtype, mode):
    """Every gate saturated (the ends of the sigmoid and tanh of the [warp-nn]
    equation block), |h| = 1 exactly on many cells (in the bf16 exchange word
    too), on the persistent (fused and hoisted), stepped and GEMM-step paths."""
    spec = Spec(32, 64, 2, True, 16, 20, dtype, 720, "normal0.1")
    print(f"case saturated gates {dtype} {mode}", flush=True)
    inp = _saturating(spec)
    rec, opts = LENGTH_MODES[mode]
    got, m = run_gpu(inp, recurrence=rec, options=opts)
    y, hn, cn = got
    assert np.all(np.abs(y) <= 1.0) and np.all(np.isfinite(cn))
    assert np.mean(np.abs(y) == 1.0) > 0.1, "the case should drive h to +-1 exactly"
    assert_parity(got, run_oracle(inp), dtype, f"saturated {mode}: {m.describe(spec.T, spec.B)}")


@pytest.mark.parametrize("mode", sorted(LENGTH_MODES))
def test_large_weights_few_steps(mode):
    """Weights x40 (the invariant pin's saturating draw) over three steps of one
    bidirectional layer in fp32: most pre-activations are far into the
    saturated ends.  (Over more steps such weights make the recurrence
    chaotic: fp32 and fp64 runs of the same inputs drift apart by more than
    any fixed tolerance, whatever the implementation.)"""
    spec = Spec(32, 64, 1, True, 3, 20, "f32", 730, "normal0.1")
    print(f"case large weights {mode}", flush=True)
    inp = make_inputs(spec)
    inp.params = [_scaled(p, 40.0, False) for p in inp.params]
    rec, opts = LENGTH_MODES[mode]
    got, m = run_gpu(inp, recurrence=rec, options=opts)
    assert np.all(np.abs(got[0]) <= 1.0)
    assert_parity(got, run_oracle(inp), "f32", f"x40 weights {mode}: {m.describe(spec.T, spec.B)}")


def test_lengths_all_full_equal_plain_forward():
    spec = Spec(48, 72, 2, True, 7, 37, "f32", 705, "normal0.1")
    inp = make_inputs(spec)
    a, _ = run_gpu(inp)
    b, _ = run_gpu(inp, lengths=[spec.T] * spec.B)
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)


@pytest.mark.parametrize("spec", SMALL[:4] + SMALL[5:7], ids=_id)
@pytest.mark.parametrize("proj_tile", [1, 2, 3, 4, 5, 6, 7],
                         ids=["proj128", "proj256", "proj256dma", "ring4", "ring5", "ring3x128", "interleaved"])
def test_projection_tiles(spec, proj_tile):
    """Both projection GEMM kernels, forced on shapes with ragged M, N and K."""
    print(f"case {_id(spec)} proj tile {proj_tile}", flush=True)
    inp = make_inputs(spec)
    got, m = run_gpu(inp, options={pkg.LSTM_OPT_PROJ_TILE: proj_tile, pkg.LSTM_OPT_FUSE_INPUT: 0})
    ref = run_oracle(inp)
    assert_parity(got, ref, spec.dtype, f"proj tile {proj_tile}")


@pytest.mark.parametrize("spec", [Spec(200, 136, 1, True, 9, 37, "bf16", 711, "normal0.1"),   # ragged K: a checked last stage
                                  Spec(512, 192, 1, False, 40, 13, "bf16", 712, "normal0.1"),  # full stages only
                                  Spec(96, 72, 1, False, 33, 9, "f32", 713, "normal0.1")], ids=_id)
def test_interleaved_projection_equals_dma(spec):
    """The projection with its loads spread over the products (tile 7) does
    the same products in the same order as the double-buffered one (tile 3):
    equal bit for bit, and within the oracle's tolerance."""
    print(f"case {_id(spec)} interleaved projection", flush=True)
    inp = make_inputs(spec)
    a, m = run_gpu(inp, options={pkg.LSTM_OPT_PROJ_TILE: 7, pkg.LSTM_OPT_FUSE_INPUT: 0, pkg.LSTM_OPT_SMALL_BATCH: 0})
    assert "k_proj_il" in m.describe(spec.T, spec.B)
    b, _ = run_gpu(inp, options={pkg.LSTM_OPT_PROJ_TILE: 3, pkg.LSTM_OPT_FUSE_INPUT: 0, pkg.LSTM_OPT_SMALL_BATCH: 0})
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)
    assert_parity(a, run_oracle(inp), spec.dtype, "interleaved projection")


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("spec", [Spec(48, 72, 2, True, 7, 37, "f32", 201, "normal0.1"),
                                  Spec(96, 136, 1, False, 6, 21, "bf16", 202, "normal0.1")], ids=_id)
def test_every_tile_persistent_equals_step(spec, tile):
    """Each recurrent tile gives oracle parity, and the persistent launch
    (step barriers inside one kernel) equals one-launch-per-step bit for bit
    (both with the hoisted projection; the fused one sums in another order)."""
    print(f"case {_id(spec)} tile {tile}", flush=True)
    inp = make_inputs(spec)
    ref = run_oracle(inp)
    hoist = {pkg.LSTM_OPT_FUSE_INPUT: 0}  # same projection on both sides: the sum order matches
    step, m = run_gpu(inp, recurrence=pkg.LSTM_REC_STEP, rec_tile=tile, options=hoist)
    assert_parity(step, ref, spec.dtype, m.describe(spec.T, spec.B))
    try:
        pers, m2 = run_gpu(inp, recurrence=pkg.LSTM_REC_PERSISTENT, rec_tile=tile, options=hoist)
    except pkg.LSTMError as e:
        assert e.status == -7  # this tile does not fit as one persistent launch
        return
    assert "persistent" in m2.describe(spec.T, spec.B)
    for a, b in zip(step, pers):
        np.testing.assert_array_equal(a, b)


def test_repeat_runs_bitwise_identical():
    spec = Spec(64, 128, 2, True, 10, 20, "bf16", 301, "normal0.1")
    inp = make_inputs(spec)
    a, m = run_gpu(inp)
    b, _ = run_gpu(inp, model=m, repeat=3)
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_zero_weights_closed_form_on_gpu(dtype):
    """All weights zero: c_n = f^n c0 + i g (1 - f^n) / (1 - f), h = o tanh(c)."""
    spec = Spec(16, 32, 2, True, 6, 4, dtype, 401, "normal0.1")
    inp = make_inputs(spec)
    H, D, L, T = 32, 2, 2, 6
    inp.params = [np.zeros_like(p) if k % 4 < 2 else p for k, p in enumerate(inp.params)]
    got, _ = run_gpu(inp)
    if dtype == "bf16":
        from layer_lstm_forward_amd.synth import bf16_bits_to_f32 as widen
    else:
        widen = np.asarray
    sig = lambda z: 1 / (1 + np.exp(-z))  # noqa: E731
    c0 = inp.c0.astype(np.float64)
    y, hn, cn = got
    tol = 2e-2 if dtype == "bf16" else 1e-5
    for l in range(L):
        for d in range(D):
            b = widen(inp.params[(l * D + d) * 4 + 2]).astype(np.float64) + \
                widen(inp.params[(l * D + d) * 4 + 3]).astype(np.float64)
            i, f, g, o = sig(b[:H]), sig(b[H:2 * H]), np.tanh(b[2 * H:3 * H]), sig(b[3 * H:])
            for n, t in [(T, None)] + [((t + 1) if d == 0 else (T - t), t) for t in range(T)]:
                cc = f ** n * c0[l * D + d] + i * g * (1 - f ** n) / (1 - f)
                if t is None:
                    np.testing.assert_allclose(cn[l * D + d], cc, atol=tol, rtol=0)
                    np.testing.assert_allclose(hn[l * D + d], o * np.tanh(cc), atol=tol, rtol=0)
                elif l == L - 1:
                    np.testing.assert_allclose(y[t, :, d * H:(d + 1) * H], o * np.tanh(cc), atol=tol, rtol=0)


def _full(name, rows, options=None):
    spec = WORKLOADS[name]
    print(f"case {name} rows {rows} options {options}", flush=True)
    inp = make_inputs(spec)
    got, m = run_gpu(inp, options=options)
    desc = m.describe(spec.T, spec.B)
    y, hn, cn = got
    assert np.all(np.isfinite(y)) and np.all(np.abs(y) <= 1.0)
    if rows is None:
        ref = run_oracle(inp)
        return assert_parity(got, ref, spec.dtype, f"{name}: {desc}")
    sub = inp.rows(rows)
    ref = run_oracle(sub)
    return assert_parity((y[:, rows], hn[:, rows], cn[:, rows]), ref, spec.dtype, f"{name}: {desc}")


def test_full_tiny_l1_in8_h16():
    _full("l1_in8_h16_t5_b1_f32", None)


def test_full_l2_in256_h512_b64_f32_sampled_rows():
    _full("l2_in256_h512_t128_b64_f32", [0, 37, 63])


def test_full_l2_in256_h512_b64_f32_hoisted_projection_sampled_rows():
    _full("l2_in256_h512_t128_b64_f32", [5, 40], options={pkg.LSTM_OPT_FUSE_INPUT: 0})


def test_full_l2_in256_h512_b64_f32_wavefront_sampled_rows():
    _full("l2_in256_h512_t128_b64_f32", [1, 32, 62], options={pkg.LSTM_OPT_LAYER_PIPE: 1})


def test_full_l2_in256_h512_b64_f32_paired_wavefront_sampled_rows():
    _full("l2_in256_h512_t128_b64_f32", [3, 31, 63], options={pkg.LSTM_OPT_LAYER_PIPE: 2})


def test_full_l2_in256_h512_b64_f32_layer_by_layer_sampled_rows():
    _full("l2_in256_h512_t128_b64_f32", [2, 33, 61], options={pkg.LSTM_OPT_LAYER_PIPE: 0})


def test_full_l2_in256_h512_b64_f32_lengths_sampled_rows():
    """The benchmark workload with a padded-bucket length mix, rows sampled."""
    from layer_lstm_forward_amd.synth import make_lengths
    spec = WORKLOADS["l2_in256_h512_t128_b64_f32"]
    inp = make_inputs(spec)
    lengths = make_lengths(spec, "mix")
    got, m = run_gpu(inp, lengths=lengths)
    rows = [0, 21, 63]
    ref = run_oracle(inp.rows(rows), lengths=lengths[rows])
    y, hn, cn = got
    assert_parity((y[:, rows], hn[:, rows], cn[:, rows]), ref, spec.dtype, m.describe(spec.T, spec.B))


def test_full_l2bi_in512_h1024_b32_bf16_all_rows():
    _full("l2bi_in512_h1024_t256_b32_bf16", None)


@pytest.mark.parametrize("name", ["l1_in1024_h1024_t1024_b1_bf16", "l1_in1024_h1024_t1024_b4_bf16"])
def test_full_l1_h1024_t1024_small_batch(name):
    _full(name, None)


@pytest.mark.slow
def test_full_l4_in2048_h2048_b256_bf16_sampled_rows():
    # the first row, the last row (the end of the last 64-row block) and one
    # seeded random row, over the full T and all four layers
    rnd = int(np.random.default_rng(1006).integers(1, 255))
    _full("l4_in2048_h2048_t512_b256_bf16", [0, rnd, 255])

"""The pins have power: each plausible mistake planted in a copy of the oracle
(on the CPU, never on a GPU) makes the pin suite fail (the forward pins for
mistakes in the forward, the backward pins for mistakes in the backward)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "lstm_oracle.c")

MUTATIONS = {
    "drop_b_hh": ("acc = b_ih[r] + b_hh[r];", "acc = b_ih[r];"),
    "swap_i_f": ("const double ig = sigmoid(pb[j]);\n                        const double fg = sigmoid(pb[H + j]);",
                 "const double ig = sigmoid(pb[H + j]);\n                        const double fg = sigmoid(pb[j]);"),
    "sigmoid_sign": ("return 1.0 / (1.0 + exp(-z));", "return 1.0 / (1.0 + exp(z));"),
    "transposed_W_hh": ("acc += wh[k] * hb[k];", "acc += W_hh[(size_t)k * G + r] * hb[k];"),
    "reverse_at_step_index": ("Y[((size_t)t * B + b)", "Y[((size_t)s * B + b)"),
    "h0_of_layer0_only": ("h[e] = h0 ? h0[st + e] : 0.0;", "h[e] = h0 ? h0[e] : 0.0;"),
    "cell_uses_o": ("const double cn = fg * c[e] + ig * gg;", "const double cn = fg * c[e] + ig * og;"),
    "h_without_o": ("const double hn = og * tanh(cn);", "const double hn = tanh(cn);"),
    "o_gate_tanh": ("const double og = sigmoid(pb[3 * H + j]);", "const double og = tanh(pb[3 * H + j]);"),
    "transposed_W_ih": ("acc += wi[k] * xt[k];", "acc += W_ih[(size_t)k * G + r] * xt[k];"),
    "next_layer_reads_h_not_y": ("in_seq = Xl;", "in_seq = Yl;"),
    # variable-length rows: the reverse direction starting at T - 1 instead of
    # at the row's own end; one step too many per row
    "varlen_reverse_from_T": ("#define PADDED(t, b) (lengths && (t) >= lengths[b])",
                              "#define PADDED(t, b) (lengths && d == 0 && (t) >= lengths[b])"),
    "varlen_one_step_long": ("#define PADDED(t, b) (lengths && (t) >= lengths[b])",
                             "#define PADDED(t, b) (lengths && (t) > lengths[b])"),
}


# mistakes in the backward pass, checked by tests/test_oracle_backward.py
BACKWARD_MUTATIONS = {
    "bwd_drop_cell_carry": ("dc[eb] = dct * gf[e];  /* to c_prev */", "dc[eb] = 0.0 * dct * gf[e];"),
    "bwd_tanh_derivative": ("const double dct = dc[eb] + dht * go[e] * (1.0 - tc * tc);",
                            "const double dct = dc[eb] + dht * go[e] * (1.0 - tc);"),
    "bwd_o_gate_from_cell": ("dz[(size_t)b * G + 3 * H + j] = dht * tc * go[e] * (1.0 - go[e]);",
                             "dz[(size_t)b * G + 3 * H + j] = dct * tc * go[e] * (1.0 - go[e]);"),
    "bwd_one_bias_only": ("dp[3][r] += z;", "dp[3][r] += 0.0 * z;"),
    "bwd_no_recurrent_gradient": ("for (size_t e = 0; e < BH; ++e) dhn[e] = dh[e];",
                                  "for (size_t e = 0; e < BH; ++e) dhn[e] = 0.0 * dh[e];"),
    # per-row lengths: the gradient of h dropped at a padded step; the state
    # before the reverse scan's first valid step taken as zero
    "bwd_padded_dh_dropped": ("dh[(size_t)b * H + k] = PADDED(t, b) ? dhn[(size_t)b * H + k] : acc;",
                              "dh[(size_t)b * H + k] = acc;"),
    "bwd_padded_state_lost": ("hs[e] = h[(size_t)b * H + j];", "hs[e] = 0.0;"),
}


# mistakes in the training dropout and its generator, checked by tests/test_oracle_dropout.py
DROPOUT_MUTATIONS = {
    "dropout_no_rescale": ("return dropout_keeps(p, seed, call, l, e) ? 1.0 / (1.0 - p) : 0.0;",
                           "return dropout_keeps(p, seed, call, l, e) ? 1.0 : 0.0;"),
    "dropout_keep_inverted": ("return u >= p;", "return u < p;"),
    "dropout_next_layer_index": ("Xl[e] *= dropout_factor(drop_p, seed, call, l, e);",
                                 "Xl[e] *= dropout_factor(drop_p, seed, call, l + 1, e);"),
    "dropout_first_word_only": ("(double)(w[e % 4] >> 11)", "(double)(w[0] >> 11)"),
    "philox_key_not_advanced": ("k1 += 0xBB67AE8584CAA73Bull;", "k1 += 0;"),
    "dropout_gradient_unmasked": ("dY[e] = l > 0 ? dX[e] * dropout_factor(drop_p, seed, call, l - 1, e) : dX[e];",
                                  "dY[e] = dX[e];"),
}
# mistakes in the other recurrent modes, checked by tests/test_oracle_modes.py
MODE_MUTATIONS = {
    "gru_reset_outside_hidden": ("const double ng = tanh(gi[2 * H + j] + rg * gh[2 * H + j]);",
                                 "const double ng = tanh(rg * (gi[2 * H + j] + gh[2 * H + j]));"),
    "gru_update_swapped": ("hv = (1.0 - zg) * ng + zg * state[(size_t)b * H + j];",
                           "hv = zg * ng + (1.0 - zg) * state[(size_t)b * H + j];"),
    "gru_r_reads_z_block": ("const double rg = sigmoid(gi[j] + gh[j]);",
                            "const double rg = sigmoid(gi[H + j] + gh[H + j]);"),
    "relu_is_identity": ("hv = mode == 2 ? tanh(v) : (v > 0.0 ? v : 0.0);", "hv = mode == 2 ? tanh(v) : v;"),
    "rnn_hidden_bias_dropped": ("double a = has_bias ? w[2][r] : 0.0, c = has_bias ? w[3][r] : 0.0;",
                                "double a = has_bias ? w[2][r] : 0.0, c = 0.0;"),
}
TARGET = {**{n: "test_oracle_pins.py" for n in MUTATIONS},
          **{n: "test_oracle_modes.py" for n in MODE_MUTATIONS},
          **{n: "test_oracle_backward.py" for n in BACKWARD_MUTATIONS},
          **{n: "test_oracle_dropout.py" for n in DROPOUT_MUTATIONS}}
ALL = {**MUTATIONS, **BACKWARD_MUTATIONS, **DROPOUT_MUTATIONS, **MODE_MUTATIONS}


@pytest.mark.parametrize("name", sorted(ALL))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = ALL[name]
    target = TARGET[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mut = tmp_path / "lstm_oracle_mut.c"
    mut.write_text(src.replace(old, new))
    lib = tmp_path / "liblstm_oracle_mut.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-o", str(lib),
                           str(mut), "-lm"])
    env = dict(os.environ, LSTM_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", target)],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"mutation {name} survived the pins:\n{r.stdout[-2000:]}"

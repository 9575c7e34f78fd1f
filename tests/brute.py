"""Per-gate scalar LSTM evaluator for tiny shapes (test helper, pure Python).

An independent formulation of the cell used to pin the oracle: it keeps the
eight weight matrices W_ii..W_ho and the eight bias vectors b_ii..b_ho as
separate objects, exactly the symbols of the equation block on the warp-nn
"Long Short-Term Memory (LSTM)" page (the per-gate buffers of the pulsatrix
"LSTMModule" class reference are the same idea), and evaluates every scalar
with Python floats and math.exp / math.tanh.  The stacked row-block layout is
unpacked here by the page's parameter table: W_ii..W_io are the four H-row
blocks of weight_ih, in that order, and likewise for weight_hh and the biases.
"""
import math

GATES = ("i", "f", "g", "o")


def unpack(W_ih, W_hh, b_ih, b_hh, H):
    """Split stacked parameters into per-gate nested lists (no numpy)."""
    g = {}
    for q, name in enumerate(GATES):
        rows = range(q * H, (q + 1) * H)
        g["W_i" + name] = [[float(W_ih[r][k]) for k in range(len(W_ih[r]))] for r in rows]
        g["W_h" + name] = [[float(W_hh[r][k]) for k in range(len(W_hh[r]))] for r in rows]
        g["b_i" + name] = [float(b_ih[r]) if b_ih is not None else 0.0 for r in rows]
        g["b_h" + name] = [float(b_hh[r]) if b_hh is not None else 0.0 for r in rows]
    return g


def _sig(z):
    return 1.0 / (1.0 + math.exp(-z))


def _affine(W, v, b):
    return [sum(W[j][k] * v[k] for k in range(len(v))) + b[j] for j in range(len(W))]


def cell(g, x, h, c):
    """One step of one direction: returns (h_t, c_t) as lists."""
    a = {n: [u + w for u, w in zip(_affine(g["W_i" + n], x, g["b_i" + n]),
                                   _affine(g["W_h" + n], h, g["b_h" + n]))]
         for n in GATES}
    i = [_sig(z) for z in a["i"]]
    f = [_sig(z) for z in a["f"]]
    gg = [math.tanh(z) for z in a["g"]]
    o = [_sig(z) for z in a["o"]]
    c_new = [f[j] * c[j] + i[j] * gg[j] for j in range(len(c))]
    h_new = [o[j] * math.tanh(c_new[j]) for j in range(len(c))]
    return h_new, c_new


def lstm(x, params, H, L, D, h0=None, c0=None, has_bias=True, lengths=None, between=None):
    """x: nested [T][B][I]; params flat in (layer, direction, W_ih, W_hh[, b_ih, b_hh]).

    between: None, or between[l][t][b][k], a factor that element (t, b, k) of
    layer l's output carries into layer l + 1 (training dropout).

    lengths: None, or the number of valid steps of each row; a row's sequence
    is then its first lengths[b] time steps only, its padded outputs stay
    zero, and the reverse direction walks that sequence backwards from its
    own last element.
    Returns y [T][B][D*H], h_n and c_n [L*D][B][H] as nested lists.
    """
    T, B = len(x), len(x[0])
    per = 4 if has_bias else 2
    seq = [[list(map(float, x[t][b])) for b in range(B)] for t in range(T)]
    hn, cn = [], []
    for l in range(L):
        out = [[[0.0] * (D * H) for _ in range(B)] for _ in range(T)]
        for d in range(D):
            p = params[(l * D + d) * per:(l * D + d + 1) * per]
            g = unpack(p[0], p[1], p[2] if has_bias else None, p[3] if has_bias else None, H)
            hl, cl = [], []
            for b in range(B):
                h = [float(v) for v in h0[l * D + d][b]] if h0 is not None else [0.0] * H
                c = [float(v) for v in c0[l * D + d][b]] if c0 is not None else [0.0] * H
                n = T if lengths is None else lengths[b]
                order = range(n) if d == 0 else range(n - 1, -1, -1)
                for t in order:
                    h, c = cell(g, seq[t][b], h, c)
                    out[t][b][d * H:(d + 1) * H] = h
                hl.append(h)
                cl.append(c)
            hn.append(hl)
            cn.append(cl)
        seq = out
        if between is not None and l + 1 < L:
            seq = [[[out[t][b][k] * between[l][t][b][k] for k in range(D * H)] for b in range(B)]
                   for t in range(T)]
    return out, hn, cn


def rnn(mode, x, params, H, L, D, h0=None, has_bias=True, lengths=None):
    """The GRU ("gru", gate blocks r, z, n) and the plain RNNs ("rnn_tanh",
    "rnn_relu") in the same per-gate scalar style: every gate keeps its own
    W_i*, W_h*, b_i*, b_h*; the GRU's candidate applies r to the hidden
    contribution including its bias.  lengths: as for lstm() (a row's own
    sequence only; padded outputs stay zero).  Returns y [T][B][D*H] and h_n
    [L*D][B][H] as nested lists."""
    T, B = len(x), len(x[0])
    per = 4 if has_bias else 2
    names = ("r", "z", "n") if mode == "gru" else ("a",)
    seq = [[list(map(float, x[t][b])) for b in range(B)] for t in range(T)]
    hn = []
    out = seq
    for l in range(L):
        out = [[[0.0] * (D * H) for _ in range(B)] for _ in range(T)]
        for d in range(D):
            p = params[(l * D + d) * per:(l * D + d + 1) * per]
            g = {}
            for q, nm in enumerate(names):
                rows = range(q * H, (q + 1) * H)
                g["Wi" + nm] = [[float(v) for v in p[0][r]] for r in rows]
                g["Wh" + nm] = [[float(v) for v in p[1][r]] for r in rows]
                g["bi" + nm] = [float(p[2][r]) if has_bias else 0.0 for r in rows]
                g["bh" + nm] = [float(p[3][r]) if has_bias else 0.0 for r in rows]
            hl = []
            for b in range(B):
                h = [float(v) for v in h0[l * D + d][b]] if h0 is not None else [0.0] * H
                n = T if lengths is None else lengths[b]
                order = range(n) if d == 0 else range(n - 1, -1, -1)
                for t in order:
                    xi = {nm: _affine(g["Wi" + nm], seq[t][b], g["bi" + nm]) for nm in names}
                    hh = {nm: _affine(g["Wh" + nm], h, g["bh" + nm]) for nm in names}
                    if mode == "gru":
                        r = [_sig(xi["r"][j] + hh["r"][j]) for j in range(H)]
                        z = [_sig(xi["z"][j] + hh["z"][j]) for j in range(H)]
                        n = [math.tanh(xi["n"][j] + r[j] * hh["n"][j]) for j in range(H)]
                        h = [(1.0 - z[j]) * n[j] + z[j] * h[j] for j in range(H)]
                    elif mode == "rnn_tanh":
                        h = [math.tanh(xi["a"][j] + hh["a"][j]) for j in range(H)]
                    else:
                        h = [max(0.0, xi["a"][j] + hh["a"][j]) for j in range(H)]
                    out[t][b][d * H:(d + 1) * H] = h
                hl.append(h)
            hn.append(hl)
        seq = out
    return out, hn

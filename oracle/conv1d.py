"""Causal depthwise conv1d of the Mamba2 mixer (the step before the scan), in
float64 numpy.

TEST INFRASTRUCTURE ONLY: imported by tests and the bench's CPU baseline
leg, never by the product path; shares no code with the HIP library.

What it computes (vLLM RFC "Mamba2: exact-replay decode ...", section 2,
item 6: the prefill form causal_conv1d_fn and the decode form
causal_conv1d_update of the same convolution; the bf16 operands are promoted
before the accumulation). For one sequence of L tokens with channels c of
the concatenated x | B | C projection (conv_dim = H*P + 2*G*N), kernel width
W and a state holding the W-1 inputs before the sequence:

    ext   = [state (W-1 rows, oldest first); inputs (L rows)]
    out_t = act(bias_c + sum_{i<W} w[c, i] * ext[t + i, c])
    state' = the last W-1 rows of ext

with act = SiLU (v / (1 + exp(-v))) or the identity. The outputs split into
x [L,H,P], B [L,G,N], C [L,G,N] by channel. The decode form is the same
definition applied to one token (L = 1).
"""
from __future__ import annotations

import numpy as np


def silu(v):
    return v / (1.0 + np.exp(-v))


def conv1d_seq(inp, weight, bias=None, state=None, activation=True):
    """One sequence. inp [L, Cd], weight [Cd, W], bias [Cd] or None, state
    [Cd, W-1] (oldest first) or None = zeros. Returns (out [L, Cd], new
    state [Cd, W-1]), float64."""
    inp = np.asarray(inp, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    L, Cd = inp.shape
    W = w.shape[1]
    st = np.zeros((Cd, W - 1)) if state is None else np.asarray(state, dtype=np.float64)
    ext = np.concatenate([st.T, inp], axis=0)                 # [W-1+L, Cd]
    out = np.zeros((L, Cd)) if bias is None else np.tile(np.asarray(bias, np.float64), (L, 1))
    for i in range(W):
        out = out + w[:, i] * ext[i:i + L]
    if activation:
        out = silu(out)
    return out, ext[L:].T.copy()


def conv1d_varlen(inp, weight, cu, bias=None, states=None, activation=True):
    """Varlen pack: sequence s is rows cu[s]..cu[s+1]-1 of inp [T, Cd] and
    starts from states[s] (None = zeros). Returns (out [T, Cd], final states
    [S, Cd, W-1])."""
    inp = np.asarray(inp, dtype=np.float64)
    W = np.asarray(weight).shape[1]
    S = len(cu) - 1
    out = np.zeros(inp.shape)
    fin = np.zeros((S, inp.shape[1], W - 1))
    for s in range(S):
        a, b = int(cu[s]), int(cu[s + 1])
        o, f = conv1d_seq(inp[a:b], weight, bias, None if states is None else states[s],
                          activation)
        out[a:b] = o
        fin[s] = f
    return out, fin


def split_xbc(out, H, G, P, N):
    """[T, H*P + 2*G*N] -> x [T,H,P], B [T,G,N], C [T,G,N]."""
    T = out.shape[0]
    hp, gn = H * P, G * N
    return (out[:, :hp].reshape(T, H, P), out[:, hp:hp + gn].reshape(T, G, N),
            out[:, hp + gn:].reshape(T, G, N))

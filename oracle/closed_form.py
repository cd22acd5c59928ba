"""Chunk-by-chunk closed form of the Mamba2 scan, in float64 numpy.

TEST INFRASTRUCTURE ONLY. An independent formulation of the recurrence in
ssd_oracle.c, used to pin it.

The ReplaySSM reproduction page ("Core equations") gives, for a checkpoint
S_ckpt followed by buffered tokens j = 1..h with decay alpha_i:

    S_h = gamma_h S_ckpt + sum_j gamma_{j+1:h} v_j k_j^T,
    gamma_{a:b} = prod_{i=a..b} alpha_i,

and outputs as the checkpoint read-out plus a decay-masked product of
key-query scores with values. With alpha_i = exp(delta_i A), v = delta x,
k = B, q = C and Lambda_t the in-chunk inclusive cumulative sum of
delta_r A, this is, for one chunk starting from state S0:

    y_t   = exp(Lambda_t) (S0 C_t) + sum_{s<=t} exp(Lambda_t - Lambda_s)
                 delta_s (C_t . B_s) x_s + D x_t
    S_end = exp(Lambda_last) S0 + sum_s exp(Lambda_last - Lambda_s)
                 delta_s x_s (outer) B_s

The chunk grid starts at each sequence's first token. Plain numpy matmul is
the only library step; there is no blocking beyond the chunk itself.
"""
from __future__ import annotations

import numpy as np


def softplus(u):
    return np.logaddexp(0.0, u)


def chunked_scan(x, dt, A, B, C, cu, chunk_size, D=None, dt_bias=None,
                 dt_softplus=True, init=None):
    """Returns (y[T,H,P], final[S,H,P,N], chunk_end_states list per seq)."""
    x = np.asarray(x, np.float64)
    dt = np.asarray(dt, np.float64)
    B = np.asarray(B, np.float64)
    C = np.asarray(C, np.float64)
    A = np.asarray(A, np.float64)
    T, H, P = x.shape
    G, N = B.shape[1:]
    hpg = H // G
    S = len(cu) - 1
    bias = np.zeros(H) if dt_bias is None else np.asarray(dt_bias, np.float64)
    Dv = np.zeros(H) if D is None else np.asarray(D, np.float64)
    u = dt + bias[None, :]
    delta = softplus(u) if dt_softplus else u              # [T, H]
    y = np.zeros((T, H, P))
    final = np.zeros((S, H, P, N))
    ends = []
    for s in range(S):
        t0, t1 = int(cu[s]), int(cu[s + 1])
        state = (np.zeros((H, P, N)) if init is None
                 else np.array(init[s], dtype=np.float64))
        seq_ends = []
        for c0 in range(t0, t1, chunk_size):
            c1 = min(c0 + chunk_size, t1)
            for h in range(H):
                g = h // hpg
                d = delta[c0:c1, h]                         # [L]
                lam = np.cumsum(d * A[h])                   # inclusive
                Ct, Bt, xt = C[c0:c1, g], B[c0:c1, g], x[c0:c1, h]
                diff = lam[:, None] - lam[None, :]
                causal = np.tril(np.ones((c1 - c0, c1 - c0), dtype=bool))
                decay = np.where(causal, np.exp(np.where(causal, diff, 0.0)), 0.0)
                scores = (Ct @ Bt.T) * decay * d[None, :]   # [L, L]
                y_state = np.exp(lam)[:, None] * (Ct @ state[h].T)
                y[c0:c1, h] = y_state + scores @ xt + Dv[h] * xt
                w = np.exp(lam[-1] - lam) * d               # [L]
                state[h] = np.exp(lam[-1]) * state[h] + (xt * w[:, None]).T @ Bt
            if c1 - c0 == chunk_size:
                seq_ends.append(state.copy())
        final[s] = state
        ends.append(seq_ends)
    return y, final, ends

"""Recurrent selective-state update with the state stored in a cache dtype
(fp32 or bf16), in float64 numpy.

TEST INFRASTRUCTURE ONLY: imported by tests and the bench's CPU baseline
leg, never by the product path; shares no code with the HIP library.

What it computes (vLLM RFC "Mamba2: exact-replay decode ...", section 3b,
packed-history recovery: generated history is replayed with a multi-token
recurrent update that rounds the state to the cache dtype after every
token, so a recovered decode continues exactly like an uninterrupted one;
section 1 names the recurrent update). Per head h, group g = h / (H/G),
token t, with the stored state widened exactly:

    delta = softplus(dt_t + dt_bias[h])
    h_new = exp(delta A[h]) * h + delta * x_t (outer) B_t        [P x N]
    y_t   = h_new . C_t + D[h] x_t
    h     = round_to_cache_dtype(h_new)

The output reads the unrounded h_new; only what is stored is rounded. With
an fp32 cache the rounding is to float32 (the fp64 reference keeps fp64 when
cache="f64").
"""
from __future__ import annotations

import numpy as np


def softplus(u):
    return np.where(u > 0, u + np.log1p(np.exp(-np.abs(u))), np.log1p(np.exp(u)))


def round_bf16(a):
    """float64 -> nearest bf16 value (ties to even), as float64. Rounds the
    float64 value directly (one rounding)."""
    a = np.asarray(a, dtype=np.float64)
    m, e = np.frexp(a)                    # a = m * 2**e, 0.5 <= |m| < 1
    # bf16 keeps 8 significant bits: m * 2**8 rounded to an integer, ties to even
    r = np.round(np.ldexp(m, 8))          # numpy rounds half to even
    return np.ldexp(r, e - 8)


def round_cache(a, cache):
    if cache == "f64":
        return np.asarray(a, dtype=np.float64)
    if cache == "f32":
        return np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)
    if cache == "bf16":
        return round_bf16(a)
    raise ValueError(cache)


def ssu_tokens(h0, x, dt, A, B, C, D=None, dt_bias=None, dt_softplus=True, cache="f32"):
    """One sequence of T tokens from stored state h0 [H,P,N] (float64 values
    of the cache dtype). x [T,H,P], dt [T,H], B/C [T,G,N]. Returns (y [T,H,P],
    stored state after the last token [H,P,N])."""
    x, dt, B, C = (np.asarray(v, dtype=np.float64) for v in (x, dt, B, C))
    T, H, P = x.shape
    G = B.shape[1]
    hpg = H // G
    A = np.asarray(A, dtype=np.float64)
    D = np.zeros(H) if D is None else np.asarray(D, dtype=np.float64)
    bias = np.zeros(H) if dt_bias is None else np.asarray(dt_bias, dtype=np.float64)
    h = np.array(h0, dtype=np.float64, copy=True)
    y = np.zeros((T, H, P))
    for t in range(T):
        for hh in range(H):
            g = hh // hpg
            u = dt[t, hh] + bias[hh]
            dl = softplus(u) if dt_softplus else u
            hn = np.exp(dl * A[hh]) * h[hh] + dl * np.outer(x[t, hh], B[t, g])
            y[t, hh] = hn @ C[t, g] + D[hh] * x[t, hh]
            h[hh] = round_cache(hn, cache)
    return y, h


def ssu_varlen(states, x, dt, A, B, C, cu, D=None, dt_bias=None, dt_softplus=True,
               cache="f32"):
    """Varlen pack: sequence s (tokens cu[s]..cu[s+1]-1) starts from
    states[s]. Returns (y [T,H,P], final states [S,H,P,N])."""
    S = len(cu) - 1
    y = np.zeros(np.asarray(x).shape)
    fin = np.array(states, dtype=np.float64, copy=True)
    for s in range(S):
        a, b = int(cu[s]), int(cu[s + 1])
        ys, fin[s] = ssu_tokens(states[s], x[a:b], dt[a:b], A, B[a:b], C[a:b], D, dt_bias,
                                dt_softplus, cache)
        y[a:b] = ys
    return y, fin

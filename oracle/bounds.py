"""Error scales of the chunked scan's outputs, for element-wise bounds in the
GPU parity tests.

TEST INFRASTRUCTURE ONLY: imported by tests, never by the product path.

Row t of a chunk (head h, chunk start state S0, in-chunk inclusive sums
Lam_t of delta*A) is, in the chunk-by-chunk closed form of the ReplaySSM
reproduction page ("Core equations") that the vLLM RFC "Mamba2: exact-replay
decode ..." (section 2, item 1) measures against an fp64 reference,

    y_t[p] = exp(Lam_t) sum_n S0[p,n] C_t[n]                       (read-out)
           + sum_{s<=t} m_ts x_s[p],  m_ts = (C_t . B_s) exp(Lam_t - Lam_s) delta_s
           + D x_t[p].

A kernel that rounds its read-out operand S0 and each weight m_ts once to a
format with unit roundoff u (and otherwise computes in a much finer
precision) errs by at most

    u * mag[t,p],  mag = exp(Lam_t) sum_n |S0[p,n] C_t[n]| + sum_s |m_ts x_s[p]|

(each rounding is a relative error of at most u on one of these terms), and,
in the probabilistic model of rounding errors -- independent, mean zero,
bounded by u (Higham and Mary, "A New Approach to Probabilistic Rounding
Error Analysis", SIAM J. Sci. Comput. 41(5), 2019, Theorem 2.4, a Hoeffding
bound) -- by at most

    lam * u * rms[t,p],  rms^2 = exp(2 Lam_t) sum_n (S0[p,n] C_t[n])^2 + sum_s (m_ts x_s[p])^2

with probability at least 1 - 2 exp(-lam^2 / 2) per element.

``chunk_error_scales`` evaluates mag and rms from the exact fp64 quantities:
the chunk start states come from the sequential oracle (``scan`` with
``max_chunks``), the chunk grid starts at each sequence's first token.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .oracle import scan


def _softplus(u):
    # log1p(exp(u)) for u <= 0, u + log1p(exp(-u)) otherwise
    return np.where(u <= 0, np.log1p(np.exp(np.minimum(u, 0.0))),
                    u + np.log1p(np.exp(-np.maximum(u, 0.0))))


@dataclass
class ErrorScales:
    mag: np.ndarray      # [T, H, P] sum of the absolute rounded terms
    rms: np.ndarray      # [T, H, P] root of the sum of their squares
    state_row: np.ndarray  # [T, H] exp(Lam_t) max|S0| sum_n |C_t[n]|
    seqs: list           # sequences covered (others are zero)


def chunk_error_scales(x, dt, A, B, C, cu, chunk_size, D=None, dt_bias=None,
                       dt_softplus=True, init=None, seqs=None) -> ErrorScales:
    """mag, rms and the per-row state scale for every output row of the
    sequences in `seqs` (default: all) of a varlen pack; inputs as for
    ``scan`` (fp64 arrays of the exact stored values)."""
    x, dt, B, C = (np.asarray(a, dtype=np.float64) for a in (x, dt, B, C))
    A = np.asarray(A, dtype=np.float64)
    cu = np.asarray(cu, dtype=np.int64)
    T, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    hpg = H // G
    Q = int(chunk_size)
    S = cu.size - 1
    seqs = list(range(S)) if seqs is None else list(seqs)
    raw = dt + (0.0 if dt_bias is None else np.asarray(dt_bias, dtype=np.float64)[None, :])
    delta = _softplus(raw) if dt_softplus else raw
    mag = np.zeros((T, H, P))
    rms = np.zeros((T, H, P))
    srow = np.zeros((T, H))
    for s in seqs:
        t0, t1 = int(cu[s]), int(cu[s + 1])
        L = t1 - t0
        if L == 0:
            continue
        nfull = L // Q
        sub_cu = np.array([0, L], dtype=np.int64)
        h0 = None if init is None else np.asarray(init, dtype=np.float64)[s:s + 1]
        starts = [np.zeros((H, P, N)) if h0 is None else h0[0]]
        if nfull > 0:
            r = scan(x[t0:t1], dt[t0:t1], A, B[t0:t1], C[t0:t1], sub_cu, Q, D=D,
                     dt_bias=dt_bias, dt_softplus=dt_softplus, init=h0, max_chunks=nfull)
            starts += [r.chunk_states[0, c] for c in range(nfull)]
        for c in range((L + Q - 1) // Q):
            a, b = t0 + c * Q, min(t0 + (c + 1) * Q, t1)
            S0 = starts[c]
            for g in range(G):
                Cc, Bc = C[a:b, g], B[a:b, g]
                Gm = Cc @ Bc.T                                  # [t, s] = C_t . B_s
                Cabs, Csq = np.abs(Cc), Cc * Cc
                for h in range(g * hpg, (g + 1) * hpg):
                    d = delta[a:b, h]
                    lam = np.cumsum(d * A[h])
                    e = np.exp(lam)
                    lower = np.tril(np.ones((b - a, b - a), dtype=bool))
                    dec = np.exp(np.where(lower, lam[:, None] - lam[None, :], -np.inf))
                    w = dec * d[None, :]
                    m = Gm * w
                    xc = x[a:b, h]
                    s0 = S0[h]
                    ro_abs = e[:, None] * (Cabs @ np.abs(s0).T)
                    ro_sq = (e * e)[:, None] * (Csq @ (s0 * s0).T)
                    mag[a:b, h] = ro_abs + np.abs(m) @ np.abs(xc)
                    rms[a:b, h] = np.sqrt(ro_sq + (m * m) @ (xc * xc))
                    srow[a:b, h] = e * np.abs(s0).max() * Cabs.sum(axis=1)
    return ErrorScales(mag, rms, srow, seqs)

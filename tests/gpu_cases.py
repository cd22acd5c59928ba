"""Shared helpers for the GPU tests: seeded problems on the device, the
oracle's view of the same values, and the tolerance metrics.

Tolerances (written in the tests that use them):
  bf16 outputs: mean|y - y_ref| / mean|y_ref| <= 0.3 %, over all outputs of
  a run, in float64 (the oracle is not rounded, so the 0.141 % bf16 floor is
  part of the budget), and the same per (sequence, head); element by element
  the bounds of check_bf16 below.
  fp32 states: per (sequence, head), max|S - S_ref| / max|S_ref| <= 1e-4.
  fp32 outputs: per (sequence, head), max|y - y_ref| / max|y_ref| <= 1e-4.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

from exact_replay_decode_amd import Shape, synth, to_device, to_f64

DEV = torch.device("cuda:0")


@dataclasses.dataclass
class Problem:
    shape: Shape
    hp: synth.HeadParams
    tok: synth.Tokens          # packed streams
    lengths: list
    A: torch.Tensor
    D: torch.Tensor
    bias: torch.Tensor

    @property
    def cu(self):
        return synth.cu_seqlens(self.lengths)

    def dev(self, a, b=None):
        """(x, dt, B, C) on the device for packed tokens [a, b)."""
        t = self.tok if a is None else self.tok.slice(a, b)
        sh = self.shape
        return (to_device(t.x, sh.io_dtype, DEV), to_device(t.dt, sh.dt_dtype, DEV),
                to_device(t.B, sh.io_dtype, DEV), to_device(t.C, sh.io_dtype, DEV))

    def oracle(self, init=None, max_chunks=0):
        from oracle import scan
        x, dt, B, C = self.tok.f64()
        return scan(x, dt, self.hp.A, B, C, self.cu, self.shape.chunk_size,
                    D=self.hp.D, dt_bias=self.hp.dt_bias,
                    dt_softplus=self.shape.dt_softplus, init=init, max_chunks=max_chunks)


def make_problem(lengths, H, G, P, N, Q, io="bf16", dt=None, seed=0) -> Problem:
    shape = Shape(H, G, P, N, Q, io, dt or io)
    hp = synth.make_head_params(H, seed)
    parts = [synth.make_tokens(L, H, G, P, N, seed, stream=i, io_dtype=io,
                               dt_dtype=dt or io) for i, L in enumerate(lengths)]
    tok = synth.concat(parts)
    f = lambda a: torch.from_numpy(a).to(DEV)  # noqa: E731
    return Problem(shape, hp, tok, list(lengths), f(hp.A), f(hp.D), f(hp.dt_bias))


def bits(t: torch.Tensor) -> torch.Tensor:
    """Raw bit pattern, so equality is byte equality (-0 != +0)."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16)
    if t.dtype == torch.float32:
        return t.view(torch.int32)
    return t


def same_bits(a: torch.Tensor, b: torch.Tensor) -> bool:
    return a.shape == b.shape and bool(torch.equal(bits(a), bits(b)))


def mean_rel_err(y: torch.Tensor, ref: np.ndarray) -> float:
    d = to_f64(y) - ref
    return float(np.abs(d).mean() / np.abs(ref).mean())


def headwise_max_rel(s: np.ndarray, ref: np.ndarray) -> float:
    """max over (seq, head) of max|s - ref| / max|ref| on the trailing dims."""
    d = np.abs(s - ref).reshape(ref.shape[0], ref.shape[1], -1).max(-1)
    m = np.abs(ref).reshape(ref.shape[0], ref.shape[1], -1).max(-1)
    m = np.where(m == 0, 1.0, m)
    return float((d / m).max())


def y_headwise_max_rel(y: torch.Tensor, ref: np.ndarray, cu) -> float:
    """Per (sequence, head) normwise error of fp32 outputs."""
    yv = to_f64(y)
    worst = 0.0
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        if b == a:
            continue
        d = np.abs(yv[a:b] - ref[a:b]).max(axis=(0, 2))
        m = np.abs(ref[a:b]).max(axis=(0, 2))
        worst = max(worst, float((d / np.where(m == 0, 1.0, m)).max()))
    return worst


def split_lengths(T: int, step: int):
    """[step|...]: calls of `step` tokens, the last one takes the rest."""
    out, t = [], 0
    while t < T:
        out.append(min(step, T - t))
        t += step
    return out


def cache_consistent(cache) -> bool:
    """The cache's bf16 state copy is the fp32 state rounded to nearest even
    (torch's float32 -> bfloat16 conversion), and the decode bookkeeping
    counters are back to zero."""
    return (same_bits(cache.state_bf_rowmajor(), cache.state.to(torch.bfloat16))
            and int(cache.work.abs().sum()) == 0)


# ---- element-wise bounds for bf16 outputs ----------------------------------
#
# The matrix-core engine rounds two operands of the chunk arithmetic to bf16
# (unit roundoff u = 2^-8, nearest even): the read-out copy of the chunk
# start state and each intra-chunk weight m_ts; every other step is fp32
# (accumulation, decays, the hi/lo-split state update, carried at ~2^-16).
# With mag, rms and state_row from oracle.bounds (exact fp64 quantities of
# the same chunk grid), and v the fp32 value before the final rounding:
#   |v - y_ref| <= (1 + 1/8) u mag + 1.02 eps_S state_row
#     (u mag: one relative rounding of at most u per term; the extra u/8
#     covers the fp32 steps -- sums of at most 256 products, exponents of
#     in-chunk decays below ~1000 -- and eps_S state_row the fp32 state's own
#     error, at most the 1e-4 per-head tolerance the states are held to);
#   |y - y_ref| <= u |y_ref| + (1 + u) |v - y_ref|       (the bf16 store)
# which is the hard bound. Under the probabilistic model of rounding
# (independent mean-zero errors, Higham and Mary 2019, Theorem 2.4) the two
# bf16 roundings contribute at most LAMBDA u rms instead of u mag, except
# with probability 2 exp(-LAMBDA^2 / 2) = 4.6e-11 per element; the fp32
# steps keep the deterministic u mag / 8.
U_BF16 = 2.0 ** -8
LAMBDA = 7.0
STATE_EPS = 1e-4


def error_scales(pr, seqs=None, init=None):
    """oracle.bounds scales of the problem's outputs (sequences `seqs`)."""
    from oracle.bounds import chunk_error_scales
    x, dt, B, C = pr.tok.f64()
    return chunk_error_scales(x, dt, pr.hp.A, B, C, pr.cu, pr.shape.chunk_size, D=pr.hp.D,
                              dt_bias=pr.hp.dt_bias, dt_softplus=pr.shape.dt_softplus,
                              init=init, seqs=seqs)


def chunk_rows(cu, Q):
    """For each sequence of a pack, the rows of its full chunks in the
    prefill's chunk_states: [(s, c, row)]."""
    cu = np.asarray(cu)
    out, row = [], 0
    for s in range(cu.size - 1):
        for c in range(int(cu[s + 1] - cu[s]) // Q):
            out.append((s, c, row))
            row += 1
    return out


def check_bf16(y, ref_y, sc, spans, rows=None, label=""):
    """Element-wise hard and probabilistic bounds, and the per-(sequence,
    head) mean relative error <= 0.3 %. y: the GPU outputs of the checked
    rows; ref_y and the scales sc (oracle.bounds) cover the problem's rows,
    of which `rows` (default: all) are the ones in y; spans are the (start,
    end) ranges of y's rows that belong to one sequence each. Prints the
    worst ratios and returns them."""
    rows = slice(None) if rows is None else rows
    yv = to_f64(y)
    ref = ref_y[rows]
    d = np.abs(yv - ref)
    mag, rms = sc.mag[rows], sc.rms[rows]
    assert mag.shape == d.shape
    base = U_BF16 * np.abs(ref) + 1.02 * STATE_EPS * sc.state_row[rows][..., None]
    det = (1 + U_BF16) * 0.125 * U_BF16 * mag
    hard = base + (1 + U_BF16) * U_BF16 * mag + det
    stat = base + (1 + U_BF16) * LAMBDA * U_BF16 * rms + det
    hard_ratio = float((d / hard).max())
    # in units of u rms, what is left after the deterministic parts
    excess = float(((d - base - det) / ((1 + U_BF16) * U_BF16 * rms)).max())
    worst_mean = 0.0
    for a, b in spans:
        if b == a:
            continue
        num = d[a:b].mean(axis=(0, 2))
        den = np.abs(ref[a:b]).mean(axis=(0, 2))
        worst_mean = max(worst_mean, float((num / den).max()))
    print(f"{label} bf16 element bounds: hard {hard_ratio:.3f} of the bound, "
          f"probabilistic {excess:.2f} u rms (limit {LAMBDA}), "
          f"worst (seq, head) mean {100 * worst_mean:.4f} %", flush=True)
    assert np.all(d <= hard), f"{label}: hard element bound exceeded ({hard_ratio:.3f})"
    assert np.all(d <= stat), f"{label}: probabilistic element bound exceeded ({excess:.2f})"
    assert worst_mean <= 3e-3, f"{label}: (seq, head) mean {worst_mean:.5f}"
    return hard_ratio, excess, worst_mean


def seq_spans(cu):
    cu = np.asarray(cu)
    return [(int(cu[s]), int(cu[s + 1])) for s in range(cu.size - 1)]


def offset_invariant(cache, lengths, Q, states) -> bool:
    """The cache's offset invariant after sequences of the given lengths
    were committed to slots 0.. in order (the invariant the prefix-cache
    poisoning fix asserts directly in its regression test, here for exact
    replay): every boundary sits on the chunk grid at floor(len / Q) * Q,
    holds bit for bit the single-shot state at that position (`states`), and
    the buffer holds the len % Q tokens after it."""
    lengths = np.asarray(lengths)
    bp = cache.boundary_pos.cpu().numpy()[:lengths.size]
    bl = cache.buf_len.cpu().numpy()[:lengths.size]
    return bool(np.all(bp % Q == 0) and np.array_equal(bp, (lengths // Q) * Q)
                and np.array_equal(bl, lengths % Q)
                and same_bits(cache.state[:lengths.size], states))

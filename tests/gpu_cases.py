"""Shared helpers for the GPU tests: seeded problems on the device, the
oracle's view of the same values, and the tolerance metrics.

Tolerances (written in the tests that use them):
  bf16 outputs: mean|y - y_ref| / mean|y_ref| <= 0.3 %, over all outputs of
  a run, in float64 (the oracle is not rounded, so the 0.141 % bf16 floor is
  part of the budget).
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

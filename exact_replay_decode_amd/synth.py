"""Seeded synthetic inputs for the Mamba2 SSD scan.

This module is shared by the tests, the bench and the smoke check. It
holds the input recipe only and none of the scan's arithmetic: it draws
numbers, rounds them to the storage dtype, and converts storage back to
float64 exactly.

Value distributions follow the kernel-level evidence setup of the vLLM RFC
"Mamba2: exact-replay decode so that prefill, chunked prefill and decode
produce identical bits" (section 2, preamble of the evidence list): A in
[-16, -1], softplus(dt_bias) in [1e-3, 1e-1] (log-uniform here), raw dt
drawn as 0.5 * N(0, 1), x / B / C drawn N(0, 1), D uniform in [0.5, 1.5].

bf16 values are stored as uint16 bit patterns (round to nearest even from
float32; the float64 draw is first rounded to float32). Every consumer
reads the stored values, so the double rounding is irrelevant to parity.
"""
from __future__ import annotations

import dataclasses

import numpy as np

IO_DTYPES = ("bf16", "f32")


def bf16_bits_from_f64(a: np.ndarray) -> np.ndarray:
    """Round float64 -> float32 (RNE) -> bf16 (RNE); returns uint16 bits."""
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    return r


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float64."""
    u = np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def store(a64: np.ndarray, dtype: str) -> np.ndarray:
    """Round a float64 array to its storage form (uint16 bits or float32)."""
    if dtype == "bf16":
        return bf16_bits_from_f64(a64)
    if dtype == "f32":
        return np.asarray(a64, dtype=np.float64).astype(np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


def widen(stored: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of a stored array."""
    if dtype == "bf16":
        return bf16_bits_to_f64(stored)
    if dtype == "f32":
        return np.asarray(stored, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


@dataclasses.dataclass
class HeadParams:
    """Per-head parameters, all float32 (the scan reads them as float32)."""
    A: np.ndarray        # [H], negative
    D: np.ndarray        # [H]
    dt_bias: np.ndarray  # [H]


def make_head_params(H: int, seed: int) -> HeadParams:
    rng = np.random.default_rng([seed, 0xA11CE])
    A = -rng.uniform(1.0, 16.0, size=H)
    # target softplus(dt_bias) = u, u log-uniform in [1e-3, 1e-1]; the
    # inverse of softplus is log(expm1(u)).
    u = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), size=H))
    dt_bias = np.log(np.expm1(u))
    D = rng.uniform(0.5, 1.5, size=H)
    return HeadParams(A=A.astype(np.float32), D=D.astype(np.float32),
                      dt_bias=dt_bias.astype(np.float32))


@dataclasses.dataclass
class Tokens:
    """Token-major inputs for one stream of T tokens, in storage form."""
    x: np.ndarray   # [T, H, P]
    dt: np.ndarray  # [T, H]   raw dt (before bias and softplus)
    B: np.ndarray   # [T, G, N]
    C: np.ndarray   # [T, G, N]
    io_dtype: str
    dt_dtype: str

    @property
    def T(self) -> int:
        return self.x.shape[0]

    def slice(self, a: int, b: int) -> "Tokens":
        return Tokens(self.x[a:b], self.dt[a:b], self.B[a:b], self.C[a:b],
                      self.io_dtype, self.dt_dtype)

    def f64(self):
        """(x, dt, B, C) as exact float64 arrays."""
        return (widen(self.x, self.io_dtype), widen(self.dt, self.dt_dtype),
                widen(self.B, self.io_dtype), widen(self.C, self.io_dtype))


def make_tokens(T: int, H: int, G: int, P: int, N: int, seed: int,
                stream: int = 0, io_dtype: str = "bf16",
                dt_dtype: str | None = None) -> Tokens:
    """Draw one token stream. (seed, stream) fixes the values, so stream i of
    a batch is the same array whatever the batch it is drawn for."""
    dt_dtype = dt_dtype or io_dtype
    rng = np.random.default_rng([seed, stream, 0x5EED])
    x = rng.standard_normal((T, H, P))
    dt = 0.5 * rng.standard_normal((T, H))
    Bm = rng.standard_normal((T, G, N))
    Cm = rng.standard_normal((T, G, N))
    return Tokens(store(x, io_dtype), store(dt, dt_dtype), store(Bm, io_dtype),
                  store(Cm, io_dtype), io_dtype, dt_dtype)


def concat(parts: list[Tokens]) -> Tokens:
    """Pack token streams back to back (varlen packing)."""
    p0 = parts[0]
    return Tokens(np.concatenate([p.x for p in parts]),
                  np.concatenate([p.dt for p in parts]),
                  np.concatenate([p.B for p in parts]),
                  np.concatenate([p.C for p in parts]),
                  p0.io_dtype, p0.dt_dtype)


def cu_seqlens(lengths) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, dtype=np.int64))]).astype(np.int32)


def replay_prefix_lengths(batch: int, chunk_size: int, seed: int) -> np.ndarray:
    """Prefix lengths for the batched decode workload: chunk_size + k_i with
    k_i uniform in [0, chunk_size), so every sequence holds a non-zero
    boundary state and k_i buffered tokens."""
    rng = np.random.default_rng([seed, 0xDEC0DE])
    return chunk_size + rng.integers(0, chunk_size, size=batch)


def make_tokens_torch(T: int, H: int, G: int, P: int, N: int, seed: int, device,
                      io_dtype: str = "bf16", dt_dtype: str | None = None):
    """Device-side draw of the same distributions for large workloads:
    x, B, C ~ N(0, 1) and raw dt ~ 0.5 N(0, 1), drawn in float32 by torch's
    generator on `device` and rounded to the storage dtype (round to nearest
    even). Returns torch tensors (x[T,H,P], dt[T,H], B[T,G,N], C[T,G,N]).
    Consumers that need float64 copies read these tensors back exactly."""
    import torch
    dt_dtype = dt_dtype or io_dtype
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32}
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1_000_003 + 0x5EED)
    x = torch.randn((T, H, P), generator=g, device=device).to(tdt[io_dtype])
    dt = (0.5 * torch.randn((T, H), generator=g, device=device)).to(tdt[dt_dtype])
    Bm = torch.randn((T, G, N), generator=g, device=device).to(tdt[io_dtype])
    Cm = torch.randn((T, G, N), generator=g, device=device).to(tdt[io_dtype])
    return x, dt, Bm, Cm


@dataclasses.dataclass
class ConvParams:
    """Depthwise conv taps and bias of the conv before the scan, float32
    holding bf16-representable values (bf16 model weights, promoted)."""
    weight: np.ndarray   # [conv_dim, W]
    bias: np.ndarray     # [conv_dim]


def make_conv_params(conv_dim: int, W: int, seed: int) -> ConvParams:
    """Taps and bias uniform in [-1/sqrt(W), 1/sqrt(W)] (fan-in init of a
    depthwise conv with W taps), rounded to bf16."""
    rng = np.random.default_rng([seed, W, 0xC0DE])
    lim = 1.0 / np.sqrt(W)
    w = widen(store(rng.uniform(-lim, lim, size=(conv_dim, W)), "bf16"), "bf16")
    b = widen(store(rng.uniform(-lim, lim, size=conv_dim), "bf16"), "bf16")
    return ConvParams(weight=w.astype(np.float32), bias=b.astype(np.float32))


def make_xbc(T: int, conv_dim: int, seed: int, stream: int = 0,
             io_dtype: str = "bf16") -> np.ndarray:
    """Conv input xBC [T, conv_dim] ~ N(0, 1) in storage form; (seed, stream)
    fixes the values."""
    rng = np.random.default_rng([seed, stream, 0xBC])
    return store(rng.standard_normal((T, conv_dim)), io_dtype)


def make_xbc_torch(T: int, conv_dim: int, seed: int, device, io_dtype: str = "bf16"):
    """Device-side draw of xBC ~ N(0, 1) for large workloads (float32 draw
    by torch's generator, rounded to the storage dtype)."""
    import torch
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32}
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1_000_003 + 0xBC)
    return torch.randn((T, conv_dim), generator=g, device=device).to(tdt[io_dtype])

"""Python binding of libssd_replay.so over torch tensors.

Argument marshalling only: tensors are checked for device, dtype, layout and
size (the C ABI cannot see extents), then their data pointers and the
current HIP stream are handed to the library. Every step of the scan runs in
the library's kernels; torch only owns memory and streams. Outputs that the
caller does not pass are allocated with torch.empty.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import numpy as np
import torch

from . import _lib

_DT = {"bf16": torch.bfloat16, "f32": torch.float32}
_CODE = {"bf16": _lib.SSD_BF16, "f32": _lib.SSD_F32}


@dataclass(frozen=True)
class Shape:
    """Problem shape: heads H, B/C groups G, head dim P, state size N, chunk
    size Q; storage dtypes of x/B/C/y (io) and of raw dt."""
    H: int
    G: int
    P: int
    N: int
    chunk_size: int
    io_dtype: str = "bf16"
    dt_dtype: str = "bf16"
    dt_softplus: bool = True
    state_dtype: str = "f32"

    def c(self) -> _lib.ssd_shape:
        return _lib.ssd_shape(self.H, self.G, self.P, self.N, self.chunk_size,
                              _CODE[self.io_dtype], _CODE[self.dt_dtype],
                              _CODE.get(self.state_dtype, 99), int(bool(self.dt_softplus)))

    @property
    def io(self) -> torch.dtype:
        return _DT[self.io_dtype]

    @property
    def dtt(self) -> torch.dtype:
        return _DT[self.dt_dtype]


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, name, shape, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype} != expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _opt(t, name, shape, dtype, device):
    return None if t is None else _need(t, name, shape, dtype, device)


def _cu_pair(cu_seqlens, cu_seqlens_host, device):
    if cu_seqlens_host is None:
        cu_seqlens_host = cu_seqlens
    host = np.ascontiguousarray(
        cu_seqlens_host.cpu().numpy() if isinstance(cu_seqlens_host, torch.Tensor)
        else np.asarray(cu_seqlens_host), dtype=np.int32)
    if isinstance(cu_seqlens, torch.Tensor) and cu_seqlens.device == device:
        dev = _need(cu_seqlens, "cu_seqlens", (host.size,), torch.int32, device)
    else:
        dev = torch.from_numpy(host).to(device)
    return host, dev


class ReplayCache:
    """Exact-replay cache for num_slots sequences: fp32 boundary state (and
    its bf16 copy, the read-out operand) plus the partial-chunk token buffers
    (all zeros = every slot fresh).

    With page_tokens, the buffers are pools of num_pages pages of page_tokens
    rows, and `buf_pages` [num_slots, Q / page_tokens] (int32, -1 = no page)
    says which page holds each slot's positions; the caller fills it."""

    def __init__(self, shape: Shape, num_slots: int, device="cuda", with_C: bool = False,
                 state_dtype: torch.dtype = torch.float32, _empty: bool = False,
                 page_tokens: int | None = None, num_pages: int | None = None):
        H, G, P, N, Q = shape.H, shape.G, shape.P, shape.N, shape.chunk_size
        self.shape = shape
        self.num_slots = num_slots
        self.device = torch.device(device)
        self.page_tokens = page_tokens
        self.num_pages = num_pages
        mk = torch.empty if _empty else torch.zeros
        self.state = mk((num_slots, H, P, N), dtype=state_dtype, device=self.device)
        # bf16 copy of the state in the read-out operand order [N/16, P, 16]
        self.state_bf = mk((num_slots, H, N // 16, P, 16), dtype=torch.bfloat16,
                           device=self.device)
        if page_tokens is None:
            lead = (num_slots, Q)
            self.buf_pages = None
        else:
            if not num_pages or Q % page_tokens:
                raise ValueError("paged cache: need num_pages > 0 and page_tokens dividing Q")
            lead = (num_pages, page_tokens)
            self.buf_pages = torch.full((num_slots, Q // page_tokens), -1, dtype=torch.int32,
                                        device=self.device)
        self.buf_x = mk(lead + (H, P), dtype=shape.io, device=self.device)
        self.buf_dt = mk(lead + (H,), dtype=shape.dtt, device=self.device)
        self.buf_B = mk(lead + (G, N), dtype=shape.io, device=self.device)
        self.buf_C = mk(lead + (G, N), dtype=shape.io, device=self.device) if with_C else None
        self.buf_len = mk((num_slots,), dtype=torch.int32, device=self.device)
        self.boundary_pos = mk((num_slots,), dtype=torch.int64, device=self.device)
        # decode bookkeeping, zero between calls (always allocated zeroed)
        self.work = torch.zeros((2 * num_slots + 34,), dtype=torch.int32, device=self.device)

    def struct(self) -> _lib.ssd_replay_cache:
        sd = _lib.SSD_F32 if self.state.dtype == torch.float32 else _lib.SSD_BF16
        paged = self.buf_pages is not None
        return _lib.ssd_replay_cache(
            self.state.data_ptr(), self.state_bf.data_ptr(), self.buf_x.data_ptr(),
            self.buf_dt.data_ptr(), self.buf_B.data_ptr(),
            None if self.buf_C is None else self.buf_C.data_ptr(),
            self.buf_len.data_ptr(), self.boundary_pos.data_ptr(), self.work.data_ptr(),
            self.num_slots, self.shape.chunk_size, sd,
            self.buf_pages.data_ptr() if paged else None,
            self.page_tokens if paged else 0, self.num_pages if paged else 0)

    def buffers_by_slot(self):
        """The buffers as [num_slots, Q, ...] (x, dt, B, C or None): for a paged
        cache, position j of a slot read through its page table (zeros where
        the entry is not a page)."""
        bufs = (self.buf_x, self.buf_dt, self.buf_B, self.buf_C)
        if self.buf_pages is None:
            return bufs
        pt, Q = self.page_tokens, self.shape.chunk_size
        pos = torch.arange(Q, device=self.device)
        pg = self.buf_pages.long()[:, pos // pt]                      # [slots, Q]
        ok = (pg >= 0) & (pg < self.num_pages)
        rows = torch.where(ok, pg * pt + pos % pt, torch.zeros_like(pg))
        out = []
        for t in bufs:
            if t is None:
                out.append(None)
                continue
            flat = t.reshape((-1,) + tuple(t.shape[2:]))
            g = flat[rows.reshape(-1)].reshape(rows.shape + tuple(t.shape[2:]))
            mask = ok.reshape(ok.shape + (1,) * (g.dim() - 2))
            out.append(torch.where(mask, g, torch.zeros_like(g)))
        return tuple(out)

    def state_bf_rowmajor(self) -> torch.Tensor:
        """The bf16 state copy as [num_slots, H, P, N]."""
        s = self.state_bf
        return s.permute(0, 1, 3, 2, 4).reshape(s.shape[0], s.shape[1], s.shape[3], -1)

    def refresh(self, stream=None) -> None:
        """Rebuild the bf16 state copy after writing `state` directly."""
        c, sh = self.struct(), self.shape.c()
        rc = _lib.load().ssd_replay_cache_refresh(ctypes.byref(sh), ctypes.byref(c),
                                                  _stream(stream))
        _lib.check(rc, "ssd_replay_cache_refresh")

    def tensors(self):
        return [t for t in (self.state, self.state_bf, self.buf_x, self.buf_dt, self.buf_B,
                            self.buf_C, self.buf_len, self.boundary_pos, self.work,
                            self.buf_pages)
                if t is not None]

    def clone(self) -> "ReplayCache":
        c = ReplayCache(self.shape, self.num_slots, self.device, self.buf_C is not None,
                        self.state.dtype, _empty=True, page_tokens=self.page_tokens,
                        num_pages=self.num_pages)
        for dst, src in zip(c.tensors(), self.tensors()):
            dst.copy_(src)
        return c

    def copy_from(self, other: "ReplayCache") -> None:
        for dst, src in zip(self.tensors(), other.tensors()):
            dst.copy_(src)


def ssd_replay_cache_bytes(shape: Shape, num_slots: int, with_C: bool = True) -> int:
    c = shape.c()
    return int(_lib.load().ssd_replay_cache_bytes(ctypes.byref(c), num_slots, int(with_C)))


def ssd_replay_page_bytes(shape: Shape, page_tokens: int, with_C: bool = True) -> int:
    c = shape.c()
    return int(_lib.load().ssd_replay_page_bytes(ctypes.byref(c), page_tokens, int(with_C)))


def _slots(slot_idx, n, device):
    if slot_idx is None:
        return None
    return _need(slot_idx, "slot_idx", (n,), torch.int32, device)


def ssd_prefill_chunk_count(cu_seqlens_host, chunk_size: int) -> int:
    """Rows of the prefill's chunk_states for a pack: its full chunks."""
    host = np.ascontiguousarray(np.asarray(cu_seqlens_host), dtype=np.int32)
    n = int(_lib.load().ssd_prefill_chunk_count(host.size - 1,
                                                host.ctypes.data_as(ctypes.c_void_p),
                                                int(chunk_size)))
    if n < 0:
        raise ValueError("ssd_prefill_chunk_count: bad cu_seqlens or chunk size")
    return n


def ssd_prefill_varlen(shape: Shape, cu_seqlens, x, dt, A, B, C, D=None, dt_bias=None,
                       init_state=None, y=None, final_state=None, boundary_state=None,
                       cu_seqlens_host=None, want_final=True, want_boundary=True, stream=None,
                       chunk_states=None, want_chunk_states=False):
    """Chunked scan of a varlen pack from init_state (None = zeros).
    Returns (y, final_state, boundary_state), and chunk_states as a fourth
    item with want_chunk_states (allocated unless passed: [F, H, P, N], the
    state after each full chunk of each sequence, sequences in order)."""
    dev = x.device
    H, G, P, N = shape.H, shape.G, shape.P, shape.N
    host, cu = _cu_pair(cu_seqlens, cu_seqlens_host, dev)
    S, T = host.size - 1, int(x.shape[0])
    _need(x, "x", (T, H, P), shape.io, dev)
    _need(dt, "dt", (T, H), shape.dtt, dev)
    _need(B, "B", (T, G, N), shape.io, dev)
    _need(C, "C", (T, G, N), shape.io, dev)
    _need(A, "A", (H,), torch.float32, dev)
    _opt(D, "D", (H,), torch.float32, dev)
    _opt(dt_bias, "dt_bias", (H,), torch.float32, dev)
    _opt(init_state, "init_state", (S, H, P, N), torch.float32, dev)
    y = torch.empty((T, H, P), dtype=shape.io, device=dev) if y is None else \
        _need(y, "y", (T, H, P), shape.io, dev)
    if final_state is None and want_final:
        final_state = torch.empty((S, H, P, N), dtype=torch.float32, device=dev)
    if boundary_state is None and want_boundary:
        boundary_state = torch.empty((S, H, P, N), dtype=torch.float32, device=dev)
    _opt(final_state, "final_state", (S, H, P, N), torch.float32, dev)
    _opt(boundary_state, "boundary_state", (S, H, P, N), torch.float32, dev)
    if chunk_states is not None or want_chunk_states:
        F = ssd_prefill_chunk_count(host, shape.chunk_size)
        if chunk_states is None:
            chunk_states = torch.empty((F, H, P, N), dtype=torch.float32, device=dev)
        _need(chunk_states, "chunk_states", (F, H, P, N), torch.float32, dev)
    sh = shape.c()
    rc = _lib.load().ssd_prefill_varlen(
        ctypes.byref(sh), S, T, host.ctypes.data_as(ctypes.c_void_p), _ptr(cu), _ptr(x),
        _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(dt_bias), _ptr(init_state), _ptr(y),
        _ptr(final_state), _ptr(boundary_state), _ptr(chunk_states), None, 0, _stream(stream))
    _lib.check(rc, "ssd_prefill_varlen")
    if want_chunk_states:
        return y, final_state, boundary_state, chunk_states
    return y, final_state, boundary_state


def ssd_commit_boundary(shape: Shape, cache: ReplayCache, cu_seqlens, x, dt, B, C,
                        boundary_state, slot_idx=None, cu_seqlens_host=None, stream=None):
    """Store a fresh prefill's boundary state and trailing partial chunk in
    the cache slots."""
    dev = cache.device
    H, G, P, N = shape.H, shape.G, shape.P, shape.N
    host, cu = _cu_pair(cu_seqlens, cu_seqlens_host, dev)
    S, T = host.size - 1, int(x.shape[0])
    _need(x, "x", (T, H, P), shape.io, dev)
    _need(dt, "dt", (T, H), shape.dtt, dev)
    _need(B, "B", (T, G, N), shape.io, dev)
    _need(C, "C", (T, G, N), shape.io, dev)
    _need(boundary_state, "boundary_state", (S, H, P, N), torch.float32, dev)
    sl = _slots(slot_idx, S, dev)
    sh, cs = shape.c(), cache.struct()
    rc = _lib.load().ssd_commit_boundary(
        ctypes.byref(sh), S, T, host.ctypes.data_as(ctypes.c_void_p), _ptr(cu), _ptr(sl),
        _ptr(x), _ptr(dt), _ptr(B), _ptr(C), _ptr(boundary_state), ctypes.byref(cs),
        _stream(stream))
    _lib.check(rc, "ssd_commit_boundary")


def ssd_replay_prefill(shape: Shape, cache: ReplayCache, cu_seqlens, x, dt, B, C, A, D=None,
                       dt_bias=None, slot_idx=None, y=None, cu_seqlens_host=None, stream=None):
    """Exact-replay (chunked) prefill: resume every sequence at its slot's
    boundary. Returns y for the new tokens."""
    dev = cache.device
    H, G, P, N = shape.H, shape.G, shape.P, shape.N
    host, cu = _cu_pair(cu_seqlens, cu_seqlens_host, dev)
    S, T = host.size - 1, int(x.shape[0])
    _need(x, "x", (T, H, P), shape.io, dev)
    _need(dt, "dt", (T, H), shape.dtt, dev)
    _need(B, "B", (T, G, N), shape.io, dev)
    _need(C, "C", (T, G, N), shape.io, dev)
    _need(A, "A", (H,), torch.float32, dev)
    _opt(D, "D", (H,), torch.float32, dev)
    _opt(dt_bias, "dt_bias", (H,), torch.float32, dev)
    sl = _slots(slot_idx, S, dev)
    y = torch.empty((T, H, P), dtype=shape.io, device=dev) if y is None else \
        _need(y, "y", (T, H, P), shape.io, dev)
    sh, cs = shape.c(), cache.struct()
    rc = _lib.load().ssd_replay_prefill(
        ctypes.byref(sh), ctypes.byref(cs), S, T, host.ctypes.data_as(ctypes.c_void_p),
        _ptr(cu), _ptr(sl), _ptr(x), _ptr(dt), _ptr(B), _ptr(C), _ptr(A), _ptr(D),
        _ptr(dt_bias), _ptr(y), _stream(stream))
    _lib.check(rc, "ssd_replay_prefill")
    return y


def ssd_replay_verify(shape: Shape, cache: ReplayCache, cu_seqlens, x, dt, B, C, A, D=None,
                      dt_bias=None, slot_idx=None, y=None, cu_seqlens_host=None, stream=None):
    """Speculative verification: outputs of every draft token, replayed after
    each slot's committed tokens; the cache is not changed. Returns y."""
    dev = cache.device
    H, G, P, N = shape.H, shape.G, shape.P, shape.N
    host, cu = _cu_pair(cu_seqlens, cu_seqlens_host, dev)
    S, T = host.size - 1, int(x.shape[0])
    _need(x, "x", (T, H, P), shape.io, dev)
    _need(dt, "dt", (T, H), shape.dtt, dev)
    _need(B, "B", (T, G, N), shape.io, dev)
    _need(C, "C", (T, G, N), shape.io, dev)
    _need(A, "A", (H,), torch.float32, dev)
    _opt(D, "D", (H,), torch.float32, dev)
    _opt(dt_bias, "dt_bias", (H,), torch.float32, dev)
    sl = _slots(slot_idx, S, dev)
    y = torch.empty((T, H, P), dtype=shape.io, device=dev) if y is None else \
        _need(y, "y", (T, H, P), shape.io, dev)
    sh, cs = shape.c(), cache.struct()
    rc = _lib.load().ssd_replay_verify(
        ctypes.byref(sh), ctypes.byref(cs), S, T, host.ctypes.data_as(ctypes.c_void_p),
        _ptr(cu), _ptr(sl), _ptr(x), _ptr(dt), _ptr(B), _ptr(C), _ptr(A), _ptr(D),
        _ptr(dt_bias), _ptr(y), _stream(stream))
    _lib.check(rc, "ssd_replay_verify")
    return y


def ssd_replay_accept(shape: Shape, cache: ReplayCache, cu_seqlens, accepted, x, dt, B, C, A,
                      dt_bias=None, slot_idx=None, cu_seqlens_host=None, stream=None):
    """Commit the first accepted[s] drafts of each sequence (accepted: int32
    device tensor [S]); the drafts are the ones given to the verification."""
    dev = cache.device
    H, G, P, N = shape.H, shape.G, shape.P, shape.N
    host, cu = _cu_pair(cu_seqlens, cu_seqlens_host, dev)
    S, T = host.size - 1, int(x.shape[0])
    _need(accepted, "accepted", (S,), torch.int32, dev)
    _need(x, "x", (T, H, P), shape.io, dev)
    _need(dt, "dt", (T, H), shape.dtt, dev)
    _need(B, "B", (T, G, N), shape.io, dev)
    _need(C, "C", (T, G, N), shape.io, dev)
    _need(A, "A", (H,), torch.float32, dev)
    _opt(dt_bias, "dt_bias", (H,), torch.float32, dev)
    sl = _slots(slot_idx, S, dev)
    sh, cs = shape.c(), cache.struct()
    rc = _lib.load().ssd_replay_accept(
        ctypes.byref(sh), ctypes.byref(cs), S, T, host.ctypes.data_as(ctypes.c_void_p),
        _ptr(cu), _ptr(sl), _ptr(accepted), _ptr(x), _ptr(dt), _ptr(B), _ptr(C), _ptr(A),
        _ptr(dt_bias), _stream(stream))
    _lib.check(rc, "ssd_replay_accept")


def ssd_replay_decode(shape: Shape, cache: ReplayCache, x, dt, B, C, A, D=None, dt_bias=None,
                      slot_idx=None, y=None, stream=None, static_work=False):
    """One exact-replay decode step for x.shape[0] sequences. static_work:
    call ssd_replay_decode_static, whose bookkeeping lives in the library's
    own per-GPU array (nothing is allocated on the device; the cache's work
    array is not passed)."""
    dev = cache.device
    H, G, P, N = shape.H, shape.G, shape.P, shape.N
    nb = int(x.shape[0])
    _need(x, "x", (nb, H, P), shape.io, dev)
    _need(dt, "dt", (nb, H), shape.dtt, dev)
    _need(B, "B", (nb, G, N), shape.io, dev)
    _need(C, "C", (nb, G, N), shape.io, dev)
    _need(A, "A", (H,), torch.float32, dev)
    _opt(D, "D", (H,), torch.float32, dev)
    _opt(dt_bias, "dt_bias", (H,), torch.float32, dev)
    sl = _slots(slot_idx, nb, dev)
    y = torch.empty((nb, H, P), dtype=shape.io, device=dev) if y is None else \
        _need(y, "y", (nb, H, P), shape.io, dev)
    sh, cs = shape.c(), cache.struct()
    lib = _lib.load()
    if static_work:
        cs.work = None
    fn = lib.ssd_replay_decode_static if static_work else lib.ssd_replay_decode
    rc = fn(ctypes.byref(sh), ctypes.byref(cs), nb, _ptr(sl), _ptr(x), _ptr(dt), _ptr(B), _ptr(C),
            _ptr(A), _ptr(D), _ptr(dt_bias), _ptr(y), _stream(stream))
    _lib.check(rc, "ssd_replay_decode_static" if static_work else "ssd_replay_decode")
    return y


def ssd_replay_decode_conv(shape: Shape, cache: ReplayCache, xBC, weight, conv_state, dt, A,
                           D=None, dt_bias=None, bias=None, slot_idx=None, activation=True,
                           out=None, y=None, stream=None):
    """The causal conv's decode form and one exact-replay decode step in one
    launch (ssd_conv1d_update, then ssd_replay_decode on its outputs, bit
    for bit): xBC [batch, conv_dim] of the new tokens, conv_state
    [num_slots, conv_dim, W-1] indexed by the cache's slots. Returns
    (y, (x, B, C))."""
    dev = cache.device
    H, P = shape.H, shape.P
    nb = int(xBC.shape[0])
    cd = conv_dim(shape)
    _need(xBC, "xBC", (nb, cd), shape.io, dev)
    W = int(weight.shape[1]) if weight.dim() == 2 else -1
    _need(weight, "weight", (cd, W), torch.float32, dev)
    _opt(bias, "bias", (cd,), torch.float32, dev)
    _need(conv_state, "conv_state", (cache.num_slots, cd, W - 1), shape.io, dev)
    _need(dt, "dt", (nb, H), shape.dtt, dev)
    _need(A, "A", (H,), torch.float32, dev)
    _opt(D, "D", (H,), torch.float32, dev)
    _opt(dt_bias, "dt_bias", (H,), torch.float32, dev)
    sl = _slots(slot_idx, nb, dev)
    x, B, C = _conv_outputs(shape, nb, dev, out)
    y = torch.empty((nb, H, P), dtype=shape.io, device=dev) if y is None else \
        _need(y, "y", (nb, H, P), shape.io, dev)
    sh, cs = shape.c(), cache.struct()
    rc = _lib.load().ssd_replay_decode_conv(
        ctypes.byref(sh), ctypes.byref(cs), nb, _ptr(sl), W, int(bool(activation)), _ptr(xBC),
        _ptr(weight), _ptr(bias), _ptr(conv_state), _ptr(x), _ptr(B), _ptr(C), _ptr(dt),
        _ptr(A), _ptr(D), _ptr(dt_bias), _ptr(y), _stream(stream))
    _lib.check(rc, "ssd_replay_decode_conv")
    return y, (x, B, C)


def conv_dim(shape: Shape) -> int:
    """Channels of the conv before the scan: x | B | C."""
    return shape.H * shape.P + 2 * shape.G * shape.N


def _conv_outputs(shape: Shape, T: int, dev, out):
    if out is None:
        return (torch.empty((T, shape.H, shape.P), dtype=shape.io, device=dev),
                torch.empty((T, shape.G, shape.N), dtype=shape.io, device=dev),
                torch.empty((T, shape.G, shape.N), dtype=shape.io, device=dev))
    x, B, C = out
    return (_need(x, "x", (T, shape.H, shape.P), shape.io, dev),
            _need(B, "B", (T, shape.G, shape.N), shape.io, dev),
            _need(C, "C", (T, shape.G, shape.N), shape.io, dev))


def ssd_conv1d_varlen(shape: Shape, cu_seqlens, xBC, weight, bias=None, conv_state=None,
                      slot_idx=None, activation=True, out=None, cu_seqlens_host=None,
                      stream=None):
    """Causal depthwise conv1d (prefill form) over a varlen pack of xBC
    [T, conv_dim]; conv_state [slots, conv_dim, W-1] is read and updated in
    place (None: zero history). Returns (x, B, C), the scan's inputs."""
    dev = xBC.device
    host, cu = _cu_pair(cu_seqlens, cu_seqlens_host, dev)
    S, T = host.size - 1, int(xBC.shape[0])
    cd = conv_dim(shape)
    _need(xBC, "xBC", (T, cd), shape.io, dev)
    W = int(weight.shape[1]) if weight.dim() == 2 else -1
    _need(weight, "weight", (cd, W), torch.float32, dev)
    _opt(bias, "bias", (cd,), torch.float32, dev)
    ns = 0
    if conv_state is not None:
        ns = int(conv_state.shape[0])
        _need(conv_state, "conv_state", (ns, cd, W - 1), shape.io, dev)
    sl = _slots(slot_idx, S, dev)
    x, B, C = _conv_outputs(shape, T, dev, out)
    sh = shape.c()
    rc = _lib.load().ssd_conv1d_varlen(
        ctypes.byref(sh), W, int(bool(activation)), S, T, host.ctypes.data_as(ctypes.c_void_p),
        _ptr(cu), _ptr(sl), ns, _ptr(xBC), _ptr(weight), _ptr(bias), _ptr(conv_state),
        _ptr(x), _ptr(B), _ptr(C), _stream(stream))
    _lib.check(rc, "ssd_conv1d_varlen")
    return x, B, C


def ssd_conv1d_update(shape: Shape, xBC, weight, conv_state, bias=None, slot_idx=None,
                      activation=True, out=None, stream=None):
    """Causal conv1d, decode form: one token per row of xBC [batch, conv_dim];
    conv_state [slots, conv_dim, W-1] updated in place. Returns (x, B, C)."""
    dev = xBC.device
    nb = int(xBC.shape[0])
    cd = conv_dim(shape)
    _need(xBC, "xBC", (nb, cd), shape.io, dev)
    W = int(weight.shape[1]) if weight.dim() == 2 else -1
    _need(weight, "weight", (cd, W), torch.float32, dev)
    _opt(bias, "bias", (cd,), torch.float32, dev)
    ns = int(conv_state.shape[0])
    _need(conv_state, "conv_state", (ns, cd, W - 1), shape.io, dev)
    sl = _slots(slot_idx, nb, dev)
    x, B, C = _conv_outputs(shape, nb, dev, out)
    sh = shape.c()
    rc = _lib.load().ssd_conv1d_update(
        ctypes.byref(sh), W, int(bool(activation)), nb, _ptr(sl), ns, _ptr(xBC), _ptr(weight),
        _ptr(bias), _ptr(conv_state), _ptr(x), _ptr(B), _ptr(C), _stream(stream))
    _lib.check(rc, "ssd_conv1d_update")
    return x, B, C


def ssm_state_update(shape: Shape, state, x, dt, B, C, A, D=None, dt_bias=None, slot_idx=None,
                     y=None, stream=None):
    """One recurrent selective-state update for x.shape[0] sequences; state
    [num_slots,H,P,N] (shape.state_dtype: fp32 or bf16) is updated in
    place."""
    dev = state.device
    H, G, P, N = shape.H, shape.G, shape.P, shape.N
    nb = int(x.shape[0])
    ns = int(state.shape[0])
    _need(state, "state", (ns, H, P, N), _DT[shape.state_dtype], dev)
    _need(x, "x", (nb, H, P), shape.io, dev)
    _need(dt, "dt", (nb, H), shape.dtt, dev)
    _need(B, "B", (nb, G, N), shape.io, dev)
    _need(C, "C", (nb, G, N), shape.io, dev)
    _need(A, "A", (H,), torch.float32, dev)
    _opt(D, "D", (H,), torch.float32, dev)
    _opt(dt_bias, "dt_bias", (H,), torch.float32, dev)
    sl = _slots(slot_idx, nb, dev)
    y = torch.empty((nb, H, P), dtype=shape.io, device=dev) if y is None else \
        _need(y, "y", (nb, H, P), shape.io, dev)
    sh = shape.c()
    rc = _lib.load().ssm_state_update(
        ctypes.byref(sh), nb, ns, _ptr(sl), _ptr(state), _ptr(x), _ptr(dt), _ptr(A), _ptr(B),
        _ptr(C), _ptr(D), _ptr(dt_bias), _ptr(y), _stream(stream))
    _lib.check(rc, "ssm_state_update")
    return y


def ssm_state_update_varlen(shape: Shape, state, cu_seqlens, x, dt, B, C, A, D=None,
                            dt_bias=None, slot_idx=None, y=None, cu_seqlens_host=None,
                            stream=None):
    """Multi-token recurrent update over a varlen pack (packed-history
    recovery): sequence s advances state[slot_idx[s]] token by token with
    the state rounded to shape.state_dtype after each token. Returns y."""
    dev = state.device
    H, G, P, N = shape.H, shape.G, shape.P, shape.N
    host, cu = _cu_pair(cu_seqlens, cu_seqlens_host, dev)
    S, T = host.size - 1, int(x.shape[0])
    ns = int(state.shape[0])
    _need(state, "state", (ns, H, P, N), _DT[shape.state_dtype], dev)
    _need(x, "x", (T, H, P), shape.io, dev)
    _need(dt, "dt", (T, H), shape.dtt, dev)
    _need(B, "B", (T, G, N), shape.io, dev)
    _need(C, "C", (T, G, N), shape.io, dev)
    _need(A, "A", (H,), torch.float32, dev)
    _opt(D, "D", (H,), torch.float32, dev)
    _opt(dt_bias, "dt_bias", (H,), torch.float32, dev)
    sl = _slots(slot_idx, S, dev)
    y = torch.empty((T, H, P), dtype=shape.io, device=dev) if y is None else \
        _need(y, "y", (T, H, P), shape.io, dev)
    sh = shape.c()
    rc = _lib.load().ssm_state_update_varlen(
        ctypes.byref(sh), S, T, host.ctypes.data_as(ctypes.c_void_p), _ptr(cu), _ptr(sl), ns,
        _ptr(state), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(dt_bias),
        _ptr(y), _stream(stream))
    _lib.check(rc, "ssm_state_update_varlen")
    return y


def to_device(a: np.ndarray, dtype: str, device) -> torch.Tensor:
    """Storage array from synth (uint16 bf16 bits or float32) -> torch tensor."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a bf16 / fp32 tensor."""
    return t.detach().to("cpu", torch.float64).numpy()


class DecodePlan:
    """Pre-marshalled ssd_replay_decode / ssm_state_update calls for a hot
    loop: argument checks and ctypes structs are built once; each call only
    passes the step's token pointers. Inputs per step are contiguous
    [batch, ...] tensors of the planned shapes."""

    def __init__(self, shape: Shape, batch: int, A, D=None, dt_bias=None, cache=None,
                 state=None, slot_idx=None, stream=None):
        if (cache is None) == (state is None):
            raise ValueError("give exactly one of cache (replay) or state (recurrent)")
        self.shape, self.batch = shape, batch
        dev = cache.device if cache is not None else state.device
        H = shape.H
        _need(A, "A", (H,), torch.float32, dev)
        _opt(D, "D", (H,), torch.float32, dev)
        _opt(dt_bias, "dt_bias", (H,), torch.float32, dev)
        self._keep = (A, D, dt_bias, cache, state, slot_idx)
        self.device = dev
        self._sh = shape.c()
        self._lib = _lib.load()
        self._st = _stream(stream)
        self._sl = _ptr(_slots(slot_idx, batch, dev))
        self._A, self._D, self._b = _ptr(A), _ptr(D), _ptr(dt_bias)
        if cache is not None:
            if slot_idx is None and batch > cache.num_slots:
                raise ValueError("batch exceeds cache slots")
            self._cs = cache.struct()
            self._state = None
        else:
            _need(state, "state", tuple(state.shape), _DT[shape.state_dtype], dev)
            if state.dim() != 4 or tuple(state.shape[1:]) != (H, shape.P, shape.N):
                raise ValueError("state must be [num_slots, H, P, N]")
            self._state = state
            self._ns = int(state.shape[0])
            if slot_idx is None and batch > self._ns:
                raise ValueError("batch exceeds state slots")

    def check(self, x, dt, B, C, y):
        sh, dev, nb = self.shape, self.device, self.batch
        _need(x, "x", (nb, sh.H, sh.P), sh.io, dev)
        _need(dt, "dt", (nb, sh.H), sh.dtt, dev)
        _need(B, "B", (nb, sh.G, sh.N), sh.io, dev)
        _need(C, "C", (nb, sh.G, sh.N), sh.io, dev)
        _need(y, "y", (nb, sh.H, sh.P), sh.io, dev)

    def __call__(self, x, dt, B, C, y):
        """Launch one step; tensors must already satisfy check()."""
        if self._state is None:
            rc = self._lib.ssd_replay_decode(
                ctypes.byref(self._sh), ctypes.byref(self._cs), self.batch, self._sl,
                x.data_ptr(), dt.data_ptr(), B.data_ptr(), C.data_ptr(), self._A, self._D,
                self._b, y.data_ptr(), self._st)
        else:
            rc = self._lib.ssm_state_update(
                ctypes.byref(self._sh), self.batch, self._ns, self._sl, self._state.data_ptr(),
                x.data_ptr(), dt.data_ptr(), self._A, B.data_ptr(), C.data_ptr(), self._D,
                self._b, y.data_ptr(), self._st)
        if rc != 0:
            _lib.check(rc, "DecodePlan")


class ConvDecodePlan:
    """Pre-marshalled ssd_replay_decode_conv calls (the conv's decode form and
    the replay step in one launch) for a hot loop: each call passes the
    step's xBC [batch, conv_dim], raw dt, the conv outputs x, B, C and y."""

    def __init__(self, shape: Shape, batch: int, A, cache, weight, conv_state, D=None,
                 dt_bias=None, bias=None, slot_idx=None, activation=True, stream=None):
        dev = cache.device
        cd = conv_dim(shape)
        self.W = int(weight.shape[1])
        _need(weight, "weight", (cd, self.W), torch.float32, dev)
        _opt(bias, "bias", (cd,), torch.float32, dev)
        _need(conv_state, "conv_state", (cache.num_slots, cd, self.W - 1), shape.io, dev)
        _need(A, "A", (shape.H,), torch.float32, dev)
        _opt(D, "D", (shape.H,), torch.float32, dev)
        _opt(dt_bias, "dt_bias", (shape.H,), torch.float32, dev)
        if slot_idx is None and batch > cache.num_slots:
            raise ValueError("batch exceeds cache slots")
        self.shape, self.batch, self.device = shape, batch, dev
        self._keep = (A, D, dt_bias, cache, weight, conv_state, bias, slot_idx)
        self._sh, self._cs = shape.c(), cache.struct()
        self._lib = _lib.load()
        self._st = _stream(stream)
        self._sl = _ptr(_slots(slot_idx, batch, dev))
        self._args = (self.W, int(bool(activation)))
        self._w, self._b, self._cst = _ptr(weight), _ptr(bias), _ptr(conv_state)
        self._A, self._D, self._db = _ptr(A), _ptr(D), _ptr(dt_bias)

    def __call__(self, xBC, dt, x, B, C, y):
        """Launch one step; tensors of the planned shapes, contiguous."""
        rc = self._lib.ssd_replay_decode_conv(
            ctypes.byref(self._sh), ctypes.byref(self._cs), self.batch, self._sl, *self._args,
            xBC.data_ptr(), self._w, self._b, self._cst, x.data_ptr(), B.data_ptr(),
            C.data_ptr(), dt.data_ptr(), self._A, self._D, self._db, y.data_ptr(), self._st)
        if rc != 0:
            _lib.check(rc, "ConvDecodePlan")


class ConvUpdatePlan:
    """Pre-marshalled ssd_conv1d_update calls for a hot loop: each call only
    passes the step's xBC [batch, conv_dim] and the x/B/C outputs."""

    def __init__(self, shape: Shape, batch: int, weight, conv_state, bias=None, slot_idx=None,
                 activation=True, stream=None):
        dev = conv_state.device
        cd = conv_dim(shape)
        self.W = int(weight.shape[1])
        _need(weight, "weight", (cd, self.W), torch.float32, dev)
        _opt(bias, "bias", (cd,), torch.float32, dev)
        self.ns = int(conv_state.shape[0])
        _need(conv_state, "conv_state", (self.ns, cd, self.W - 1), shape.io, dev)
        if slot_idx is None and batch > self.ns:
            raise ValueError("batch exceeds conv state slots")
        self.shape, self.batch, self.device = shape, batch, dev
        self._keep = (weight, conv_state, bias, slot_idx)
        self._sh = shape.c()
        self._lib = _lib.load()
        self._st = _stream(stream)
        self._sl = _ptr(_slots(slot_idx, batch, dev))
        self._w, self._b, self._cs = _ptr(weight), _ptr(bias), _ptr(conv_state)
        self._act = int(bool(activation))

    def check(self, xBC, x, B, C):
        sh, dev, nb = self.shape, self.device, self.batch
        _need(xBC, "xBC", (nb, conv_dim(sh)), sh.io, dev)
        _conv_outputs(sh, nb, dev, (x, B, C))

    def __call__(self, xBC, x, B, C):
        """Launch one step; tensors must already satisfy check()."""
        rc = self._lib.ssd_conv1d_update(
            ctypes.byref(self._sh), self.W, self._act, self.batch, self._sl, self.ns,
            xBC.data_ptr(), self._w, self._b, self._cs, x.data_ptr(), B.data_ptr(),
            C.data_ptr(), self._st)
        if rc != 0:
            _lib.check(rc, "ConvUpdatePlan")

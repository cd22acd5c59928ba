"""Mixed-offset batches over contiguous and paged replay caches, through the
C ABI (vLLM RFC "Mamba2: exact-replay decode ...", section 6: mixed-offset
multi-request batches -- unaligned prefill splits, resumes and interleaved
decode in the same batches -- verified bitwise at the kernel level, with
contiguous and paged buffer layouts; the buffers live in the paged mamba
cache, so slot and position are indexed separately).

Every schedule is checked bit for bit against one single-shot prefill of
each whole sequence: outputs, committed boundary states, buffers and the
slot metadata. Pages are handed out only for the positions a call touches
and returned when a chunk completes, so pages move between slots.
"""
import numpy as np
import pytest
import torch

import exact_replay_decode_amd as erd
from exact_replay_decode_amd import synth
from gpu_cases import DEV, cache_consistent, make_problem, mean_rel_err, same_bits

pytestmark = pytest.mark.gpu

BF16_MEAN_REL = 3e-3


class PagePool:
    """Host-side page allocator of a paged cache: hands out pages for the
    positions a call touches, returns them when a chunk completes. Pages are
    drawn at random, so a slot's pages are scattered over the pool and reused
    by other slots."""

    def __init__(self, cache, seed):
        self.cache = cache
        self.pt = cache.page_tokens
        self.table = np.full(tuple(cache.buf_pages.shape), -1, dtype=np.int32)
        self.free = list(range(cache.num_pages))
        self.rng = np.random.default_rng(seed)

    def need(self, slot, npos):
        for i in range((npos + self.pt - 1) // self.pt):
            if self.table[slot, i] < 0:
                j = int(self.rng.integers(len(self.free)))
                self.table[slot, i] = self.free.pop(j)

    def trim(self, slot, nbuf):
        for i in range((nbuf + self.pt - 1) // self.pt, self.table.shape[1]):
            if self.table[slot, i] >= 0:
                self.free.append(int(self.table[slot, i]))
                self.table[slot, i] = -1

    def push(self):
        self.cache.buf_pages.copy_(torch.from_numpy(self.table))


def touched(nbuf, n, Q, decode):
    """Buffer positions a call with n new tokens reads or writes."""
    if decode:
        return nbuf + 1
    total = nbuf + n
    return total if total < Q else max(nbuf, total % Q)


def run_schedule(pr, caches, seed, steps_cap=400):
    """Drive every sequence of pr through a random engine schedule on each
    cache in `caches` (same calls on all). Returns per-cache outputs [T,H,P]
    and the pools."""
    Q = pr.shape.chunk_size
    lengths = np.array(pr.lengths)
    S = len(lengths)
    cu = pr.cu
    x, dt, B, C = pr.dev(None)
    rng = np.random.default_rng(seed)
    done = np.zeros(S, dtype=np.int64)
    ys = [torch.full_like(x, float("nan")) for _ in caches]
    pools = [PagePool(c, seed + 7) if c.buf_pages is not None else None for c in caches]
    for _ in range(steps_cap):
        live = np.flatnonzero(done < lengths)
        if live.size == 0:
            break
        pick = rng.permutation(live)[:int(rng.integers(1, live.size + 1))]
        decode = bool(rng.random() < 0.35)
        if decode:
            n = np.ones(len(pick), dtype=np.int64)
        else:
            # mixed: one-token entries, unaligned chunks, zero-length entries
            n = np.where(rng.random(len(pick)) < 0.3, 1, rng.integers(0, 160, len(pick)))
            n = np.minimum(n, lengths[pick] - done[pick])
        idx = np.concatenate([np.arange(cu[s] + done[s], cu[s] + done[s] + k)
                              for s, k in zip(pick, n)]).astype(np.int64)
        it = torch.from_numpy(idx).to(DEV)
        sl = torch.from_numpy(pick.astype(np.int32)).to(DEV)
        for c, pool, yv in zip(caches, pools, ys):
            if pool is not None:
                for s, k in zip(pick, n):
                    if decode or k > 0:
                        pool.need(s, touched(int(done[s] % Q), int(k), Q, decode))
                pool.push()
            if decode:
                out = erd.ssd_replay_decode(pr.shape, c, x[it], dt[it], B[it], C[it], pr.A,
                                            pr.D, pr.bias, slot_idx=sl)
            else:
                out = erd.ssd_replay_prefill(pr.shape, c, synth.cu_seqlens(n), x[it], dt[it],
                                             B[it], C[it], pr.A, pr.D, pr.bias, slot_idx=sl)
            yv[it] = out
            if pool is not None:
                for s, k in zip(pick, n):
                    pool.trim(s, int((done[s] + k) % Q))
                pool.push()
        done[pick] += n
    assert np.array_equal(done, lengths), "schedule did not finish"
    return ys, pools


def check_final(pr, cache, y, y_ss, bnd_ss):
    Q = pr.shape.chunk_size
    lengths = np.array(pr.lengths)
    x, dt, B, C = pr.dev(None)
    assert same_bits(y, y_ss)
    assert same_bits(cache.state, bnd_ss) and cache_consistent(cache)
    assert np.array_equal(cache.buf_len.cpu().numpy(), lengths % Q)
    assert np.array_equal(cache.boundary_pos.cpu().numpy(), lengths - lengths % Q)
    bx, bdt, bB, _ = cache.buffers_by_slot()
    cu = pr.cu
    for s, L in enumerate(lengths):
        k = int(L % Q)
        a = int(cu[s + 1]) - k
        assert same_bits(bx[s, :k], x[a:a + k]) and same_bits(bdt[s, :k], dt[a:a + k])
        assert same_bits(bB[s, :k], B[a:a + k])


@pytest.mark.parametrize("H,G,P,N,Q,io,pt", [
    (8, 2, 64, 128, 64, "bf16", 16),     # matrix-core engine, 4 pages per chunk
    (8, 2, 64, 128, 256, "bf16", 64),    # the RFC's chunk size
    (4, 1, 32, 32, 16, "bf16", 16),      # chunk 16: one page per chunk
    (4, 1, 16, 16, 32, "f32", 16),       # fp32-FMA engine
])
def test_mixed_offset_batches_contiguous_and_paged(H, G, P, N, Q, io, pt):
    rng = np.random.default_rng(Q + H)
    lengths = [int(v) for v in rng.integers(1, 700, 10)] + [Q, 3 * Q + 1]
    pr = make_problem(lengths, H=H, G=G, P=P, N=N, Q=Q, io=io, seed=21)
    x, dt, B, C = pr.dev(None)
    y_ss, _, bnd_ss = erd.ssd_prefill_varlen(pr.shape, pr.cu, x, dt, pr.A, B, C, pr.D,
                                             pr.bias)
    S = len(lengths)
    npages = S * (Q // pt) + 5
    contig = erd.ReplayCache(pr.shape, S, DEV)
    paged = erd.ReplayCache(pr.shape, S, DEV, page_tokens=pt, num_pages=npages)
    # stale data everywhere in the pool: pages are never cleared between owners
    paged.buf_x.normal_()
    paged.buf_B.normal_()
    (y_c, y_p), pools = run_schedule(pr, [contig, paged], seed=Q * 3 + P)
    check_final(pr, contig, y_c, y_ss, bnd_ss)
    check_final(pr, paged, y_p, y_ss, bnd_ss)
    # the pool ends holding exactly the pages of the buffered positions
    pool = pools[1]
    held = (pool.table >= 0).sum()
    assert held == sum((L % Q + pt - 1) // pt for L in lengths)
    assert held + len(pool.free) == npages
    if io == "bf16":
        ref = pr.oracle()
        assert mean_rel_err(y_p, ref.y) <= BF16_MEAN_REL


def test_paged_batched_decode_b256():
    """256 slots at offsets 0..255 of chunk 256, pages of 64 rows scattered
    over the pool, 48 batched decode steps (about one slot in five crosses a
    chunk boundary): bitwise equal to the contiguous cache."""
    S, H, P, N, Q, pt, steps = 256, 32, 64, 128, 256, 64, 48
    shape = erd.Shape(H, 1, P, N, Q, "bf16", "bf16")
    hp = synth.make_head_params(H, 3)
    pre = synth.replay_prefix_lengths(S, Q, 3)
    lengths = pre + steps
    cu = synth.cu_seqlens(lengths)
    x, dt, B, C = synth.make_tokens_torch(int(cu[-1]), H, 1, P, N, 3, DEV)
    A, D, bias = (torch.from_numpy(v).to(DEV) for v in (hp.A, hp.D, hp.dt_bias))
    y_ss, _, bnd_ss = erd.ssd_prefill_varlen(shape, cu, x, dt, A, B, C, D, bias)
    npages = S * (Q // pt)
    contig = erd.ReplayCache(shape, S, DEV)
    paged = erd.ReplayCache(shape, S, DEV, page_tokens=pt, num_pages=npages)
    perm = np.random.default_rng(5).permutation(npages).astype(np.int32)
    paged.buf_pages.copy_(torch.from_numpy(perm.reshape(S, Q // pt)))
    ip = torch.from_numpy(np.concatenate([np.arange(cu[s], cu[s] + pre[s])
                                          for s in range(S)])).to(DEV)
    for c in (contig, paged):
        erd.ssd_replay_prefill(shape, c, synth.cu_seqlens(pre), x[ip], dt[ip], B[ip], C[ip],
                               A, D, bias)
    for k in range(steps):
        it = torch.from_numpy((cu[:-1] + pre + k).astype(np.int64)).to(DEV)
        yc = erd.ssd_replay_decode(shape, contig, x[it], dt[it], B[it], C[it], A, D, bias)
        yp = erd.ssd_replay_decode(shape, paged, x[it], dt[it], B[it], C[it], A, D, bias)
        assert same_bits(yp, yc) and same_bits(yp, y_ss[it])
    assert same_bits(paged.state, contig.state) and same_bits(paged.state, bnd_ss)
    assert cache_consistent(paged)
    for a, b in zip(paged.buffers_by_slot()[:3], contig.buffers_by_slot()[:3]):
        assert same_bits(a, b)


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_missing_page_skips_the_sequence(io):
    """A call whose page-table entry for a touched position is not a page of
    the pool leaves that sequence alone (no output, no cache change) and
    serves the others."""
    P, N = (64, 128) if io == "bf16" else (16, 16)
    Q, pt = 64, 16
    pr = make_problem([100, 100, 100], H=4, G=1, P=P, N=N, Q=Q, io=io, seed=2)
    x, dt, B, C = pr.dev(None)
    y_ss, _, _ = erd.ssd_prefill_varlen(pr.shape, pr.cu, x, dt, pr.A, B, C, pr.D, pr.bias)
    cache = erd.ReplayCache(pr.shape, 3, DEV, page_tokens=pt, num_pages=12)
    table = torch.arange(12, dtype=torch.int32, device=DEV).reshape(3, 4)
    cache.buf_pages.copy_(table)
    cu = pr.cu
    first = torch.from_numpy(np.concatenate([np.arange(cu[s], cu[s] + 40)
                                             for s in range(3)])).to(DEV)
    erd.ssd_replay_prefill(pr.shape, cache, [0, 40, 80, 120], x[first], dt[first], B[first],
                           C[first], pr.A, pr.D, pr.bias)
    before = cache.clone()
    # slot 1 would write positions 40..47 (page entry 2): take that page away;
    # slot 2 gets an entry past the pool
    cache.buf_pages[1, 2] = -1
    cache.buf_pages[2, 2] = 12
    nxt = torch.from_numpy(np.concatenate([np.arange(cu[s] + 40, cu[s] + 48)
                                           for s in range(3)])).to(DEV)
    y = erd.ssd_replay_prefill(pr.shape, cache, [0, 8, 16, 24], x[nxt], dt[nxt], B[nxt],
                               C[nxt], pr.A, pr.D, pr.bias,
                               y=torch.full((24, 4, P), 7.0, dtype=x.dtype, device=DEV))
    assert same_bits(y[:8], y_ss[nxt[:8]])
    assert bool((y[8:] == 7.0).all())
    assert int(cache.buf_len[0]) == 48
    for s in (1, 2):
        assert int(cache.buf_len[s]) == 40
        assert same_bits(cache.state[s], before.state[s])
    # decode: slot 1 needs position 40 (entry 2) -> skipped, slot 0 served
    tok = torch.tensor([int(cu[0]) + 48, int(cu[1]) + 40], device=DEV)
    yd = erd.ssd_replay_decode(pr.shape, cache, x[tok], dt[tok], B[tok], C[tok], pr.A, pr.D,
                               pr.bias, slot_idx=torch.tensor([0, 1], dtype=torch.int32,
                                                              device=DEV),
                               y=torch.full((2, 4, P), 7.0, dtype=x.dtype, device=DEV))
    assert same_bits(yd[0], y_ss[tok[0]]) and bool((yd[1] == 7.0).all())
    assert int(cache.buf_len[0]) == 49 and int(cache.buf_len[1]) == 40
    assert cache_consistent(cache)


def test_paged_commit_boundary_then_decode():
    """A plain prefill committed into a paged cache (pages of 32 rows, with C
    buffered) equals the contiguous commit; decoding on continues bitwise."""
    lengths = [600, 77, 256, 1000]
    pr = make_problem(lengths, H=8, G=2, P=64, N=128, Q=256, seed=9)
    x, dt, B, C = pr.dev(None)
    y_ss, _, _ = erd.ssd_prefill_varlen(pr.shape, pr.cu, x, dt, pr.A, B, C, pr.D, pr.bias)
    cu = pr.cu
    pre = np.array([L - 40 for L in lengths])
    ip = torch.from_numpy(np.concatenate([np.arange(cu[s], cu[s] + pre[s])
                                          for s in range(4)])).to(DEV)
    cpre = synth.cu_seqlens(pre)
    _, _, b_pre = erd.ssd_prefill_varlen(pr.shape, cpre, x[ip], dt[ip], pr.A, B[ip], C[ip],
                                         pr.D, pr.bias)
    slots = torch.tensor([3, 0, 2, 1], dtype=torch.int32, device=DEV)
    contig = erd.ReplayCache(pr.shape, 4, DEV, with_C=True)
    paged = erd.ReplayCache(pr.shape, 4, DEV, with_C=True, page_tokens=32, num_pages=40)
    perm = np.random.default_rng(1).permutation(40)[:32].astype(np.int32)
    paged.buf_pages.copy_(torch.from_numpy(perm.reshape(4, 8)))
    for c in (contig, paged):
        erd.ssd_commit_boundary(pr.shape, c, cpre, x[ip], dt[ip], B[ip], C[ip], b_pre,
                                slot_idx=slots)
    assert same_bits(paged.state, contig.state) and cache_consistent(paged)
    assert same_bits(paged.buf_len, contig.buf_len)
    assert same_bits(paged.boundary_pos, contig.boundary_pos)
    for a, b in zip(paged.buffers_by_slot(), contig.buffers_by_slot()):
        assert same_bits(a, b)
    for k in range(40):
        it = torch.from_numpy((cu[:-1] + pre + k).astype(np.int64)).to(DEV)
        yc = erd.ssd_replay_decode(pr.shape, contig, x[it], dt[it], B[it], C[it], pr.A, pr.D,
                                   pr.bias, slot_idx=slots)
        yp = erd.ssd_replay_decode(pr.shape, paged, x[it], dt[it], B[it], C[it], pr.A, pr.D,
                                   pr.bias, slot_idx=slots)
        assert same_bits(yp, yc) and same_bits(yp, y_ss[it])
    assert same_bits(paged.state, contig.state)
    for a, b in zip(paged.buffers_by_slot(), contig.buffers_by_slot()):
        assert same_bits(a, b)

"""Speculative verification and acceptance through the C ABI (ReplaySSM
reproduction README, "Motivation and method": output-only verification of
drafts; the acceptance length advances only the committed-input pointer,
rejected drafts never enter the recurrence).

Each round drafts T tokens per sequence: the first a_s are the sequence's
true continuation, the rest junk (large values, so any leak would show).
Checked bit for bit against one single-shot prefill of every true sequence:
the verified outputs of the accepted drafts, the committed boundary states,
buffers and slot metadata after every acceptance; and that verification
writes nothing.
"""
import numpy as np
import pytest
import torch

import exact_replay_decode_amd as erd
from exact_replay_decode_amd import synth
from gpu_cases import DEV, cache_consistent, make_problem, mean_rel_err, same_bits

pytestmark = pytest.mark.gpu


def cache_bits(cache):
    return [t.clone() for t in cache.tensors()]


def unchanged(cache, before):
    return all(same_bits(a, b) for a, b in zip(cache.tensors(), before))


def run_spec(pr, prompt, T, seed, cache):
    """Prefill the prompts, then speculative rounds until every sequence is
    consumed. Returns the verified outputs of all accepted drafts [T,H,P]."""
    lengths = np.array(pr.lengths)
    S = len(lengths)
    cu = pr.cu
    x, dt, B, C = pr.dev(None)
    rng = np.random.default_rng(seed)
    ip = torch.from_numpy(np.concatenate([np.arange(cu[s], cu[s] + prompt[s])
                                          for s in range(S)])).to(DEV)
    y_all = torch.full_like(x, float("nan"))
    y_all[ip] = erd.ssd_replay_prefill(pr.shape, cache, synth.cu_seqlens(prompt), x[ip], dt[ip],
                                       B[ip], C[ip], pr.A, pr.D, pr.bias)
    done = prompt.astype(np.int64).copy()
    junk = 8.0
    while (done < lengths).any():
        live = np.flatnonzero(done < lengths)
        rem = lengths[live] - done[live]
        nd = np.minimum(T, rem + 1)                      # drafts per sequence (>= 1)
        acc = np.minimum(rng.integers(0, T + 1, len(live)), np.minimum(nd, rem))
        if rng.random() < 0.25:
            acc = np.minimum(nd, rem)                    # everything accepted
        # draft rows: true tokens for j < acc, junk after
        src = np.concatenate([np.minimum(cu[s] + done[s] + np.arange(k), cu[s + 1] - 1)
                              for s, k in zip(live, nd)]).astype(np.int64)
        ok = np.concatenate([np.arange(k) < a for k, a in zip(nd, acc)])
        dx, ddt, dB, dC = (t[torch.from_numpy(src).to(DEV)].clone() for t in (x, dt, B, C))
        bad = torch.from_numpy(~ok).to(DEV)
        dx[bad] = junk
        dB[bad] = -junk
        ddt[bad] = 2.0
        dcu = synth.cu_seqlens(nd)
        sl = torch.from_numpy(live.astype(np.int32)).to(DEV)
        before = cache_bits(cache)
        yv = erd.ssd_replay_verify(pr.shape, cache, dcu, dx, ddt, dB, dC, pr.A, pr.D, pr.bias,
                                   slot_idx=sl)
        assert unchanged(cache, before), "verification wrote to the cache"
        good = torch.from_numpy(np.flatnonzero(ok)).to(DEV)
        y_all[torch.from_numpy(src[ok]).to(DEV)] = yv[good]
        erd.ssd_replay_accept(pr.shape, cache, dcu, torch.from_numpy(acc.astype(np.int32)).to(DEV),
                              dx, ddt, dB, dC, pr.A, pr.bias, slot_idx=sl)
        done[live] += acc
    return y_all


def check_cache(pr, cache, bnd_ss):
    Q = pr.shape.chunk_size
    lengths = np.array(pr.lengths)
    x, dt, B, C = pr.dev(None)
    assert same_bits(cache.state, bnd_ss) and cache_consistent(cache)
    assert np.array_equal(cache.buf_len.cpu().numpy(), lengths % Q)
    assert np.array_equal(cache.boundary_pos.cpu().numpy(), lengths - lengths % Q)
    bx, bdt, bB, _ = cache.buffers_by_slot()
    for s, L in enumerate(lengths):
        k = int(L % Q)
        a = int(pr.cu[s + 1]) - k
        assert same_bits(bx[s, :k], x[a:a + k]) and same_bits(bB[s, :k], B[a:a + k])
        assert same_bits(bdt[s, :k], dt[a:a + k])


@pytest.mark.parametrize("H,G,P,N,Q,io,T,pt", [
    (8, 2, 64, 128, 16, "bf16", 4, None),    # drafts cross chunk ends often
    (8, 2, 64, 128, 256, "bf16", 4, None),   # the RFC's chunk size
    (8, 2, 64, 128, 64, "bf16", 7, 16),      # paged buffers
    (6, 3, 32, 64, 32, "bf16", 3, None),     # 2 heads per group: C.B^T per head; a half workgroup
    (8, 1, 32, 32, 64, "bf16", 5, 16),       # C.B^T shared by a workgroup's heads; small tiles
    (4, 1, 16, 16, 16, "f32", 5, None),      # fp32-FMA engine
])
def test_speculative_rounds_bitwise(H, G, P, N, Q, io, T, pt):
    rng = np.random.default_rng(Q + T)
    S = 9
    lengths = [int(v) for v in rng.integers(40, 600, S)]
    prompt = np.array([int(rng.integers(1, L)) for L in lengths])
    pr = make_problem(lengths, H=H, G=G, P=P, N=N, Q=Q, io=io, seed=31)
    x, dt, B, C = pr.dev(None)
    y_ss, _, bnd_ss = erd.ssd_prefill_varlen(pr.shape, pr.cu, x, dt, pr.A, B, C, pr.D, pr.bias)
    if pt is None:
        cache = erd.ReplayCache(pr.shape, S, DEV)
    else:
        npg = Q // pt
        cache = erd.ReplayCache(pr.shape, S, DEV, page_tokens=pt, num_pages=S * npg)
        perm = np.random.default_rng(2).permutation(S * npg).astype(np.int32)
        cache.buf_pages.copy_(torch.from_numpy(perm.reshape(S, npg)))
    y = run_spec(pr, prompt, T, seed=Q * 7 + T, cache=cache)
    assert same_bits(y, y_ss)
    check_cache(pr, cache, bnd_ss)
    if io == "bf16":
        assert mean_rel_err(y, pr.oracle().y) <= 3e-3


def test_verify_equals_decode_steps():
    """Verified outputs of T drafts equal T decode steps on a copy of the
    cache, for slots at every offset of the chunk (drafts crossing its end)."""
    S, H, P, N, Q, T = 64, 8, 64, 128, 64, 6
    shape = erd.Shape(H, 1, P, N, Q, "bf16", "bf16")
    hp = synth.make_head_params(H, 4)
    pre = Q + np.arange(S) % Q                     # every buffer fill 0..Q-1
    lengths = pre + T
    cu = synth.cu_seqlens(lengths)
    x, dt, B, C = synth.make_tokens_torch(int(cu[-1]), H, 1, P, N, 4, DEV)
    A, D, bias = (torch.from_numpy(v).to(DEV) for v in (hp.A, hp.D, hp.dt_bias))
    cache = erd.ReplayCache(shape, S, DEV)
    ip = torch.from_numpy(np.concatenate([np.arange(cu[s], cu[s] + pre[s])
                                          for s in range(S)])).to(DEV)
    erd.ssd_replay_prefill(shape, cache, synth.cu_seqlens(pre), x[ip], dt[ip], B[ip], C[ip],
                           A, D, bias)
    idr = torch.from_numpy(np.concatenate([np.arange(cu[s] + pre[s], cu[s + 1])
                                           for s in range(S)])).to(DEV)
    dcu = synth.cu_seqlens([T] * S)
    yv = erd.ssd_replay_verify(shape, cache, dcu, x[idr], dt[idr], B[idr], C[idr], A, D, bias)
    dec = cache.clone()
    yd = []
    for k in range(T):
        it = torch.from_numpy((cu[:-1] + pre + k).astype(np.int64)).to(DEV)
        yd.append(erd.ssd_replay_decode(shape, dec, x[it], dt[it], B[it], C[it], A, D, bias))
    assert same_bits(yv.view(S, T, H, P), torch.stack(yd, 1))
    # accepting everything gives the decoded cache (buffer rows past buf_len
    # hold nothing: decode leaves a completed chunk's rows there)
    erd.ssd_replay_accept(shape, cache, dcu, torch.full((S,), T, dtype=torch.int32, device=DEV),
                          x[idr], dt[idr], B[idr], C[idr], A, bias)
    for name in ("state", "state_bf", "buf_len", "boundary_pos", "work"):
        assert same_bits(getattr(cache, name), getattr(dec, name)), name
    n = cache.buf_len.tolist()
    for a, b in zip(cache.buffers_by_slot()[:3], dec.buffers_by_slot()[:3]):
        for s in range(S):
            assert same_bits(a[s, :n[s]], b[s, :n[s]])


@pytest.mark.parametrize("S", [200, 256])
def test_large_verify_equals_decode_steps(S):
    """A batch with more workgroups than run at once (H=32: 8 per sequence,
    S x 8 > 768), buffers at every offset, so that drafts cross the chunk
    end for the last offsets and the crossing sweep takes several listed
    sequences. Outputs equal T decode steps on a copy of the cache; the
    cache, work array included, is unchanged."""
    H, P, N, Q, T = 32, 64, 128, 64, 4
    shape = erd.Shape(H, 1, P, N, Q, "bf16", "bf16")
    hp = synth.make_head_params(H, 5)
    pre = Q + (np.arange(S) * 7) % Q               # every buffer fill, shuffled
    lengths = pre + T
    cu = synth.cu_seqlens(lengths)
    x, dt, B, C = synth.make_tokens_torch(int(cu[-1]), H, 1, P, N, 5, DEV)
    A, D, bias = (torch.from_numpy(v).to(DEV) for v in (hp.A, hp.D, hp.dt_bias))
    cache = erd.ReplayCache(shape, S, DEV)
    ip = torch.from_numpy(np.concatenate([np.arange(cu[s], cu[s] + pre[s])
                                          for s in range(S)])).to(DEV)
    erd.ssd_replay_prefill(shape, cache, synth.cu_seqlens(pre), x[ip], dt[ip], B[ip], C[ip],
                           A, D, bias)
    idr = torch.from_numpy(np.concatenate([np.arange(cu[s] + pre[s], cu[s + 1])
                                           for s in range(S)])).to(DEV)
    dcu = synth.cu_seqlens([T] * S)
    before = cache_bits(cache)
    yv = erd.ssd_replay_verify(shape, cache, dcu, x[idr], dt[idr], B[idr], C[idr], A, D, bias)
    assert unchanged(cache, before), "verification wrote to the cache"
    dec = cache.clone()
    yd = []
    for k in range(T):
        it = torch.from_numpy((cu[:-1] + pre + k).astype(np.int64)).to(DEV)
        yd.append(erd.ssd_replay_decode(shape, dec, x[it], dt[it], B[it], C[it], A, D, bias))
    assert same_bits(yv.view(S, T, H, P), torch.stack(yd, 1))


def test_accept_clamps_and_zero():
    """accepted < 0 commits nothing, accepted > drafts commits all drafts."""
    pr = make_problem([100, 100], H=4, G=1, P=64, N=128, Q=32, seed=6)
    x, dt, B, C = pr.dev(None)
    y_ss, _, _ = erd.ssd_prefill_varlen(pr.shape, pr.cu, x, dt, pr.A, B, C, pr.D, pr.bias)
    cache = erd.ReplayCache(pr.shape, 2, DEV)
    ip = torch.tensor(list(range(0, 30)) + list(range(100, 130)), device=DEV)
    erd.ssd_replay_prefill(pr.shape, cache, [0, 30, 60], x[ip], dt[ip], B[ip], C[ip], pr.A,
                           pr.D, pr.bias)
    idr = torch.tensor(list(range(30, 35)) + list(range(130, 135)), device=DEV)
    before = cache_bits(cache)
    erd.ssd_replay_accept(pr.shape, cache, [0, 5, 10],
                          torch.tensor([-3, 0], dtype=torch.int32, device=DEV),
                          x[idr], dt[idr], B[idr], C[idr], pr.A, pr.bias)
    assert unchanged(cache, before)
    erd.ssd_replay_accept(pr.shape, cache, [0, 5, 10],
                          torch.tensor([99, 5], dtype=torch.int32, device=DEV),
                          x[idr], dt[idr], B[idr], C[idr], pr.A, pr.bias)
    assert cache.buf_len.tolist() == [3, 3] and cache.boundary_pos.tolist() == [32, 32]
    assert cache_consistent(cache)
    nxt = torch.tensor([35, 135], device=DEV)
    yd = erd.ssd_replay_decode(pr.shape, cache, x[nxt], dt[nxt], B[nxt], C[nxt], pr.A, pr.D,
                               pr.bias)
    assert same_bits(yd, y_ss[nxt])

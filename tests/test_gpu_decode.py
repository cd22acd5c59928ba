"""GPU exact-replay decode and recurrent update, through the C ABI.

Replay decode must reproduce single-shot prefill bit for bit (outputs,
committed boundary states, buffers); both paths are checked against the
fp64 oracle within tolerance.
"""
import numpy as np
import pytest
import torch

import exact_replay_decode_amd as erd
from exact_replay_decode_amd import synth
from gpu_cases import (DEV, cache_consistent, check_bf16, headwise_max_rel, make_problem,
                       mean_rel_err, offset_invariant,
                       same_bits, y_headwise_max_rel)

pytestmark = pytest.mark.gpu

BF16_MEAN_REL = 3e-3
STATE_REL = 1e-4
F32_Y_REL = 1e-4


def decode_tokens(shape, cache, x, dt, B, C, A, D, bias, slot=0):
    """Decode tokens x[0..n) one at a time for one slot; returns y[n,H,P]."""
    sl = torch.tensor([slot], dtype=torch.int32, device=DEV)
    ys = []
    for t in range(x.shape[0]):
        ys.append(erd.ssd_replay_decode(shape, cache, x[t:t + 1], dt[t:t + 1], B[t:t + 1],
                                        C[t:t + 1], A, D, bias, slot_idx=sl))
    return torch.cat(ys)


# ---- C0: decode every token of a tiny fp32 scan ----------------------------

def test_c0_decode_every_token():
    pr = make_problem([64], H=4, G=1, P=16, N=16, Q=16, io="f32")
    x, dt, B, C = pr.dev(None)
    y, fin, bnd = erd.ssd_prefill_varlen(pr.shape, pr.cu, x, dt, pr.A, B, C, pr.D, pr.bias)
    cache = erd.ReplayCache(pr.shape, 1, DEV, with_C=True)
    yd = decode_tokens(pr.shape, cache, x, dt, B, C, pr.A, pr.D, pr.bias)
    assert same_bits(yd, y)
    assert same_bits(cache.state[0], bnd[0]) and cache_consistent(cache)
    assert int(cache.buf_len[0]) == 0 and int(cache.boundary_pos[0]) == 64
    ref = pr.oracle()
    assert y_headwise_max_rel(yd, ref.y, pr.cu) <= F32_Y_REL


def test_c0_decode_after_split_prefill():
    pr = make_problem([64], H=4, G=1, P=16, N=16, Q=16, io="f32", seed=4)
    x, dt, B, C = pr.dev(None)
    y, _, _ = erd.ssd_prefill_varlen(pr.shape, pr.cu, x, dt, pr.A, B, C, pr.D, pr.bias)
    cache = erd.ReplayCache(pr.shape, 1, DEV)
    y0 = erd.ssd_replay_prefill(pr.shape, cache, [0, 24], x[:24], dt[:24], B[:24], C[:24],
                                pr.A, pr.D, pr.bias)
    assert int(cache.buf_len[0]) == 8 and int(cache.boundary_pos[0]) == 16
    yd = decode_tokens(pr.shape, cache, x[24:], dt[24:], B[24:], C[24:], pr.A, pr.D, pr.bias)
    assert same_bits(torch.cat([y0, yd]), y)


# ---- C1: 2048 token-by-token decode steps ---------------------------------

@pytest.fixture(scope="module")
def c1():
    pr = make_problem([2048], H=32, G=1, P=64, N=128, Q=256)
    x, dt, B, C = pr.dev(None)
    y, fin, bnd = erd.ssd_prefill_varlen(pr.shape, pr.cu, x, dt, pr.A, B, C, pr.D, pr.bias)
    return pr, (x, dt, B, C), y, fin, bnd


def test_c1_decode_2048_steps_bitwise(c1):
    pr, (x, dt, B, C), y, fin, bnd = c1
    cache = erd.ReplayCache(pr.shape, 1, DEV, with_C=True)
    yd = decode_tokens(pr.shape, cache, x, dt, B, C, pr.A, pr.D, pr.bias)
    assert same_bits(yd, y)
    assert same_bits(cache.state[0], bnd[0]) and cache_consistent(cache)
    # the buffer holds the last chunk's tokens, C included
    assert int(cache.buf_len[0]) == 0 and int(cache.boundary_pos[0]) == 2048
    assert same_bits(cache.buf_x[0], x[1792:]) and same_bits(cache.buf_C[0], C[1792:])
    assert same_bits(cache.buf_B[0], B[1792:]) and same_bits(cache.buf_dt[0], dt[1792:])


def test_c1_commit_boundary_then_decode(c1):
    """Plain prefill of 600 tokens + ssd_commit_boundary, then decode the
    rest: rows 600..767 replay the partial chunk, 768.. follow a commit."""
    pr, (x, dt, B, C), y, fin, bnd = c1
    y6, f6, b6 = erd.ssd_prefill_varlen(pr.shape, [0, 600], x[:600], dt[:600], pr.A, B[:600],
                                        C[:600], pr.D, pr.bias)
    cache = erd.ReplayCache(pr.shape, 1, DEV)
    erd.ssd_commit_boundary(pr.shape, cache, [0, 600], x[:600], dt[:600], B[:600], C[:600], b6)
    assert int(cache.buf_len[0]) == 88 and int(cache.boundary_pos[0]) == 512
    assert cache_consistent(cache)
    yd = decode_tokens(pr.shape, cache, x[600:900], dt[600:900], B[600:900], C[600:900],
                       pr.A, pr.D, pr.bias)
    assert same_bits(torch.cat([y6, yd]), y[:900])
    mism = (yd.view(torch.int16) != y[600:900].view(torch.int16)).flatten(1).any(1)
    assert int(mism.sum()) == 0


def test_c1_preemption_recompute(c1):
    """Decode to token 600, drop everything but the cache snapshot, recompute
    tokens 600..899 as one unaligned prefill, then keep decoding."""
    pr, (x, dt, B, C), y, _, _ = c1
    cache = erd.ReplayCache(pr.shape, 1, DEV)
    decode_tokens(pr.shape, cache, x[:600], dt[:600], B[:600], C[:600], pr.A, pr.D, pr.bias)
    snap = cache.clone()
    del cache
    y_re = erd.ssd_replay_prefill(pr.shape, snap, [0, 300], x[600:900], dt[600:900],
                                  B[600:900], C[600:900], pr.A, pr.D, pr.bias)
    yd = decode_tokens(pr.shape, snap, x[900:1000], dt[900:1000], B[900:1000], C[900:1000],
                       pr.A, pr.D, pr.bias)
    assert same_bits(y_re, y[600:900]) and same_bits(yd, y[900:1000])


def test_c1_ssu_differs_in_bits_but_matches_oracle(c1):
    """Negative control: the recurrent update is a different rounding of the
    same math, so its rows differ in bits from the chunked scan while both
    sit within tolerance of the oracle."""
    pr, (x, dt, B, C), y, _, _ = c1
    state = torch.zeros((1, 32, 64, 128), dtype=torch.float32, device=DEV)
    ys = []
    for t in range(512):
        ys.append(erd.ssm_state_update(pr.shape, state, x[t:t + 1], dt[t:t + 1], B[t:t + 1],
                                       C[t:t + 1], pr.A, pr.D, pr.bias))
    ys = torch.cat(ys)
    assert not same_bits(ys, y[:512])
    frac_equal = float((ys.view(torch.int16) == y[:512].view(torch.int16)).float().mean())
    print(f"SSU vs SSD bit-identical elements: {100 * frac_equal:.1f} %")
    ref = pr.oracle()
    assert mean_rel_err(ys, ref.y[:512]) <= BF16_MEAN_REL


# ---- grouped heads (C2's shape) and head counts that are not a multiple of
# the heads per decode workgroup ---------------------------------------------

@pytest.mark.parametrize("H,G,P,N,Q,io", [(64, 8, 64, 128, 256, "bf16"),
                                           (6, 2, 32, 64, 32, "bf16"),
                                           (5, 5, 64, 32, 16, "bf16"),
                                           (3, 1, 32, 128, 64, "bf16")])
def test_decode_grouped_and_ragged_heads(H, G, P, N, Q, io):
    lengths = [600, 300, 900, 248] if H == 64 else [300, 77, 129]
    pr = make_problem(lengths, H=H, G=G, P=P, N=N, Q=Q, io=io, seed=11)
    x, dt, B, C = pr.dev(None)
    y, _, bnd = erd.ssd_prefill_varlen(pr.shape, pr.cu, x, dt, pr.A, B, C, pr.D, pr.bias)
    cu = pr.cu
    S = len(lengths)
    # replay-prefill a prefix of each sequence, then decode the rest in
    # batched steps (finished sequences drop out of the batch)
    pre = np.array([L // 3 + 5 for L in lengths])
    ip = torch.from_numpy(np.concatenate([np.arange(cu[s], cu[s] + pre[s])
                                          for s in range(S)])).to(DEV)
    cache = erd.ReplayCache(pr.shape, S, DEV)
    y_pre = erd.ssd_replay_prefill(pr.shape, cache, synth.cu_seqlens(pre), x[ip], dt[ip],
                                   B[ip], C[ip], pr.A, pr.D, pr.bias)
    assert same_bits(y_pre, y[ip])
    yd = torch.empty_like(y)
    for k in range(max(lengths) - int(pre.min())):
        live = [s for s in range(S) if pre[s] + k < lengths[s]]
        if not live:
            break
        it = torch.tensor([int(cu[s] + pre[s] + k) for s in live], device=DEV)
        sl = torch.tensor(live, dtype=torch.int32, device=DEV)
        yd[it] = erd.ssd_replay_decode(pr.shape, cache, x[it], dt[it], B[it], C[it], pr.A,
                                       pr.D, pr.bias, slot_idx=sl)
    idec = torch.from_numpy(np.concatenate([np.arange(cu[s] + pre[s], cu[s + 1])
                                            for s in range(S)])).to(DEV)
    assert same_bits(yd[idec], y[idec])
    assert same_bits(cache.state, bnd) and cache_consistent(cache)
    assert np.array_equal(cache.buf_len.cpu().numpy(), np.array(lengths) % Q)


# ---- C3: batched decode, B = 256 ------------------------------------------

def _c3_setup(Q, steps=300, seed=0):
    S, H, P, N = 256, 32, 64, 128
    shape = erd.Shape(H, 1, P, N, Q, "bf16", "bf16")
    hp = synth.make_head_params(H, seed)
    pre = synth.replay_prefix_lengths(S, 256, seed)   # 256 + k_i, k_i in [0, 256)
    lengths = pre + steps
    cu = synth.cu_seqlens(lengths)
    x, dt, B, C = synth.make_tokens_torch(int(cu[-1]), H, 1, P, N, seed, DEV)
    A, D, bias = (torch.from_numpy(v).to(DEV) for v in (hp.A, hp.D, hp.dt_bias))
    return shape, hp, pre, lengths, cu, (x, dt, B, C), (A, D, bias)


def _c3_run(Q):
    shape, hp, pre, lengths, cu, (x, dt, B, C), (A, D, bias) = _c3_setup(Q)
    S = len(pre)
    y_ss, fin_ss, bnd_ss = erd.ssd_prefill_varlen(shape, cu, x, dt, A, B, C, D, bias)
    # replay: prefill the prefixes, then 300 batched decode steps
    idx_pre = np.concatenate([np.arange(cu[s], cu[s] + pre[s]) for s in range(S)])
    ip = torch.from_numpy(idx_pre).to(DEV)
    cache = erd.ReplayCache(shape, S, DEV)
    y_pre = erd.ssd_replay_prefill(shape, cache, synth.cu_seqlens(pre), x[ip], dt[ip], B[ip],
                                   C[ip], A, D, bias)
    assert same_bits(y_pre, y_ss[ip])
    steps = int(lengths[0] - pre[0])
    ydec = []
    for k in range(steps):
        it = torch.from_numpy((cu[:-1] + pre + k).astype(np.int64)).to(DEV)
        ydec.append(erd.ssd_replay_decode(shape, cache, x[it], dt[it], B[it], C[it], A, D, bias))
    ydec = torch.stack(ydec, 1)                       # [S, steps, H, P]
    idx_dec = np.stack([cu[:-1] + pre + k for k in range(steps)], 1)
    want = y_ss[torch.from_numpy(idx_dec.astype(np.int64)).to(DEV)]
    return shape, hp, pre, lengths, cu, (x, dt, B, C), ydec, want, cache, bnd_ss, fin_ss


@pytest.mark.parametrize("Q", [256, 16])
def test_c3_batched_replay_decode_bitwise(Q):
    shape, hp, pre, lengths, cu, (x, dt, B, C), ydec, want, cache, bnd, fin = _c3_run(Q)
    assert same_bits(ydec, want)
    # offset invariant: every committed boundary sits on the chunk grid and
    # holds exactly the single-shot state at that position
    assert offset_invariant(cache, lengths, Q, bnd) and cache_consistent(cache)
    # the ranked launches leave the bookkeeping array zero
    assert not cache.work.any()
    # oracle parity on sampled sequences (decode rows and boundary state)
    from oracle import scan
    from oracle.bounds import chunk_error_scales
    for s in (0, 131, 255):
        a, b = int(cu[s]), int(cu[s + 1])
        args = (erd.to_f64(x[a:b]), erd.to_f64(dt[a:b]), hp.A, erd.to_f64(B[a:b]),
                erd.to_f64(C[a:b]), [0, b - a], Q)
        ref = scan(*args, D=hp.D, dt_bias=hp.dt_bias)
        assert mean_rel_err(ydec[s], ref.y[pre[s]:]) <= BF16_MEAN_REL
        check_bf16(ydec[s], ref.y, chunk_error_scales(*args, D=hp.D, dt_bias=hp.dt_bias),
                   [(0, b - a - int(pre[s]))], rows=slice(int(pre[s]), None),
                   label=f"C3 chunk {Q} decode rows, sequence {s}")
        assert headwise_max_rel(cache.state[s:s + 1].cpu().numpy(), ref.boundary_state) <= STATE_REL


def test_offset_invariant_catches_poisoned_slots():
    """Negative control of the offset invariant the batched-decode test
    asserts: a correct commit passes it, and each way of committing a slot
    at the wrong position fails it -- a boundary state taken one token off
    the chunk grid, a boundary position moved by a chunk, a buffer count off
    by one (the prefix-cache poisoning page's regression test asserts the
    same invariant directly)."""
    Q = 64
    lengths = [200, 64, 1, 130, 255, 0]
    pr = make_problem(lengths, H=8, G=1, P=64, N=128, Q=Q, seed=21)
    x, dt, B, C = pr.dev(None)
    cu = pr.cu
    _, _, bnd = erd.ssd_prefill_varlen(pr.shape, cu, x, dt, pr.A, B, C, pr.D, pr.bias)

    def committed(states):
        cache = erd.ReplayCache(pr.shape, len(lengths), DEV)
        erd.ssd_commit_boundary(pr.shape, cache, cu, x, dt, B, C, states)
        return cache

    good = committed(bnd)
    assert offset_invariant(good, lengths, Q, bnd)
    # sequence 3's boundary state computed one token late: the chunk grid of
    # a run that starts at its second token
    a, b = int(cu[3]), int(cu[4])
    _, _, off = erd.ssd_prefill_varlen(pr.shape, [0, b - a - 1], x[a + 1:b], dt[a + 1:b], pr.A,
                                       B[a + 1:b], C[a + 1:b], pr.D, pr.bias)
    poisoned = bnd.clone()
    poisoned[3] = off[0]
    assert not offset_invariant(committed(poisoned), lengths, Q, bnd)
    moved = committed(bnd)
    moved.boundary_pos[0] += Q
    assert not offset_invariant(moved, lengths, Q, bnd)
    counted = committed(bnd)
    counted.buf_len[4] -= 1
    assert not offset_invariant(counted, lengths, Q, bnd)


def test_c3_replay_batch_invariance():
    """A slot's decode output does not depend on which other slots share
    the call, nor on their offsets."""
    shape, hp, pre, lengths, cu, (x, dt, B, C), (A, D, bias) = _c3_setup(256, steps=4)
    S = len(pre)
    idx_pre = np.concatenate([np.arange(cu[s], cu[s] + pre[s]) for s in range(S)])
    ip = torch.from_numpy(idx_pre).to(DEV)
    cache = erd.ReplayCache(shape, S, DEV)
    erd.ssd_replay_prefill(shape, cache, synth.cu_seqlens(pre), x[ip], dt[ip], B[ip], C[ip],
                           A, D, bias)
    it = torch.from_numpy((cu[:-1] + pre).astype(np.int64)).to(DEV)
    full = erd.ssd_replay_decode(shape, cache.clone(), x[it], dt[it], B[it], C[it], A, D, bias)
    # (101 slots: more workgroups than run at once, a batch that is not a
    # multiple of 8)
    for sub in ([5], [17, 200, 3], list(range(0, 256, 7)), list(range(255, 53, -2))):
        sl = torch.tensor(sub, dtype=torch.int32, device=DEV)
        c2 = cache.clone()
        ys = erd.ssd_replay_decode(shape, c2, x[it][sl.long()], dt[it][sl.long()],
                                   B[it][sl.long()], C[it][sl.long()], A, D, bias, slot_idx=sl)
        assert same_bits(ys, full[sl.long()])
        assert not c2.work.any()


def test_ssu_batch_invariance():
    shape, hp, pre, lengths, cu, (x, dt, B, C), (A, D, bias) = _c3_setup(256, steps=1)
    S = 256
    st0 = torch.randn((S, 32, 64, 128), generator=torch.Generator(device=DEV).manual_seed(3),
                      device=DEV)
    it = torch.from_numpy((cu[:-1] + pre).astype(np.int64)).to(DEV)
    xs, dts, Bs, Cs = x[it], dt[it], B[it], C[it]
    st_full = st0.clone()
    y_full = erd.ssm_state_update(shape, st_full, xs, dts, Bs, Cs, A, D, bias)
    for b in (1, 4, 16, 64, 256):
        st = st0.clone()
        yb = erd.ssm_state_update(shape, st, xs[:b], dts[:b], Bs[:b], Cs[:b], A, D, bias)
        assert same_bits(yb, y_full[:b]) and same_bits(st[:b], st_full[:b])
        assert same_bits(st[b:], st0[b:])


def test_ssu_matches_oracle_from_a_state():
    """40 recurrent steps from the fp32 state after each prefix."""
    shape, hp, pre, lengths, cu, (x, dt, B, C), (A, D, bias) = _c3_setup(256, steps=40)
    from oracle import scan
    S = len(pre)
    ip = torch.from_numpy(np.concatenate([np.arange(cu[s], cu[s] + pre[s])
                                          for s in range(S)])).to(DEV)
    _, state, _ = erd.ssd_prefill_varlen(shape, synth.cu_seqlens(pre), x[ip], dt[ip], A,
                                         B[ip], C[ip], D, bias)
    ys = []
    for k in range(40):
        it = torch.from_numpy((cu[:-1] + pre + k).astype(np.int64)).to(DEV)
        ys.append(erd.ssm_state_update(shape, state, x[it], dt[it], B[it], C[it], A, D, bias))
    ys = torch.stack(ys, 1)
    for s in (0, 99):
        a, b = int(cu[s]), int(cu[s + 1])
        ref = scan(erd.to_f64(x[a:b]), erd.to_f64(dt[a:b]), hp.A, erd.to_f64(B[a:b]),
                   erd.to_f64(C[a:b]), [0, b - a], 256, D=hp.D, dt_bias=hp.dt_bias)
        assert mean_rel_err(ys[s], ref.y[pre[s]:]) <= BF16_MEAN_REL
        assert headwise_max_rel(state[s:s + 1].cpu().numpy(), ref.final_state) <= STATE_REL


# ---- C4: 24-layer scan stack, 600-token prompt + 300 decode steps ---------

def test_c4_layer_stack():
    H, P, N, Q = 24, 64, 128, 256
    for layer in range(24):
        pr = make_problem([900], H=H, G=1, P=P, N=N, Q=Q, seed=100 + layer)
        x, dt, B, C = pr.dev(None)
        y, _, bnd = erd.ssd_prefill_varlen(pr.shape, [0, 900], x, dt, pr.A, B, C, pr.D, pr.bias)
        cache = erd.ReplayCache(pr.shape, 1, DEV)
        y0 = erd.ssd_replay_prefill(pr.shape, cache, [0, 600], x[:600], dt[:600], B[:600],
                                    C[:600], pr.A, pr.D, pr.bias)
        yd = decode_tokens(pr.shape, cache, x[600:], dt[600:], B[600:], C[600:], pr.A, pr.D,
                           pr.bias)
        rows = (yd.view(torch.int16) != y[600:].view(torch.int16)).flatten(1).any(1)
        assert same_bits(y0, y[:600]) and int(rows.sum()) == 0, layer
        assert same_bits(cache.state[0], bnd[0]) and cache_consistent(cache)
        # chunked prefill at most 100 tokens per call
        c2 = erd.ReplayCache(pr.shape, 1, DEV)
        parts = []
        for a in range(0, 900, 100):
            parts.append(erd.ssd_replay_prefill(pr.shape, c2, [0, 100], x[a:a + 100],
                                                dt[a:a + 100], B[a:a + 100], C[a:a + 100],
                                                pr.A, pr.D, pr.bias))
        assert same_bits(torch.cat(parts), y), layer
        if layer == 0:
            ref = pr.oracle()
            assert mean_rel_err(yd, ref.y[600:]) <= BF16_MEAN_REL


def test_cache_refresh_after_direct_state_write():
    """A caller that writes the fp32 state itself rebuilds the bf16 copy with
    ssd_replay_cache_refresh; decode then continues from that state exactly
    as a prefill resumed from it (init_state) does."""
    pr = make_problem([300], H=8, G=2, P=64, N=64, Q=64, seed=21)
    x, dt, B, C = pr.dev(None)
    st0 = torch.randn((1, 8, 64, 64), generator=torch.Generator(device=DEV).manual_seed(5),
                      device=DEV)
    y, _, _ = erd.ssd_prefill_varlen(pr.shape, pr.cu, x, dt, pr.A, B, C, pr.D, pr.bias,
                                     init_state=st0)
    cache = erd.ReplayCache(pr.shape, 1, DEV)
    cache.state.copy_(st0)
    assert not cache_consistent(cache)
    cache.refresh()
    assert cache_consistent(cache)
    yd = decode_tokens(pr.shape, cache, x, dt, B, C, pr.A, pr.D, pr.bias)
    assert same_bits(yd, y) and cache_consistent(cache)


@pytest.mark.parametrize("S,H,G,P,N", [(4500, 4, 1, 32, 32),   # one workgroup per slot
                                       (500, 6, 3, 32, 64)])   # 2 heads per group, half workgroups
def test_large_batch_ranked_launch(S, H, G, P, N):
    """Ranked launches of small shapes: 4500 slots (more positions than the
    ranking kernel holds in registers) and 500 slots of 6 heads (two per
    group: per-head C.B^T and chunk-state update, the second workgroup of a
    slot half empty); neither batch is a multiple of 8, and about one slot in
    32 fills its chunk per step. Four steps, every slot in a shuffled order,
    bit-identical to the single-shot prefill; the bookkeeping array is left
    zero."""
    Q, steps = 32, 4
    shape = erd.Shape(H, G, P, N, Q, "bf16", "bf16")
    rng = np.random.default_rng(77)
    pre = rng.integers(0, 100, S)
    lengths = pre + steps
    cu = synth.cu_seqlens(lengths)
    x, dt, B, C = synth.make_tokens_torch(int(cu[-1]), H, G, P, N, 77, DEV)
    hp = synth.make_head_params(H, 77)
    A, D, bias = (torch.from_numpy(v).to(DEV) for v in (hp.A, hp.D, hp.dt_bias))
    y_ss, _, bnd = erd.ssd_prefill_varlen(shape, cu, x, dt, A, B, C, D, bias)
    ip = torch.from_numpy(np.concatenate([np.arange(cu[s], cu[s] + pre[s])
                                          for s in range(S)])).to(DEV)
    cache = erd.ReplayCache(shape, S, DEV)
    erd.ssd_replay_prefill(shape, cache, synth.cu_seqlens(pre), x[ip], dt[ip], B[ip], C[ip],
                           A, D, bias)
    for k in range(steps):
        perm = rng.permutation(S)
        it = torch.from_numpy((cu[:-1] + pre + k)[perm].astype(np.int64)).to(DEV)
        sl = torch.from_numpy(perm.astype(np.int32)).to(DEV)
        yd = erd.ssd_replay_decode(shape, cache, x[it], dt[it], B[it], C[it], A, D, bias,
                                   slot_idx=sl)
        assert same_bits(yd, y_ss[it]), k
        assert not cache.work.any()
    assert same_bits(cache.state, bnd) and cache_consistent(cache)


def test_batch_longer_than_slot_count():
    """Positions whose slot is outside [0, num_slots) are skipped (their
    output rows are not written). A batch with more positions than slots
    (here 1000 positions, 100 slots, more workgroups than run at once) takes
    the unranked launch with the separate chunk-state update; the valid
    positions' outputs and the caches equal the single-shot prefill's."""
    S, nb, H, G, P, N, Q, steps = 100, 1000, 4, 1, 32, 32, 32, 40
    shape = erd.Shape(H, G, P, N, Q, "bf16", "bf16")
    rng = np.random.default_rng(78)
    pre = rng.integers(0, 70, S)
    lengths = pre + steps
    cu = synth.cu_seqlens(lengths)
    x, dt, B, C = synth.make_tokens_torch(int(cu[-1]), H, G, P, N, 78, DEV)
    hp = synth.make_head_params(H, 78)
    A, D, bias = (torch.from_numpy(v).to(DEV) for v in (hp.A, hp.D, hp.dt_bias))
    y_ss, _, bnd = erd.ssd_prefill_varlen(shape, cu, x, dt, A, B, C, D, bias)
    ip = torch.from_numpy(np.concatenate([np.arange(cu[s], cu[s] + pre[s])
                                          for s in range(S)])).to(DEV)
    cache = erd.ReplayCache(shape, S, DEV)
    erd.ssd_replay_prefill(shape, cache, synth.cu_seqlens(pre), x[ip], dt[ip], B[ip], C[ip],
                           A, D, bias)
    for k in range(steps):
        order = rng.permutation(nb)
        pos, rest = order[:S], order[S:]              # where the slots sit in the batch
        slots = np.full(nb, -1, dtype=np.int32)
        slots[rest[:300]] = -7                        # other out-of-range entries
        slots[rest[300:600]] = S + 3
        slots[pos] = np.arange(S, dtype=np.int32)
        tok = np.zeros(nb, dtype=np.int64)            # skipped positions read token 0
        tok[pos] = cu[:-1] + pre + k
        it = torch.from_numpy(tok).to(DEV)
        y = torch.full((nb, H, P), float("nan"), dtype=torch.bfloat16, device=DEV)
        erd.ssd_replay_decode(shape, cache, x[it], dt[it], B[it], C[it], A, D, bias,
                              slot_idx=torch.from_numpy(slots).to(DEV), y=y)
        pv = torch.from_numpy(pos).to(DEV)
        assert same_bits(y[pv], y_ss[it[pv]]), k
        skipped = torch.ones(nb, dtype=torch.bool, device=DEV)
        skipped[pv] = False
        assert torch.isnan(y[skipped].float()).all()
    assert same_bits(cache.state, bnd) and cache_consistent(cache)


def test_ranked_launch_with_skipped_positions():
    """A ranked launch (more workgroups than run at once, batch <= slots)
    whose batch holds out-of-range slot entries: their workgroups only count
    themselves out, their output rows are not written, and the valid
    positions equal the single-shot prefill bit for bit."""
    S, nb, H, G, P, N, Q, steps = 1000, 900, 4, 1, 32, 32, 32, 6
    shape = erd.Shape(H, G, P, N, Q, "bf16", "bf16")
    rng = np.random.default_rng(79)
    pre = rng.integers(0, 70, S)
    lengths = pre + steps
    cu = synth.cu_seqlens(lengths)
    x, dt, B, C = synth.make_tokens_torch(int(cu[-1]), H, G, P, N, 79, DEV)
    hp = synth.make_head_params(H, 79)
    A, D, bias = (torch.from_numpy(v).to(DEV) for v in (hp.A, hp.D, hp.dt_bias))
    y_ss, _, _ = erd.ssd_prefill_varlen(shape, cu, x, dt, A, B, C, D, bias)
    ip = torch.from_numpy(np.concatenate([np.arange(cu[s], cu[s] + pre[s])
                                          for s in range(S)])).to(DEV)
    cache = erd.ReplayCache(shape, S, DEV)
    erd.ssd_replay_prefill(shape, cache, synth.cu_seqlens(pre), x[ip], dt[ip], B[ip], C[ip],
                           A, D, bias)
    live = rng.permutation(S)[:800]                   # slots decoded in these steps
    for k in range(steps):
        pos = rng.permutation(nb)
        slots = np.full(nb, -1, dtype=np.int32)
        slots[pos[800:850]] = S                       # other out-of-range entries
        slots[pos[:800]] = live
        tok = np.zeros(nb, dtype=np.int64)
        tok[pos[:800]] = cu[live] + pre[live] + k
        it = torch.from_numpy(tok).to(DEV)
        y = torch.full((nb, H, P), float("nan"), dtype=torch.bfloat16, device=DEV)
        erd.ssd_replay_decode(shape, cache, x[it], dt[it], B[it], C[it], A, D, bias,
                              slot_idx=torch.from_numpy(slots).to(DEV), y=y)
        pv = torch.from_numpy(pos[:800]).to(DEV)
        assert same_bits(y[pv], y_ss[it[pv]]), k
        skipped = torch.from_numpy(pos[800:]).to(DEV)
        assert torch.isnan(y[skipped].float()).all()
        assert not cache.work.any()
    n = cache.buf_len.cpu().numpy()
    assert np.array_equal(n[live], (pre[live] + steps) % Q)
    rest = np.setdiff1d(np.arange(S), live)
    assert np.array_equal(n[rest], pre[rest] % Q)

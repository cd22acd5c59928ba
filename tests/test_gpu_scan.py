"""GPU parity and bit-identity of the chunked scan (prefill), through the
C ABI: against the fp64 oracle within tolerance, and against itself
bit for bit under splits, prefixes and packing."""
import numpy as np
import pytest
import torch

import exact_replay_decode_amd as erd
from gpu_cases import (DEV, check_bf16, chunk_rows, error_scales, headwise_max_rel,
                       make_problem, mean_rel_err, same_bits, seq_spans, split_lengths,
                       y_headwise_max_rel)

pytestmark = pytest.mark.gpu

BF16_MEAN_REL = 3e-3   # mean|dy| / mean|y| for bf16 outputs
STATE_REL = 1e-4       # per (seq, head) max|dS| / max|S|
F32_Y_REL = 1e-4       # per (seq, head) max|dy| / max|y| for fp32 outputs


def prefill(pr, a=None, b=None, cu=None, init=None):
    x, dt, B, C = pr.dev(a, b)
    cu = pr.cu if cu is None else cu
    return erd.ssd_prefill_varlen(pr.shape, cu, x, dt, pr.A, B, C, pr.D, pr.bias,
                                  init_state=init)


def replay_in_pieces(pr, pieces, cache=None, slot=0):
    """Feed one sequence (packed stream 0) through ssd_replay_prefill in
    pieces; returns (y, cache)."""
    cache = cache or erd.ReplayCache(pr.shape, 1, DEV, with_C=True)
    ys, t = [], 0
    sl = torch.tensor([slot], dtype=torch.int32, device=DEV)
    for L in pieces:
        x, dt, B, C = pr.dev(t, t + L)
        ys.append(erd.ssd_replay_prefill(pr.shape, cache, [0, L], x, dt, B, C, pr.A, pr.D,
                                         pr.bias, slot_idx=sl))
        t += L
    return torch.cat(ys), cache


# ---- C0: tiny fp32 scan --------------------------------------------------

def test_c0_fp32_matches_oracle_and_splits():
    pr = make_problem([64], H=4, G=1, P=16, N=16, Q=16, io="f32")
    y, fin, bnd = prefill(pr)
    ref = pr.oracle()
    assert y_headwise_max_rel(y, ref.y, pr.cu) <= F32_Y_REL
    assert headwise_max_rel(fin.cpu().numpy(), ref.final_state) <= STATE_REL
    assert headwise_max_rel(bnd.cpu().numpy(), ref.boundary_state) <= STATE_REL
    for pieces in ([24, 40], [1] * 64, [16, 16, 32], [7, 9, 48], [63, 1]):
        y2, cache = replay_in_pieces(pr, pieces)
        assert same_bits(y2, y), pieces
        assert same_bits(cache.state[0], bnd[0])
        assert int(cache.buf_len[0]) == 0 and int(cache.boundary_pos[0]) == 64


def test_c0_every_single_split():
    pr = make_problem([64], H=4, G=1, P=16, N=16, Q=16, io="f32", seed=1)
    y, _, _ = prefill(pr)
    for s in range(1, 64):
        y2, _ = replay_in_pieces(pr, [s, 64 - s])
        assert same_bits(y2, y), s


# ---- C1: one long sequence, bf16 I/O --------------------------------------

@pytest.fixture(scope="module")
def c1():
    pr = make_problem([2048], H=32, G=1, P=64, N=128, Q=256)
    y, fin, bnd = prefill(pr)
    return pr, y, fin, bnd


def check_chunk_states(pr, y, bnd, ref):
    """The prefill's chunk_states output: against the oracle's state after
    every full chunk (per (seq, head) 1e-4), the last full chunk of each
    sequence bit for bit equal to its boundary state, and y unchanged by
    asking for them."""
    x, dt, B, C = pr.dev(None)
    y2, _, bnd2, cs = erd.ssd_prefill_varlen(pr.shape, pr.cu, x, dt, pr.A, B, C, pr.D, pr.bias,
                                             want_chunk_states=True)
    assert same_bits(y2, y) and same_bits(bnd2, bnd)
    rows = chunk_rows(pr.cu, pr.shape.chunk_size)
    assert cs.shape[0] == len(rows)
    got = cs.cpu().numpy()
    want = np.stack([ref.chunk_states[s, c] for s, c, _ in rows])
    assert headwise_max_rel(got, want) <= STATE_REL
    for s in range(len(pr.lengths)):
        mine = [r for t, _, r in rows if t == s]
        if mine:
            assert same_bits(cs[mine[-1]], bnd[s]), s
    return cs


def test_c1_oracle_parity(c1):
    pr, y, fin, bnd = c1
    ref = pr.oracle(max_chunks=8)
    err = mean_rel_err(y, ref.y)
    print(f"C1 mean|dy|/mean|y| = {100 * err:.4f} %")
    assert err <= BF16_MEAN_REL
    assert headwise_max_rel(fin.cpu().numpy(), ref.final_state) <= STATE_REL
    assert headwise_max_rel(bnd.cpu().numpy(), ref.boundary_state) <= STATE_REL
    check_bf16(y, ref.y, error_scales(pr), seq_spans(pr.cu), label="C1")
    check_chunk_states(pr, y, bnd, ref)


@pytest.mark.parametrize("step", [256, 100, 257])
def test_c1_repeated_splits_bitwise(c1, step):
    pr, y, fin, bnd = c1
    y2, cache = replay_in_pieces(pr, split_lengths(2048, step))
    assert same_bits(y2, y)
    assert same_bits(cache.state[0], bnd[0])
    assert int(cache.buf_len[0]) == 0 and int(cache.boundary_pos[0]) == 2048


@pytest.mark.parametrize("s", [1, 100, 255, 256, 257, 1000, 2047])
def test_c1_single_split_bitwise(c1, s):
    pr, y, _, _ = c1
    y2, _ = replay_in_pieces(pr, [s, 2048 - s])
    assert same_bits(y2, y)


def test_c1_aligned_split_through_plain_prefill(c1):
    """An aligned split run with the plain API: the second call starts from
    the first call's fp32 final state."""
    pr, y, fin, _ = c1
    y_a, fin_a, _ = prefill(pr, 0, 768, cu=[0, 768])
    y_b, fin_b, _ = prefill(pr, 768, 2048, cu=[0, 1280], init=fin_a)
    assert same_bits(torch.cat([y_a, y_b]), y)
    assert same_bits(fin_b, fin)


def test_c1_prefix_invariance(c1):
    """Prefixes 1..511 give the 512-token run's rows bit for bit."""
    pr, y, _, _ = c1
    for L in range(1, 512):
        yL, _, _ = prefill(pr, 0, L, cu=[0, L])
        assert same_bits(yL, y[:L]), L


def test_c1_bf16_state_resume_breaks_aligned_split(c1):
    """Negative control: resuming from a bf16-rounded state changes bits
    after an aligned split (the fp32 state is what keeps splits exact)."""
    pr, y, _, _ = c1
    _, fin_a, _ = prefill(pr, 0, 512, cu=[0, 512])
    rounded = fin_a.to(torch.bfloat16).to(torch.float32)
    y_b, _, _ = prefill(pr, 512, 2048, cu=[0, 1536], init=rounded)
    assert not same_bits(y_b, y[512:])


def test_c1_empty_and_tiny_sequences():
    pr = make_problem([0, 1, 0, 300, 0], H=32, G=1, P=64, N=128, Q=256)
    y, fin, bnd = prefill(pr)
    ref = pr.oracle()
    assert mean_rel_err(y, ref.y) <= BF16_MEAN_REL
    f = fin.cpu().numpy()
    assert np.all(f[0] == 0) and np.all(f[2] == 0) and np.all(f[4] == 0)
    assert headwise_max_rel(f[[1, 3]], ref.final_state[[1, 3]]) <= STATE_REL
    b = bnd.cpu().numpy()
    assert np.all(b[3] != 0) and np.all(b[1] == 0)
    assert headwise_max_rel(b[[3]], ref.boundary_state[[3]]) <= STATE_REL


# ---- C2: grouped heads, varlen pack ---------------------------------------

@pytest.fixture(scope="module")
def c2():
    lengths = [600, 300, 900, 248]
    pr = make_problem(lengths, H=64, G=8, P=64, N=128, Q=256, seed=2)
    y, fin, bnd = prefill(pr)
    return pr, y, fin, bnd


def test_c2_oracle_parity(c2):
    pr, y, fin, bnd = c2
    ref = pr.oracle(max_chunks=4)
    err = mean_rel_err(y, ref.y)
    print(f"C2 mean|dy|/mean|y| = {100 * err:.4f} %")
    assert err <= BF16_MEAN_REL
    assert headwise_max_rel(fin.cpu().numpy(), ref.final_state) <= STATE_REL
    assert headwise_max_rel(bnd.cpu().numpy(), ref.boundary_state) <= STATE_REL
    check_bf16(y, ref.y, error_scales(pr), seq_spans(pr.cu), label="C2")
    check_chunk_states(pr, y, bnd, ref)


def test_ssd_error_level_printed_by_the_rfc(c1, c2):
    """[RFC] section 2, item 1 prints the chunked scan at 0.166-0.169 % of
    mean |y| against fp64 on these two shapes (H=32 G=1 and H=64 G=8, P=64,
    N=128, chunk 256, 2048 tokens, bf16 I/O), against a 0.141 % floor from
    rounding the outputs alone. This engine rounds the same two operands to
    bf16 as the chunked kernel there (the read-out state and the masked
    C.B^T weights), so it lands in the same place: within 0.02 points of
    the printed band (one seed here, one there), and above the floor."""
    levels, floors = {}, {}
    for name, (pr, y, _, _) in (("C1", c1), ("C2", c2)):
        ref = pr.oracle()
        levels[name] = mean_rel_err(y, ref.y)
        floors[name] = mean_rel_err(torch.from_numpy(ref.y).to(torch.bfloat16), ref.y)
    print("chunked-scan error vs fp64: " +
          ", ".join(f"{k} {100 * v:.4f} % (floor {100 * floors[k]:.4f} %)"
                    for k, v in levels.items()), flush=True)
    for k, v in levels.items():
        assert 1.46e-3 <= v <= 1.89e-3, levels
        assert v > floors[k]


def test_c2_packing_invariance(c2):
    pr, y, fin, bnd = c2
    cu = pr.cu
    for s, L in enumerate(pr.lengths):
        a, b = int(cu[s]), int(cu[s + 1])
        ys, fs, bs = prefill(pr, a, b, cu=[0, L])
        assert same_bits(ys, y[a:b]), s
        assert same_bits(fs[0], fin[s]) and same_bits(bs[0], bnd[s])


def test_c2_permuted_pack(c2):
    pr, y, fin, _ = c2
    cu = pr.cu
    order = [2, 0, 3, 1]
    idx = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in order])
    x, dt, B, C = pr.dev(None)
    it = torch.from_numpy(idx).to(DEV)
    lens = [pr.lengths[s] for s in order]
    cu2 = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    y2, fin2, _ = erd.ssd_prefill_varlen(pr.shape, cu2, x[it].contiguous(), dt[it].contiguous(),
                                         pr.A, B[it].contiguous(), C[it].contiguous(), pr.D,
                                         pr.bias)
    assert same_bits(y2, y[it])
    for k, s in enumerate(order):
        assert same_bits(fin2[k], fin[s])


def test_c2_group_map_zeroed_group():
    """Heads of a group whose B is zero produce exactly D*x (rounded)."""
    pr = make_problem([300], H=64, G=8, P=64, N=128, Q=256, seed=3)
    x, dt, B, C = pr.dev(None)
    B = B.clone()
    B[:, 3] = 0
    y, _, _ = erd.ssd_prefill_varlen(pr.shape, pr.cu, x, dt, pr.A, B, C, pr.D, pr.bias)
    want = (pr.D[None, 24:32, None] * x[:, 24:32].float()).to(torch.bfloat16)
    assert same_bits(y[:, 24:32], want)
    assert not same_bits(y[:, 16:24], (pr.D[None, 16:24, None] * x[:, 16:24].float()).to(torch.bfloat16))


# ---- W1b-shaped launch: 256 x 2048 tokens, sampled oracle checks ----------

def test_full_batch_prefill_sampled_parity():
    """The 256 x 2048-token launch the bench times, checked on sampled
    sequences against the oracle and for packing invariance."""
    from exact_replay_decode_amd import synth
    from oracle import scan
    S, T, H, P, N, Q = 256, 2048, 32, 64, 128, 256
    shape = erd.Shape(H, 1, P, N, Q, "bf16", "bf16")
    hp = synth.make_head_params(H, 0)
    x, dt, B, C = synth.make_tokens_torch(S * T, H, 1, P, N, 0, DEV)
    cu = synth.cu_seqlens([T] * S)
    A, D, bias = (torch.from_numpy(v).to(DEV) for v in (hp.A, hp.D, hp.dt_bias))
    y, fin, _ = erd.ssd_prefill_varlen(shape, cu, x, dt, A, B, C, D, bias)
    from oracle.bounds import chunk_error_scales
    for s in (0, 77, 255):
        sl = slice(s * T, (s + 1) * T)
        args = (erd.to_f64(x[sl]), erd.to_f64(dt[sl]), hp.A, erd.to_f64(B[sl]),
                erd.to_f64(C[sl]), [0, T], Q)
        ref = scan(*args, D=hp.D, dt_bias=hp.dt_bias)
        assert mean_rel_err(y[sl], ref.y) <= BF16_MEAN_REL
        check_bf16(y[sl], ref.y, chunk_error_scales(*args, D=hp.D, dt_bias=hp.dt_bias),
                   [(0, T)], label=f"256 x 2048 launch, sequence {s}")
        assert headwise_max_rel(fin[s:s + 1].cpu().numpy(), ref.final_state) <= STATE_REL
        ys, fs, _ = erd.ssd_prefill_varlen(shape, [0, T], x[sl], dt[sl], A, B[sl], C[sl], D,
                                           bias)
        assert same_bits(ys, y[sl]) and same_bits(fs[0], fin[s])


# ---- whole heads and split columns ----------------------------------------

def test_split_columns_equal_whole_heads():
    """With few (sequence, head) pairs the prefill runs each head as two
    workgroups on its column halves, with many as one workgroup per head.
    Each sequence of an 8-sequence pack (H=32: 256 pairs, whole heads) run
    alone (32 pairs, split columns) gives the same outputs, final, boundary
    and chunk states bit for bit, from seeded initial states; and continuing
    a replay cache sequence by sequence (split) or as one pack (whole) leaves
    the same outputs and cache."""
    H, G, P, N, Q = 32, 1, 64, 128, 256
    lengths = [700, 300, 900, 256, 130, 512, 1000, 77]
    S = len(lengths)
    pr = make_problem(lengths, H=H, G=G, P=P, N=N, Q=Q, seed=11)
    x, dt, B, C = pr.dev(None)
    g = torch.Generator(device="cpu").manual_seed(5)
    init = (torch.randn((S, H, P, N), generator=g) * 0.1).to(DEV)
    y, fin, bnd, cst = erd.ssd_prefill_varlen(pr.shape, pr.cu, x, dt, pr.A, B, C, pr.D, pr.bias,
                                              init_state=init, want_chunk_states=True)
    cu = pr.cu
    f0 = 0
    for s in range(S):
        a, b = int(cu[s]), int(cu[s + 1])
        ys, fs, bs, cs = erd.ssd_prefill_varlen(pr.shape, [0, b - a], x[a:b], dt[a:b], pr.A,
                                                B[a:b], C[a:b], pr.D, pr.bias,
                                                init_state=init[s:s + 1].contiguous(),
                                                want_chunk_states=True)
        nf = (b - a) // Q
        assert same_bits(ys, y[a:b]), s
        assert same_bits(fs, fin[s:s + 1]) and same_bits(bs, bnd[s:s + 1]), s
        assert same_bits(cs, cst[f0:f0 + nf]), s
        f0 += nf
    # replay: the first 60 % of every sequence as one pack, then the rest as
    # one pack (cache A) or sequence by sequence (cache B)
    first = [int(L * 0.6) for L in lengths]
    rest = [L - f for L, f in zip(lengths, first)]
    i1 = torch.from_numpy(np.concatenate([np.arange(cu[s], cu[s] + first[s])
                                          for s in range(S)])).to(DEV)
    i2 = [torch.arange(int(cu[s]) + first[s], int(cu[s + 1]), device=DEV) for s in range(S)]
    caches = []
    for mode in ("pack", "each"):
        cache = erd.ReplayCache(pr.shape, S, DEV, with_C=True)
        erd.ssd_replay_prefill(pr.shape, cache, np.cumsum([0] + first), x[i1], dt[i1], B[i1],
                               C[i1], pr.A, pr.D, pr.bias)
        if mode == "pack":
            i = torch.cat(i2)
            y2 = erd.ssd_replay_prefill(pr.shape, cache, np.cumsum([0] + rest), x[i], dt[i],
                                        B[i], C[i], pr.A, pr.D, pr.bias)
        else:
            y2 = torch.cat([erd.ssd_replay_prefill(
                pr.shape, cache, [0, rest[s]], x[i2[s]], dt[i2[s]], B[i2[s]], C[i2[s]], pr.A,
                pr.D, pr.bias, slot_idx=torch.tensor([s], dtype=torch.int32, device=DEV))
                for s in range(S)])
        caches.append((y2, cache))
    (ya, ca), (yb, cb) = caches
    assert same_bits(ya, yb)
    for name in ("state", "state_bf", "buf_len", "boundary_pos", "work"):
        assert same_bits(getattr(ca, name), getattr(cb, name)), name

"""Pins of the fp64 oracle to facts outside itself (CPU only).

Each test ties the sequential oracle to something it cannot agree with by
construction: a hand-worked dyadic example, an independent chunked closed
form, textbook special cases, linearity, and numbers the pages print.
"""
import json
import math
import os

import numpy as np
import pytest

from exact_replay_decode_amd import synth
from oracle import closed_form, scan

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rand_problem(seed, lengths, H, G, P, N, init=False, scale_dt=1.0):
    rng = np.random.default_rng(seed)
    T = int(sum(lengths))
    x = rng.standard_normal((T, H, P))
    dt = 0.5 * rng.standard_normal((T, H)) * scale_dt
    B = rng.standard_normal((T, G, N))
    C = rng.standard_normal((T, G, N))
    A = -rng.uniform(1, 16, H)
    D = rng.uniform(0.5, 1.5, H)
    bias = np.log(np.expm1(np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), H))))
    S = len(lengths)
    h0 = rng.standard_normal((S, H, P, N)) if init else None
    cu = np.concatenate([[0], np.cumsum(lengths)])
    return dict(x=x, dt=dt, B=B, C=C, A=A, D=D, dt_bias=bias, cu=cu, init=h0)


def test_dyadic_worked_example_bitexact():
    g = json.load(open(os.path.join(GOLD, "dyadic_recurrence.json")))
    T = len(g["x"])
    x = np.array(g["x"]).reshape(T, 1, 1)
    dt = np.array(g["dt"]).reshape(T, 1)
    B = np.array(g["B"]).reshape(T, 1, 1)
    C = np.array(g["C"]).reshape(T, 1, 1)
    r = scan(x, dt, np.array([g["A"]]), B, C, [0, T], g["chunk_size"],
             D=np.array([g["D"]]), dt_softplus=False, max_chunks=2)
    assert r.y.ravel().tolist() == g["y"]
    assert r.final_state.ravel().tolist() == [g["h"][-1]]
    assert r.boundary_state.ravel().tolist() == [g["boundary_state_after_4"]]
    assert r.chunk_states.ravel().tolist() == g["chunk_states"]
    assert r.boundary_len.tolist() == [0]


@pytest.mark.parametrize("Q,G,lengths,P,N", [
    (4, 1, [13], 4, 4), (16, 2, [64], 8, 16), (16, 1, [5, 33, 16], 16, 8),
    (8, 2, [1, 17], 4, 12)])
@pytest.mark.parametrize("init", [False, True])
def test_closed_form_equals_sequential(Q, G, lengths, P, N, init):
    H = 2 * G
    pr = _rand_problem(7, lengths, H, G, P, N, init=init)
    r = scan(pr["x"], pr["dt"], pr["A"], pr["B"], pr["C"], pr["cu"], Q,
             D=pr["D"], dt_bias=pr["dt_bias"], init=pr["init"],
             max_chunks=max(lengths) // Q)
    y2, fin2, ends = closed_form.chunked_scan(
        pr["x"], pr["dt"], pr["A"], pr["B"], pr["C"], pr["cu"], Q, D=pr["D"],
        dt_bias=pr["dt_bias"], init=pr["init"])
    scale = np.abs(r.y).max()
    assert np.abs(r.y - y2).max() <= 1e-12 * scale
    assert np.abs(r.final_state - fin2).max() <= 1e-12 * max(np.abs(fin2).max(), 1e-300)
    for s, seq_ends in enumerate(ends):
        for c, st in enumerate(seq_ends):
            assert np.abs(r.chunk_states[s, c] - st).max() <= 1e-12 * np.abs(st).max()
        if seq_ends:
            np.testing.assert_array_equal(r.boundary_state[s], r.chunk_states[s, len(seq_ends) - 1])
        assert r.boundary_len[s] == lengths[s] % Q


def test_split_continuation_is_bitexact():
    pr = _rand_problem(3, [57], 3, 1, 8, 8)
    full = scan(pr["x"], pr["dt"], pr["A"], pr["B"], pr["C"], pr["cu"], 16,
                D=pr["D"], dt_bias=pr["dt_bias"])
    for split in (1, 16, 24, 40, 56):
        a = scan(pr["x"][:split], pr["dt"][:split], pr["A"], pr["B"][:split],
                 pr["C"][:split], [0, split], 16, D=pr["D"], dt_bias=pr["dt_bias"])
        b = scan(pr["x"][split:], pr["dt"][split:], pr["A"], pr["B"][split:],
                 pr["C"][split:], [0, 57 - split], 16, D=pr["D"],
                 dt_bias=pr["dt_bias"], init=a.final_state)
        np.testing.assert_array_equal(np.concatenate([a.y, b.y]), full.y)
        np.testing.assert_array_equal(b.final_state, full.final_state)


def test_prefix_invariance_bitexact():
    pr = _rand_problem(4, [40], 2, 1, 4, 8)
    full = scan(pr["x"], pr["dt"], pr["A"], pr["B"], pr["C"], pr["cu"], 8,
                D=pr["D"], dt_bias=pr["dt_bias"])
    for L in range(1, 40):
        r = scan(pr["x"][:L], pr["dt"][:L], pr["A"], pr["B"][:L], pr["C"][:L],
                 [0, L], 8, D=pr["D"], dt_bias=pr["dt_bias"])
        np.testing.assert_array_equal(r.y, full.y[:L])


def test_packing_changes_nothing():
    pr = _rand_problem(5, [9, 30, 17], 4, 2, 4, 4, init=True)
    packed = scan(pr["x"], pr["dt"], pr["A"], pr["B"], pr["C"], pr["cu"], 8,
                  D=pr["D"], dt_bias=pr["dt_bias"], init=pr["init"])
    cu = pr["cu"]
    for s in range(3):
        a, b = cu[s], cu[s + 1]
        r = scan(pr["x"][a:b], pr["dt"][a:b], pr["A"], pr["B"][a:b],
                 pr["C"][a:b], [0, b - a], 8, D=pr["D"], dt_bias=pr["dt_bias"],
                 init=pr["init"][s:s + 1])
        np.testing.assert_array_equal(r.y, packed.y[a:b])
        np.testing.assert_array_equal(r.final_state[0], packed.final_state[s])


def test_single_token_zero_state():
    """T=1 from zero: y = delta (C.B) x + D x, delta = softplus(dt + bias)."""
    pr = _rand_problem(11, [1], 3, 1, 5, 7)
    r = scan(pr["x"], pr["dt"], pr["A"], pr["B"], pr["C"], pr["cu"], 4,
             D=pr["D"], dt_bias=pr["dt_bias"])
    delta = np.logaddexp(0.0, pr["dt"][0] + pr["dt_bias"])
    cb = float(pr["C"][0, 0] @ pr["B"][0, 0])
    want = (delta * cb + pr["D"])[:, None] * pr["x"][0]
    np.testing.assert_allclose(r.y[0], want, rtol=4e-16 * 8, atol=0)
    want_state = (delta[:, None, None] * pr["x"][0][:, :, None]
                  * pr["B"][0, 0][None, None, :])
    np.testing.assert_allclose(r.final_state[0], want_state, rtol=4e-16, atol=0)


def test_no_decay_is_masked_linear_attention():
    """A = 0: y = tril(C B^T) (delta * x) + D x, a plain masked matmul."""
    pr = _rand_problem(12, [37], 2, 1, 6, 9)
    A0 = np.zeros(2)
    r = scan(pr["x"], pr["dt"], A0, pr["B"], pr["C"], pr["cu"], 8,
             D=pr["D"], dt_bias=pr["dt_bias"])
    delta = np.logaddexp(0.0, pr["dt"] + pr["dt_bias"][None, :])
    Cm, Bm = pr["C"][:, 0], pr["B"][:, 0]
    M = np.tril(Cm @ Bm.T)
    for h in range(2):
        want = M @ (delta[:, h:h + 1] * pr["x"][:, h]) + pr["D"][h] * pr["x"][:, h]
        assert np.abs(r.y[:, h] - want).max() <= 1e-13 * np.abs(want).max()


def test_zero_input_is_pure_decay():
    """x = 0 from h0: y_t = exp(A sum_{r<=t} delta_r) (h0 . C_t)."""
    pr = _rand_problem(13, [29], 2, 1, 3, 5, init=True)
    x0 = np.zeros_like(pr["x"])
    r = scan(x0, pr["dt"], pr["A"], pr["B"], pr["C"], pr["cu"], 8,
             D=pr["D"], dt_bias=pr["dt_bias"], init=pr["init"])
    delta = np.logaddexp(0.0, pr["dt"] + pr["dt_bias"][None, :])
    for h in range(2):
        lam = np.cumsum(delta[:, h]) * pr["A"][h]
        want = np.exp(lam)[:, None] * (pr["C"][:, 0] @ pr["init"][0, h].T)
        assert np.abs(r.y[:, h] - want).max() <= 1e-13 * np.abs(want).max()


def test_scalar_geometric_series():
    """H=P=N=1 with constant a = exp(dA), b = dx B: h_t = a^t h0 + b (1-a^t)/(1-a)."""
    T, d, A, xv, Bv, Cv, h0 = 50, 0.3, -0.7, 1.3, 0.9, 1.0, 2.0
    r = scan(np.full((T, 1, 1), xv), np.full((T, 1), d), np.array([A]),
             np.full((T, 1, 1), Bv), np.full((T, 1, 1), Cv), [0, T], 16,
             dt_softplus=False, init=np.full((1, 1, 1, 1), h0))
    a, b = math.exp(d * A), d * xv * Bv
    t = np.arange(1, T + 1)
    want = a ** t * h0 + b * (1 - a ** t) / (1 - a)
    assert np.abs(r.y.ravel() - want).max() <= 1e-13 * np.abs(want).max()


@pytest.mark.parametrize("which", ["B", "C"])
def test_zero_B_or_C_leaves_skip_term(which):
    pr = _rand_problem(14, [21], 2, 1, 4, 4)
    pr[which] = np.zeros_like(pr[which])
    r = scan(pr["x"], pr["dt"], pr["A"], pr["B"], pr["C"], pr["cu"], 8,
             D=pr["D"], dt_bias=pr["dt_bias"])
    np.testing.assert_array_equal(r.y, pr["D"][None, :, None] * pr["x"])


def test_contiguous_head_to_group_map():
    """Heads h read group h // (H/G): zeroing group 1's B leaves heads 2,3
    (and only them) with y = D x when H=4, G=2."""
    pr = _rand_problem(15, [19], 4, 2, 3, 4)
    pr["B"][:, 1] = 0.0
    r = scan(pr["x"], pr["dt"], pr["A"], pr["B"], pr["C"], pr["cu"], 8,
             D=pr["D"], dt_bias=pr["dt_bias"])
    skip = pr["D"][None, :, None] * pr["x"]
    np.testing.assert_array_equal(r.y[:, 2:], skip[:, 2:])
    assert np.abs(r.y[:, :2] - skip[:, :2]).max() > 1e-3


def test_state_layout_is_p_by_n():
    """State[p, n] accumulates delta x[p] B[n]: with one token and P != N the
    final state is the outer product x (outer) B, not its transpose."""
    x = np.arange(1, 4, dtype=float).reshape(1, 1, 3)
    B = np.array([1.0, 10.0, 100.0, 1000.0, 1e4]).reshape(1, 1, 5)
    C = np.zeros((1, 1, 5))
    r = scan(x, np.ones((1, 1)), np.array([-1.0]), B, C, [0, 1], 4,
             dt_softplus=False)
    np.testing.assert_array_equal(r.final_state[0, 0], np.outer(x.ravel(), B.ravel()))


def test_linearity():
    pr = _rand_problem(16, [23], 2, 1, 4, 6, init=True)
    kw = dict(D=pr["D"], dt_bias=pr["dt_bias"])
    rng = np.random.default_rng(99)
    x2 = rng.standard_normal(pr["x"].shape)
    h2 = rng.standard_normal(pr["init"].shape)
    r1 = scan(pr["x"], pr["dt"], pr["A"], pr["B"], pr["C"], pr["cu"], 8, init=pr["init"], **kw)
    r2 = scan(x2, pr["dt"], pr["A"], pr["B"], pr["C"], pr["cu"], 8, init=h2, **kw)
    r12 = scan(pr["x"] + x2, pr["dt"], pr["A"], pr["B"], pr["C"], pr["cu"], 8,
               init=pr["init"] + h2, **kw)
    s = np.abs(r12.y).max()
    assert np.abs(r12.y - (r1.y + r2.y)).max() <= 1e-12 * s
    assert np.abs(r12.final_state - (r1.final_state + r2.final_state)).max() <= \
        1e-12 * np.abs(r12.final_state).max()


def test_bf16_rounding_floor_matches_printed_value():
    """Rounding N(0,1) to bf16 gives mean|err|/mean|x| = 0.141 percent, the
    floor the RFC prints; pins the quantiser and the error metric."""
    g = json.load(open(os.path.join(GOLD, "rfc_printed_numbers.json")))
    rng = np.random.default_rng(0)
    v = rng.standard_normal(2_000_000)
    q = synth.bf16_bits_to_f64(synth.bf16_bits_from_f64(v))
    pct = 100 * np.abs(q - v).mean() / np.abs(v).mean()
    assert abs(pct - g["bf16_rounding_floor_percent"]["value"]) < 0.0015


def test_bf16_round_to_nearest_even_cases():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8,
                     1.0 + 2 ** -8 + 2 ** -20, 0.0, -0.0, 65504.0])
    want = np.array([1.0, 1.0, 1.0 + 2 ** -6, -1.0, 1.0 + 2 ** -7, 0.0, -0.0, 65536.0])
    got = synth.bf16_bits_to_f64(synth.bf16_bits_from_f64(vals))
    np.testing.assert_array_equal(got, want)
    assert np.signbit(got[6])


def test_generator_retention_of_slow_heads():
    """Slowest head keeps roughly 42-73 percent of its state per 256-token
    chunk (RFC section 2, item 4); a loose check of the dt recipe."""
    for seed in (0, 1, 2):
        hp = synth.make_head_params(32, seed)
        tok = synth.make_tokens(2048, 32, 1, 1, 1, seed)
        _, dt, _, _ = tok.f64()
        delta = np.logaddexp(0.0, dt + hp.dt_bias.astype(np.float64)[None, :])
        per_chunk = np.exp((delta * hp.A.astype(np.float64)).reshape(8, 256, 32).sum(1))
        slowest = np.median(per_chunk, axis=0).max()
        assert 0.35 <= slowest <= 0.85, slowest
        assert np.all(hp.A < 0) and np.all(hp.A >= -16) and np.all(hp.A <= -1)
        sp = np.logaddexp(0.0, hp.dt_bias.astype(np.float64))
        assert np.all(sp > 0.99e-3) and np.all(sp < 1.01e-1)


def test_streams_are_batch_independent():
    a = synth.make_tokens(10, 2, 1, 4, 4, seed=5, stream=3)
    b = synth.make_tokens(10, 2, 1, 4, 4, seed=5, stream=3)
    c = synth.make_tokens(10, 2, 1, 4, 4, seed=5, stream=4)
    np.testing.assert_array_equal(a.x, b.x)
    assert not np.array_equal(a.x, c.x)


def test_softplus_both_branches():
    """delta = softplus(dt + bias) on both signs of the argument, against
    numpy's logaddexp(0, u) (single token from zero state)."""
    u = np.array([-40.0, -20.0, -3.0, -0.5, 0.0, 0.5, 3.0, 20.0, 40.0])
    H = u.size
    x = np.ones((1, H, 1))
    B = np.ones((1, 1, 1))
    C = np.ones((1, 1, 1))
    r = scan(x, u.reshape(1, H), -np.ones(H), B, C, [0, 1], 4,
             dt_bias=np.zeros(H))
    np.testing.assert_allclose(r.y.ravel(), np.logaddexp(0.0, u), rtol=4e-16, atol=0)

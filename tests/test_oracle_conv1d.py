"""Pins of the conv1d oracle (oracle/conv1d.py) to facts outside itself:
numpy's full convolution, scipy's logistic function, closed forms of
special kernels, and the continuation property a causal filter must have.
Each plausible slip (reversed kernel taps, dropped bias, state rows in the
wrong order, a missing activation, an x/B/C split at the wrong channel)
fails at least one of them."""
import numpy as np
import pytest
from scipy.special import expit

from oracle.conv1d import conv1d_seq, conv1d_varlen, silu, split_xbc


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("W", [2, 3, 4])
def test_matches_numpy_convolve_from_zero_state(W):
    L, Cd = 37, 5
    inp, w, b = rnd(1, L, Cd), rnd(2, Cd, W), rnd(3, Cd)
    out, _ = conv1d_seq(inp, w, b, activation=False)
    for c in range(Cd):
        # np.convolve(a, v)[n] = sum_m a[m] v[n - m]; the causal filter uses
        # tap w[c, i] on input n - (W - 1) + i, i.e. v = w[c, ::-1]
        ref = b[c] + np.convolve(inp[:, c], w[c, ::-1])[:L]
        np.testing.assert_allclose(out[:, c], ref, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("W", [2, 4])
def test_tap_on_current_token_is_identity_and_tap_zero_is_a_shift(W):
    L, Cd = 9, 3
    inp, st = rnd(4, L, Cd), rnd(5, Cd, W - 1)
    ident = np.zeros((Cd, W))
    ident[:, W - 1] = 1.0
    out, fin = conv1d_seq(inp, ident, None, st, activation=False)
    assert np.array_equal(out, inp)
    shift = np.zeros((Cd, W))
    shift[:, 0] = 1.0
    out, _ = conv1d_seq(inp, shift, None, st, activation=False)
    # output t sees the input W-1 steps back; the first W-1 come from the
    # state, oldest first
    assert np.array_equal(out[:W - 1], st.T)
    assert np.array_equal(out[W - 1:], inp[:L - (W - 1)])
    assert np.array_equal(fin, inp[L - (W - 1):].T)


def test_constant_input_gives_bias_plus_tap_sum():
    Cd, W = 4, 4
    w, b = rnd(6, Cd, W), rnd(7, Cd)
    inp = np.full((6, Cd), 0.75)
    st = np.full((Cd, W - 1), 0.75)
    out, _ = conv1d_seq(inp, w, b, st, activation=False)
    np.testing.assert_allclose(out, np.tile(b + 0.75 * w.sum(1), (6, 1)), rtol=1e-14)


def test_activation_is_silu():
    v = np.linspace(-30, 30, 121)
    np.testing.assert_allclose(silu(v), v * expit(v), rtol=1e-12, atol=1e-300)
    assert silu(np.array([0.0]))[0] == 0.0
    inp, w, b = rnd(8, 11, 6), rnd(9, 6, 4), rnd(10, 6)
    lin, _ = conv1d_seq(inp, w, b, activation=False)
    act, _ = conv1d_seq(inp, w, b, activation=True)
    np.testing.assert_allclose(act, lin * expit(lin), rtol=1e-12)


@pytest.mark.parametrize("W", [2, 3, 4])
def test_split_continuation_is_exact(W):
    """Running a prefix, then the rest from the prefix's final state, gives
    the bits of the whole run (every output is the same fp64 sum)."""
    L, Cd = 40, 7
    inp, w, b, st = rnd(11, L, Cd), rnd(12, Cd, W), rnd(13, Cd), rnd(14, Cd, W - 1)
    whole, fin = conv1d_seq(inp, w, b, st)
    for a in (0, 1, W - 2, W - 1, 17, L - 1, L):
        o1, f1 = conv1d_seq(inp[:a], w, b, st)
        o2, f2 = conv1d_seq(inp[a:], w, b, f1)
        assert np.array_equal(np.concatenate([o1, o2]), whole)
        assert np.array_equal(f2, fin)


def test_short_sequences_keep_older_state_rows():
    Cd, W = 3, 4
    st = rnd(15, Cd, W - 1)
    inp = rnd(16, 1, Cd)
    _, fin = conv1d_seq(inp, rnd(17, Cd, W), None, st)
    assert np.array_equal(fin, np.concatenate([st[:, 1:], inp.T], axis=1))
    _, fin0 = conv1d_seq(np.zeros((0, Cd)), rnd(17, Cd, W), None, st)
    assert np.array_equal(fin0, st)


def test_varlen_is_per_sequence():
    Cd, W = 5, 4
    lengths = [7, 0, 1, 12]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    inp, w, b = rnd(18, int(cu[-1]), Cd), rnd(19, Cd, W), rnd(20, Cd)
    sts = rnd(21, 4, Cd, W - 1)
    out, fin = conv1d_varlen(inp, w, cu, b, sts)
    for s in range(4):
        o, f = conv1d_seq(inp[cu[s]:cu[s + 1]], w, b, sts[s])
        assert np.array_equal(out[cu[s]:cu[s + 1]], o) and np.array_equal(fin[s], f)


def test_split_xbc_channel_order():
    H, G, P, N = 2, 1, 3, 4
    out = np.arange(2 * (H * P + 2 * G * N), dtype=np.float64).reshape(2, -1)
    x, B, C = split_xbc(out, H, G, P, N)
    assert x[1, 1, 2] == out[1, 1 * P + 2]
    assert B[0, 0, 3] == out[0, H * P + 3]
    assert C[1, 0, 0] == out[1, H * P + G * N]

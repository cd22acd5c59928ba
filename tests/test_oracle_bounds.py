"""Pins of oracle/bounds.py, the error scales behind the element-wise GPU
output bounds: each against something other than its own formula -- the
sequential fp64 oracle, the triangle inequality, and term-by-term brute
force on tiny inputs."""
import numpy as np
import pytest

from exact_replay_decode_amd import synth
from oracle import scan
from oracle.bounds import chunk_error_scales


def problem(lengths, H, G, P, N, seed, init=False, nonneg=False):
    hp = synth.make_head_params(H, seed)
    tok = synth.concat([synth.make_tokens(L, H, G, P, N, seed, stream=i, io_dtype="f32",
                                          dt_dtype="f32") for i, L in enumerate(lengths)])
    x, dt, B, C = tok.f64()
    rng = np.random.default_rng(seed + 100)
    h0 = rng.standard_normal((len(lengths), H, P, N)) if init else None
    if nonneg:
        x, B, C = np.abs(x), np.abs(B), np.abs(C)
        h0 = None if h0 is None else np.abs(h0)
    return hp, x, dt, B, C, synth.cu_seqlens(lengths), h0


@pytest.mark.parametrize("lengths,Q,G", [([40], 16, 1), ([7, 33, 16], 16, 2), ([70], 32, 1)])
def test_triangle_inequality_against_the_sequential_oracle(lengths, Q, G):
    # y - D x is the sum of the rounded terms, so |y - D x| <= mag; and the
    # root of the summed squares never exceeds the summed magnitudes
    hp, x, dt, B, C, cu, h0 = problem(lengths, 4, G, 8, 8, seed=3, init=True)
    ref = scan(x, dt, hp.A, B, C, cu, Q, D=hp.D, dt_bias=hp.dt_bias, init=h0)
    sc = chunk_error_scales(x, dt, hp.A, B, C, cu, Q, D=hp.D, dt_bias=hp.dt_bias, init=h0)
    core = np.abs(ref.y - hp.D[None, :, None] * x)
    assert np.all(core <= sc.mag * (1 + 1e-12) + 1e-300)
    assert np.all(sc.rms <= sc.mag * (1 + 1e-12))
    assert np.all(sc.rms > 0)


@pytest.mark.parametrize("lengths,Q", [([50], 16), ([17, 64, 3], 16), ([100], 32)])
def test_nonnegative_inputs_give_the_output_itself(lengths, Q):
    # with x, B, C, h0 >= 0 and positive decays every term is >= 0: mag is
    # then exactly y - D x of the sequential recurrence (chunk grid, chunk
    # start states, decays and the C.B contraction all pinned at once)
    hp, x, dt, B, C, cu, h0 = problem(lengths, 3, 1, 6, 5, seed=5, init=True, nonneg=True)
    ref = scan(x, dt, hp.A, B, C, cu, Q, D=hp.D, dt_bias=hp.dt_bias, init=h0)
    sc = chunk_error_scales(x, dt, hp.A, B, C, cu, Q, D=hp.D, dt_bias=hp.dt_bias, init=h0)
    core = ref.y - hp.D[None, :, None] * x
    np.testing.assert_allclose(sc.mag, core, rtol=1e-12, atol=1e-300)


def test_single_token_from_zero_state():
    # T = 1, h0 = 0: one term delta (C . B) x; mag = rms = its magnitude
    hp, x, dt, B, C, cu, _ = problem([1], 2, 1, 4, 3, seed=7)
    sc = chunk_error_scales(x, dt, hp.A, B, C, cu, 16, D=hp.D, dt_bias=hp.dt_bias)
    d = np.log1p(np.exp(dt[0] + hp.dt_bias))
    term = np.abs(d[:, None] * (C[0, 0] @ B[0, 0]) * x[0])
    np.testing.assert_allclose(sc.mag[0], term, rtol=1e-13)
    np.testing.assert_allclose(sc.rms[0], term, rtol=1e-13)


def test_brute_force_terms():
    # every term of every output enumerated one by one: the read-out terms
    # exp(Lam_t) S0[p,n] C_t[n] and the in-chunk terms m_ts x_s[p]
    H, G, P, N, Q = 2, 1, 3, 4, 8
    hp, x, dt, B, C, cu, h0 = problem([20], H, G, P, N, seed=11, init=True)
    sc = chunk_error_scales(x, dt, hp.A, B, C, cu, Q, D=hp.D, dt_bias=hp.dt_bias, init=h0)
    ref = scan(x, dt, hp.A, B, C, cu, Q, D=hp.D, dt_bias=hp.dt_bias, init=h0, max_chunks=2)
    d = np.log1p(np.exp(dt + hp.dt_bias[None, :]))
    for h in range(H):
        for t in range(20):
            c0 = (t // Q) * Q
            S0 = h0[0, h] if c0 == 0 else ref.chunk_states[0, c0 // Q - 1, h]
            for p in range(P):
                terms = []
                for n in range(N):
                    lam_t = sum(d[r, h] * hp.A[h] for r in range(c0, t + 1))
                    terms.append(np.exp(lam_t) * S0[p, n] * C[t, 0, n])
                for s in range(c0, t + 1):
                    lam_ts = sum(d[r, h] * hp.A[h] for r in range(s + 1, t + 1))
                    cb = sum(C[t, 0, n] * B[s, 0, n] for n in range(N))
                    terms.append(cb * np.exp(lam_ts) * d[s, h] * x[s, h, p])
                terms = np.array(terms)
                assert np.isclose(sc.mag[t, h, p], np.abs(terms).sum(), rtol=1e-11)
                assert np.isclose(sc.rms[t, h, p], np.sqrt((terms ** 2).sum()), rtol=1e-11)
                # the terms add up to the sequential recurrence's output
                assert np.isclose(terms.sum() + hp.D[h] * x[t, h, p], ref.y[t, h, p],
                                  rtol=1e-10, atol=1e-12)


def test_state_row_scale():
    hp, x, dt, B, C, cu, h0 = problem([24], 2, 1, 4, 4, seed=13, init=True)
    sc = chunk_error_scales(x, dt, hp.A, B, C, cu, 16, D=hp.D, dt_bias=hp.dt_bias, init=h0)
    d = np.log1p(np.exp(dt + hp.dt_bias[None, :]))
    t, h = 5, 1
    lam = (d[:t + 1, h] * hp.A[h]).sum()
    want = np.exp(lam) * np.abs(h0[0, h]).max() * np.abs(C[t, 0]).sum()
    assert np.isclose(sc.state_row[t, h], want, rtol=1e-12)


def test_sequence_subset_leaves_others_zero():
    hp, x, dt, B, C, cu, _ = problem([10, 12, 9], 2, 1, 4, 4, seed=17)
    sc = chunk_error_scales(x, dt, hp.A, B, C, cu, 16, D=hp.D, dt_bias=hp.dt_bias, seqs=[1])
    assert np.all(sc.mag[:10] == 0) and np.all(sc.mag[22:] == 0)
    assert np.all(sc.mag[10:22] > 0)

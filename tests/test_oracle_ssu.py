"""Pins of the cache-dtype recurrent-update oracle (oracle/ssu.py): its bf16
rounding against torch's float32 -> bfloat16 cast, its recurrence against
the independently pinned sequential scan oracle (a C program), and closed
forms where the rounding does or does not act."""
import numpy as np
import pytest
import torch

from oracle import scan
from oracle.ssu import round_bf16, ssu_tokens, ssu_varlen


def test_round_bf16_matches_torch_on_float32_values():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-6, 6, 20000),
                        [0.0, -0.0, 1.0, -1.0, 3.0e38, 1e-30]]).astype(np.float32)
    # exact ties: a bf16 value plus half its ulp, both parities of the last bit
    base = torch.tensor(rng.standard_normal(2000), dtype=torch.bfloat16).float().numpy()
    half = np.ldexp(np.ones_like(base), (np.frexp(base)[1] - 9).astype(np.int32))
    ties = (base + np.sign(base) * half).astype(np.float32)
    for arr in (v, ties):
        want = torch.from_numpy(arr).to(torch.bfloat16).double().numpy()
        assert np.array_equal(round_bf16(arr.astype(np.float64)), want)


def _inputs(T, H, G, P, N, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((T, H, P)), 0.5 * rng.standard_normal((T, H)),
            -rng.uniform(1, 16, H), rng.standard_normal((T, G, N)),
            rng.standard_normal((T, G, N)), rng.uniform(0.5, 1.5, H),
            np.log(np.expm1(np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), H)))))


def test_unrounded_recurrence_is_the_scan_oracle():
    T, H, G, P, N = 37, 4, 2, 8, 16
    x, dt, A, B, C, D, bias = _inputs(T, H, G, P, N, 1)
    h0 = np.random.default_rng(2).standard_normal((H, P, N))
    y, h = ssu_tokens(h0, x, dt, A, B, C, D, bias, cache="f64")
    ref = scan(x, dt, A, B, C, [0, T], 16, D=D, dt_bias=bias, init=h0[None])
    np.testing.assert_allclose(y, ref.y, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(h, ref.final_state[0], rtol=1e-11, atol=1e-12)


def test_split_replay_is_exact():
    T, H, G, P, N = 30, 2, 1, 4, 8
    x, dt, A, B, C, D, bias = _inputs(T, H, G, P, N, 3)
    h0 = round_bf16(np.random.default_rng(4).standard_normal((H, P, N)))
    y, h = ssu_tokens(h0, x, dt, A, B, C, D, bias, cache="bf16")
    for a in (1, 13, 29):
        y1, h1 = ssu_tokens(h0, x[:a], dt[:a], A, B[:a], C[:a], D, bias, cache="bf16")
        y2, h2 = ssu_tokens(h1, x[a:], dt[a:], A, B[a:], C[a:], D, bias, cache="bf16")
        assert np.array_equal(np.concatenate([y1, y2]), y) and np.array_equal(h2, h)


def test_representable_states_are_not_perturbed():
    """A = 0 (no decay), delta = 0.5 exactly (softplus off), small integer x
    and B: every state is a multiple of 0.5 below 2**7, exact in bf16, so the
    bf16 run equals the unrounded one."""
    T, H, G, P, N = 12, 2, 1, 4, 4
    rng = np.random.default_rng(5)
    x = rng.integers(-2, 3, (T, H, P)).astype(np.float64)
    B = rng.integers(-2, 3, (T, G, N)).astype(np.float64)
    C = rng.standard_normal((T, G, N))
    dt = np.full((T, H), 0.5)
    A = np.zeros(H)
    y16, h16 = ssu_tokens(np.zeros((H, P, N)), x, dt, A, B, C, dt_softplus=False, cache="bf16")
    y64, h64 = ssu_tokens(np.zeros((H, P, N)), x, dt, A, B, C, dt_softplus=False, cache="f64")
    assert np.array_equal(h16, h64) and np.array_equal(y16, y64)


def test_output_reads_the_unrounded_state_and_the_store_is_rounded():
    """One element: state 1, no decay, delta x B = 2**-10 (below half a bf16
    ulp of 1). The first output sees 1 + 2**-10, the stored state is 1, and
    the second output sees 1 + 2**-10 again (not 1 + 2**-9)."""
    one = np.ones((1, 1, 1))
    x = np.full((2, 1, 1), 2.0 ** -10)
    B = np.ones((2, 1, 1))
    C = np.ones((2, 1, 1))
    dt = np.ones((2, 1))
    y, h = ssu_tokens(one, x, dt, np.zeros(1), B, C, dt_softplus=False, cache="bf16")
    assert y[0, 0, 0] == 1 + 2.0 ** -10 and y[1, 0, 0] == 1 + 2.0 ** -10
    assert h[0, 0, 0] == 1.0
    y32, h32 = ssu_tokens(one, x, dt, np.zeros(1), B, C, dt_softplus=False, cache="f32")
    assert y32[1, 0, 0] == 1 + 2.0 ** -9 and h32[0, 0, 0] == 1 + 2.0 ** -9


def test_varlen_is_per_sequence():
    H, G, P, N = 2, 1, 4, 8
    lengths = [5, 0, 9]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    x, dt, A, B, C, D, bias = _inputs(int(cu[-1]), H, G, P, N, 6)
    st = np.random.default_rng(7).standard_normal((3, H, P, N)).astype(np.float32)
    y, fin = ssu_varlen(st, x, dt, A, B, C, cu, D, bias, cache="f32")
    for s in range(3):
        ys, hs = ssu_tokens(st[s], x[cu[s]:cu[s + 1]], dt[cu[s]:cu[s + 1]], A,
                            B[cu[s]:cu[s + 1]], C[cu[s]:cu[s + 1]], D, bias, cache="f32")
        assert np.array_equal(y[cu[s]:cu[s + 1]], ys) and np.array_equal(fin[s], hs)


@pytest.mark.parametrize("cache", ["f32", "bf16"])
def test_state_dtype_of_the_store(cache):
    T, H, G, P, N = 4, 2, 1, 4, 8
    x, dt, A, B, C, D, bias = _inputs(T, H, G, P, N, 8)
    _, h = ssu_tokens(np.zeros((H, P, N)), x, dt, A, B, C, D, bias, cache=cache)
    if cache == "f32":
        assert np.array_equal(h, h.astype(np.float32).astype(np.float64))
    else:
        assert np.array_equal(h, torch.from_numpy(h).to(torch.bfloat16).double().numpy())

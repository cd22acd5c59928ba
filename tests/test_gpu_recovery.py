"""Packed-history recovery through the C ABI (vLLM RFC "Mamba2: exact-replay
decode ...", section 3b: generated history is replayed with a multi-token
recurrent update that rounds the state to the cache dtype after every
token; recovered decode then equals uninterrupted decode, 28/28 recoveries
of 255 tokens in the RFC). The mirror property of exact replay.

Tolerances: outputs mean|y - ref| / mean|ref| <= 0.3 % (bf16, as for every
output); fp32 states per (sequence, head) max relative 1e-4 against the
fp64 recurrence; bf16 states against the bf16-rounding oracle within 8
units of 2^-8 times the head's largest element (fp32 and fp64 arithmetic can
round a near-tie to neighbouring bf16 values, one bf16 ulp apart, and the
element then carries the difference: up to four such flips of the largest
element over the 255 tokens; 4.8 units seen).
"""
import numpy as np
import pytest
import torch

import exact_replay_decode_amd as erd
from exact_replay_decode_amd import synth
from gpu_cases import DEV, headwise_max_rel, make_problem, mean_rel_err, same_bits
from oracle import scan
from oracle.ssu import ssu_varlen

pytestmark = pytest.mark.gpu

SDT = {"f32": torch.float32, "bf16": torch.bfloat16}


def shape_with_state(pr, cache):
    s = pr.shape
    return erd.Shape(s.H, s.G, s.P, s.N, s.chunk_size, s.io_dtype, s.dt_dtype,
                     state_dtype=cache)


@pytest.mark.parametrize("cache", ["f32", "bf16"])
@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_multi_token_update_equals_single_steps(cache, io):
    lengths = [255, 0, 1, 40, 300]
    P, N = (64, 128) if io == "bf16" else (32, 16)
    pr = make_problem(lengths, H=8, G=2, P=P, N=N, Q=16, io=io, seed=12)
    sh = shape_with_state(pr, cache)
    x, dt, B, C = pr.dev(None)
    S = len(lengths)
    st0 = torch.randn((S + 2, 8, P, N), device=DEV,
                      generator=torch.Generator(device=DEV).manual_seed(13)).to(SDT[cache])
    sl = torch.tensor([3, 0, 6, 1, 5], dtype=torch.int32, device=DEV)
    st_multi = st0.clone()
    y_multi = erd.ssm_state_update_varlen(sh, st_multi, pr.cu, x, dt, B, C, pr.A, pr.D,
                                          pr.bias, slot_idx=sl)
    st_one = st0.clone()
    y_one = torch.empty_like(y_multi)
    cu = pr.cu
    for k in range(max(lengths)):
        live = [s for s in range(S) if k < lengths[s]]
        it = torch.tensor([int(cu[s]) + k for s in live], device=DEV)
        y_one[it] = erd.ssm_state_update(sh, st_one, x[it], dt[it], B[it], C[it], pr.A, pr.D,
                                         pr.bias, slot_idx=sl[live])
    assert same_bits(y_multi, y_one)
    assert same_bits(st_multi, st_one)
    for k in (2, 4):                       # slots no sequence names
        assert same_bits(st_multi[k], st0[k])


@pytest.mark.parametrize("cache", ["f32", "bf16"])
def test_packed_history_recovery(cache):
    """28 requests: prompt prefill, 255 generated tokens decoded one by one
    with the recurrent update (state stored in the cache dtype), then 16
    more. Recovery after a preemption: prefill the prompt again, replay the
    255 generated tokens with one multi-token update, decode the 16: the
    state and the 16 outputs equal the uninterrupted run bit for bit."""
    S, H, P, N, gen, more = 28, 8, 64, 128, 255, 16
    rng = np.random.default_rng(28)
    prompt = rng.integers(50, 500, S)
    lengths = prompt + gen + more
    pr = make_problem(list(lengths), H=H, G=1, P=P, N=N, Q=256, seed=13)
    sh = shape_with_state(pr, cache)
    x, dt, B, C = pr.dev(None)
    cu = pr.cu
    ip = torch.from_numpy(np.concatenate([np.arange(cu[s], cu[s] + prompt[s])
                                          for s in range(S)])).to(DEV)

    def prefill_state():
        _, fin, _ = erd.ssd_prefill_varlen(pr.shape, synth.cu_seqlens(prompt), x[ip], dt[ip],
                                           pr.A, B[ip], C[ip], pr.D, pr.bias,
                                           want_boundary=False)
        return fin.to(SDT[cache])          # stored in the cache dtype

    def decode(state, k0, k1):
        ys = []
        for k in range(k0, k1):
            it = torch.from_numpy((cu[:-1] + prompt + k).astype(np.int64)).to(DEV)
            ys.append(erd.ssm_state_update(sh, state, x[it], dt[it], B[it], C[it], pr.A, pr.D,
                                           pr.bias))
        return torch.stack(ys, 1)

    run = prefill_state()
    decode(run, 0, gen)
    y_after = decode(run, gen, gen + more)
    # preemption: everything but the token history is lost
    rec = prefill_state()
    ih = torch.from_numpy(np.concatenate([np.arange(cu[s] + prompt[s], cu[s] + prompt[s] + gen)
                                          for s in range(S)])).to(DEV)
    erd.ssm_state_update_varlen(sh, rec, synth.cu_seqlens([gen] * S), x[ih], dt[ih], B[ih],
                                C[ih], pr.A, pr.D, pr.bias)
    y_rec = decode(rec, gen, gen + more)
    assert same_bits(rec, run)
    assert same_bits(y_rec, y_after)
    mism = (y_rec.view(torch.int16) != y_after.view(torch.int16)).flatten(1).any(1)
    assert int(mism.sum()) == 0          # 28/28 recoveries bit-identical


@pytest.mark.parametrize("cache", ["f32", "bf16"])
def test_multi_token_update_matches_oracle(cache):
    lengths = [200, 7, 64]
    pr = make_problem(lengths, H=4, G=2, P=64, N=128, Q=16, seed=14)
    sh = shape_with_state(pr, cache)
    x, dt, B, C = pr.dev(None)
    st0 = torch.randn((3, 4, 64, 128), device=DEV,
                      generator=torch.Generator(device=DEV).manual_seed(14)).to(SDT[cache])
    st = st0.clone()
    y = erd.ssm_state_update_varlen(sh, st, pr.cu, x, dt, B, C, pr.A, pr.D, pr.bias)
    xs, dts, Bs, Cs = pr.tok.f64()
    h0 = erd.to_f64(st0)
    ref_y, ref_h = ssu_varlen(h0, xs, dts, pr.hp.A, Bs, Cs, pr.cu, pr.hp.D, pr.hp.dt_bias,
                              cache=cache)
    assert mean_rel_err(y, ref_y) <= 3e-3
    if cache == "f32":
        exact = scan(xs, dts, pr.hp.A, Bs, Cs, pr.cu, 16, D=pr.hp.D, dt_bias=pr.hp.dt_bias,
                     init=h0)
        assert headwise_max_rel(st.cpu().numpy(), exact.final_state) <= 1e-4
    else:
        # both sides round the state to bf16 after every token; where the
        # fp32 and fp64 values straddle a rounding boundary they land one
        # bf16 ulp (2^-8 of the element) apart and later tokens carry the
        # difference. Over random initial states the worst head of this case
        # reached 4.8 ulps of its largest element: bound 8.
        d = np.abs(erd.to_f64(st) - ref_h).reshape(3, 4, -1).max(-1)
        m = np.abs(ref_h).reshape(3, 4, -1).max(-1)
        assert np.all(d <= 8 * 2.0 ** -8 * m)


def test_recurrent_error_levels_printed_by_the_rfc():
    """[RFC] section 2, item 1: against the fp64 reference, the recurrent
    update sits at 0.141 % with an fp32 state and 0.245-0.269 % with a bf16
    state (32 heads, 1 group, P=64, N=128, 2048 tokens, bf16 activations).
    The same shape and input recipe here lands in the same places."""
    T, H, G, P, N = 2048, 32, 1, 64, 128
    pr = make_problem([T], H=H, G=G, P=P, N=N, Q=256, seed=15)
    x, dt, B, C = pr.dev(None)
    ref = pr.oracle()
    got = {}
    for cache in ("f32", "bf16"):
        st = torch.zeros((1, H, P, N), dtype=SDT[cache], device=DEV)
        y = erd.ssm_state_update_varlen(shape_with_state(pr, cache), st, pr.cu, x, dt, B, C,
                                        pr.A, pr.D, pr.bias)
        got[cache] = mean_rel_err(y, ref.y)
    assert 1.3e-3 <= got["f32"] <= 1.6e-3, got
    assert 2.0e-3 <= got["bf16"] <= 3.5e-3, got
    assert got["bf16"] > got["f32"]

"""Degenerate parameter cases through the C ABI: the raw dt taken as delta
(softplus off), absent D and dt_bias (optional arguments), a head with
A = 0 (no decay at all), and tokens whose delta underflows to zero in fp32
(softplus of a very negative dt: the token adds nothing to the state).

Each run is checked against the oracle (fp64) within the usual tolerances
and, bit for bit, against the same tokens fed as a chunked replay (uneven
splits) followed by one-token decode steps: the exact-replay property must
hold in these corners too.
"""
import numpy as np
import pytest
import torch

import exact_replay_decode_amd as erd
from exact_replay_decode_amd import synth, to_device
from gpu_cases import DEV, check_bf16, mean_rel_err, same_bits, seq_spans
from oracle import scan
from oracle.bounds import chunk_error_scales

pytestmark = pytest.mark.gpu


def storage(vals, dtype):
    """float values -> synth's storage form (bf16 bits as uint16, or fp32)."""
    v = np.asarray(vals, dtype=np.float32)
    if dtype == "bf16":
        return torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return v


def run_case(shape, lengths, tok, A, D, bias, seed):
    """Single-shot prefill vs replay (random splits, then decode of each
    sequence's last 5 tokens); returns (y, final, oracle)."""
    io, dtd = shape.io_dtype, shape.dt_dtype
    x, dt, B, C = (to_device(tok.x, io, DEV), to_device(tok.dt, dtd, DEV),
                   to_device(tok.B, io, DEV), to_device(tok.C, io, DEV))
    At = torch.from_numpy(A).to(DEV)
    Dt = None if D is None else torch.from_numpy(D).to(DEV)
    bt = None if bias is None else torch.from_numpy(bias).to(DEV)
    cu = synth.cu_seqlens(lengths)
    y, fin, _ = erd.ssd_prefill_varlen(shape, cu, x, dt, At, B, C, Dt, bt)

    S = len(lengths)
    cache = erd.ReplayCache(shape, S, DEV)
    rng = np.random.default_rng(seed)
    done = np.zeros(S, dtype=np.int64)
    pre = np.maximum(np.array(lengths) - 5, 0)
    y_rep = torch.full_like(y, float("nan"))
    while (done < pre).any():
        n = np.minimum(rng.integers(1, 200, S), pre - done)
        idx = torch.from_numpy(np.concatenate(
            [np.arange(cu[s] + done[s], cu[s] + done[s] + n[s]) for s in range(S)])).to(DEV)
        y_rep[idx] = erd.ssd_replay_prefill(shape, cache, synth.cu_seqlens(n), x[idx], dt[idx],
                                            B[idx], C[idx], At, Dt, bt)
        done += n
    for _ in range(5):
        live = np.flatnonzero(done < np.array(lengths))
        if live.size == 0:
            break
        it = torch.from_numpy((cu[live] + done[live]).astype(np.int64)).to(DEV)
        y_rep[it] = erd.ssd_replay_decode(shape, cache, x[it], dt[it], B[it], C[it], At, Dt, bt,
                                          slot_idx=torch.from_numpy(live.astype(np.int32)).to(DEV))
        done[live] += 1
    assert same_bits(y_rep, y), "replay and decode differ from the single-shot prefill"

    xs, dts, Bs, Cs = tok.f64()
    ref = scan(xs, dts, A, Bs, Cs, cu, shape.chunk_size, D=D, dt_bias=bias,
               dt_softplus=shape.dt_softplus)
    sc = chunk_error_scales(xs, dts, A, Bs, Cs, cu, shape.chunk_size, D=D, dt_bias=bias,
                            dt_softplus=shape.dt_softplus)
    return y, fin, ref, sc, cu


def check(shape, y, fin, ref, scales=None, cu=None):
    if shape.io_dtype == "bf16":
        assert mean_rel_err(y, ref.y) <= 3e-3
        check_bf16(y, ref.y, scales, seq_spans(cu), label="degenerate")
    else:
        H = shape.H
        yy = erd.to_f64(y)
        # per head, over all tokens: max |y - ref| / max |ref|
        d = np.abs(yy - ref.y).reshape(-1, H, shape.P).max(axis=(0, 2))
        m = np.abs(ref.y).reshape(-1, H, shape.P).max(axis=(0, 2))
        assert np.all(d <= 1e-4 * m)
    # fp32 states per (sequence, head), relative to the largest element; a
    # state whose every contribution is below fp32's range (all deltas
    # underflow) has the reference's magnitude ~1e-87 and is 0 in fp32
    S, H = ref.final_state.shape[:2]
    st = fin.cpu().numpy().astype(np.float64)
    d = np.abs(st - ref.final_state).reshape(S, H, -1).max(-1)
    m = np.abs(ref.final_state).reshape(S, H, -1).max(-1)
    assert np.all(d <= 1e-4 * np.maximum(m, 1e-30))


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_raw_dt_without_D_and_bias(io):
    """dt_softplus off: delta = dt (no bias), dt drawn positive; D absent."""
    H, G, P, N, Q = (8, 2, 64, 128, 64) if io == "bf16" else (4, 2, 32, 16, 32)
    lengths = [300, 17, 0, 129]
    shape = erd.Shape(H, G, P, N, Q, io, io, dt_softplus=False)
    tok = synth.concat([synth.make_tokens(L, H, G, P, N, 40, stream=i, io_dtype=io, dt_dtype=io)
                        for i, L in enumerate(lengths)])
    rng = np.random.default_rng(40)
    tok.dt = storage(rng.uniform(0.002, 0.1, tok.dt.shape), io)
    A = synth.make_head_params(H, 40).A
    y, fin, ref, sc, cu = run_case(shape, lengths, tok, A, None, None, seed=40)
    check(shape, y, fin, ref, sc, cu)


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_zero_decay_head_and_vanishing_delta(io):
    """Head 1 has A = 0 (its state only accumulates); every 7th token of
    head 0 and all of head 2's tokens in one sequence get dt = -200, so
    softplus(dt + bias) underflows to zero in fp32."""
    H, G, P, N, Q = (8, 1, 64, 128, 256) if io == "bf16" else (4, 1, 32, 16, 32)
    lengths = [513, 40, 256]
    shape = erd.Shape(H, G, P, N, Q, io, io)
    tok = synth.concat([synth.make_tokens(L, H, G, P, N, 41, stream=i, io_dtype=io, dt_dtype=io)
                        for i, L in enumerate(lengths)])
    hp = synth.make_head_params(H, 41)
    A = hp.A.copy()
    A[1] = 0.0
    dt = tok.dt.copy()
    m200 = storage([-200.0], io)[0]
    dt[::7, 0] = m200
    dt[lengths[0]:lengths[0] + lengths[1], 2] = m200
    tok.dt = dt
    y, fin, ref, sc, cu = run_case(shape, lengths, tok, A, hp.D, hp.dt_bias, seed=41)
    check(shape, y, fin, ref, sc, cu)
    # head 2 of sequence 1 never had a nonzero delta: its state stays zero
    assert not fin[1, 2].any()
    assert float(np.abs(ref.final_state[1, 2]).max()) < 1e-80

"""Replay decode captured in a HIP graph (torch.cuda.CUDAGraph): one decode
step of a 3-layer stack is captured once and replayed for 40 steps. Between
replays the step's token inputs are copied into the captured input buffers
and the outputs copied out (eager work between replays, so a replay that
reused stale values would show). The cache keeps buf_len on the device, so
nothing on the host changes from step to step. Every step's outputs and the
final caches equal the eager run bit for bit; with chunk 16 every slot
crosses chunk ends, so the chunk-state update runs inside the graph too.
With 200 slots (more workgroups than run at once) each captured step is the
ranking launch followed by the ranked decode launch."""
import numpy as np
import pytest
import torch

import exact_replay_decode_amd as erd
from exact_replay_decode_amd import synth
from gpu_cases import DEV, same_bits

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("S,H", [(8, 8),      # all workgroups at once: one launch per step
                                 (200, 16)])  # ranked: a ranking launch, then the step
def test_decode_steps_replayed_from_a_graph(S, H):
    L, G, P, N, Q, steps = 3, 2, 64, 128, 16, 40
    sh = erd.Shape(H, G, P, N, Q, "bf16", "bf16")
    pre = [5 + 3 * s for s in range(S)]          # buffers at different offsets
    layers = []
    for li in range(L):
        hp = synth.make_head_params(H, 50 + li)
        prm = tuple(torch.from_numpy(v).to(DEV) for v in (hp.A, hp.D, hp.dt_bias))
        ptoks = synth.make_tokens_torch(sum(pre), H, G, P, N, 50 + li, DEV)
        dtoks = [t.view(steps, S, *t.shape[1:])
                 for t in synth.make_tokens_torch(steps * S, H, G, P, N, 60 + li, DEV)]
        c_e = erd.ReplayCache(sh, S, DEV)
        erd.ssd_replay_prefill(sh, c_e, synth.cu_seqlens(pre), *ptoks, *prm)
        layers.append((prm, dtoks, c_e, c_e.clone()))

    y_e = torch.empty((steps, L, S, H, P), dtype=torch.bfloat16, device=DEV)
    for k in range(steps):
        for li, (prm, dtoks, c_e, _) in enumerate(layers):
            y_e[k, li] = erd.ssd_replay_decode(sh, c_e, *(t[k] for t in dtoks), *prm)

    stream = torch.cuda.Stream()
    xin = [[torch.empty_like(t[0]) for t in dtoks] for (_, dtoks, _, _) in layers]
    yout = [torch.empty((S, H, P), dtype=torch.bfloat16, device=DEV) for _ in layers]
    plans = [erd.DecodePlan(sh, S, *prm, cache=c_g, stream=stream)
             for (prm, _, _, c_g) in layers]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for plan, xs, yo in zip(plans, xin, yout):
            plan(*xs, yo)
    torch.cuda.synchronize()
    y_g = torch.empty_like(y_e)
    for k in range(steps):
        for li, (_, dtoks, _, _) in enumerate(layers):
            for buf, t in zip(xin[li], dtoks):
                buf.copy_(t[k])
        g.replay()
        for li in range(L):
            y_g[k, li].copy_(yout[li])
        torch.cuda.synchronize()
    assert same_bits(y_g, y_e)
    for _, _, c_e, c_g in layers:
        for name in ("state", "state_bf", "buf_len", "boundary_pos", "work"):
            assert same_bits(getattr(c_g, name), getattr(c_e, name)), name
        n = c_e.buf_len.tolist()
        for a, b in zip(c_g.buffers_by_slot()[:3], c_e.buffers_by_slot()[:3]):
            for s in range(S):
                assert same_bits(a[s, :n[s]], b[s, :n[s]])


def test_speculative_rounds_replayed_from_a_graph():
    """One speculative round (verification of T drafts, then acceptance of a
    device-side count of them) captured once and replayed for 24 rounds.
    Drafts and counts are copied into the captured buffers between replays;
    with chunk 16 drafts cross chunk ends and accepted drafts fill chunks in
    most rounds, so the listed sweeps (their list kept in the cache's work
    array) run inside the graph. Outputs and caches equal the eager run bit
    for bit, and the work array is zero after every replay."""
    S, H, G, P, N, Q, T, rounds = 64, 16, 4, 64, 128, 16, 4, 24
    sh = erd.Shape(H, G, P, N, Q, "bf16", "bf16")
    hp = synth.make_head_params(H, 70)
    A, D, bias = (torch.from_numpy(v).to(DEV) for v in (hp.A, hp.D, hp.dt_bias))
    pre = [1 + (7 * s) % (3 * Q) for s in range(S)]
    c_e = erd.ReplayCache(sh, S, DEV)
    erd.ssd_replay_prefill(sh, c_e, synth.cu_seqlens(pre),
                           *synth.make_tokens_torch(sum(pre), H, G, P, N, 70, DEV), A, D, bias)
    c_g = c_e.clone()
    drafts = [t.view(rounds, S * T, *t.shape[1:])
              for t in synth.make_tokens_torch(rounds * S * T, H, G, P, N, 71, DEV)]
    acc = torch.from_numpy(
        np.random.default_rng(72).integers(0, T + 1, size=(rounds, S)).astype(np.int32)).to(DEV)
    cu_h = synth.cu_seqlens([T] * S)
    cu_d = torch.from_numpy(cu_h).to(DEV)

    y_e = torch.empty((rounds, S * T, H, P), dtype=torch.bfloat16, device=DEV)
    for r in range(rounds):
        d = [t[r] for t in drafts]
        erd.ssd_replay_verify(sh, c_e, cu_d, *d, A, D, bias, y=y_e[r], cu_seqlens_host=cu_h)
        erd.ssd_replay_accept(sh, c_e, cu_d, acc[r], *d, A, bias, cu_seqlens_host=cu_h)

    stream = torch.cuda.Stream()
    din = [torch.empty_like(t[0]) for t in drafts]
    ain = torch.empty_like(acc[0])
    yout = torch.empty((S * T, H, P), dtype=torch.bfloat16, device=DEV)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        erd.ssd_replay_verify(sh, c_g, cu_d, *din, A, D, bias, y=yout, cu_seqlens_host=cu_h,
                              stream=stream)
        erd.ssd_replay_accept(sh, c_g, cu_d, ain, *din, A, bias, cu_seqlens_host=cu_h,
                              stream=stream)
    torch.cuda.synchronize()
    y_g = torch.empty_like(y_e)
    for r in range(rounds):
        for buf, t in zip(din, drafts):
            buf.copy_(t[r])
        ain.copy_(acc[r])
        g.replay()
        y_g[r].copy_(yout)
        torch.cuda.synchronize()
        assert not c_g.work.any(), r
    assert same_bits(y_g, y_e)
    for name in ("state", "state_bf", "buf_len", "boundary_pos", "work"):
        assert same_bits(getattr(c_g, name), getattr(c_e, name)), name
    n = c_e.buf_len.tolist()
    for a, b in zip(c_g.buffers_by_slot()[:3], c_e.buffers_by_slot()[:3]):
        for s in range(S):
            assert same_bits(a[s, :n[s]], b[s, :n[s]])

"""GPU causal conv1d (the step before the scan) through the C ABI: parity
with the fp64 oracle, and the bit identity of its prefill and decode forms
(vLLM RFC "Mamba2: exact-replay decode ...", section 2, item 6), alone and
chained into the scan.

Tolerance, derived from the arithmetic: each output is an fmaf chain of W
products from the bias, then SiLU with the hardware exp2 and reciprocal, in
fp32. The chain's error is below W+1 fp32 half-ulps of M = |bias| +
sum |w_i v_i|. exp(-v) as exp2(-v log2 e) is off by |v| 2**-24 relative
from the product's rounding plus an ulp, the reciprocal and product add two
more, and SiLU passes the relative error of exp(-v) through at most 1:1, so
|silu error| <= |ref| (|v| 2**-24 + 4 * 2**-23) <= 1e-6 |ref| + 2e-6 M
(|v| <= M, |ref| <= |v| + 1). fp32 outputs: |y32 - ref| <= 2e-6 * M +
1e-6 * |ref|. bf16 outputs add the storage rounding, half a bf16 ulp:
|y - ref| <= 2**-8 * |ref| + 2e-6 * M.
"""
import numpy as np
import pytest
import torch

import exact_replay_decode_amd as erd
from exact_replay_decode_amd import synth
from gpu_cases import DEV, same_bits
from oracle.conv1d import conv1d_varlen

pytestmark = pytest.mark.gpu

def setup(lengths, H, G, P, N, W, io, seed=0, with_state=True, slots=None):
    shape = erd.Shape(H, G, P, N, 16, io, io)
    cd = erd.conv_dim(shape)
    cp = synth.make_conv_params(cd, W, seed)
    parts = [synth.make_xbc(L, cd, seed, stream=i, io_dtype=io) for i, L in enumerate(lengths)]
    xbc_s = np.concatenate(parts) if parts else np.zeros((0, cd))
    S = len(lengths)
    ns = slots or S
    st_s = synth.make_xbc(ns * (W - 1), cd, seed, stream=999, io_dtype=io)
    # state [slots, conv_dim, W-1] from rows of the same distribution
    st64 = synth.widen(st_s, io).reshape(ns, W - 1, cd).transpose(0, 2, 1).copy()
    dev = lambda a: erd.to_device(a, io, DEV)  # noqa: E731
    state = dev(synth.store(st64, io)).contiguous() if with_state else None
    return dict(shape=shape, cd=cd, W=W, io=io, cu=synth.cu_seqlens(lengths),
                xbc=dev(xbc_s), xbc64=synth.widen(xbc_s, io), st64=st64 if with_state else None,
                state=state, weight=torch.from_numpy(cp.weight).to(DEV),
                bias=torch.from_numpy(cp.bias).to(DEV), w64=cp.weight.astype(np.float64),
                b64=cp.bias.astype(np.float64))


def cat_out(x, B, C):
    T = x.shape[0]
    return torch.cat([x.reshape(T, -1), B.reshape(T, -1), C.reshape(T, -1)], 1)


def check_parity(y, ref, mag, io):
    d = np.abs(erd.to_f64(y) - ref)
    if io == "bf16":
        bound = 2.0 ** -8 * np.abs(ref) + 2e-6 * mag
    else:
        bound = 1e-6 * np.abs(ref) + 2e-6 * mag
    assert np.all(d <= bound), float((d / np.maximum(bound, 1e-300)).max())


@pytest.mark.parametrize("W", [2, 3, 4])
@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("act", [True, False])
def test_conv_prefill_matches_oracle(W, io, act):
    # lengths: empty, shorter than the window, one run, several tiles with
    # a ragged tail
    lengths = [0, 1, 2, 3, 31, 300, 517]
    c = setup(lengths, H=4, G=2, P=32, N=16, W=W, io=io, seed=W)
    st0 = None if c["state"] is None else c["state"].clone()
    x, B, C = erd.ssd_conv1d_varlen(c["shape"], c["cu"], c["xbc"], c["weight"], c["bias"],
                                    conv_state=c["state"], activation=act)
    ref, fin = conv1d_varlen(c["xbc64"], c["w64"], c["cu"], c["b64"], c["st64"], act)
    mag, _ = conv1d_varlen(np.abs(c["xbc64"]), np.abs(c["w64"]), c["cu"], np.abs(c["b64"]),
                           np.abs(c["st64"]), activation=False)
    check_parity(cat_out(x, B, C), ref, mag, io)
    # final states are copies of inputs (exact)
    assert np.array_equal(erd.to_f64(c["state"]), fin)
    # an empty sequence leaves its slot alone
    assert same_bits(c["state"][0], st0[0])


@pytest.mark.parametrize("W", [2, 3, 4])
@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_conv_update_token_by_token_equals_prefill(W, io):
    lengths = [300, 1, 77]
    c = setup(lengths, H=8, G=1, P=64, N=128, W=W, io=io, seed=10 + W)
    st_pre = c["state"].clone()
    x, B, C = erd.ssd_conv1d_varlen(c["shape"], c["cu"], c["xbc"], c["weight"], c["bias"],
                                    conv_state=st_pre)
    y_pre = cat_out(x, B, C)
    st = c["state"].clone()
    cu = c["cu"]
    ys = torch.empty_like(y_pre)
    for k in range(max(lengths)):
        live = [s for s in range(3) if k < lengths[s]]
        it = torch.tensor([int(cu[s]) + k for s in live], device=DEV)
        sl = torch.tensor(live, dtype=torch.int32, device=DEV)
        xd, Bd, Cd = erd.ssd_conv1d_update(c["shape"], c["xbc"][it], c["weight"], st,
                                           c["bias"], slot_idx=sl)
        ys[it] = cat_out(xd, Bd, Cd)
    assert same_bits(ys, y_pre)
    assert same_bits(st, st_pre)


@pytest.mark.parametrize("W", [2, 4])
def test_conv_split_prefill_bitwise(W):
    """Chunked prefill at any split, with the state carried in place,
    reproduces the unsplit prefill."""
    L = 700
    c = setup([L], H=4, G=1, P=64, N=64, W=W, io="bf16", seed=3)
    st = c["state"].clone()
    x, B, C = erd.ssd_conv1d_varlen(c["shape"], c["cu"], c["xbc"], c["weight"], c["bias"],
                                    conv_state=st)
    whole = cat_out(x, B, C)
    for splits in ([1, 1, 1, 697], [2, 255, 256, 187], [W - 1, 1, L - W], [333, 367],
                   [256] * 2 + [188]):
        s2 = c["state"].clone()
        parts, t = [], 0
        for n in splits:
            xo, Bo, Co = erd.ssd_conv1d_varlen(c["shape"], [0, n], c["xbc"][t:t + n],
                                               c["weight"], c["bias"], conv_state=s2)
            parts.append(cat_out(xo, Bo, Co))
            t += n
        assert same_bits(torch.cat(parts), whole), splits
        assert same_bits(s2, st)


def test_conv_packing_and_slots_invariance():
    """A sequence's outputs and final state do not depend on the rest of the
    pack, its position in it, or which slot holds its state."""
    lengths = [260, 5, 129, 0, 64]
    c = setup(lengths, H=4, G=2, P=32, N=32, W=4, io="bf16", seed=5, slots=8)
    sl = torch.tensor([6, 1, 3, 0, 7], dtype=torch.int32, device=DEV)
    st = c["state"].clone()
    x, B, C = erd.ssd_conv1d_varlen(c["shape"], c["cu"], c["xbc"], c["weight"], c["bias"],
                                    conv_state=st, slot_idx=sl)
    y = cat_out(x, B, C)
    cu = c["cu"]
    for s in (0, 2, 4):
        a, b = int(cu[s]), int(cu[s + 1])
        one = c["state"][sl[s].long():sl[s].long() + 1].clone()
        xo, Bo, Co = erd.ssd_conv1d_varlen(c["shape"], [0, b - a], c["xbc"][a:b], c["weight"],
                                           c["bias"], conv_state=one)
        assert same_bits(cat_out(xo, Bo, Co), y[a:b])
        assert same_bits(one[0], st[sl[s].long()])
    # slots not named are untouched; the empty sequence's slot too
    for k in (2, 4, 5, 0):
        assert same_bits(st[k], c["state"][k])


def test_conv_without_state_is_zero_history():
    c = setup([40, 3], H=4, G=1, P=16, N=16, W=4, io="f32", seed=8)
    x, B, C = erd.ssd_conv1d_varlen(c["shape"], c["cu"], c["xbc"], c["weight"], c["bias"])
    z = torch.zeros_like(c["state"])
    x2, B2, C2 = erd.ssd_conv1d_varlen(c["shape"], c["cu"], c["xbc"], c["weight"], c["bias"],
                                       conv_state=z)
    assert same_bits(cat_out(x, B, C), cat_out(x2, B2, C2))


def test_conv_then_scan_decode_equals_prefill():
    """The mixer's front end end to end: conv -> scan over a 600-token
    prompt plus 300 generated tokens, once as a single prefill and once as a
    prompt prefill followed by token-by-token conv updates and replay decode:
    the scan outputs are bit-identical."""
    H, G, P, N, Q, W = 8, 1, 64, 128, 256, 4
    shape = erd.Shape(H, G, P, N, Q, "bf16", "bf16")
    cd = erd.conv_dim(shape)
    T, T0 = 900, 600
    cp = synth.make_conv_params(cd, W, 1)
    weight, bias = torch.from_numpy(cp.weight).to(DEV), torch.from_numpy(cp.bias).to(DEV)
    xbc = erd.to_device(synth.make_xbc(T, cd, 1), "bf16", DEV)
    hp = synth.make_head_params(H, 1)
    A, D, dtb = (torch.from_numpy(v).to(DEV) for v in (hp.A, hp.D, hp.dt_bias))
    dt = erd.to_device(synth.make_tokens(T, H, G, P, N, 1).dt, "bf16", DEV)
    # single shot
    x, B, C = erd.ssd_conv1d_varlen(shape, [0, T], xbc, weight, bias)
    y_ss, _, _ = erd.ssd_prefill_varlen(shape, [0, T], x, dt, A, B, C, D, dtb)
    # prompt, then decode
    cst = torch.zeros((1, cd, W - 1), dtype=torch.bfloat16, device=DEV)
    cache = erd.ReplayCache(shape, 1, DEV)
    x0, B0, C0 = erd.ssd_conv1d_varlen(shape, [0, T0], xbc[:T0], weight, bias, conv_state=cst)
    y0 = erd.ssd_replay_prefill(shape, cache, [0, T0], x0, dt[:T0], B0, C0, A, D, dtb)
    ys = [y0]
    for t in range(T0, T):
        xt, Bt, Ct = erd.ssd_conv1d_update(shape, xbc[t:t + 1], weight, cst, bias)
        ys.append(erd.ssd_replay_decode(shape, cache, xt, dt[t:t + 1], Bt, Ct, A, D, dtb))
    assert same_bits(torch.cat(ys), y_ss)


def test_conv_full_size_sampled_parity():
    """256 sequences x 2048 tokens at H=32, G=1, P=64, N=128, W=4 (the
    bench workload): sampled sequences against the oracle, and the final
    states."""
    S, T, H, G, P, N, W = 256, 2048, 32, 1, 64, 128, 4
    shape = erd.Shape(H, G, P, N, 256, "bf16", "bf16")
    cd = erd.conv_dim(shape)
    cu = synth.cu_seqlens([T] * S)
    xbc = synth.make_xbc_torch(S * T, cd, 2, DEV)
    cp = synth.make_conv_params(cd, W, 2)
    weight, bias = torch.from_numpy(cp.weight).to(DEV), torch.from_numpy(cp.bias).to(DEV)
    st = torch.zeros((S, cd, W - 1), dtype=torch.bfloat16, device=DEV)
    x, B, C = erd.ssd_conv1d_varlen(shape, cu, xbc, weight, bias, conv_state=st)
    for s in (0, 97, 255):
        a = s * T
        inp = erd.to_f64(xbc[a:a + T])
        ref, fin = conv1d_varlen(inp, cp.weight, [0, T], cp.bias)
        mag, _ = conv1d_varlen(np.abs(inp), np.abs(cp.weight), [0, T], np.abs(cp.bias),
                               activation=False)
        check_parity(cat_out(x[a:a + T], B[a:a + T], C[a:a + T]), ref, mag, "bf16")
        assert np.array_equal(erd.to_f64(st[s]), fin[0])


def _fused_setup(B, H, G, P, N, Q, W, seed):
    shape = erd.Shape(H, G, P, N, Q, "bf16", "bf16")
    cd = erd.conv_dim(shape)
    cp = synth.make_conv_params(cd, W, seed)
    hp = synth.make_head_params(H, seed)
    prm = tuple(torch.from_numpy(v).to(DEV) for v in (hp.A, hp.D, hp.dt_bias))
    pre = synth.replay_prefix_lengths(B, Q, seed)
    px, pdt, pB, pC = synth.make_tokens_torch(int(pre.sum()), H, G, P, N, seed, DEV)
    caches = []
    for _ in range(2):
        c = erd.ReplayCache(shape, B, DEV)
        erd.ssd_replay_prefill(shape, c, synth.cu_seqlens(pre), px, pdt, pB, pC, *prm)
        caches.append(c)
    st = erd.to_device(synth.make_xbc(B * (W - 1), cd, seed + 1), "bf16", DEV)
    cstate = st.view(W - 1, B, cd).permute(1, 2, 0).contiguous()
    return shape, cd, cp, prm, caches, [cstate.clone(), cstate.clone()]


@pytest.mark.parametrize("Q,G,W,Bn", [(256, 1, 4, 128), (16, 8, 3, 64), (256, 8, 2, 64)])
def test_fused_conv_decode_equals_two_launches(Q, G, W, Bn):
    """ssd_replay_decode_conv (the conv's decode form and the replay step in
    one launch) against ssd_conv1d_update then ssd_replay_decode, over
    enough steps to fill chunks (buffers holding 0..Q-1 tokens):
    outputs, the conv's x | B | C, the conv state and every cache array
    bit for bit; positions in permuted slot order with one skipped. B=128
    at H=32 has more workgroups than run at once (the ranked launch)."""
    H, P, N = 32, 64, 128
    shape, cd, cp, prm, caches, cst = _fused_setup(Bn, H, G, P, N, Q, W, 31)
    A, D, dtb = prm
    weight, bias = torch.from_numpy(cp.weight).to(DEV), torch.from_numpy(cp.bias).to(DEV)
    slots = torch.from_numpy(np.random.default_rng(5).permutation(Bn).astype(np.int32)).to(DEV)
    slots[7] = -1                                   # skipped: no conv, no step
    steps = 40 if Q == 256 else 20
    xbc = erd.to_device(synth.make_xbc(steps * Bn, cd, 32), "bf16", DEV).view(steps, Bn, cd)
    dts = erd.to_device(synth.make_tokens(steps * Bn, H, G, P, N, 33).dt, "bf16",
                        DEV).view(steps, Bn, H)
    for i in range(steps):
        x, Bt, Ct = erd.ssd_conv1d_update(shape, xbc[i], weight, cst[0], bias, slot_idx=slots)
        y0 = erd.ssd_replay_decode(shape, caches[0], x, dts[i], Bt, Ct, A, D, dtb,
                                   slot_idx=slots)
        y1, (x1, B1, C1) = erd.ssd_replay_decode_conv(shape, caches[1], xbc[i], weight, cst[1],
                                                       dts[i], A, D, dtb, bias=bias,
                                                       slot_idx=slots)
        keep = torch.arange(Bn, device=DEV) != 7
        assert same_bits(y1[keep], y0[keep]), i
        assert same_bits(x1[keep], x[keep]) and same_bits(B1[keep], Bt[keep]) and \
            same_bits(C1[keep], Ct[keep]), i
        assert same_bits(cst[1], cst[0]), i
    c0, c1 = caches
    for name in ("state", "buf_x", "buf_dt", "buf_B", "buf_len", "boundary_pos", "work"):
        assert same_bits(getattr(c1, name), getattr(c0, name)), name
    assert same_bits(c1.state_bf_rowmajor(), c0.state_bf_rowmajor())

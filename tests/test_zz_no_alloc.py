"""The allocation-free decode entry point (ssd_replay_decode_static, for
callers that cannot allocate device memory) against ssd_replay_decode,
through the C ABI: two calls in a row, the second with a smaller batch, on
twin caches prepared identically; outputs and every cache array bit for
bit, and the library's array left zero (a third call on a fresh twin
agrees too). Covers a batch that runs in one launch and one that is ranked
first, and chunks that fill during the calls."""
import numpy as np
import pytest
import torch

import exact_replay_decode_amd as erd
from exact_replay_decode_amd import synth
from gpu_cases import DEV, same_bits

pytestmark = pytest.mark.gpu


def twin_caches(shape, S, seed):
    hp = synth.make_head_params(shape.H, seed)
    rng = np.random.default_rng(seed)
    pre = rng.integers(1, 3 * shape.chunk_size, S)
    # a few slots one token short of a full chunk, so the calls fill them
    pre[::5] = shape.chunk_size - 1
    total = int(pre.sum()) + 4 * S
    x, dt, B, C = synth.make_tokens_torch(total, shape.H, shape.G, shape.P, shape.N, seed, DEV)
    A, D, bias = (torch.from_numpy(v).to(DEV) for v in (hp.A, hp.D, hp.dt_bias))
    cu = synth.cu_seqlens(pre)
    caches = []
    for _ in range(2):
        c = erd.ReplayCache(shape, S, DEV)
        erd.ssd_replay_prefill(shape, c, cu, x[:cu[-1]], dt[:cu[-1]], B[:cu[-1]], C[:cu[-1]], A,
                               D, bias)
        caches.append(c)
    return caches, (x, dt, B, C), (A, D, bias), int(cu[-1])


def same_cache(a, b):
    return (same_bits(a.state, b.state) and same_bits(a.state_bf, b.state_bf)
            and same_bits(a.buf_x, b.buf_x) and same_bits(a.buf_dt, b.buf_dt)
            and same_bits(a.buf_B, b.buf_B) and torch.equal(a.buf_len, b.buf_len)
            and torch.equal(a.boundary_pos, b.boundary_pos))


@pytest.mark.parametrize("S,H,G,Q,batches", [
    (16, 8, 2, 64, [16, 5]),        # every workgroup resident at once: one launch
    (300, 32, 1, 256, [300, 130]),  # ranked launch (more workgroups than run at once)
])
def test_static_decode_matches_plain_decode(S, H, G, Q, batches):
    shape = erd.Shape(H, G, 64, 128, Q, "bf16", "bf16")
    (plain, static), (x, dt, B, C), (A, D, bias), t = twin_caches(shape, S, seed=S + Q)
    rng = np.random.default_rng(7)
    for nb in batches:
        sl = torch.from_numpy(rng.permutation(S)[:nb].astype(np.int32)).to(DEV)
        it = torch.arange(t, t + nb, device=DEV)
        t += nb
        y0 = erd.ssd_replay_decode(shape, plain, x[it], dt[it], B[it], C[it], A, D, bias,
                                   slot_idx=sl)
        y1 = erd.ssd_replay_decode(shape, static, x[it], dt[it], B[it], C[it], A, D, bias,
                                   slot_idx=sl, static_work=True)
        torch.cuda.synchronize()
        assert same_bits(y1, y0), nb
        assert same_cache(static, plain), nb
        assert not plain.work.any()


def test_static_decode_rejects_large_caches():
    shape = erd.Shape(1, 1, 16, 16, 16, "bf16", "bf16")
    c = erd.ReplayCache(shape, 32769, DEV)
    x = torch.zeros((1, 1, 16), dtype=torch.bfloat16, device=DEV)
    dt = torch.zeros((1, 1), dtype=torch.bfloat16, device=DEV)
    BC = torch.zeros((1, 1, 16), dtype=torch.bfloat16, device=DEV)
    A = torch.zeros(1, device=DEV)
    with pytest.raises(erd.SsdError) as e:
        erd.ssd_replay_decode(shape, c, x, dt, BC, BC, A, static_work=True)
    assert e.value.code == -6

"""C ABI checks that need no GPU: the library loads, exports every entry
point include/ssd_replay.h declares, and rejects bad arguments on the host
with the documented status before launching anything."""
import ctypes
import os
import re

import numpy as np
import pytest

import exact_replay_decode_amd as erd
from exact_replay_decode_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "ssd_replay.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    want = {"ssd_status_string", "ssd_replay_cache_bytes", "ssd_prefill_workspace_bytes",
            "ssd_prefill_varlen", "ssd_commit_boundary", "ssd_replay_prefill",
            "ssd_replay_decode", "ssm_state_update", "ssd_replay_cache_refresh",
            "ssd_replay_page_bytes", "ssd_conv1d_varlen", "ssd_conv1d_update",
            "ssd_replay_verify", "ssd_replay_accept", "ssm_state_update_varlen",
            "ssd_prefill_chunk_count", "ssd_replay_decode_static", "ssd_replay_decode_conv"}
    assert set(declared_functions()) == want
    assert set(_lib.EXPORTS) == want


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    for code, name in _lib.STATUS.items():
        assert _lib.status_string(code).startswith(name)
    assert _lib.status_string(12345) == "unknown ssd_status"


def test_cache_bytes_match_printed_memory():
    """RFC section 4: about 1.16 MiB of buffer (x, dt, B, C with 4-byte dt)
    plus 1 MiB of fp32 state per layer and sequence at H=32, G=1, P=64,
    N=128, chunk 256."""
    import json
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                    "rfc_printed_numbers.json")))
    sh = erd.Shape(32, 1, 64, 128, 256, "bf16", "f32")
    total = erd.ssd_replay_cache_bytes(sh, 1, with_C=True)
    state = 32 * 64 * 128 * 4
    state_bf = 32 * 64 * 128 * 2      # bf16 copy of the state (read-out operand)
    buf = total - state - state_bf - 3 * 4 - 8 - 34 * 4
    assert state / 2 ** 20 == g["fp32_state_mib_per_layer_per_seq"]["value"]
    assert round(buf / 2 ** 20, 2) == g["buffer_mib_per_layer_per_seq"]["value"]
    # per slot, plus two shared bookkeeping words
    assert erd.ssd_replay_cache_bytes(sh, 27, with_C=True) == 27 * (total - 136) + 136
    # the scan never reads buffered C: without it the buffer shrinks by G*N*2*Q
    assert total - erd.ssd_replay_cache_bytes(sh, 1, with_C=False) == 256 * 128 * 2


# ---- fail-closed validation (no launch; fake device pointers) -------------

FAKE = ctypes.c_void_p(0x1000)


def shape(**kw):
    base = dict(H=4, G=1, P=16, N=16, chunk_size=16, io_dtype=1, dt_dtype=1, state_dtype=0,
                dt_softplus=1)
    base.update(kw)
    return _lib.ssd_shape(**base)


def prefill(sh, cu=(0, 8), T=8, **over):
    lib = _lib.load()
    cu = np.asarray(cu, dtype=np.int32)
    args = dict(x=FAKE, dt=FAKE, A=FAKE, B=FAKE, C=FAKE, y=FAKE, cu_dev=FAKE)
    args.update(over)
    return lib.ssd_prefill_varlen(ctypes.byref(sh), len(cu) - 1, T,
                                  cu.ctypes.data_as(ctypes.c_void_p), args["cu_dev"], args["x"],
                                  args["dt"], args["A"], args["B"], args["C"], None, None, None,
                                  args["y"], None, None, args.get("cs"), None, 0, None)


@pytest.mark.parametrize("kw,code", [
    (dict(state_dtype=1), -4), (dict(io_dtype=7), -3), (dict(dt_dtype=-1), -3),
    (dict(H=6, G=4), -2), (dict(H=0), -2), (dict(G=0), -2),
    (dict(chunk_size=512), -7), (dict(chunk_size=48), -7), (dict(P=256), -7),
    (dict(N=8), -7), (dict(P=24), -7)])
def test_prefill_rejects_bad_shapes(kw, code):
    assert prefill(shape(**kw)) == code


def test_prefill_rejects_bad_seqlens_and_nulls():
    sh = shape()
    assert prefill(sh, cu=(0, 5), T=8) == -2          # cu[S] != T
    assert prefill(sh, cu=(1, 8), T=8) == -2          # cu[0] != 0
    assert prefill(sh, cu=(0, 6, 4, 8), T=8) == -2    # decreasing
    assert prefill(sh, x=None) == -1
    assert prefill(sh, A=None) == -1
    assert prefill(sh, cu_dev=None) == -1
    assert prefill(shape(), cu=(0,), T=0) == 0        # nothing to do, no launch
    assert prefill(sh, x=ctypes.c_void_p(0x1002)) == -9   # misaligned x
    assert prefill(sh, y=ctypes.c_void_p(0x1008)) == -9
    assert prefill(sh, cs=ctypes.c_void_p(0x1004)) == -9  # misaligned chunk_states


def test_prefill_chunk_count():
    lib = _lib.load()

    def count(cu, Q):
        cu = np.asarray(cu, dtype=np.int32)
        return lib.ssd_prefill_chunk_count(len(cu) - 1, cu.ctypes.data_as(ctypes.c_void_p), Q)

    # full chunks per sequence, summed: 600 // 256 + 300 // 256 + 900 // 256 + 248 // 256
    assert count([0, 600, 900, 1800, 2048], 256) == 2 + 1 + 3 + 0
    assert count([0, 2048], 256) == 8 and count([0, 2047], 256) == 7
    assert count([0, 16, 16, 48], 16) == 1 + 0 + 2
    assert count([0], 16) == 0
    assert count([0, 8, 4], 16) == -1                 # decreasing
    assert count([0, 8], 0) == -1
    assert lib.ssd_prefill_chunk_count(1, None, 16) == -1
    assert erd.api.ssd_prefill_chunk_count([0, 600, 900, 1800, 2048], 256) == 6


def cache(sh_c, **kw):
    base = dict(state=0x1000, state_bf=0x1000, buf_x=0x1000, buf_dt=0x1000, buf_B=0x1000,
                buf_C=None, buf_len=0x1000, boundary_pos=0x1000, work=0x1000, num_slots=4,
                chunk_size=16, state_dtype=0)
    base.update(kw)
    return _lib.ssd_replay_cache(**base)


def decode(sh, c, batch=2):
    lib = _lib.load()
    return lib.ssd_replay_decode(ctypes.byref(sh), ctypes.byref(c), batch, None, FAKE, FAKE,
                                 FAKE, FAKE, FAKE, None, None, FAKE, None)


def test_static_decode_checks():
    # the allocation-free decode needs no work array, takes at most 32768
    # slots, and fails closed like the plain one
    lib = _lib.load()

    def dec(sh, c, batch=2):
        return lib.ssd_replay_decode_static(ctypes.byref(sh), ctypes.byref(c), batch, None, FAKE,
                                            FAKE, FAKE, FAKE, FAKE, None, None, FAKE, None)
    sh = shape()
    assert dec(sh, cache(sh, work=None, num_slots=32769), batch=0) == -6
    assert dec(sh, cache(sh, work=None, state_dtype=1)) == -4
    assert dec(sh, cache(sh, work=None, chunk_size=32)) == -5
    assert dec(sh, cache(sh, work=None), batch=0) == 0     # nothing to do, no launch
    assert dec(sh, cache(sh, work=None, buf_B=None)) == -1
    assert decode(sh, cache(sh, work=None)) == -1          # the plain form needs it


def test_replay_fails_closed():
    sh = shape()
    assert decode(sh, cache(sh, state_dtype=1)) == -4        # non-fp32 state
    assert decode(sh, cache(sh, chunk_size=32)) == -5        # chunk mismatch
    assert decode(sh, cache(sh, buf_B=None)) == -1
    assert decode(sh, cache(sh, state_bf=None)) == -1
    assert decode(sh, cache(sh, work=None)) == -1
    assert decode(sh, cache(sh, state_bf=0x1008)) == -9      # misaligned
    lib = _lib.load()
    assert lib.ssd_replay_cache_refresh(ctypes.byref(sh), ctypes.byref(cache(sh, state=None)),
                                        None) == -1
    assert lib.ssd_replay_cache_refresh(ctypes.byref(sh), ctypes.byref(cache(sh, chunk_size=32)),
                                        None) == -5
    assert decode(sh, cache(sh, num_slots=0)) == -2
    assert decode(sh, cache(sh), batch=5) == -2              # more rows than slots
    assert decode(shape(state_dtype=1), cache(sh)) == -4
    assert decode(sh, cache(sh), batch=0) == 0
    lib = _lib.load()
    cu = np.asarray([0, 8], dtype=np.int32)
    c = cache(sh, chunk_size=64)
    assert lib.ssd_replay_prefill(ctypes.byref(sh), ctypes.byref(c), 1, 8,
                                  cu.ctypes.data_as(ctypes.c_void_p), FAKE, None, FAKE, FAKE,
                                  FAKE, FAKE, FAKE, None, None, FAKE, None) == -5
    assert lib.ssd_commit_boundary(ctypes.byref(sh), 1, 8, cu.ctypes.data_as(ctypes.c_void_p),
                                   FAKE, None, FAKE, FAKE, FAKE, FAKE, None,
                                   ctypes.byref(cache(sh)), None) == -1
    # the recurrent update takes fp32 or bf16 state; any other code fails closed
    assert lib.ssm_state_update(ctypes.byref(shape(state_dtype=2)), 1, 1, None, FAKE, FAKE,
                                FAKE, FAKE, FAKE, FAKE, None, None, FAKE, None) == -4
    assert lib.ssm_state_update(ctypes.byref(sh), 3, 2, None, FAKE, FAKE, FAKE, FAKE, FAKE,
                                FAKE, None, None, FAKE, None) == -2


def test_speculative_entry_points_fail_closed():
    sh = shape()
    lib = _lib.load()
    cu = np.asarray([0, 4], dtype=np.int32)
    cup = cu.ctypes.data_as(ctypes.c_void_p)
    verify = lambda c, **k: lib.ssd_replay_verify(  # noqa: E731
        ctypes.byref(sh), ctypes.byref(c), 1, 4, cup, FAKE, None, FAKE, FAKE, FAKE,
        k.get("C", FAKE), FAKE, None, None, k.get("y", FAKE), None)
    accept = lambda c, **k: lib.ssd_replay_accept(  # noqa: E731
        ctypes.byref(sh), ctypes.byref(c), 1, 4, cup, FAKE, None, k.get("acc", FAKE), FAKE,
        FAKE, FAKE, k.get("C", None), FAKE, None, None)
    assert verify(cache(sh, chunk_size=32)) == -5
    assert verify(cache(sh, state_dtype=1)) == -4
    assert verify(cache(sh), y=None) == -1
    assert verify(cache(sh), C=None) == -1
    assert accept(cache(sh), acc=None) == -1
    assert accept(cache(sh, buf_C=0x1000)) == -1             # C buffered: C needed
    assert accept(cache(sh, chunk_size=64)) == -5


def test_varlen_ssu_checks():
    lib = _lib.load()
    cu = np.asarray([0, 4, 9], dtype=np.int32)
    cup = cu.ctypes.data_as(ctypes.c_void_p)
    call = lambda sh, **k: lib.ssm_state_update_varlen(  # noqa: E731
        ctypes.byref(sh), 2, 9, cup, FAKE, None, k.get("ns", 2), k.get("state", FAKE), FAKE,
        FAKE, FAKE, FAKE, FAKE, None, None, k.get("y", FAKE), None)
    assert call(shape(state_dtype=2)) == -4
    assert call(shape(), ns=1) == -2                        # more sequences than slots
    assert call(shape(), state=None) == -1
    assert call(shape(), y=None) == -1
    assert call(shape(), state=ctypes.c_void_p(0x1004)) == -9


def test_paged_cache_checks():
    """Paged buffers: page_tokens a power of two in [16, Q], num_pages > 0."""
    sh = shape(chunk_size=64)
    ok = dict(chunk_size=64, buf_pages=0x2000, page_tokens=32, num_pages=8)
    assert decode(sh, cache(sh, **ok), batch=0) == 0
    for bad in (dict(page_tokens=8), dict(page_tokens=128), dict(page_tokens=48),
                dict(page_tokens=0), dict(num_pages=0), dict(num_pages=-3)):
        assert decode(sh, cache(sh, **{**ok, **bad}), batch=0) == -2, bad
    # page_tokens and num_pages are ignored without a page table
    assert decode(sh, cache(sh, chunk_size=64, page_tokens=3, num_pages=-1), batch=0) == 0


def test_page_bytes():
    sh = erd.Shape(32, 1, 64, 128, 256, "bf16", "f32")
    per_tok = 32 * 64 * 2 + 32 * 4 + 2 * 128 * 2
    assert erd.ssd_replay_page_bytes(sh, 64, with_C=True) == 64 * per_tok
    assert erd.ssd_replay_page_bytes(sh, 16, with_C=False) == 16 * (per_tok - 128 * 2)
    # a whole chunk of pages is the contiguous buffer of one slot
    slot = erd.ssd_replay_cache_bytes(sh, 1, with_C=True) - 34 * 4
    assert slot - erd.ssd_replay_page_bytes(sh, 256, with_C=True) == \
        32 * 64 * 128 * 6 + 3 * 4 + 8
    for bad in (8, 512, 48, 0):
        assert erd.ssd_replay_page_bytes(sh, bad, with_C=True) == 0


def conv_prefill(sh, W=4, S=1, T=8, cu=None, state=None, num_slots=0, **over):
    lib = _lib.load()
    cu = np.asarray(cu if cu is not None else [0] + [T] * S, dtype=np.int32)
    a = dict(xBC=FAKE, weight=FAKE, x=FAKE, B=FAKE, C=FAKE, cu_dev=FAKE)
    a.update(over)
    return lib.ssd_conv1d_varlen(ctypes.byref(sh), W, 1, len(cu) - 1, int(cu[-1]),
                                 cu.ctypes.data_as(ctypes.c_void_p), a["cu_dev"], None,
                                 num_slots, a["xBC"], a["weight"], None, state, a["x"],
                                 a["B"], a["C"], None)


def test_conv_checks():
    sh = shape()
    assert conv_prefill(sh, W=1) == -7 and conv_prefill(sh, W=5) == -7
    assert conv_prefill(sh, weight=None) == -1
    assert conv_prefill(sh, x=None) == -1
    assert conv_prefill(sh, xBC=ctypes.c_void_p(0x1004)) == -9
    assert conv_prefill(sh, state=ctypes.c_void_p(0x1008), num_slots=1) == -9
    assert conv_prefill(sh, state=FAKE, num_slots=0) == -2     # state but no slots
    assert conv_prefill(sh, weight=ctypes.c_void_p(0x1004)) == -9   # taps read in 16 B
    assert conv_prefill(sh, cu=[0, 4, 2, 8]) == -2
    assert conv_prefill(sh, cu=[0, 0]) == 0                    # empty sequence: nothing to do
    assert conv_prefill(shape(state_dtype=1)) == -4
    big = np.zeros(65537, dtype=np.int32)
    assert conv_prefill(sh, cu=big) == -2                      # more than 65535 sequences
    lib = _lib.load()
    upd = lambda **k: lib.ssd_conv1d_update(  # noqa: E731
        ctypes.byref(sh), k.get("W", 4), 1, k.get("batch", 2), None, k.get("ns", 4),
        k.get("xBC", FAKE), FAKE, None, k.get("state", FAKE), FAKE, FAKE, FAKE, None)
    assert upd(W=6) == -7
    assert upd(state=None) == -1
    assert upd(batch=5) == -2                                  # more rows than slots
    assert upd(batch=0) == 0
    assert upd(xBC=ctypes.c_void_p(0x1002)) == -9


def test_fused_conv_decode_checks():
    # the conv + decode step fails closed on the conv's arguments and on the
    # decode's, before any launch
    sh = shape()
    lib = _lib.load()

    def dec(c=None, W=4, batch=2, xBC=FAKE, weight=FAKE, state=FAKE):
        c = cache(sh) if c is None else c
        return lib.ssd_replay_decode_conv(ctypes.byref(sh), ctypes.byref(c), batch, None, W, 1,
                                          xBC, weight, None, state, FAKE, FAKE, FAKE, FAKE,
                                          FAKE, None, None, FAKE, None)
    assert dec(W=1) == -7 and dec(W=5) == -7
    assert dec(xBC=None) == -1 and dec(weight=None) == -1 and dec(state=None) == -1
    assert dec(xBC=ctypes.c_void_p(0x1002)) == -9
    assert dec(weight=ctypes.c_void_p(0x1004)) == -9
    assert dec(c=cache(sh, state_dtype=1)) == -4                 # the decode's own checks
    assert dec(c=cache(sh, chunk_size=32)) == -5
    assert dec(c=cache(sh, work=None)) == -1
    assert dec(batch=5) == -2                                    # more rows than slots
    assert dec(batch=0) == 0


def test_python_binding_checks_extents():
    torch = pytest.importorskip("torch")
    sh = erd.Shape(4, 1, 16, 16, 16, "f32", "f32")
    x = torch.zeros((8, 4, 16))
    with pytest.raises(ValueError):
        erd.ssd_prefill_varlen(sh, [0, 8], x, torch.zeros((8, 3)), torch.zeros(4),
                               torch.zeros((8, 1, 16)), torch.zeros((8, 1, 16)))

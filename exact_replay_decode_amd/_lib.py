"""ctypes declarations of libssd_replay.so (include/ssd_replay.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libssd_replay.so")

SSD_F32, SSD_BF16 = 0, 1

STATUS = {
    0: "SSD_OK", -1: "SSD_ERR_NULL", -2: "SSD_ERR_SHAPE", -3: "SSD_ERR_DTYPE",
    -4: "SSD_ERR_STATE_NOT_FP32", -5: "SSD_ERR_CHUNK_MISMATCH",
    -6: "SSD_ERR_WORKSPACE", -7: "SSD_ERR_UNSUPPORTED", -8: "SSD_ERR_HIP", -9: "SSD_ERR_ALIGN",
}

# every symbol include/ssd_replay.h declares
EXPORTS = ("ssd_status_string", "ssd_replay_cache_bytes", "ssd_prefill_workspace_bytes",
           "ssd_prefill_varlen", "ssd_commit_boundary", "ssd_replay_prefill",
           "ssd_replay_decode", "ssm_state_update", "ssd_replay_cache_refresh",
           "ssd_replay_page_bytes", "ssd_conv1d_varlen", "ssd_conv1d_update",
           "ssd_replay_verify", "ssd_replay_accept", "ssm_state_update_varlen",
           "ssd_prefill_chunk_count", "ssd_replay_decode_static", "ssd_replay_decode_conv")


class ssd_shape(ctypes.Structure):
    _fields_ = [("H", ctypes.c_int32), ("G", ctypes.c_int32), ("P", ctypes.c_int32),
                ("N", ctypes.c_int32), ("chunk_size", ctypes.c_int32),
                ("io_dtype", ctypes.c_int32), ("dt_dtype", ctypes.c_int32),
                ("state_dtype", ctypes.c_int32), ("dt_softplus", ctypes.c_int32)]


class ssd_replay_cache(ctypes.Structure):
    _fields_ = [("state", ctypes.c_void_p), ("state_bf", ctypes.c_void_p),
                ("buf_x", ctypes.c_void_p), ("buf_dt", ctypes.c_void_p),
                ("buf_B", ctypes.c_void_p), ("buf_C", ctypes.c_void_p),
                ("buf_len", ctypes.c_void_p), ("boundary_pos", ctypes.c_void_p),
                ("work", ctypes.c_void_p), ("num_slots", ctypes.c_int32),
                ("chunk_size", ctypes.c_int32), ("state_dtype", ctypes.c_int32),
                ("buf_pages", ctypes.c_void_p), ("page_tokens", ctypes.c_int32),
                ("num_pages", ctypes.c_int32)]


_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m exact_replay_decode_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    shp = ctypes.POINTER(ssd_shape)
    cp = ctypes.POINTER(ssd_replay_cache)
    lib.ssd_status_string.restype = ctypes.c_char_p
    lib.ssd_status_string.argtypes = [ctypes.c_int]
    lib.ssd_replay_cache_bytes.restype = sz
    lib.ssd_replay_cache_bytes.argtypes = [shp, i32, i32]
    lib.ssd_prefill_workspace_bytes.restype = sz
    lib.ssd_prefill_workspace_bytes.argtypes = [shp, i32, i64]
    lib.ssd_prefill_varlen.restype = ctypes.c_int
    lib.ssd_prefill_varlen.argtypes = [shp, i32, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                       vp, vp, vp, vp, vp, vp, sz, vp]
    lib.ssd_prefill_chunk_count.restype = i64
    lib.ssd_prefill_chunk_count.argtypes = [i32, vp, i32]
    lib.ssd_replay_page_bytes.restype = sz
    lib.ssd_replay_page_bytes.argtypes = [shp, i32, i32]
    lib.ssd_replay_cache_refresh.restype = ctypes.c_int
    lib.ssd_replay_cache_refresh.argtypes = [shp, cp, vp]
    lib.ssd_commit_boundary.restype = ctypes.c_int
    lib.ssd_commit_boundary.argtypes = [shp, i32, i64, vp, vp, vp, vp, vp, vp, vp, vp, cp, vp]
    lib.ssd_replay_prefill.restype = ctypes.c_int
    lib.ssd_replay_prefill.argtypes = [shp, cp, i32, i64, vp, vp, vp, vp, vp, vp, vp, vp,
                                       vp, vp, vp, vp]
    lib.ssd_replay_verify.restype = ctypes.c_int
    lib.ssd_replay_verify.argtypes = [shp, cp, i32, i64, vp, vp, vp, vp, vp, vp, vp, vp,
                                      vp, vp, vp, vp]
    lib.ssd_replay_accept.restype = ctypes.c_int
    lib.ssd_replay_accept.argtypes = [shp, cp, i32, i64, vp, vp, vp, vp, vp, vp, vp, vp,
                                      vp, vp, vp]
    lib.ssd_replay_decode.restype = ctypes.c_int
    lib.ssd_replay_decode.argtypes = [shp, cp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.ssd_replay_decode_static.restype = ctypes.c_int
    lib.ssd_replay_decode_static.argtypes = [shp, cp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.ssd_replay_decode_conv.restype = ctypes.c_int
    lib.ssd_replay_decode_conv.argtypes = [shp, cp, i32, vp, i32, i32, vp, vp, vp, vp, vp, vp,
                                           vp, vp, vp, vp, vp, vp, vp]
    lib.ssd_conv1d_varlen.restype = ctypes.c_int
    lib.ssd_conv1d_varlen.argtypes = [shp, i32, i32, i32, i64, vp, vp, vp, i32, vp, vp, vp,
                                      vp, vp, vp, vp, vp]
    lib.ssd_conv1d_update.restype = ctypes.c_int
    lib.ssd_conv1d_update.argtypes = [shp, i32, i32, i32, vp, i32, vp, vp, vp, vp, vp, vp, vp,
                                      vp]
    lib.ssm_state_update_varlen.restype = ctypes.c_int
    lib.ssm_state_update_varlen.argtypes = [shp, i32, i64, vp, vp, vp, i32, vp, vp, vp, vp, vp,
                                            vp, vp, vp, vp, vp]
    lib.ssm_state_update.restype = ctypes.c_int
    lib.ssm_state_update.argtypes = [shp, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    _lib = lib
    return lib


def status_string(code: int) -> str:
    return load().ssd_status_string(int(code)).decode()


class SsdError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {status_string(code)} ({code})")


def check(code: int, where: str) -> None:
    if code != 0:
        raise SsdError(code, where)

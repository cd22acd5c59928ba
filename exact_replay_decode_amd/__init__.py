"""Mamba2 SSD chunked scan with exact-replay decode for MI355X (gfx950).

The compute lives in libssd_replay.so (hand-written HIP, C ABI in
include/ssd_replay.h); this package is its torch binding plus the seeded
synthetic input generator (synth).
"""
from .api import (Shape, ReplayCache, DecodePlan, ConvUpdatePlan, ConvDecodePlan, ssd_prefill_varlen, ssd_commit_boundary,  # noqa: F401
                  ssd_replay_prefill, ssd_replay_decode, ssm_state_update,
                  ssd_replay_verify, ssd_replay_accept, ssm_state_update_varlen,
                  ssd_replay_cache_bytes, ssd_replay_page_bytes, ssd_conv1d_varlen,
                  ssd_conv1d_update, ssd_prefill_chunk_count, conv_dim, to_device,
                  ssd_replay_decode_conv,
                  to_f64)
from ._lib import SsdError, load as load_library  # noqa: F401

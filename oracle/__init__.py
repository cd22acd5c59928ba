"""fp64 CPU oracle for the Mamba2 SSD scan.

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the bench's
CPU baseline leg, never by the product path. It shares no code with the HIP
library.

- ``scan``: the sequential recurrence (plain C, OpenMP over sequence x head),
  the definition of what the scan computes.
- ``closed_form.chunked_scan``: the chunk-by-chunk closed form in numpy, an
  independent formulation used to pin ``scan``.
- ``conv1d``: the causal depthwise conv1d before the scan (prefill and decode
  forms are one definition), in numpy.
- ``ssu``: the recurrent update with the state rounded to the cache dtype
  after every token (packed-history recovery), in numpy.
"""
from .oracle import scan, threads, set_threads, ensure_built  # noqa: F401

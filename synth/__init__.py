"""Seeded synthetic inputs for the paged quantized-KV decode step.

This package only *prepares* inputs: it draws Q, K and V, writes K/V into a
paged cache the way a cache-write step would (e4m3 through torch's own cast,
e2m3 through a nearest-value table search), and builds block tables.  It holds
none of the decode step's arithmetic (no planning, no Q quantization, no
attention, no merge), so both the oracle and the HIP path can consume the
same inputs without sharing any of the computation under test.
"""

from .workloads import (  # noqa: F401
    Spec,
    Workload,
    SPECS,
    spec_for,
    build,
    e2m3_encode_table,
    pack_codes_6bit,
)

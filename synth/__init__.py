"""Seeded synthetic inputs for combined sparse decode attention.

This package draws and lays out inputs only: queries, paged K/V pools, page
tables, sequence lengths, per-layer configurations and planted needle keys.
It holds none of the attention method's arithmetic and imports neither the
CPU oracle nor the GPU library; both of those consume what it produces.

The random source is the counter-based SplitMix64 generator in ``synth.c``,
compiled with gcc into ``libfsa_synth.so`` next to this file.
"""
from .core import (  # noqa: F401
    build_lib,
    bf16_bits_to_f64,
    f64_to_bf16_bits,
    lib,
    normal_bf16,
    normal_f64,
    raw_u64,
    stream_key,
    uniform,
)
from .workloads import Workload, make_workload, WORKLOADS  # noqa: F401

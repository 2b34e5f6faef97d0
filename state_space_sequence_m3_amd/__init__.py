"""MI355X-native Mamba-3 SSM layer core.

The compute lives in ``libm3scan.so`` (hand-written HIP for gfx950, C ABI declared in
``include/m3scan.h``).  ``state_space_sequence_m3_amd.m3scan`` is the thin ctypes binding with
the same entry-point names; ``state_space_sequence_m3_amd.inputs`` draws the seeded synthetic
workloads.  Importing this package does not load the GPU library; the binding loads it on first
use and raises if it is missing.
"""
from . import inputs  # noqa: F401

__all__ = ["inputs"]

"""PACE-style periodic-rounding GDN decode with a column-scaled 4/8-bit state, for MI355X.

The compute path is the HIP library ``libpace.so`` (C ABI in include/pace.h);
``linear_attn_decode_pace_amd.pace`` is its ctypes binding and
``linear_attn_decode_pace_amd.runtime`` the torch-side helpers (device
buffers, streams, timing).  ``inputs`` generates seeded synthetic workloads.
"""

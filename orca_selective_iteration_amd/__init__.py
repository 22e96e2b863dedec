"""MI355X-native selective-batched Orca iteration.

The compute path lives in ``liborca.so`` (HIP kernels for gfx950 behind a
C ABI declared in ``include/orca.h``); ``orca_selective_iteration_amd.lib``
is a thin ctypes binding with the same entry-point names.  The library is
loaded on first use and a missing or stale build raises an error: there is no
fallback path.  Import submodules explicitly (``from
orca_selective_iteration_amd import lib, synth``).
"""

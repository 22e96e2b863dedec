"""MI355X-native selective-batched Orca iteration.

The compute path lives in ``liborca.so`` (HIP kernels for gfx950 behind a
C ABI declared in ``include/orca.h``); ``orca_selective_iteration_amd.lib``
is a thin ctypes binding with the same entry-point names.  The library is
loaded on first use; if it has not been built it is built in-tree first
(hipcc, no GPU needed), and a build older than its sources loads with a
warning.  There is no other implementation and no fallback path: an entry
point the library cannot run raises ``OrcaError``.  Import submodules explicitly (``from
orca_selective_iteration_amd import lib, synth``).
"""

"""Plain CPU oracle for one Orca iteration computed by selective batching.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link anything in this package: only ``tests/``, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` use it.  It
shares no code, constants or helpers with the HIP library; both sides receive
their inputs from the seeded generators in ``orca_selective_iteration_amd.synth``,
which hold none of the method's arithmetic.

Modules
-------
model   the transformer-layer math, the selective-batched iteration and the two
        reference formulations the method claims equality with (each request
        alone; padding + masking).
sched   the iteration-level scheduler, the request-level (static) baseline
        and the first-fit token allocator of the Attention K/V manager.

Every function cites the page and section it follows.  Functions that no page
value, closed form or library routine pins are marked "parity unpinned".
"""

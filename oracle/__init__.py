"""Plain fp64 CPU oracle for the owner-side DMuon Muon step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product package may import, call or
execute anything in this directory.  Only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` use it.

The oracle is deliberately slow and obvious: NumPy float64, dense matrix
products, one matrix at a time, in the order the method states its steps.  It
shares no code with the HIP path; the only module both sides read is ``synth``
(seeded synthetic inputs and shape tables, no arithmetic of the method).

Modules
-------
``oracle.muon``       momentum, Frobenius normalisation, wide orientation,
                      Newton-Schulz iteration, scaled update, whole step.
``oracle.pack``       per-owner contiguous buffer: pack / unpack (bit copies).
``oracle.partition``  balanced (LPT greedy) owner assignment and pack offsets.
``oracle.adamw``      AdamW step for the parameters Muon does not own.

Every function is pinned by a ``-m "not gpu"`` test against something other
than itself (closed forms, library routines, invariants, brute force).  No
function is "parity unpinned".
"""

from . import adamw, muon, pack, partition  # noqa: F401

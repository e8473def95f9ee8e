"""MI355X (gfx950) owner-side DMuon Muon step.

The computation lives in ``libdmuon.so`` (C ABI: ``include/dmuon.h``), built
from the HIP sources in ``csrc/``.  This package is its thin binding.
"""

from ._lib import DmuonError, load  # noqa: F401
from .api import (QUINTIC, AdamWOptions, StepOptions, Workspace, adamw_step,  # noqa: F401
                  chain_status, muon_step, muon_step_noalloc, nonfinite_flags, pack, pack_offsets,
                  partition_lpt, step_launches, unpack, workspace_bytes)

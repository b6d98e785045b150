"""Float64 CPU oracle for the mHC hot path.

TEST INFRASTRUCTURE ONLY.  Only tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no
code with the HIP path (``birkhoff_projection_amd``) and imports nothing from
it; the two meet only through the seeded generators in ``workloads.py``.

Modules:
  birkhoff -- projection onto the doubly stochastic matrices and its gradient
  mix      -- n-stream mix, forward and backward
  layer    -- one full mHC residual-layer step, forward and backward
"""
from .birkhoff import (birkhoff_project, birkhoff_project_bwd, residual,
                       sinkhorn, sinkhorn_fixed)
from .mix import stream_mix, stream_mix_bwd
from .layer import layer_fwd, layer_bwd

__all__ = ["birkhoff_project", "birkhoff_project_bwd", "residual", "sinkhorn",
           "sinkhorn_fixed", "stream_mix", "stream_mix_bwd", "layer_fwd",
           "layer_bwd"]

"""MI355X (gfx950) implementation of the mHC hot path.

The Birkhoff projection of per-token 4x4 residual-mixing logits (Newton on
the reduced dual, or Sinkhorn-Knopp), its implicit-differentiation backward,
and the n = 4 stream mix, as hand-written HIP kernels behind the C ABI of
``include/mhc.h``; ``ops`` is a thin ctypes binding that uses PyTorch only
for device memory and streams.
"""
from ._lib import LIB_PATH, MHCError, lib
from .ops import (BirkhoffProjection, birkhoff_bwd, birkhoff_bwd_n, birkhoff_bwd_recompute,
                  birkhoff_fwd, birkhoff_fwd_bwd, birkhoff_fwd_n, birkhoff_pipeline_step,
                  birkhoff_project,
                  layer_bwd, layer_bwd_noalloc, layer_fwd, layer_workspace, make_opts,
                  stream_mix, stream_mix_bwd)

__all__ = ["LIB_PATH", "MHCError", "lib", "BirkhoffProjection", "birkhoff_bwd",
           "birkhoff_bwd_n", "birkhoff_bwd_recompute", "birkhoff_fwd_bwd", "birkhoff_fwd_n",
           "birkhoff_fwd", "birkhoff_pipeline_step", "birkhoff_project", "layer_bwd", "layer_bwd_noalloc", "layer_fwd",
           "layer_workspace",
           "make_opts", "stream_mix", "stream_mix_bwd"]

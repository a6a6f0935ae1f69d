"""MI355X-native Block / Full Attention Residuals depth aggregation.

The compute lives in ``libattnres.so`` (hand-written gfx950 HIP kernels behind
a C ABI declared in ``include/attnres.h``); ``_lib`` binds it with ctypes and
``driver`` schedules the two-phase computation over a model's depth.
"""
from ._lib import (attnres_block_accumulate, attnres_full, attnres_phase1, attnres_phase1_first_prenorm,
                   attnres_phase1_noalloc, attnres_phase1_accumulate,
                   attnres_phase1_workspace_bytes,
                   attnres_phase2_merge, attnres_phase2_merge_multi, attnres_site_backward,
                   attnres_site_backward_accumulate,
                   attnres_site_backward_workspace_bytes, attnres_phase2_backward,
                   attnres_phase2_backward_workspace_bytes, attnres_phase1_backward,
                   attnres_phase1_backward_workspace_bytes, attnres_stream_probe, AttnResError, load,
                   status_string)
from .driver import BlockAttnRes, FullAttnRes, prefill_chunked

__all__ = ["attnres_phase1", "attnres_phase1_first_prenorm", "attnres_phase1_noalloc", "attnres_phase1_accumulate", "attnres_phase1_workspace_bytes", "attnres_phase2_merge", "attnres_phase2_merge_multi",
           "attnres_full", "attnres_block_accumulate", "attnres_site_backward",
           "attnres_site_backward_accumulate", "attnres_site_backward_workspace_bytes", "attnres_phase2_backward", "attnres_phase2_backward_workspace_bytes",
           "attnres_phase1_backward", "attnres_phase1_backward_workspace_bytes", "attnres_stream_probe", "AttnResError", "load", "status_string", "BlockAttnRes",
           "FullAttnRes", "prefill_chunked"]

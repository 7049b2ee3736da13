"""MI355X (gfx950) Mamba2 causal conv1d + SSD chunked scan with segment-local state passing.

The compute path is libssd.so (hand-written HIP for CDNA4, C ABI in
include/ssd.h).  This package only marshals torch tensors into that ABI.
"""
from ._lib import (SSD_BF16, SSD_F32, SSD_WS_BACKWARD, SSD_WS_FORWARD, SSD_WS_FORWARD_CONV,
                   SSDError, load)
from .ops import (BackwardBuffers, ForwardBuffers, Segments, backward, forward, make_problem,
                  ssd_apply_init_state, ssd_boundary_scan, ssd_conv1d_bwd, ssd_conv1d_fwd,
                  ssd_conv_segment_output, ssd_conv_segment_states,
                  ssd_segment_bwd, ssd_segment_bwd_chunks, ssd_segment_bwd_pass,
                  ssd_segment_bwd_summary,
                  ssd_segment_fwd, ssd_segment_fwd_noalloc, ssd_segment_output, ssd_segment_output_fused,
                  ssd_segment_states, ssd_workspace_bytes, summary_numel)

__all__ = ["SSD_BF16", "SSD_F32", "SSD_WS_BACKWARD", "SSD_WS_FORWARD", "SSD_WS_FORWARD_CONV",
           "SSDError", "load",
           "BackwardBuffers", "ForwardBuffers", "Segments", "backward", "forward",
           "make_problem", "ssd_apply_init_state", "ssd_boundary_scan", "ssd_conv1d_bwd",
           "ssd_conv1d_fwd", "ssd_conv_segment_output", "ssd_conv_segment_states",
           "ssd_segment_bwd", "ssd_segment_bwd_chunks", "ssd_segment_bwd_pass",
           "ssd_segment_bwd_summary", "ssd_segment_fwd", "ssd_segment_fwd_noalloc", "ssd_segment_output",
           "ssd_segment_output_fused", "ssd_segment_states", "ssd_workspace_bytes", "summary_numel"]

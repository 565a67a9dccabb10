"""Falcon fast-weight attention on MI355X (gfx950): chunked forward pass and
single-token recurrent step, and the backward pass of the chunked form, behind a
C ABI (include/falcon.h)."""

from .falcon import (VARIANTS, FalconError, ForwardCall, chunk_fwd, chunk_fwd_varlen, recurrent_step, new_state, lib,  # noqa: F401
                     make_shape, status_string, chunk_bwd, bwd_workspace_bytes, chunk_fwd_segmented,
                     segmented_workspace_bytes)

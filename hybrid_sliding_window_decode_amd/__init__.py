"""Hybrid sliding-window decode attention for AMD Instinct MI355X (gfx950).

The compute path is the HIP library `libhswd.so` (C ABI, `include/hswd.h`);
this package is a thin ctypes binding over it.  Torch tensors supply device
memory and the stream; every step of the decode path runs in the library's
kernels.  Calling an op when the library has not been built raises.
"""

from .binding import (AttnDesc, BoundCall, HswdError, HswdUnavailable,  # noqa: F401
                      bind_layer_step, bind_layer_step_gproj, check_errors, decode_attn_full,
                      decode_attn_partials, decode_attn_sliding, gate_proj, head_gate,
                      kv_slot_write, layer_step, layer_step_gproj, layer_step_noalloc,
                      lse_merge, make_desc,
                      num_splits, ring_mask, rope_apply, status_string, stream_read, version,
                      workspace, workspace_bytes, workspace_init)

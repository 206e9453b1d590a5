"""MI355X (gfx950) Transformer-based linear attention: forward and backward of
one head-batch, as hand-written HIP kernels behind a C ABI (include/la.h).

The Python layer only marshals arguments to liblinattn.so; see _binding.py.
"""
from ._binding import (KernelTrace, LA_BF16, LA_FP16, LA_FP32, LIB_PATH, NATIVE_D, STATUS,
                       SUPPORTED_D, LAError, LinearAttention, alloc_workspace, backward,
                       backward_segment, decode_step, forward, forward_noalloc,
                       forward_segment, layer_backward,
                       layer_forward, layer_sizes, linear_attention, load_library, new_record,
                       num_segments, record_size, state_size, status_string, workspace_size)

__all__ = ["KernelTrace", "LA_BF16", "LA_FP16", "LA_FP32", "LIB_PATH", "NATIVE_D", "STATUS",
           "SUPPORTED_D", "LAError", "LinearAttention", "alloc_workspace", "backward",
           "backward_segment", "decode_step", "forward", "forward_noalloc", "forward_segment",
           "layer_backward",
           "layer_forward", "layer_sizes", "linear_attention", "load_library", "new_record",
           "num_segments", "record_size", "state_size", "status_string", "workspace_size"]

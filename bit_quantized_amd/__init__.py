"""MI355X (gfx950) W4A8 linear layer: per-token int8 activations x GPTQ int4
weights (group 128, asymmetric scale and zero) -> bf16, in hand-written HIP.

The public API is the C ABI in include/w4a8.h; this package is its thin
Python binding (torch for device memory and streams only).
"""
from ._lib import (  # noqa: F401
    BF16, F32, GROUP, PATH_AUTO, PATH_GEMV, PATH_PREFILL, PATH_PREFILL_N128, PATH_PREFILL_N256, PATH_SKINNY, PackedWeight, SiblingWeight,
    W4A8Error, gemm, gemm_debug, linear, linear_siblings, linear_workspace_bytes, load,
    pack_siblings, pack_weights, packed_weight_bytes, quant_act, select_path, unpack_weights,
    workspace_bytes, PackedW8, quant_act_hadamard, linear_hadamard, w4a16_linear,
    w4a16_select_path, w4a16_workspace_bytes, w8a8_gemm, w8a8_gemm_debug, w8a8_linear, w8a8_linear_workspace_bytes,
    w8a8_pack_weights, w8a8_select_path, w8a8_unpack_weights, w8a8_workspace_bytes,
    peak_mfma_i8, peak_stream_read, NOALLOC_SCRATCH_BYTES, linear_noalloc,
)

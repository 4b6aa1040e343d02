"""MI355X-native Kimi Delta Attention (KDA): Python binding of the C ABI.

The computation lives in hand-written HIP kernels for gfx950 behind the C ABI
declared in ``include/kda.h`` (library ``libkda.so`` in this directory). This
package only marshals torch tensors into that ABI.
"""
from ._binding import (  # noqa: F401
    GatedRMSNorm,
    KdaError,
    Overlap,
    NOALLOC_SCRATCH_BYTES,
    PREFILL_BAD_CU_SEQLENS,
    kda_chunk_prefill,
    kda_chunk_prefill_noalloc,
    kda_chunk_prefill_workspace_maps,
    kda_chunk_prefill_workspace_min_size,
    kda_chunk_prefill_workspace_size,
    kda_conv_decode_packed,
    kda_decode_packed,
    kda_mixed_batch,
    kda_mixed_batch_workspace_size,
    kda_short_conv,
    kda_spec_decode,
    lib,
    prefill_status,
)

__all__ = [
    "GatedRMSNorm",
    "KdaError",
    "Overlap",
    "NOALLOC_SCRATCH_BYTES",
    "PREFILL_BAD_CU_SEQLENS",
    "kda_chunk_prefill",
    "kda_chunk_prefill_noalloc",
    "kda_chunk_prefill_workspace_maps",
    "kda_chunk_prefill_workspace_min_size",
    "kda_chunk_prefill_workspace_size",
    "kda_conv_decode_packed",
    "kda_decode_packed",
    "kda_mixed_batch",
    "kda_mixed_batch_workspace_size",
    "kda_short_conv",
    "kda_spec_decode",
    "lib",
    "prefill_status",
]

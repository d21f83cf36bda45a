"""Mamba-2 (SSD) mixer-core prefill and decode step for AMD MI355X (gfx950).

The computation lives in libm2ssd.so (hand-written HIP kernels behind the C ABI
of include/m2ssd.h); this package is its ctypes binding.  Build the library
with ``python -m mamba_ssd_selective_amd.build``.
"""
from ._lib import (M2_BF16, M2_F32, M2Error, cu_seqlens_of, gated_rmsnorm_group, get_counters,
                   load, mamba2_conv_rows, mamba2_decode, mamba2_prefill, mamba2_prefill_workspace_size,
                   mamba2_prefill_noalloc, mamba2_prefill_noalloc_scratch_bytes,
                   mamba2_prefill_inproj, mamba2_prefill_inproj_workspace_size,
                   mamba2_decode_inproj, mamba2_mixed_inproj, mamba2_mixed_inproj_workspace_size,
                   reset_counters, ssd_chunk_scan, ssd_chunk_scan_plan, ssd_chunk_scan_workspace_size,
                   timing_enable,
                   timing_read, version, LIB_PATH)

__all__ = ["M2_BF16", "M2_F32", "M2Error", "cu_seqlens_of", "gated_rmsnorm_group",
           "get_counters", "load", "mamba2_conv_rows", "mamba2_decode", "mamba2_prefill",
           "mamba2_prefill_workspace_size", "mamba2_prefill_noalloc",
           "mamba2_prefill_noalloc_scratch_bytes", "mamba2_prefill_inproj",
           "mamba2_prefill_inproj_workspace_size", "mamba2_decode_inproj", "mamba2_mixed_inproj",
           "mamba2_mixed_inproj_workspace_size", "reset_counters", "ssd_chunk_scan",
           "ssd_chunk_scan_plan", "ssd_chunk_scan_workspace_size", "timing_enable",
           "timing_read", "version",
           "LIB_PATH"]

"""MI355X-native Mamba-2 SSD chunked selective-scan forward.

The scan runs in hand-written HIP kernels for gfx950 behind the C ABI of
``include/ssd.h`` (``libssd.so``, built in-tree); ``binding`` marshals torch
tensors to it.
"""
from .binding import (KERNEL_PATHS, NOALLOC_SCRATCH_BYTES, SSD_BF16, SSD_ERR_WAIT, SSD_F32, STAGES, SsdError, Timing,
                      abi_version, block_workspace_size, bwd_workspace_size, load_library,
                      path_code, scan_bwd, scan_bwd_raw, scan_fwd, scan_fwd_noalloc_raw, scan_fwd_path_raw,
                      scan_fwd_raw, scan_fwd_varlen_raw, split_conv1d_scan_fwd,
                      split_conv1d_scan_fwd_raw, status_string, taken_path,
                      varlen_workspace_size, wait_status, workspace_size)

__all__ = ["scan_fwd", "scan_fwd_raw", "scan_fwd_noalloc_raw", "scan_fwd_path_raw", "scan_fwd_varlen_raw", "scan_bwd",
           "scan_bwd_raw", "bwd_workspace_size", "split_conv1d_scan_fwd",
           "split_conv1d_scan_fwd_raw", "workspace_size", "varlen_workspace_size",
           "block_workspace_size", "wait_status", "taken_path", "status_string", "abi_version",
           "load_library", "path_code", "KERNEL_PATHS", "Timing", "SsdError", "SSD_F32",
           "SSD_BF16", "SSD_ERR_WAIT", "NOALLOC_SCRATCH_BYTES", "STAGES"]

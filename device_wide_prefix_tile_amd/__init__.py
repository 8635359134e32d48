"""MI355X (gfx950) device-wide prefix scan.

The work is done by hand-written HIP kernels in libdwpt_scan.so (C ABI in
include/dwpt_scan.h); this package is a thin torch-tensor binding of it.
"""
from .binding import (SCAN_SMALL_N_AUTO, ScanError, compact, csr_row_offsets, lib, radix_split, scan_copy_probe, scan_exclusive, scan_get_device_error,
                      scan_inclusive, scan_noalloc, scan_release_workspace, scan_set_multi_tile_mode, scan_set_small_n_max,
                      scan_set_spin_limit,
                      scan_status_string, segmented_scan)

__all__ = ["SCAN_SMALL_N_AUTO", "ScanError", "compact", "csr_row_offsets", "lib", "radix_split", "scan_copy_probe", "scan_exclusive", "scan_get_device_error",
           "scan_inclusive", "scan_noalloc", "scan_release_workspace", "scan_set_multi_tile_mode", "scan_set_small_n_max",
           "scan_set_spin_limit",
           "scan_status_string", "segmented_scan"]

"""MI355X-native Mamba-2 SSD selective scan.

The work is done by libssd.so (hand-written gfx950 HIP kernels behind the C ABI
in include/ssd.h).  This package is its thin Python binding plus the seeded
synthetic input generator used by the tests and the benchmark.

    from mamba_ssd_chunked_scan_amd import scan_fwd, step
    y, final_state = scan_fwd(x, dt, A, B, C, D, chunk=256, init_state=h0)
    y_t = step(state, x_t, dt_t, A, B_t, C_t, D)      # state updated in place
    y, finals = scan_fwd_varlen(x, dt, A, B, C, cu_seqlens, D)   # ragged batch
"""
from .binding import (  # noqa: F401
    SSDError, chunk_cb, chunk_cumsum, chunk_scan, chunk_scan_workspace_size, chunk_state, lib,
    scan_bwd, scan_bwd_varlen, scan_fwd, scan_fwd_varlen, state_passing, step, step_multi,
    varlen_workspace_size, workspace_size,
)

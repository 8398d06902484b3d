"""MI355X (gfx950) RG-LRU temporal branch: causal Conv1D (width 4) -> RG-LRU, and the
recurrent block around it (input linears, GeLU branch, output linear), the gated MLP block and
the local (sliding-window) multi-query attention block.

The compute path is librglru.so (hand-written HIP kernels behind a C ABI, declared in
include/rglru.h); this package is its thin ctypes binding.  Importing the package does not
load the library; load() (or the first call) does, and raises if it is not built.
"""
from ._binding import (EXPORTS, LIB_PATH, RGLRU_BF16, RGLRU_F32, RgluError,  # noqa: F401
                       backward, block_forward, block_fwd_workspace_bytes, bwd_workspace_bytes,
                       conv1d_causal4, decode_workspace_bytes,
                       forward, fwd_workspace_bytes, gated_mlp_fwd, io_code, load,
                       local_mqa_decode_step, local_mqa_fwd, mlp_forward,
                       mqa_decode_workspace_bytes, mlp_fwd_workspace_bytes, mqa_forward,
                       mqa_fwd_workspace_bytes, rglru_block_fwd, rglru_bwd,
                       rglru_block_decode_step, block_decode_workspace_bytes,
                       rglru_decode_step, rglru_fwd, rglru_gates, rglru_lru, rglru_scan,
                       rglru_workspace_status, RGLRU_ESTALL, rglru_decode_step_noalloc,
                       NOALLOC_SCRATCH_BYTES, rglru_fwd_train, rglru_bwd_saved,
                       forward_train, train_saved_bytes, fwd_train_workspace_bytes,
                       bwd_saved_workspace_bytes,
                       lru_workspace_bytes, scan_workspace_bytes, status_string, workspace)

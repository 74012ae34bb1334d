"""MI355X-native selective state-space scan (Mamba S6) and its Mamba-2 SSD form.

Thin Python binding over the C ABI in ``include/ssm_mi355x.h`` (library
``libssm_mi355x.so`` built in-tree by ``build.py``).  The functions carry the
C names, take torch tensors on the current ROCm device, allocate outputs with
torch, and pass raw device pointers plus the current HIP stream.  All
computation happens in the library's HIP kernels; there is no fallback.
"""
from ._binding import (  # noqa: F401
    SSM_SCAN_DELTA_PER_TOKEN,
    SSM_SCAN_EULER,
    SSM_SCAN_REVERSE,
    SSMError,
    library_path,
    load_library,
    ssm_causal_conv1d_fwd,
    ssm_scan_bwd,
    ssm_scan_bwd_ex,
    ssm_scan_bwd_ex_workspace_bytes,
    ssm_scan_bwd_train,
    ssm_scan_bwd_train_workspace_bytes,
    ssm_scan_bwd_workspace_bytes,
    ssd_chunk_scan_fwd,
    ssd_state_update,
    ssd_workspace_bytes,
    ssm_scan_final_state,
    ssm_scan_fwd,
    ssm_scan_fwd_ex,
    ssm_scan_fwd_noalloc,
    ssm_scan_fwd_noalloc_max_workspace_bytes,
    ssm_scan_fwd_train,
    ssm_scan_train_states_bytes,
    ssm_state_update,
    ssm_scan_workspace_bytes,
)

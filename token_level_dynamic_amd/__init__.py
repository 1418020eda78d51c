"""Token-level dynamic local-global attention (forward) for AMD MI355X.

The computation lives in liblogo.so (HIP kernels for gfx950 behind the C ABI
of include/logo.h). This package is its Python binding: the same entry
points, taking torch tensors for device memory and a HIP stream.
"""
from ._lib import (  # noqa: F401
    LOGO_BF16,
    LOGO_F32,
    STAGES,
    LogoError,
    alloc_backward_buffers,
    alloc_forward_buffers,
    alloc_routed_buffers,
    alloc_train_buffers,
    io_dtype,
    lib,
    logo_backward,
    logo_backward_workspace_size,
    logo_calibrate_threshold,
    logo_combine,
    logo_decode_step,
    logo_decode_workspace_size,
    logo_decode_problem,
    logo_forward,
    logo_forward_routed,
    logo_forward_train,
    logo_global_attn_sparse,
    logo_local_attn,
    logo_problem,
    logo_profile_begin,
    logo_profile_end,
    logo_routed_workspace_size,
    logo_select_queries,
    logo_select_threshold,
    logo_target_count,
    logo_varlen_selected_count,
    logo_varlen_workspace_size,
    logo_forward_varlen,
    logo_workspace_size,
    make_decode_problem,
    make_problem,
    view_strides,
)

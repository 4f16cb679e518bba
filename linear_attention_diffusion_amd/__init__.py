"""SANA ReLU linear attention on MI355X (gfx950): HIP kernels behind a C ABI.

Entry points (same names as the C ABI in include/sana_linattn.h):
  sana_linattn_forward, sana_linattn_state_update, sana_linattn_block_forward,
  sana_linattn_block_causal, sana_linattn_apply, sana_linattn_backward,
  sana_linattn_state_update_backward, sana_linattn_backward_saved,
  rope3d_table / rope3d_device (host builder of the 3D RoPE tables),
  rope3d_axes / rope3d_axes_device (the same RoPE as per-axis tables).
"""

from .binding import (  # noqa: F401
    EXPORTED,
    SANA_DT_BF16,
    SANA_DT_F32,
    SANA_ERR_HIP,
    SANA_ERR_INVALID,
    SANA_ERR_UNSUPPORTED,
    SANA_ERR_WORKSPACE,
    SANA_OK,
    Rope,
    sana_layout,
    SanaError,
    lib,
    make_workspace,
    rope3d_axes,
    rope3d_axes_device,
    rope3d_device,
    rope3d_table,
    backward_workspace_bytes,
    block_causal_workspace_bytes,
    sana_linattn_apply,
    sana_linattn_backward,
    sana_linattn_backward_saved,
    sana_linattn_block_causal,
    sana_linattn_block_forward,
    sana_linattn_forward,
    sana_linattn_state_update,
    sana_linattn_state_update_backward,
    sana_linattn_temporal_conv3,
    sana_linattn_status_string,
    workspace_bytes,
)

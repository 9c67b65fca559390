"""Fused non-GEMM operator chain of a video+audio DiT block, for MI355X (gfx950).

The package is a thin Python face over ``libdit_ops.so``, a C-ABI library of
hand-written HIP kernels (``csrc/``; declarations in ``include/dit_ops.h``):

  dit_adaln_modulate      y = LayerNorm(x) * (1 + scale) + shift
  dit_gated_residual      out = x + gate * y
  dit_gated_residual_adaln  the two fused: x_out = x + gate * y, z = AdaLN(x_out)
  dit_swiglu              out = silu(a) * b over [a | b] rows
  dit_qk_rmsnorm_rope3d   per-head RMSNorm of q and k, then 3D (t, h, w) RoPE
  dit_qk_rmsnorm_rope3d_layout  the same, reading q/k from a fused QKV buffer and
                          writing head-major outputs
  dit_residual_change     Cache-DiT statistic: sum |r - r_cached| / sum |r_cached| per sample
  dit_residual_change_noalloc  the same with no workspace (a static scratch array), for callers
                          that cannot allocate
  dit_subblock_pool       SubBlock routing: means of each 64-token block of q' and k'
  dit_qk_rmsnorm_rope3d_pool  QK RMSNorm + RoPE that also writes those block means
  dit_subblock_route      SubBlock routing: block scores and the kept key blocks per query block
  dit_packed_positions    (t, h, w) coordinates of a packed token sequence
  dit_copy16              plain 16-byte-vector copy (bandwidth ceiling)
  dit_stream_pattern      each kernel's memory traffic with no arithmetic (its own ceiling)

PyTorch supplies device memory and streams only.  Build the library with
``python -m video_diffusion_transformer_dit_amd.build``.
"""
from ._binding import (  # noqa: F401
    DIT_ERR_ALIGN,
    DIT_ERR_ARG,
    DIT_ERR_HIP,
    DIT_ERR_SCRATCH,
    DIT_ERR_NULL,
    DIT_ERR_SHAPE,
    DIT_OK,
    DIT_QK_HEAD_MAJOR,
    DIT_QK_TOKEN_MAJOR,
    DIT_STREAM_HEAD_MAJOR,
    DIT_STREAM_READ,
    DIT_STREAM_ROW_GROUP,
    DIT_STREAM_ROW_GROUP_2X2,
    DIT_STREAM_SCORE_TILES,
    DIT_STREAM_TOPK_ROWS,
    DIT_STREAM_SPLIT_ROWS,
    DIT_STREAM_TWO_IN,
    DIT_STREAM_WRITE,
    DIT_SUBBLOCK_TOKENS,
    LIB_PATH,
    SIGNATURES,
    DitError,
    dit_abi_version,
    dit_adaln_modulate,
    dit_copy16,
    dit_gated_residual,
    dit_gated_residual_adaln,
    dit_packed_positions,
    dit_qk_rmsnorm_rope3d,
    dit_qk_rmsnorm_rope3d_layout,
    dit_qk_rmsnorm_rope3d_pool,
    dit_residual_change,
    dit_residual_change_noalloc,
    dit_residual_change_workspace_bytes,
    dit_status_str,
    dit_stream_pattern,
    dit_subblock_keep,
    dit_subblock_pool,
    dit_subblock_route,
    dit_subblock_scores_ld,
    dit_swiglu,
    load_library,
)

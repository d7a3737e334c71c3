"""QoQ W4A8 GEMM for MI355X (gfx950): Python binding of libqoq.so.

The C ABI (include/qoq.h) is the product; this package only marshals
arguments to it.  Names mirror the C entry points.
"""

from ._native import (  # noqa: F401
    EXPORTS,
    GROUP,
    LIB_PATH,
    PackedWeight,
    PackedWeightW8,
    QoQError,
    load_library,
    qoq_hadamard_rotate,
    qoq_kv4_decode_attention,
    qoq_kv4_decode_attention_workspace_size,
    qoq_kv4_decode_attention_plan,
    qoq_kv4_quant,
    qoq_pack_codes,
    qoq_pack_weights,
    qoq_quant_act_per_token,
    qoq_rmsnorm_quant_per_token,
    qoq_scale_columns,
    qoq_smoothing_factors,
    qoq_swiglu_quant_per_token,
    qoq_unpack_weights,
    qoq_w4a8_forward,
    qoq_w4a8_gemm,
    qoq_w4a8_gemm_i32,
    qoq_w4a8_gemm_noalloc,
    qoq_w4a8_gemm_plan,
    NOALLOC_SCRATCH_BYTES,
    qoq_w4a8_gemm_saturating,
    qoq_w4a8_gemm_saturating_i32,
    qoq_pack_weights_w8,
    qoq_w8a8_gemm,
    qoq_w8a8_gemm_i32,
    qoq_weight_layout_query,
)

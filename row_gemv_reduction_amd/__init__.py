"""MI355X-native row-parallel decode projections and ring-ordered reduction.

The compute path is libtpdecode.so (HIP, gfx950); this package holds its
build script, a thin ctypes binding with the C interface's names, the seeded
input generators and the workload shapes. Nothing here computes on the CPU.
"""
from . import synth, workloads  # noqa: F401
from .binding import (  # noqa: F401
    TP_PATH_MFMA, TP_PATH_VALU, TP_POINT_ATTN_OUT, TP_POINT_FFN_DOWN, TP_WEIGHTS_BF16,
    TP_WEIGHTS_MXFP4, TP_WEIGHTS_MXFP8, Plan, TPError, mx_codes_shape, mx_scales_shape, packed_dtype,
    tp_pack_weights_mx, tp_quantize_mx, prefill_packed_shape, tp_prefill_pack_weights, tp_prefill_layers,
    moe_packed_shape, packed_act_shape, packed_shape, tp_decode_layers, tp_decode_layers_packed,
    tp_decode_layers_packed_noalloc,
    tp_decode_point, tp_gate_up_swiglu, tp_moe_decode, tp_pack_activations, tp_qkv_proj,
    tp_moe_pack_experts, tp_moe_partial, tp_moe_route, tp_pack_weights,
    moe_attn_packed_shape, tp_moe_pack_attn, tp_moe_layer_decode,
    tp_plan, tp_ring_reduce, tp_rowparallel_partial, tp_rowparallel_partials,
    tp_rowparallel_partials_packed, tp_set_debug_sync, tp_stream_read_probe, tp_workspace_init,
    tp_workspace_status,
)

"""motattn: MI355X-native hot path of the Cosmos 3 Mixture-of-Transformers
denoiser forward — region-split QKV/O projection, 3D mRoPE, masked flash
attention (AR-causal/DM-full and chunk-causal against a KV cache) and the
flow-matching Euler step with its flow-shifted noise schedule — as
hand-written HIP kernels for gfx950 behind the C ABI in include/motattn.h.  This package is the thin ctypes binding.
"""
from ._binding import (  # noqa: F401
    EXPORTED, LIB_PATH, MOT_AR_CAUSAL_DM_FULL, MOT_BF16, MOT_CHUNK_CAUSAL_KV, MOT_ERR_HIP,
    MOT_ERR_INVALID_ARG, MOT_ERR_UNSUPPORTED, MOT_FP32, MOT_OK, MotError, attn_args,
    flow_cfg_euler_step, flow_euler_step, mask_args, mot_layernorm_region, mot_region_linear,
    MOT_EPI_NONE, MOT_EPI_GELU, MOT_EPI_ADD, mot_abi_version, mot_attention_fwd, mot_attention_fwd_args,
    mot_build_layout, mot_mask_materialize, mot_qkv_project, mot_sigma_schedule, mot_status_string,
    mot_tile_classes_host, mrope_apply, raw_call, mot_attn_args, mot_segment, mot_attention_merge,
)

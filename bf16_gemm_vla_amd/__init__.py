"""MI355X (gfx950) FP8/BF16-weight GEMM path for small-batch VLA inference.

The compute lives in hand-written HIP kernels behind the C ABI of
include/vla.h (libvla.so, built in-tree by ``python -m
bf16_gemm_vla_amd.build``).  This package is the thin Python binding of that
ABI: the same entry-point names, torch tensors standing in for device
pointers.  PyTorch provides device memory and streams only.
"""
from ._lib import (  # noqa: F401
    LIB_PATH, SIGNATURES, VLA_EALIGN, VLA_EHIP, VLA_EINVAL, VLA_ESHAPE, VLA_ESTATE,
    VLA_EWORKSPACE, VLA_LAYOUT_MFMA, VLA_LAYOUT_ROWMAJOR, VLA_OK, VLA_WFMT_BF16,
    VLA_WFMT_E4M3_FNUZ, VLA_WFMT_E4M3_OCP, VLA_WFMT_MXFP4, last_error, load, status_string,
    vla_decoder_chain_create, vla_decoder_chain_enqueue, vla_decoder_chain_enqueue_staged,
    vla_decoder_chain_scratch_bytes,
    vla_gate_residual_ada_norm, vla_gemm_bf16, vla_gemm_fp8w, vla_gemm_fp8w_noalloc, vla_gemm_mxfp4w, vla_gemm_fp8w_gelu_mul, vla_gemm_supported, vla_gemm_workspace_bytes,
    vla_gemm_plan, vla_mlp_chain_create, vla_mlp_chain_destroy, vla_mlp_chain_enqueue, vla_mlp_chain_enqueue_staged, vla_mlp_chain_fused_supported, vla_decoder_chain_fused_supported,
    vla_mlp_chain_replay, vla_set_wait_limit, vla_workspace_status,
    vla_mlp_chain_scratch_bytes, vla_pack_fp8, vla_packed_bytes, vla_probe_mfma_rate, vla_probe_stream_read, vla_quantize_act,
    VLA_MFMA_BF16_32X32X16, VLA_MFMA_BF16_16X16X32, VLA_MFMA_FP8_32X32X64, VLA_MFMA_FP8_16X16X128,
    vla_quantize_act_static, vla_quantize_act_workspace_bytes, vla_quantize_pack, vla_reencode_fnuz_to_ocp,
)

"""MI355X-native NVFP4 forward / MXFP8 backward MoE expert layer.

Thin Python binding over the C-ABI library ``libnvfp4moe.so`` (built from
``csrc/`` by ``precision_moe_numerics_nvfp4_amd.build``). Every function here
only checks and marshals its arguments -- torch tensors are used for device
memory and the current HIP stream -- and calls the library entry point of the
same name; all arithmetic runs in the HIP kernels. There is no CPU fallback:
if the library is missing or the tensors are not on a GPU, the calls raise.
"""

from .binding import (  # noqa: F401
    LIB_PATH,
    NVFP4MOE_BF16,
    NVFP4MOE_F32,
    Nvfp4moeError,
    abi_version,
    lib,
    moe_bwd_dgrad,
    moe_bwd_wgrad,
    moe_combine,
    moe_combine_bwd,
    moe_fwd_grouped_gemm,
    moe_bwd_wgrad_nvfp4,
    moe_fwd_grouped_gemm_mxfp8,
    moe_padded_offsets,
    moe_permute,
    moe_permute_noalloc,
    mxfp8_gather_rows,
    mxfp8_quantize,
    mxfp8_quantize_dual,
    mxfp8_requant_sr,
    nvfp4_quantize,
    nvfp4_quantize_live,
    nvfp4_quantize_sr,
    nvfp4_quantize_sr_colwise,
    nvfp4_quantize_tile16,
    nvfp4_requant_sr,
    permute_workspace_size,
    status_string,
)

"""MI355X (gfx950) fused residual-add + Gemma RMSNorm + FP8/NVFP4 activation
quant: a HIP library behind a C ABI (include/gemma_norm_quant.h), with a thin
ctypes/PyTorch binding."""

from .ops import (  # noqa: F401
    gemma_add_rms_norm_quant, gemma_add_rms_norm_quant_out, add_rms_norm_quant,
    add_rms_norm_quant_out, gemma_add_rms_norm, quant_fp8_static, quant_nvfp4, block_scale_bytes,
)
from ._lib import (  # noqa: F401
    nq_gemma_add_rms_norm_quant, nq_add_rms_norm_quant, nq_quant_fp8_static, nq_quant_nvfp4,
    nq_block_scale_bytes, nq_status_string, nq_abi_version, nq_convert_probe, NqError, LIB_PATH,
)

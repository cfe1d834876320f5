"""MI355X (gfx950) fused residual-add + Gemma RMSNorm + FP8/NVFP4 activation
quant: a HIP library behind a C ABI (include/gemma_norm_quant.h), with a thin
ctypes/PyTorch binding."""

from .ops import gemma_add_rms_norm_quant, gemma_add_rms_norm_quant_out, block_scale_bytes  # noqa: F401
from ._lib import (  # noqa: F401
    nq_gemma_add_rms_norm_quant, nq_block_scale_bytes, nq_status_string, nq_abi_version,
    nq_convert_probe, NqError, LIB_PATH,
)

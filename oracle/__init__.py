"""CPU oracle for the fused residual-add + Gemma RMSNorm + input-quant op.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this
package: only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg
of ``bench.py`` use it.  It shares no code with the HIP library and imports
nothing from it.

The op is the one stated on the ``fused_norm_quant`` page
(``gemma_add_rms_norm_quant``): ``residual <- x + residual``; a Gemma RMSNorm
that scales by ``(1 + weight)``; the normed activation rounded to x's dtype;
then either static per-tensor FP8 E4M3 codes or NVFP4 (packed E2M1 codes with
one E4M3 scale per 16-element block, stored in the 128x4-tiled scale layout).
Its variants: a plain (w instead of 1 + w) norm, no quant, and MXFP8 (E4M3
codes with one E8M0 power-of-two scale per 32-element block, the
``allreduce_gemma_rms_norm_mxfp8`` variant on the
``fused_allreduce_gemma_rms_norm`` page).  ``gemm.py`` is the consumer linear
that reads the quantized activation (static FP8 or MXFP8) directly.
The page says the fused kernel computes the same codes as the unfused chain
(add+norm, then a standalone quant); the oracle is written as that chain.

Arithmetic: every rounding to a storage format (bf16, fp16, E4M3, E2M1) is
round-to-nearest-even to the nearest representable value, written out from
the format definition in ``formats.py``.  The norm is evaluated in fp64 and
rounded once to x's dtype.  The quant stage takes its decisions in IEEE fp32
(numpy float32 operations), the precision of the conversion instructions the
pages use.

Parity status per function is in each module's header.
"""

from .formats import (  # noqa: F401
    BF16, FP16, E4M3FN, E2M1, round_rne, encode, decode, decode_table,
    decode_e8m0, bits_to_f64, f64_to_bits,
)
from .norm_quant import (  # noqa: F401
    add_residual, gemma_rms_norm, rms_norm, quant_fp8_static, quant_nvfp4,
    nvfp4_block_scale_codes, nvfp4_element_codes,
    mxfp8_block_exponent, quant_mxfp8,
    swizzle_128x4_offset, block_scale_buffer_shape, scatter_block_scales,
    gemma_add_rms_norm_quant, add_rms_norm_quant,
)
from .gemm import (  # noqa: F401
    dequant_fp8_static, dequant_mxfp8, dequant_nvfp4, gemm_f64, gemm_fp8_static, gemm_mxfp8, gemm_nvfp4,
)

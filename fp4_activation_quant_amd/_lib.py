"""ctypes binding of libgemma_norm_quant.so (include/gemma_norm_quant.h).

Argument marshalling only: every step of the op runs in the HIP library.  The
library is loaded from this package directory; there is no fallback.  Build
it with ``python -m fp4_activation_quant_amd.build``.
"""

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgemma_norm_quant.so")

NQ_OK, NQ_EINVAL, NQ_EUNSUPPORTED, NQ_EHIP = 0, 1, 2, 3
NQ_BF16, NQ_FP16 = 0, 1
NQ_MODE_FP8_STATIC, NQ_MODE_NVFP4, NQ_MODE_NONE, NQ_MODE_MXFP8 = 0, 1, 2, 3
NQ_NORM_GEMMA, NQ_NORM_PLAIN = 0, 1
EXPORTS = ("nq_gemma_add_rms_norm_quant", "nq_add_rms_norm_quant", "nq_quant_fp8_static",
           "nq_quant_nvfp4", "nq_quant_mxfp8", "nq_gemm_mxfp8", "nq_gemm_fp8_static", "nq_gemm_nvfp4",
           "nq_block_scale_bytes", "nq_status_string", "nq_abi_version", "nq_convert_probe",
           "nq_traffic_probe", "nq_gemma_add_rms_norm_quant_gemm_fp8")

_lib = None


class NqError(RuntimeError):
    def __init__(self, status, what):
        super().__init__(f"{what}: {nq_status_string(status)} (status {status})")
        self.status = status


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing "
                               "(python -m fp4_activation_quant_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
        L.nq_gemma_add_rms_norm_quant.argtypes = [vp, vp, vp, f32, vp, i64, i64, i32, i32, i32,
                                                  vp, vp, vp, vp]
        L.nq_gemma_add_rms_norm_quant.restype = i32
        L.nq_add_rms_norm_quant.argtypes = [vp, vp, vp, f32, vp, i64, i64, i32, i32, i32, i32,
                                            vp, vp, vp, vp]
        L.nq_add_rms_norm_quant.restype = i32
        L.nq_quant_fp8_static.argtypes = [vp, vp, i64, i64, i32, vp, vp]
        L.nq_quant_fp8_static.restype = i32
        L.nq_quant_nvfp4.argtypes = [vp, vp, i64, i64, i32, vp, vp, vp]
        L.nq_quant_nvfp4.restype = i32
        L.nq_quant_mxfp8.argtypes = [vp, i64, i64, i32, vp, vp, vp]
        L.nq_quant_mxfp8.restype = i32
        L.nq_gemm_mxfp8.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, vp]
        L.nq_gemm_mxfp8.restype = i32
        L.nq_gemm_fp8_static.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, vp]
        L.nq_gemm_fp8_static.restype = i32
        L.nq_gemm_nvfp4.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, vp, vp]
        L.nq_gemm_nvfp4.restype = i32
        L.nq_block_scale_bytes.argtypes = [i64, i64]
        L.nq_block_scale_bytes.restype = ctypes.c_size_t
        L.nq_status_string.argtypes = [i32]
        L.nq_status_string.restype = ctypes.c_char_p
        L.nq_abi_version.argtypes = []
        L.nq_abi_version.restype = i32
        L.nq_convert_probe.argtypes = [i32, vp, i64, f32, vp, vp]
        L.nq_convert_probe.restype = i32
        pp = ctypes.POINTER(ctypes.c_void_p)
        pi64 = ctypes.POINTER(ctypes.c_int64)
        L.nq_traffic_probe.argtypes = [pp, pi64, i32, pp, pi64, i32, i64, i32, i32, i32, vp]
        L.nq_traffic_probe.restype = i32
        L.nq_gemma_add_rms_norm_quant_gemm_fp8.argtypes = [vp, vp, vp, vp, f32, vp, i64, i64, i32, i32, vp, vp,
                                                           vp, vp, i64, vp, vp]
        L.nq_gemma_add_rms_norm_quant_gemm_fp8.restype = i32
        _lib = L
    return _lib


def nq_gemma_add_rms_norm_quant(x, residual, weight, eps, scale, M, H, dtype, mode, write_y,
                                q, block_scale, y, stream):
    """Raw call with integer device addresses (0 for NULL); returns the status."""
    return lib().nq_gemma_add_rms_norm_quant(x or None, residual or None, weight or None,
                                             float(eps), scale or None, int(M), int(H), int(dtype),
                                             int(mode), int(bool(write_y)), q or None,
                                             block_scale or None, y or None, stream or None)


def nq_add_rms_norm_quant(x, residual, weight, eps, scale, M, H, dtype, norm, mode, write_y,
                          q, block_scale, y, stream):
    """Raw call (integer device addresses, 0 for NULL); returns the status."""
    return lib().nq_add_rms_norm_quant(x or None, residual or None, weight or None, float(eps),
                                       scale or None, int(M), int(H), int(dtype), int(norm),
                                       int(mode), int(bool(write_y)), q or None,
                                       block_scale or None, y or None, stream or None)


def nq_quant_fp8_static(y, scale, M, H, dtype, q, stream):
    return lib().nq_quant_fp8_static(y or None, scale or None, int(M), int(H), int(dtype),
                                     q or None, stream or None)


def nq_quant_nvfp4(y, global_scale, M, H, dtype, q, block_scale, stream):
    return lib().nq_quant_nvfp4(y or None, global_scale or None, int(M), int(H), int(dtype),
                                q or None, block_scale or None, stream or None)


def nq_quant_mxfp8(y, M, H, dtype, q, scales, stream):
    return lib().nq_quant_mxfp8(y or None, int(M), int(H), int(dtype), q or None, scales or None,
                                stream or None)


def nq_gemm_mxfp8(a, a_scales, b, b_scales, M, N, K, out, stream):
    return lib().nq_gemm_mxfp8(a or None, a_scales or None, b or None, b_scales or None, int(M),
                               int(N), int(K), out or None, stream or None)


def nq_gemm_fp8_static(a, a_scale, b, b_scale, M, N, K, out, stream):
    return lib().nq_gemm_fp8_static(a or None, a_scale or None, b or None, b_scale or None, int(M),
                                    int(N), int(K), out or None, stream or None)


def nq_gemm_nvfp4(a, a_scales, a_gs, b, b_scales, b_gs, M, N, K, out, stream):
    return lib().nq_gemm_nvfp4(a or None, a_scales or None, a_gs or None, b or None, b_scales or None,
                               b_gs or None, int(M), int(N), int(K), out or None, stream or None)


def nq_block_scale_bytes(M, H):
    return int(lib().nq_block_scale_bytes(int(M), int(H)))


def nq_status_string(status):
    return lib().nq_status_string(int(status)).decode()


def nq_abi_version():
    return int(lib().nq_abi_version())


def nq_convert_probe(kind, inp, n, param, out, stream):
    """Raw call: ``inp``/``out`` are device addresses (see the header)."""
    return lib().nq_convert_probe(int(kind), inp or None, int(n), float(param), out or None,
                                  stream or None)


NQ_PROBE_PREFETCH, NQ_PROBE_TILED_SCALES = 1, 2


def nq_traffic_probe(src, src_row_bytes, dst, dst_row_bytes, rows, threads, grid, flags, stream):
    """Raw call: ``src`` / ``dst`` are lists of device addresses, the row
    byte counts lists of ints, ``flags`` NQ_PROBE_* bits (see the header)."""
    vpa = ctypes.c_void_p * max(1, len(src))
    vpd = ctypes.c_void_p * max(1, len(dst))
    i64a = ctypes.c_int64 * max(1, len(src))
    i64d = ctypes.c_int64 * max(1, len(dst))
    return lib().nq_traffic_probe(vpa(*src), i64a(*src_row_bytes), len(src), vpd(*dst) if dst else None,
                                  i64d(*dst_row_bytes) if dst else None, len(dst), int(rows), int(threads),
                                  int(grid), int(flags), stream or None)


def nq_gemma_add_rms_norm_quant_gemm_fp8(x, residual, residual_out, weight, eps, scale, M, H, dtype,
                                         write_y, q, y, b, b_scale, N, out, stream):
    return lib().nq_gemma_add_rms_norm_quant_gemm_fp8(x or None, residual or None, residual_out or None,
                                                      weight or None, float(eps), scale or None, int(M), int(H),
                                                      int(dtype), int(write_y), q or None, y or None, b or None,
                                                      b_scale or None, int(N), out or None, stream or None)

"""MI355X-native fused diagonal-GMM EM step (Flash-GMM method) behind a C ABI.

The compute runs in the HIP kernels of libflashgmm.so; this package holds the
ctypes binding (argument marshalling only) and the seeded input generators.
Importing it fails loudly when the library has not been built.
"""
from ._lib import (GMM, GMMError, PATH_AUTO, PATH_FUSED, PATH_TWO_SWEEP, PREC_FP32, PREC_FP64, PREC_REFINED,  # noqa: F401
                   MFMA_FP32, MFMA_SPLIT_BF16, MFMA_SPLIT_LOGITS, EXPORTS, LIB_PATH, raw_library,
                   estep_stats_noalloc)

__all__ = ["GMM", "GMMError", "PATH_AUTO", "PATH_FUSED", "PATH_TWO_SWEEP", "PREC_FP32", "PREC_FP64", "PREC_REFINED",
           "MFMA_FP32", "MFMA_SPLIT_BF16", "MFMA_SPLIT_LOGITS", "EXPORTS", "LIB_PATH", "raw_library",
           "estep_stats_noalloc"]

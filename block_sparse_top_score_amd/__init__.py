"""Decode-step block-sparse top-score attention on MI355X (gfx950).

The compute path is libsparse_decode.so (hand-written HIP kernels behind the
C ABI in include/sparse_decode.h); this package is its thin Python binding.
"""
from ._abi import (EXPORTS, LIB_PATH, SDConfig, SDError, SparseDecode, load,
                   make_config, validate_config, SD_OK, SD_EINVAL, SD_ENOMEM,
                   SD_EHIP, SD_EUNSUPPORTED, SD_ESTATE, SD_DEBUG_PAGE_TABLE,
                   SD_DEBUG_SUMMARY, SD_DEBUG_MAW, SD_DEBUG_K, SD_DEBUG_V)

__all__ = ["EXPORTS", "LIB_PATH", "SDConfig", "SDError", "SparseDecode", "load",
           "make_config", "validate_config"]

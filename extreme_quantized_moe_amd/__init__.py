"""MiLo W3A16 + low-rank-compensated MoE expert GEMM for MI355X (gfx950).

The compute lives in libmilo.so (HIP, C ABI in include/milo.h); this package
is the ctypes binding.  Importing it loads the library and raises if it has
not been built: there is no CPU or PyTorch fallback.
"""
from ._lib import (  # noqa: F401
    EPI_NONE, EPI_ROUTE_SCALE, EPI_SWIGLU, GEMM_PREPASS_DONE, LR_FP16, LR_INT3, PATH_AUTO, PATH_DECODE,
    PATH_PREFILL, LIB_PATH, MiloError, lib,
)

lib()  # fail loudly at import if libmilo.so is missing

from .ops import (  # noqa: E402,F401
    Family, MoELayer, build_compensator, expert_counts, lowrank_svd, lr_words, moe_combine, rank_policy,
    weight_kurtosis, moe_lowrank_prepass, moe_w3a16_lowrank_gemm, pack_int3,
    pack_lr_int3, packed_words, quantize_hqq_int3, quantize_rtn_int3, route_sort, sz_words,
)

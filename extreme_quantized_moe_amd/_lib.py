"""ctypes view of libmilo.so (include/milo.h).  Argument marshalling only."""
import ctypes as C
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmilo.so")

MILO_OK = 0
STATUS_NAMES = {0: "MILO_OK", 1: "MILO_ERR_NULL", 2: "MILO_ERR_SHAPE", 3: "MILO_ERR_ALIGN",
                4: "MILO_ERR_RANK", 5: "MILO_ERR_WORKSPACE", 6: "MILO_ERR_ARG", 7: "MILO_ERR_HIP"}
EPI_NONE, EPI_SWIGLU, EPI_ROUTE_SCALE = 0, 1, 2
PATH_AUTO, PATH_DECODE, PATH_PREFILL = 0, 1, 2
GEMM_PREPASS_DONE = 1
STATIC_WORKSPACE_BYTES = 64 << 20
LR_FP16, LR_INT3 = 0, 1
QUANT_RTN, QUANT_HQQ = 0, 1


class MiloWeights(C.Structure):
    _fields_ = [("packed", C.c_void_p), ("sz", C.c_void_p), ("U", C.c_void_p),
                ("V", C.c_void_p), ("rank", C.c_void_p), ("lr_format", C.c_int32),
                ("Uq", C.c_void_p), ("Usz", C.c_void_p), ("Vq", C.c_void_p),
                ("Vsz", C.c_void_p)]


class MiloGemmDesc(C.Structure):
    _fields_ = [
        ("num_experts", C.c_int32), ("N", C.c_int32), ("K", C.c_int32),
        ("max_rank", C.c_int32), ("n_w", C.c_int32),
        ("w", MiloWeights * 2),
        ("x", C.c_void_p), ("x_rows", C.c_int32), ("gather_div", C.c_int32),
        ("sorted_pairs", C.c_void_p), ("offsets", C.c_void_p),
        ("num_pairs", C.c_int32), ("max_rows_per_expert", C.c_int32),
        ("slot_w", C.c_void_p), ("y_rows", C.c_int32), ("epilogue", C.c_int32),
        ("y", C.c_void_p), ("path", C.c_int32), ("flags", C.c_int32),
    ]


class MiloError(RuntimeError):
    def __init__(self, fn, code, detail):
        self.code = code
        super().__init__(f"{fn} failed: {STATUS_NAMES.get(code, code)}: {detail}")


_lib = None


def lib():
    """Load libmilo.so (built in-tree by extreme_quantized_moe_amd.build).
    Raises if it is missing: there is no fallback implementation."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} not found: build it with "
                          "`python extreme_quantized_moe_amd/build.py` (no fallback path exists)")
    L = C.CDLL(LIB_PATH)
    i32, i64, vp, sz = C.c_int32, C.c_int64, C.c_void_p, C.c_size_t
    sig = {
        "milo_abi_version": (i32, []),
        "milo_layout_version": (i32, []),
        "milo_status_string": (C.c_char_p, [i32]),
        "milo_last_error": (C.c_char_p, []),
        "milo_packed_words": (i64, [i64, i64]),
        "milo_sz_words": (i64, [i64, i64]),
        "milo_quantize_rtn_int3": (i32, [vp, i64, i64, vp, vp, vp, vp]),
        "milo_quantize_rtn_int3_grouped": (i32, [vp, i64, i64, i32, vp, vp, vp, vp]),
        "milo_pack_int3": (i32, [vp, vp, vp, i64, i64, vp, vp, vp]),
        "milo_quantize_hqq_int3": (i32, [vp, i64, i64, i32, C.c_double, C.c_double, C.c_double, vp, vp, vp,
                                          vp]),
        "milo_lr_v_words": (i64, [i32, i64]),
        "milo_lr_v_sz_words": (i64, [i32, i64]),
        "milo_lr_u_words": (i64, [i64, i32]),
        "milo_lr_u_sz_words": (i64, [i64]),
        "milo_pack_lr_int3": (i32, [vp, vp, vp, vp, vp, vp, i64, i64, i32, i32, vp, vp, vp, vp, vp]),
        "milo_lowrank_svd_workspace_bytes": (sz, [i64, i64, i32, i32]),
        "milo_lowrank_svd": (i32, [vp, i64, i64, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]),
        "milo_build_compensator_workspace_bytes": (sz, [i64, i64, i32, i32]),
        "milo_build_compensator": (i32, [vp, i64, i64, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp,
                                          vp, vp, sz, vp]),
        "milo_weight_kurtosis_workspace_bytes": (sz, [i64]),
        "milo_weight_kurtosis": (i32, [vp, i64, i64, vp, vp, vp, sz, vp]),
        "milo_expert_counts": (i32, [vp, i32, vp, vp]),
        "milo_rank_policy": (i32, [vp, vp, vp, i32, i32, i32, i32, i32, vp]),
        "milo_route_workspace_bytes": (sz, [i32, i32, i32, i32]),
        "milo_route_sort": (i32, [vp, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "milo_moe_gemm_workspace_bytes": (sz, [C.POINTER(MiloGemmDesc)]),
        "milo_moe_w3a16_lowrank_gemm": (i32, [C.POINTER(MiloGemmDesc), vp, sz, vp]),
        "milo_moe_lowrank_prepass": (i32, [C.POINTER(MiloGemmDesc), vp, sz, vp]),
        "milo_moe_w3a16_lowrank_gemm_static": (i32, [C.POINTER(MiloGemmDesc), vp]),
        "milo_moe_combine": (i32, [vp, i32, i32, i32, vp, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def check(fn_name, rc):
    if rc != MILO_OK:
        detail = lib().milo_last_error().decode(errors="replace")
        raise MiloError(fn_name, rc, detail)
    return rc

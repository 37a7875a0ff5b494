"""ctypes loader for libbsa.so (the HIP kernels behind the C ABI in include/bsa.h).

Argument marshalling only.  The library must have been built in-tree
(`python -m block_sparse_attention_fractal_amd.build`); there is no fallback:
loading fails loudly when it is missing.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbsa.so")

BSA_OK = 0
BSA_F32, BSA_BF16 = 0, 1
BSA_LAYOUT_ORIGINAL, BSA_LAYOUT_FRACTAL = 0, 1
BSA_MASK_CDF, BSA_MASK_SIP = 0, 1
BSA_ORDER_FRACTAL, BSA_ORDER_TILE_MAJOR, BSA_ORDER_HILBERT = 0, 1, 2

# every symbol declared in include/bsa.h
EXPORTED = ["bsa_query_sizes", "bsa_permute", "bsa_order_table", "bsa_permute_table", "bsa_pool",
            "bsa_block_map", "bsa_build_mask", "bsa_forward", "bsa_prepare_v", "bsa_query_attend_ws", "bsa_attend",
            "bsa_attend_static", "bsa_query_backward_ws", "bsa_backward", "bsa_attend_train", "bsa_backward_train",
            "bsa_query_group_sizes", "bsa_build_group_mask",
            "bsa_forward_groups", "bsa_prepare_v_groups", "bsa_query_attend_groups_ws", "bsa_attend_groups", "bsa_status_str", "bsa_last_error",
            "bsa_version"]


KEY_GROUP = 4   # BSA_KEY_GROUP


class Problem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("T", ctypes.c_int32),
                ("H", ctypes.c_int32), ("W", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("patch", ctypes.c_int32), ("block", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("layout", ctypes.c_int32)]


class MaskParams(ctypes.Structure):
    _fields_ = [("thr", ctypes.c_double), ("win_t", ctypes.c_int32), ("win_h", ctypes.c_int32),
                ("win_w", ctypes.c_int32), ("mode", ctypes.c_int32), ("seed", ctypes.c_uint64)]


class CSR(ctypes.Structure):
    _fields_ = [("row_ptr", ctypes.c_void_p), ("col_idx", ctypes.c_void_p),
                ("capacity", ctypes.c_int64), ("nnz", ctypes.c_void_p), ("shift", ctypes.c_void_p)]


class BSAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


_lib = None


def lib():
    """Load libbsa.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m block_sparse_attention_fractal_amd.build`")
    l = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    P = ctypes.POINTER
    l.bsa_query_sizes.argtypes = [P(Problem), P(i64), P(i64), P(i64), P(i64)]
    l.bsa_permute.argtypes = [P(Problem), vp, vp, ctypes.c_int, vp]
    l.bsa_order_table.argtypes = [P(Problem), ctypes.c_int, vp]
    l.bsa_permute_table.argtypes = [P(Problem), vp, vp, vp, ctypes.c_int, vp]
    l.bsa_pool.argtypes = [P(Problem), vp, vp, vp, vp, vp]
    l.bsa_block_map.argtypes = [P(Problem), vp, vp, vp, vp]
    l.bsa_build_mask.argtypes = [P(Problem), P(MaskParams), vp, vp, P(CSR), vp, i64, vp]
    l.bsa_forward.argtypes = [P(Problem), vp, vp, vp, P(CSR), vp, vp, vp, i64, vp]
    l.bsa_prepare_v.argtypes = [P(Problem), vp, vp, vp]
    l.bsa_query_attend_ws.argtypes = [P(Problem), P(i64)]
    l.bsa_attend.argtypes = [P(Problem), vp, vp, vp, P(CSR), vp, vp, vp, i64, vp]
    l.bsa_attend_static.argtypes = [P(Problem), vp, vp, vp, P(CSR), vp, vp, vp]
    l.bsa_query_backward_ws.argtypes = [P(Problem), P(i64)]
    l.bsa_backward.argtypes = [P(Problem), vp, vp, vp, P(CSR), vp, vp, vp, vp, vp, vp, i64, vp]
    l.bsa_attend_train.argtypes = [P(Problem), vp, vp, vp, P(CSR), vp, vp, vp, vp, i64, vp]
    l.bsa_backward_train.argtypes = [P(Problem), vp, vp, vp, P(CSR), vp, vp, vp, vp, vp, vp, vp, vp, i64, vp]
    l.bsa_query_group_sizes.argtypes = [P(Problem), ctypes.c_int, P(i64), P(i64), P(i64)]
    l.bsa_build_group_mask.argtypes = [P(Problem), ctypes.c_int, P(MaskParams), vp, vp, P(CSR), vp, i64, vp]
    l.bsa_forward_groups.argtypes = [P(Problem), ctypes.c_int, vp, vp, vp, P(CSR), vp, vp, vp, i64, vp]
    l.bsa_prepare_v_groups.argtypes = [P(Problem), ctypes.c_int, vp, vp, vp]
    l.bsa_query_attend_groups_ws.argtypes = [P(Problem), ctypes.c_int, P(i64)]
    l.bsa_attend_groups.argtypes = [P(Problem), ctypes.c_int, vp, vp, vp, P(CSR), vp, vp, vp, i64, vp]
    l.bsa_status_str.argtypes = [ctypes.c_int]
    l.bsa_status_str.restype = ctypes.c_char_p
    l.bsa_last_error.argtypes = []
    l.bsa_last_error.restype = ctypes.c_char_p
    l.bsa_version.argtypes = []
    for name in ("bsa_query_sizes", "bsa_permute", "bsa_order_table", "bsa_permute_table", "bsa_pool",
                 "bsa_block_map", "bsa_build_mask", "bsa_forward", "bsa_prepare_v", "bsa_query_attend_ws",
                 "bsa_attend", "bsa_attend_static", "bsa_query_backward_ws", "bsa_backward", "bsa_attend_train",
                 "bsa_backward_train", "bsa_version"):
        getattr(l, name).restype = ctypes.c_int
    _lib = l
    return l


def check(status: int):
    if status != BSA_OK:
        l = lib()
        raise BSAError(status, f"{l.bsa_status_str(status).decode()}: {l.bsa_last_error().decode()}")

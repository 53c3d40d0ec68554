"""ctypes view of libabsa.so (declarations in include/absa.h)."""
import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libabsa.so")

ABSA_OK = 0
ABSA_ERR_INVALID_ARG = -1
ABSA_ERR_SHAPE = -2
ABSA_ERR_UNSUPPORTED = -3
ABSA_ERR_WORKSPACE = -4
ABSA_ERR_HIP = -5
ABSA_ERR_ALIGNMENT = -6
ABSA_ERR_TOO_LARGE = -7

SEL_SIP, SEL_TOPK, SEL_ALL = 0, 1, 2

EXPORTED = (
    "absa_version", "absa_status_string", "absa_num_blocks", "absa_select_workspace",
    "absa_select_workspace_layout", "absa_select", "absa_attend", "absa_dense",
    "absa_fp8_workspace", "absa_quantize_fp8", "absa_attend_fp8",
    "absa_select_clusters_workspace", "absa_select_clusters", "absa_attend_clusters",
    "absa_select_noalloc", "absa_select_profile", "absa_attend_pairs_workspace", "absa_attend_pairs",
    "absa_attend_balanced_workspace", "absa_attend_balanced",
)


class AbsaProblem(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("L", ctypes.c_int32), ("d", ctypes.c_int32),
        ("T", ctypes.c_int32), ("Hs", ctypes.c_int32), ("Ws", ctypes.c_int32),
        ("q_block", ctypes.c_int32), ("kv_block", ctypes.c_int32),
        ("scale", ctypes.c_float), ("out_bf16", ctypes.c_int32),
    ]


class AbsaSelectParams(ctypes.Structure):
    _fields_ = [
        ("keep", ctypes.c_float), ("clusters", ctypes.c_int32), ("kmeans_steps", ctypes.c_int32),
        ("select_scale_log2", ctypes.c_float), ("seed", ctypes.c_uint64), ("stream", ctypes.c_uint32),
        ("mode", ctypes.c_int32),
    ]


class AbsaBlockList(ctypes.Structure):
    _fields_ = [
        ("count", ctypes.c_void_p), ("kv_idx", ctypes.c_void_p), ("inv_pi", ctypes.c_void_p),
        ("cap", ctypes.c_int32),
    ]


class AbsaClusterLists(ctypes.Structure):
    _fields_ = [
        ("count", ctypes.c_void_p), ("kv_idx", ctypes.c_void_p), ("w", ctypes.c_void_p),
        ("label", ctypes.c_void_p), ("cap", ctypes.c_int32), ("clusters", ctypes.c_int32),
    ]


class AbsaFp8Operands(ctypes.Structure):
    _fields_ = [
        ("q8", ctypes.c_void_p), ("sq", ctypes.c_void_p), ("k8", ctypes.c_void_p), ("sk", ctypes.c_void_p),
        ("kbar", ctypes.c_void_p), ("v8t", ctypes.c_void_p), ("sv", ctypes.c_void_p), ("mu", ctypes.c_void_p),
        ("qk_int8", ctypes.c_int32),
    ]


class AbsaError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)} ({status})")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load libabsa.so; raises if it has not been built (there is no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m block_sparse_attention_34_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, SP, BL = ctypes.POINTER(AbsaProblem), ctypes.POINTER(AbsaSelectParams), ctypes.POINTER(AbsaBlockList)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    lib.absa_version.restype = ctypes.c_int32
    lib.absa_version.argtypes = []
    lib.absa_status_string.restype = ctypes.c_char_p
    lib.absa_status_string.argtypes = [ctypes.c_int32]
    lib.absa_num_blocks.restype = ctypes.c_int
    lib.absa_num_blocks.argtypes = [P, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)]
    lib.absa_select_workspace.restype = ctypes.c_int
    lib.absa_select_workspace.argtypes = [P, SP, ctypes.POINTER(sz)]
    lib.absa_select_workspace_layout.restype = ctypes.c_int
    lib.absa_select_workspace_layout.argtypes = [P, SP, ctypes.POINTER(sz)]
    lib.absa_select.restype = ctypes.c_int
    lib.absa_select.argtypes = [P, SP, vp, vp, BL, vp, vp, sz, vp]
    lib.absa_select_noalloc.restype = ctypes.c_int
    lib.absa_select_noalloc.argtypes = [P, SP, vp, vp, BL, vp, vp]
    lib.absa_select_profile.restype = ctypes.c_int
    lib.absa_select_profile.argtypes = [P, SP, vp, vp, BL, vp, ctypes.c_size_t, vp, ctypes.POINTER(ctypes.c_float),
                                        ctypes.c_int32]
    lib.absa_attend.restype = ctypes.c_int
    lib.absa_attend.argtypes = [P, vp, vp, vp, BL, vp, vp]
    lib.absa_dense.restype = ctypes.c_int
    lib.absa_dense.argtypes = [P, vp, vp, vp, vp, vp]
    lib.absa_attend_balanced_workspace.restype = ctypes.c_int
    lib.absa_attend_balanced_workspace.argtypes = [ctypes.POINTER(sz)]
    lib.absa_attend_balanced.restype = ctypes.c_int
    lib.absa_attend_balanced.argtypes = [P, vp, vp, vp, BL, vp, vp, sz, vp]
    lib.absa_attend_pairs_workspace.restype = ctypes.c_int
    lib.absa_attend_pairs_workspace.argtypes = [P, ctypes.POINTER(sz)]
    lib.absa_attend_pairs.restype = ctypes.c_int
    lib.absa_attend_pairs.argtypes = [P, vp, vp, vp, BL, vp, vp, sz, vp]
    CL = ctypes.POINTER(AbsaClusterLists)
    lib.absa_select_clusters_workspace.restype = ctypes.c_int
    lib.absa_select_clusters_workspace.argtypes = [P, SP, ctypes.POINTER(sz)]
    lib.absa_select_clusters.restype = ctypes.c_int
    lib.absa_select_clusters.argtypes = [P, SP, vp, vp, CL, vp, sz, vp]
    lib.absa_attend_clusters.restype = ctypes.c_int
    lib.absa_attend_clusters.argtypes = [P, vp, vp, vp, CL, vp, vp]
    F8 = ctypes.POINTER(AbsaFp8Operands)
    lib.absa_fp8_workspace.restype = ctypes.c_int
    lib.absa_fp8_workspace.argtypes = [P, ctypes.POINTER(sz)]
    lib.absa_quantize_fp8.restype = ctypes.c_int
    lib.absa_quantize_fp8.argtypes = [P, vp, vp, vp, F8, vp, sz, vp]
    lib.absa_attend_fp8.restype = ctypes.c_int
    lib.absa_attend_fp8.argtypes = [P, F8, BL, vp, vp]
    _lib = lib
    return lib


def status_string(status: int) -> str:
    try:
        return load().absa_status_string(status).decode()
    except ImportError:
        return "status %d" % status


def check(status: int, where: str) -> None:
    if status != ABSA_OK:
        raise AbsaError(status, where)

"""ctypes loader for ``liblosa.so``: argument marshalling only.

The library is loaded on first use.  If it has not been built, every call
raises :class:`LosaLibraryMissing`; there is no fallback implementation.
"""

import ctypes
import os
import threading

# LOSA_LIBRARY names another build of the same library (the host-sanitizer
# test build); by default the in-tree liblosa.so is loaded
LIB_PATH = os.environ.get("LOSA_LIBRARY") or \
    os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblosa.so")

LOSA_OK = 0
STATUS_NAMES = {
    0: "LOSA_OK",
    1: "LOSA_ERR_NULL_POINTER",
    2: "LOSA_ERR_BAD_SHAPE",
    3: "LOSA_ERR_BAD_DTYPE",
    4: "LOSA_ERR_BAD_THRESHOLD",
    5: "LOSA_ERR_MISALIGNED",
    6: "LOSA_ERR_DEVICE",
    7: "LOSA_ERR_BAD_ARGUMENT",
    8: "LOSA_ERR_WORKSPACE",
    9: "LOSA_ERR_SCRATCH_LIMIT",
}
LOSA_BF16 = 0
LOSA_FP32 = 1
MAX_BLOCKS = 1024
NOALLOC_MAX_ROWS = 4194304


class LosaLibraryMissing(RuntimeError):
    pass


class LosaError(RuntimeError):
    def __init__(self, fn, status, text):
        super().__init__(f"{fn} failed: {STATUS_NAMES.get(status, status)} ({text})")
        self.status = status


class AttnDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("heads", ctypes.c_int32),
        ("seq_len", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("stride_batch", ctypes.c_int64),
        ("stride_head", ctypes.c_int64),
        ("stride_token", ctypes.c_int64),
        ("o_stride_batch", ctypes.c_int64),
        ("o_stride_head", ctypes.c_int64),
        ("o_stride_token", ctypes.c_int64),
    ]


_lock = threading.Lock()
_lib = None

_VP = ctypes.c_void_p
_DESC = ctypes.POINTER(AttnDesc)
SIGNATURES = {
    "losa_num_blocks": (ctypes.c_int32, [_DESC]),
    "losa_dense_attn": (ctypes.c_int, [_DESC, _VP, _VP, _VP, _VP, _VP, _VP]),
    "losa_block_mass": (ctypes.c_int, [_DESC, _VP, _VP, _VP, _VP, _VP, _VP]),
    "losa_block_mass_noalloc": (ctypes.c_int, [_DESC, _VP, _VP, _VP, _VP]),
    "losa_dense_attn_mass_workspace": (ctypes.c_int64, [_DESC]),
    "losa_dense_attn_mass_workspace_min": (ctypes.c_int64, [_DESC]),
    "losa_dense_attn_mass": (ctypes.c_int, [_DESC, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                            ctypes.c_int64, _VP]),
    "losa_select": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, _VP, ctypes.c_double,
                                   _VP, _VP, _VP]),
    "losa_select_per_row": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, _VP, _VP,
                                           ctypes.c_int32, _VP, _VP, _VP]),
    "losa_block_mask": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, _VP, _VP, _VP, _VP]),
    "losa_retained_mass": (ctypes.c_int, [_DESC, _VP, _VP, _VP, _VP]),
    "losa_sparse_attn": (ctypes.c_int, [_DESC, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP]),
    "losa_sparse_plan_size": (ctypes.c_int64, [_DESC]),
    "losa_sparse_plan": (ctypes.c_int, [_DESC, _VP, _VP, ctypes.c_int64, _VP]),
    "losa_sparse_attn_planned": (ctypes.c_int, [_DESC, _VP, _VP, _VP, _VP, _VP, _VP,
                                                ctypes.c_int64, _VP, _VP, _VP]),
    "losa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "losa_version": (ctypes.c_int32, []),
}


def load(path: str = LIB_PATH):
    """Load (once) and return the ctypes handle of liblosa.so."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(path):
                raise LosaLibraryMissing(
                    f"{path} is not built; run `python -m block_sparse_attention_losa_amd.build`")
            lib = ctypes.CDLL(path)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(lib, name)
                fn.restype = res
                fn.argtypes = args
            _lib = lib
        return _lib


def check(fn_name: str, status: int):
    if status != LOSA_OK:
        text = load().losa_status_string(status)
        raise LosaError(fn_name, status, text.decode() if text else "")

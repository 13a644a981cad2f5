"""ctypes view of libwkv7.so (declarations mirror include/wkv7.h).

WKV7_LIB, when set, names another build of the library to load instead of
the in-tree one (for A/B timing of builds); it must exist.
"""
import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("WKV7_LIB") or os.path.join(PKG, "libwkv7.so")

WKV7_F32, WKV7_BF16 = 0, 1
WKV7_ALGO_AUTO, WKV7_ALGO_SCAN, WKV7_ALGO_CHUNKED = 0, 1, 2
WKV7_OK, WKV7_ERR_INVALID, WKV7_ERR_UNSUPPORTED, WKV7_ERR_WORKSPACE, WKV7_ERR_HIP = 0, -1, -2, -3, -4

# Every function the C header declares, for the symbol-export test.
EXPORTS = ("wkv7_checkpoint_bytes", "wkv7_backward_workspace_bytes", "wkv7_forward",
           "wkv7_backward", "wkv7_epilogue_workspace_bytes", "wkv7_epilogue_forward",
           "wkv7_epilogue_backward", "wkv7_status_string", "wkv7_abi_version",
           "wkv7_fault_status", "wkv7_test_hook", "wkv7_backward_noalloc")
# ... and every function include/rwkv8.h declares
RWKV8_EXPORTS = ("rwkv8_checkpoint_bytes", "rwkv8_backward_workspace_bytes", "rwkv8_forward",
                 "rwkv8_backward")
WKV7_FAULT_RWKV8_DECAY = 2

WKV7_NOALLOC_SCRATCH_BYTES = 128 << 20

WKV7_FAULT_HELPER_WAIT = 1
WKV7_HOOK_FAULT_INJECT, WKV7_HOOK_FAIL_LAUNCHES = 1, 2


WKV7_FUSED_INPUTS = 1   # wkv7_shape.flags bit


class Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("T", ctypes.c_int64), ("H", ctypes.c_int64),
                ("N", ctypes.c_int64), ("dtype", ctypes.c_int32), ("chunk", ctypes.c_int32),
                ("algo", ctypes.c_int32), ("flags", ctypes.c_int32)]


class Rwkv8Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("T", ctypes.c_int64), ("H", ctypes.c_int64),
                ("Hv", ctypes.c_int64), ("L", ctypes.c_int64), ("E", ctypes.c_int64)]


class Wkv7Error(RuntimeError):
    def __init__(self, func, status, text):
        super().__init__(f"{func} failed: {status} ({text})")
        self.status = status


_LIB = None


def lib():
    """Load libwkv7.so; raise if it has not been built (there is no fallback)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m linear_attention_rnn_wkv7_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    sp = ctypes.POINTER(Shape)
    L.wkv7_checkpoint_bytes.argtypes = [sp]
    L.wkv7_checkpoint_bytes.restype = sz
    L.wkv7_backward_workspace_bytes.argtypes = [sp, i32]
    L.wkv7_backward_workspace_bytes.restype = sz
    L.wkv7_forward.argtypes = [sp] + [vp] * 10 + [vp]
    L.wkv7_forward.restype = i32
    L.wkv7_backward.argtypes = [sp] + [vp] * 17 + [vp, sz, vp]
    L.wkv7_backward.restype = i32
    L.wkv7_backward_noalloc.argtypes = [sp] + [vp] * 17 + [vp]
    L.wkv7_backward_noalloc.restype = i32
    L.wkv7_epilogue_workspace_bytes.argtypes = [sp]
    L.wkv7_epilogue_workspace_bytes.restype = sz
    L.wkv7_epilogue_forward.argtypes = [sp] + [vp] * 9 + [vp]
    L.wkv7_epilogue_forward.restype = i32
    L.wkv7_epilogue_backward.argtypes = [sp] + [vp] * 17 + [vp, sz, vp]
    L.wkv7_epilogue_backward.restype = i32
    L.wkv7_status_string.argtypes = [i32]
    L.wkv7_status_string.restype = ctypes.c_char_p
    L.wkv7_abi_version.argtypes = []
    L.wkv7_abi_version.restype = i32
    L.wkv7_fault_status.argtypes = [ctypes.POINTER(ctypes.c_uint), i32, vp]
    L.wkv7_fault_status.restype = i32
    L.wkv7_test_hook.argtypes = [i32, ctypes.c_int64]
    L.wkv7_test_hook.restype = i32
    s8 = ctypes.POINTER(Rwkv8Shape)
    L.rwkv8_checkpoint_bytes.argtypes = [s8]
    L.rwkv8_checkpoint_bytes.restype = sz
    L.rwkv8_backward_workspace_bytes.argtypes = [s8, i32]
    L.rwkv8_backward_workspace_bytes.restype = sz
    L.rwkv8_forward.argtypes = [s8] + [vp] * 9 + [vp]
    L.rwkv8_forward.restype = i32
    L.rwkv8_backward.argtypes = [s8] + [vp] * 14 + [vp, sz, vp]
    L.rwkv8_backward.restype = i32
    _LIB = L
    return L


def status_text(status):
    return lib().wkv7_status_string(status).decode()


def check(func, status):
    if status != WKV7_OK:
        raise Wkv7Error(func, status, status_text(status))

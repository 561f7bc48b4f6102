"""ctypes binding of libadasum.so (argument marshalling only).

torch is imported before the library is loaded: torch ships its own HIP
runtime under the same soname (libamdhip64.so.7), so the dynamic loader then
binds the library to that already-loaded runtime and both share one HIP
context, one set of streams and one address space.
"""

import ctypes
import os

import torch  # noqa: F401  (must be loaded first, see above)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libadasum.so")

F32, F16, BF16 = 0, 1, 2
TREE, CHAIN = 0, 1
OK, EINVAL, ENOMEM, EHIP = 0, -1, -2, -3

# name -> (restype, argtypes); mirrors include/adasum.h
_VP = ctypes.c_void_p
_I64P = ctypes.POINTER(ctypes.c_int64)
SIGNATURES = {
    "adasum_combine": (ctypes.c_int, [_VP, ctypes.c_int, _I64P, ctypes.c_int, ctypes.c_int, _VP, _VP]),
    "adasum_workspace_bytes": (ctypes.c_int64, [ctypes.c_int, _I64P, ctypes.c_int, ctypes.c_int, ctypes.c_int]),
    "adasum_combine_ex": (ctypes.c_int, [_VP, ctypes.c_int, _I64P, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         _VP, _VP, ctypes.c_size_t, _VP, _VP, _VP, _VP]),
    "adasum_combine_noalloc": (ctypes.c_int, [_VP, ctypes.c_int, _I64P, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                              _VP, _VP, _VP, _VP, _VP]),
    "adasum_sum": (ctypes.c_int, [_VP, ctypes.c_int, ctypes.c_int64, ctypes.c_int, _VP, _VP, ctypes.c_size_t,
                                  _VP]),
    "adasum_sum_workspace_bytes": (ctypes.c_int64, [ctypes.c_int, ctypes.c_int64, ctypes.c_int]),
    "adasum_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "adasum_last_error": (ctypes.c_char_p, []),
    "adasum_version": (ctypes.c_int, []),
}



class KernelTime(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_char * 32), ("launches", ctypes.c_int),
                ("milliseconds", ctypes.c_double), ("bytes", ctypes.c_double)]


SIGNATURES["adasum_profile_begin"] = (ctypes.c_int, [])
SIGNATURES["adasum_profile_end"] = (ctypes.c_int, [ctypes.POINTER(KernelTime), ctypes.c_int])

_lib = None


class AdasumError(RuntimeError):
    def __init__(self, code, message):
        super().__init__(message)
        self.code = code


def lib():
    """Load libadasum.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python distributed_sgd_gradient_amd/build.py`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def profile_begin():
    check(lib().adasum_profile_begin())


def profile_end():
    """Per-kernel-kind {launches, milliseconds, bytes} recorded since profile_begin()."""
    rows = (KernelTime * 8)()
    n = check(lib().adasum_profile_end(rows, 8))
    return {r.kernel.decode(): {"launches": r.launches, "milliseconds": r.milliseconds, "bytes": r.bytes}
            for r in rows[:n]}


def check(code):
    """Raise AdasumError for a negative return code."""
    if code < 0:
        L = lib()
        detail = L.adasum_last_error().decode()
        raise AdasumError(code, f"{L.adasum_strerror(code).decode()}: {detail}")
    return code

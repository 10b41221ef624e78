"""ctypes view of ``libdcn_mi355x.so`` (the C ABI in ``include/dcn.h``).

Loading fails loudly when the library has not been built: there is no
fallback implementation anywhere in the package.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdcn_mi355x.so")

# dcn_status
DCN_OK = 0
STATUS_NAMES = {0: "DCN_OK", 1: "DCN_E_NULL", 2: "DCN_E_SHAPE", 3: "DCN_E_DTYPE",
                4: "DCN_E_UNSUPPORTED", 5: "DCN_E_ALIGN", 6: "DCN_E_HIP",
                7: "DCN_E_INTERNAL", 8: "DCN_E_WORKSPACE"}
# dcn_dtype / dcn_layout
DCN_F32, DCN_BF16 = 0, 1
DCN_OUT_NCHW, DCN_OUT_NHWC = 0, 1

# every symbol include/dcn.h declares
EXPORTS = ("dcn_create", "dcn_destroy", "dcn_output_size", "dcn_workspace_bytes",
           "dcn_tap_schedule", "dcn_packed_weight_bytes",
           "dcn_pack_weight", "dcn_forward_packed", "dcn_forward", "dcn_forward_rows",
           "dcn_forward_multi", "dcn_nchw_to_nhwc", "dcn_backward_workspace_bytes",
           "dcn_backward", "dcn_msda_create", "dcn_msda_destroy", "dcn_msda_value_positions",
           "dcn_msda_forward", "dcn_dsample_create", "dcn_dsample_destroy",
           "dcn_dsample_output_size", "dcn_dsample_forward", "dcn_forward_noalloc", "dcn_debug_coords", "dcn_debug_corner_table",
           "dcn_status_string", "dcn_last_error",
           "dcn_version")


class DcnDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "in_ch", "height", "width", "out_ch", "kernel_h", "kernel_w",
        "pad_h", "pad_w", "in_dtype", "out_dtype", "out_layout")]


class MsdaDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "num_queries", "num_heads", "head_dim", "num_levels", "num_points", "dtype",
        "softmax")]


class DsDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "groups", "group_ch", "height", "width", "kernel_h", "kernel_w", "pad_h",
        "pad_w", "dtype", "softmax", "out_layout")]


class DcnError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__("%s failed: %s (%s)" % (where, STATUS_NAMES.get(status, status), detail))


_lib = None


def load():
    """Load the shared library once; raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            "libdcn_mi355x.so is not built (expected at %s); run "
            "`python -m modulated_deformable_convolution_dcn_amd.build`" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
    st = ctypes.c_int
    sig = {
        "dcn_create": (st, [ctypes.POINTER(DcnDesc), ctypes.POINTER(vp)]),
        "dcn_destroy": (st, [vp]),
        "dcn_output_size": (st, [vp, ctypes.POINTER(i32), ctypes.POINTER(i32)]),
        "dcn_workspace_bytes": (st, [vp, ctypes.POINTER(sz)]),
        "dcn_tap_schedule": (st, [vp, ctypes.POINTER(ctypes.c_int32),
                                  ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)]),
        "dcn_packed_weight_bytes": (st, [vp, ctypes.POINTER(sz)]),
        "dcn_pack_weight": (st, [vp, vp, vp, sz, vp]),
        "dcn_forward_packed": (st, [vp, vp, vp, vp, vp, sz, vp, vp, vp]),
        "dcn_forward": (st, [vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "dcn_forward_rows": (st, [vp, i32, i32, vp, vp, vp, vp, sz, vp, vp, vp]),
        "dcn_nchw_to_nhwc": (st, [vp, vp, i32, i32, i32, i32, i32, vp]),
        "dcn_backward_workspace_bytes": (st, [vp, ctypes.POINTER(sz)]),
        "dcn_backward": (st, [vp] * 12 + [sz, vp]),
        "dcn_msda_create": (st, [ctypes.POINTER(MsdaDesc), ctypes.POINTER(i32),
                                 ctypes.POINTER(vp)]),
        "dcn_msda_destroy": (st, [vp]),
        "dcn_msda_value_positions": (st, [vp, ctypes.POINTER(i32)]),
        "dcn_msda_forward": (st, [vp, vp, vp, vp, vp, vp]),
        "dcn_forward_multi": (st, [i32, ctypes.POINTER(vp), vp, ctypes.POINTER(vp),
                                   ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(sz),
                                   ctypes.POINTER(vp), ctypes.POINTER(vp), vp]),
        "dcn_forward_noalloc": (st, [vp, vp, vp, vp, vp, vp, vp, vp]),
        "dcn_dsample_create": (st, [ctypes.POINTER(DsDesc), ctypes.POINTER(vp)]),
        "dcn_dsample_destroy": (st, [vp]),
        "dcn_dsample_output_size": (st, [vp, ctypes.POINTER(i32), ctypes.POINTER(i32)]),
        "dcn_dsample_forward": (st, [vp, vp, vp, vp, vp, vp]),
        "dcn_debug_coords": (st, [vp, vp, vp, vp, vp]),
        "dcn_debug_corner_table": (st, [vp, vp, vp, vp, vp, sz, vp, vp, vp, vp, vp]),
        "dcn_status_string": (ctypes.c_char_p, [st]),
        "dcn_last_error": (ctypes.c_char_p, []),
        "dcn_version": (i32, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def check(status: int, where: str) -> None:
    if status != DCN_OK:
        detail = load().dcn_last_error().decode(errors="replace")
        raise DcnError(status, where, detail)

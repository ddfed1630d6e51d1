"""ctypes view of libmssm.so (include/mssm.h).  Argument marshalling only."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmssm.so")

MSSM_F32 = 0
MSSM_BF16 = 1
MSSM_FLAG_LOAD_STATE = 1
MSSM_FLAG_LAYOUT_BLD = 2
MSSM_FLAG_BC_STATE_MAJOR = 4
MSSM_FLAG_STATE_STREAM = 8

STATUS = {
    0: "MSSM_OK", -1: "MSSM_ERR_NULL", -2: "MSSM_ERR_DIMS",
    -3: "MSSM_ERR_UNSUPPORTED", -4: "MSSM_ERR_ALIGN", -5: "MSSM_ERR_ALIAS",
    -6: "MSSM_ERR_HIP", -7: "MSSM_ERR_WORKSPACE",
}

MSSM_OP_SCAN_FWD = 0
MSSM_OP_SCAN_FWD_CONV = 1
MSSM_OP_SCAN_BWD = 2
MSSM_OP_MAMBA2_FWD = 3

# every symbol include/mssm.h declares
EXPORTS = ("mssm_selective_scan_fwd", "mssm_selective_scan_bwd",
           "mssm_selective_scan_fwd_conv", "mssm_causal_conv1d_fwd",
           "mssm_selective_state_update", "mssm_mamba2_scan_fwd",
           "mssm_selective_scan_fwd_plan", "mssm_set_scan_timing_events",
           "mssm_status_string", "mssm_last_error", "mssm_abi_version",
           "mssm_selective_scan_fwd_ws", "mssm_selective_scan_fwd_conv_ws",
           "mssm_selective_scan_bwd_ws", "mssm_mamba2_scan_fwd_ws",
           "mssm_workspace_size", "mssm_selective_scan_fwd_noalloc",
           "mssm_valu_probe", "mssm_causal_conv1d_bwd")


class Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("dim", ctypes.c_int64),
                ("dstate", ctypes.c_int64), ("seqlen", ctypes.c_int64),
                ("io_dtype", ctypes.c_int32), ("flags", ctypes.c_uint32),
                ("time_segments", ctypes.c_int32), ("ngroups", ctypes.c_int32)]


class Plan(ctypes.Structure):
    _fields_ = [("groups", ctypes.c_int32), ("whole_groups", ctypes.c_int32),
                ("split_groups", ctypes.c_int32), ("segments", ctypes.c_int32),
                ("segment_len", ctypes.c_int64),
                ("waves_per_group", ctypes.c_int32), ("kernels", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_int64),
                ("vector_path", ctypes.c_int32), ("reserved", ctypes.c_int32)]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_ if k != "reserved"}


_lib = None


def lib():
    """The loaded library; raises if it has not been built (no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                "libmssm.so is not built (%s); run "
                "`python -m selective_state_space_52_amd.build`" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        vp, fp, i = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int
        L.mssm_selective_scan_fwd.argtypes = [vp, vp, fp, vp, vp, fp, vp, fp, i,
                                              vp, fp, ctypes.POINTER(Dims), vp]
        L.mssm_selective_scan_fwd.restype = i
        L.mssm_selective_scan_bwd.argtypes = [vp, vp, fp, vp, vp, fp, vp, fp, i,
                                              fp, vp, fp, vp, vp, fp, fp, fp,
                                              fp, vp, fp, fp,
                                              ctypes.POINTER(Dims), vp]
        L.mssm_selective_scan_bwd.restype = i
        L.mssm_selective_scan_fwd_conv.argtypes = [vp, fp, fp, vp, vp, fp, vp, vp,
                                                   fp, vp, fp, i, vp, fp, vp,
                                                   ctypes.POINTER(Dims), vp]
        L.mssm_selective_scan_fwd_conv.restype = i
        L.mssm_causal_conv1d_fwd.argtypes = [vp, fp, fp, vp, i, i, vp,
                                             ctypes.POINTER(Dims), vp]
        L.mssm_causal_conv1d_fwd.restype = i
        L.mssm_selective_state_update.argtypes = [fp, vp, vp, fp, vp, vp, fp, vp,
                                                  fp, i, vp, ctypes.POINTER(Dims), vp]
        L.mssm_selective_state_update.restype = i
        L.mssm_mamba2_scan_fwd.argtypes = [vp, vp, fp, vp, vp, fp, vp, fp, i,
                                           ctypes.c_int64, vp, fp,
                                           ctypes.POINTER(Dims), vp]
        L.mssm_mamba2_scan_fwd.restype = i
        i64 = ctypes.c_int64
        L.mssm_selective_scan_fwd_ws.argtypes = [vp, vp, fp, vp, vp, fp, vp, fp, i,
                                                 vp, fp, vp, i64, ctypes.POINTER(Dims), vp]
        L.mssm_selective_scan_fwd_ws.restype = i
        L.mssm_selective_scan_fwd_conv_ws.argtypes = [vp, fp, fp, vp, vp, fp, vp, vp,
                                                      fp, vp, fp, i, vp, fp, vp, vp, i64,
                                                      ctypes.POINTER(Dims), vp]
        L.mssm_selective_scan_fwd_conv_ws.restype = i
        L.mssm_selective_scan_bwd_ws.argtypes = [vp, vp, fp, vp, vp, fp, vp, fp, i,
                                                 fp, vp, fp, vp, vp, fp, fp, fp,
                                                 fp, vp, fp, fp, vp, i64,
                                                 ctypes.POINTER(Dims), vp]
        L.mssm_selective_scan_bwd_ws.restype = i
        L.mssm_mamba2_scan_fwd_ws.argtypes = [vp, vp, fp, vp, vp, fp, vp, fp, i,
                                              i64, vp, fp, vp, i64,
                                              ctypes.POINTER(Dims), vp]
        L.mssm_mamba2_scan_fwd_ws.restype = i
        L.mssm_selective_scan_fwd_noalloc.argtypes = [vp, vp, fp, vp, vp, fp, vp, fp, i,
                                                      vp, fp, ctypes.POINTER(Dims), vp]
        L.mssm_selective_scan_fwd_noalloc.restype = i
        L.mssm_workspace_size.argtypes = [i, ctypes.POINTER(Dims), i64,
                                          ctypes.POINTER(i64)]
        L.mssm_workspace_size.restype = i
        L.mssm_selective_scan_fwd_plan.argtypes = [ctypes.POINTER(Dims),
                                                   ctypes.POINTER(Plan)]
        L.mssm_selective_scan_fwd_plan.restype = i
        L.mssm_status_string.argtypes = [i]
        L.mssm_status_string.restype = ctypes.c_char_p
        L.mssm_last_error.argtypes = []
        L.mssm_last_error.restype = ctypes.c_char_p
        L.mssm_set_scan_timing_events.argtypes = [vp, vp]
        L.mssm_set_scan_timing_events.restype = i
        L.mssm_abi_version.argtypes = []
        L.mssm_abi_version.restype = i
        L.mssm_causal_conv1d_bwd.argtypes = [vp, fp, fp, vp, i, i, vp, vp, fp, fp, vp,
                                             ctypes.POINTER(Dims), vp]
        L.mssm_causal_conv1d_bwd.restype = i
        L.mssm_valu_probe.argtypes = [i, i, i, vp, vp]
        L.mssm_valu_probe.restype = i
        _lib = L
    return _lib


class MssmError(RuntimeError):
    def __init__(self, code: int):
        L = lib()
        msg = L.mssm_status_string(code).decode()
        if code in (-6, -7):
            msg += ": " + L.mssm_last_error().decode()
        super().__init__("%s (%d): %s" % (STATUS.get(code, "?"), code, msg))
        self.code = code


def check(code: int) -> None:
    if code != 0:
        raise MssmError(code)

"""ctypes view of libpkd.so (include/pkd.h).  Argument marshalling only."""

from __future__ import annotations

import ctypes
import os
import re

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpkd.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "pkd.h")

PKD_OK = 0
PKD_ERR_INVALID_ARG = 1
PKD_ERR_UNSUPPORTED = 2
PKD_ERR_DTYPE_MISMATCH = 3
PKD_ERR_WORKSPACE_TOO_SMALL = 4
PKD_ERR_STALE_PLAN = 5
PKD_ERR_HIP = 6

PKD_DTYPE_BF16 = 1
PKD_DTYPE_FP16 = 2
PKD_DTYPE_FP8_E4M3 = 3
PKD_LAYOUT_NHD = 0
PKD_LAYOUT_HND = 1
PKD_DEVERR_PAGE_ID = 1
PKD_VARIANT_AUTO = 0
PKD_VARIANT_DOT2 = 1
PKD_VARIANT_MFMA = 2
PKD_VARIANT_MFMA_PV = 3
VARIANTS = {"auto": PKD_VARIANT_AUTO, "dot2": PKD_VARIANT_DOT2, "mfma": PKD_VARIANT_MFMA,
            "mfma_pv": PKD_VARIANT_MFMA_PV}

HEADER_BASE = 32
PKD_PLAN_DECODE, PKD_PLAN_SHARED = 0, 1
PKD_PLAN_ALL_PARTIALS = 1
H_FIELDS = ["MAGIC", "VERSION", "BATCH", "QO_HEADS", "KV_HEADS", "HEAD_DIM", "PAGE_SIZE",
            "SLOTS", "CHUNK_PAGES", "ITEMS", "PARTIALS", "SPLIT", "ALPHA", "BETA", "NNZ",
            "PLAN_ID", "OFF_SLOTS", "OFF_ITEMS", "OFF_MERGE", "OFF_INDICES",
            "TOTAL_TOKENS_LO", "TOTAL_TOKENS_HI", "OFF_FIRST", "KIND", "NUM_GROUPS",
            "OFF_GROUPS", "ROWS_PER_BLOCK", "MIN_CHUNKS", "MAX_CHUNKS", "FLAGS"]
H = {name: i for i, name in enumerate(H_FIELDS)}

_STATUS_NAMES = {0: "PKD_OK", 1: "PKD_ERR_INVALID_ARG", 2: "PKD_ERR_UNSUPPORTED",
                 3: "PKD_ERR_DTYPE_MISMATCH", 4: "PKD_ERR_WORKSPACE_TOO_SMALL",
                 5: "PKD_ERR_STALE_PLAN", 6: "PKD_ERR_HIP"}


class PkdError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{_STATUS_NAMES.get(code, code)}: {message}")
        self.code = code


class pkd_plan_opts(ctypes.Structure):
    _fields_ = [("fixed_chunk_pages", ctypes.c_int32), ("min_chunk_tokens", ctypes.c_int32),
                ("alpha", ctypes.c_int32), ("beta", ctypes.c_int32), ("variant", ctypes.c_int32),
                ("flags", ctypes.c_int32)]


_i32, _i64, _sz, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p
_pi32 = ctypes.POINTER(ctypes.c_int32)
_pf32 = ctypes.POINTER(ctypes.c_float)

SIGNATURES = {
    "pkd_create": (ctypes.c_int, [ctypes.POINTER(_vp), _i32, _i32]),
    "pkd_destroy": (ctypes.c_int, [_vp]),
    "pkd_num_slots": (_i32, [_vp]),
    "pkd_plan_id": (_i64, [_vp]),
    "pkd_planned_variant": (_i32, [_vp]),
    "pkd_plan_shape": (ctypes.c_int, [_vp, _pi32]),
    "pkd_last_error": (ctypes.c_char_p, []),
    "pkd_int_workspace_bytes": (_sz, [_i32, _i32, _i32]),
    "pkd_float_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32]),
    "pkd_host_workspace_bytes": (_sz, [_i32, _i32]),
    "pkd_plan": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                _vp, _sz, _vp, _sz, _vp, _sz, ctypes.POINTER(pkd_plan_opts), _vp]),
    "pkd_plan_static": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                                       _i32, _i32, ctypes.POINTER(pkd_plan_opts), _vp]),
    "pkd_plan_host": (ctypes.c_int, [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                                     ctypes.POINTER(pkd_plan_opts), _vp, _sz,
                                     ctypes.POINTER(_i64)]),
    "pkd_plan_shared": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                       _i32, _i32, _i32, _vp, _sz, _vp, _sz, _vp, _sz,
                                       ctypes.POINTER(pkd_plan_opts), _vp]),
    "pkd_plan_shared_host": (ctypes.c_int, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                                            ctypes.POINTER(pkd_plan_opts), _vp, _sz,
                                            ctypes.POINTER(_i64)]),
    "pkd_shared_workspace_bytes": (ctypes.c_int, [_i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                                  ctypes.POINTER(_sz), ctypes.POINTER(_sz),
                                                  ctypes.POINTER(_sz)]),
    "pkd_append_positions": (ctypes.c_int, [_vp, _vp, _vp, _i32, _i32, _vp, _vp, _vp]),
    "pkd_append_paged_kv": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _vp, _vp, _i32, _i32, _i32,
                                           _i32, _i32, _i32, _vp, _i64, _vp, _vp]),
    "pkd_append_paged_kv_scaled": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _vp, _vp, _i32, _i32,
                                                  _i32, _i32, _i32, _i32, _vp, _i64,
                                                  ctypes.c_float, ctypes.c_float, _vp, _vp]),
    "pkd_run": (ctypes.c_int, [_vp, _vp, _i32, _vp, _i64, _i32, _i32, _vp, _vp, ctypes.c_float,
                               _vp]),
    "pkd_run_scaled": (ctypes.c_int, [_vp, _vp, _i32, _vp, _i64, _i32, _i32, _vp, _vp,
                                      ctypes.c_float, ctypes.c_float, ctypes.c_float, _vp]),
    "pkd_run_composable": (ctypes.c_int, [_vp, _vp, _vp, _i32, _vp, _i64, _i32, _i32, _vp, _vp,
                                          ctypes.c_float, _vp]),
    "pkd_run_composable_scaled": (ctypes.c_int, [_vp, _vp, _vp, _i32, _vp, _i64, _i32, _i32, _vp,
                                                 _vp, ctypes.c_float, ctypes.c_float,
                                                 ctypes.c_float, _vp]),
    "pkd_read_device_error": (ctypes.c_int, [_vp, _pi32, _vp]),
    "pkd_merge_state": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp]),
    "pkd_merge_states": (ctypes.c_int, [_vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp]),
    "pkd_profile_enable": (ctypes.c_int, [_vp, _i32]),
    "pkd_read_sink_words": (_i32, [_i32]),
    "pkd_read_stream": (ctypes.c_int, [_vp, _i64, _vp, _i32, _vp]),
    "pkd_read_pages": (ctypes.c_int, [_vp, _i64, _i64, _vp, _i64, _vp, _i32, _vp]),
    "pkd_profile_read": (ctypes.c_int, [_vp, ctypes.POINTER(ctypes.c_double),
                                        ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_i64)]),
}

_LIB = None


def header_functions():
    """Names of the functions include/pkd.h declares."""
    text = open(HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkd_[a-z_0-9]+)\s*\(", text)))


def load():
    """Load libpkd.so from the package directory; raise if it is not built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m paged_kv_decode_11_amd.build` "
                           "(or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib


def check(rc: int) -> None:
    if rc != PKD_OK:
        msg = load().pkd_last_error()
        raise PkdError(rc, msg.decode() if msg else "")

"""ctypes loader for libkda.so (the C ABI declared in include/kda.h).

Argument marshalling only: nothing here computes any part of the method. If
the shared library is missing or fails to load, every call raises; there is no
fallback path.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

LIB_PATH = Path(__file__).resolve().parent / "libkda.so"

KDA_DTYPE_FP32 = 0
KDA_DTYPE_BF16 = 1
KDA_GATE_LOG_DECAY = 0
KDA_GATE_SCALED_SIGMOID = 1
GATES = {"log_decay": KDA_GATE_LOG_DECAY, "scaled_sigmoid": KDA_GATE_SCALED_SIGMOID}
KDA_QK_AS_GIVEN = 0
KDA_QK_L2NORM = 1
CONVS = {"none": 0, "short4": 1, "short4_silu": 2}
OPERANDS = {"bf16": 0, "fp16": 1}
# device-side error bits of a prefill workspace (kda_workspace_status)
WS_ERR_WAIT_TIMEOUT = 1
WS_ERR_HEADER_MISMATCH = 2
STATUS = {0: "KDA_SUCCESS", 1: "KDA_ERROR_INVALID_VALUE", 2: "KDA_ERROR_NOT_SUPPORTED",
          3: "KDA_ERROR_WORKSPACE_TOO_SMALL", 4: "KDA_ERROR_NO_DEVICE", 5: "KDA_ERROR_HIP"}
EXPORTS = ("kda_abi_version", "kda_status_string", "kda_chunk_fwd_workspace_bytes", "kda_chunk_fwd_min_workspace_bytes",
           "kda_chunk_prep_workspace_bytes",
           "kda_workspace_status", "kda_chunk_fwd", "kda_chunk_prep", "kda_chunk_state", "kda_decode_step",
           "kda_chunk_bwd_workspace_bytes", "kda_chunk_bwd_segmented_workspace_bytes", "kda_chunk_bwd",
           "kda_chunk_fwd_no_alloc")

NO_ALLOC_SCRATCH_BYTES = 16 * 1024 * 1024  # KDA_NO_ALLOC_SCRATCH_BYTES

ABI_VERSION = 11
_lib = None


class KDAError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__("%s: %s" % (what, STATUS.get(status, "status %d" % status)))
        self.status = status


def load() -> ctypes.CDLL:
    """Load libkda.so once; raise if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not LIB_PATH.exists():
        raise RuntimeError("libkda.so is not built (%s); run kda_gated_delta_chunk_amd/build.py" % LIB_PATH)
    lib = ctypes.CDLL(str(LIB_PATH))
    lib.kda_abi_version.argtypes = []
    lib.kda_abi_version.restype = ctypes.c_int
    if lib.kda_abi_version() != ABI_VERSION:
        raise RuntimeError("%s has ABI version %d, this binding expects %d; rebuild it"
                           % (LIB_PATH, lib.kda_abi_version(), ABI_VERSION))
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.kda_abi_version.argtypes = []
    lib.kda_abi_version.restype = ctypes.c_int
    lib.kda_status_string.argtypes = [ctypes.c_int]
    lib.kda_status_string.restype = ctypes.c_char_p
    ci = ctypes.c_int
    for fn in (lib.kda_chunk_fwd_workspace_bytes, lib.kda_chunk_fwd_min_workspace_bytes,
               lib.kda_chunk_prep_workspace_bytes):
        fn.argtypes = [i64, i64, i32, i32, i32, i32, i32, ci, ci, ci]
        fn.restype = sz
    lib.kda_workspace_status.argtypes = [vp, sz, ctypes.POINTER(i32), vp]
    lib.kda_workspace_status.restype = ci
    lib.kda_chunk_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i32, i32, i32, i32, i32,
                                  ci, ci, ci, ci, vp, ci, ci, vp, vp, vp, sz, vp]
    lib.kda_chunk_fwd.restype = ctypes.c_int
    lib.kda_chunk_fwd_no_alloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i32, i32, i32, i32, i32,
                                           ci, ci, ci, ci, vp, ci, ci, vp, vp, vp]
    lib.kda_chunk_fwd_no_alloc.restype = ctypes.c_int
    lib.kda_chunk_prep.argtypes = [vp, vp, vp, vp, vp, i64, i64, i32, i32, i32, i32, i32, ci,
                                   ci, ci, ci, vp, ci, vp, sz, vp]
    lib.kda_chunk_prep.restype = ctypes.c_int
    lib.kda_chunk_state.argtypes = [vp, vp, vp, vp, i64, i64, i32, i32, i32, i32, i32, ctypes.c_int, ctypes.c_int,
                                    vp, ctypes.c_int, vp, vp, vp, sz, vp]
    lib.kda_chunk_state.restype = ctypes.c_int
    lib.kda_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_int, vp, vp, ctypes.c_int, vp]
    lib.kda_decode_step.restype = ctypes.c_int
    lib.kda_chunk_bwd_workspace_bytes.argtypes = [i64, i64, i32, i32, i32, i32, ctypes.c_int, ctypes.c_int]
    lib.kda_chunk_bwd_workspace_bytes.restype = sz
    lib.kda_chunk_bwd_segmented_workspace_bytes.argtypes = [i64, i64, i32, i32, i32, i32, ctypes.c_int, ctypes.c_int,
                                                            i64]
    lib.kda_chunk_bwd_segmented_workspace_bytes.restype = sz
    lib.kda_chunk_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i32, i32, i32, i32, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                  sz, vp]
    lib.kda_chunk_bwd.restype = ctypes.c_int
    _lib = lib
    return lib


def check(status: int, what: str) -> None:
    if status != 0:
        raise KDAError(status, what)

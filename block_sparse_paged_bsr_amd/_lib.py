"""ctypes declarations of libbsr_attn.so (include/bsr_attn.h).

Loading fails loudly when the library has not been built: there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbsr_attn.so")
PROBE_PATH = os.path.join(HERE, "libbsr_probe.so")  # include/bsr_probe.h: HBM read and rate probes

BSR_OK = 0
BSR_INVALID_ARG = -1
BSR_UNSUPPORTED = -2
BSR_CAPACITY = -3
BSR_HIP_ERROR = -4
STATUS_NAMES = {
    BSR_OK: "BSR_OK",
    BSR_INVALID_ARG: "BSR_INVALID_ARG",
    BSR_UNSUPPORTED: "BSR_UNSUPPORTED",
    BSR_CAPACITY: "BSR_CAPACITY",
    BSR_HIP_ERROR: "BSR_HIP_ERROR",
}
DTYPE_F32 = 0
DTYPE_BF16 = 1

i32p = C.POINTER(C.c_int32)
i64p = C.POINTER(C.c_int64)


class PlanDesc(C.Structure):
    _fields_ = [
        ("batch", C.c_int32),
        ("qo_indptr", i32p),
        ("kv_indptr", i32p),
        ("kv_indices", i32p),
        ("last_page_len", i32p),
        ("num_pages", C.c_int32),
        ("num_qo_heads", C.c_int32),
        ("num_kv_heads", C.c_int32),
        ("head_dim", C.c_int32),
        ("page_size", C.c_int32),
        ("causal", C.c_int32),
        ("num_workers", C.c_int32),
        ("tile_q", C.c_int32),
        ("alpha", C.c_int32),
        ("beta", C.c_int32),
        ("window_size", C.c_int32),
        ("logits_soft_cap", C.c_float),
    ]


class PlanView(C.Structure):
    _fields_ = [
        ("batch", C.c_int32),
        ("num_qo_heads", C.c_int32),
        ("num_kv_heads", C.c_int32),
        ("head_dim", C.c_int32),
        ("page_size", C.c_int32),
        ("causal", C.c_int32),
        ("group_size", C.c_int32),
        ("tile_q", C.c_int32),
        ("num_workers", C.c_int32),
        ("num_slots", C.c_int32),
        ("total_work", C.c_int64),
        ("chunk_limit", C.c_int64),
        ("num_tiles", C.c_int32),
        ("tiles", i32p),
        ("num_items", C.c_int32),
        ("items", i32p),
        ("queue_ptr", i32p),
        ("queue_items", i32p),
        ("worker_cost", i64p),
        ("num_merge", C.c_int32),
        ("merge_tiles", i32p),
        ("merge_ptr", i32p),
        ("merge_slots", i32p),
        ("window_left", C.c_int32),
        ("logits_soft_cap", C.c_float),
        ("tile_lo", i32p),
        ("custom_mask_bits", C.c_int64),
        ("num_levels", C.c_int32),
        ("level_req_start", i32p),
        ("merge_row_off", i32p),
    ]


EXPORTED = [
    "bsr_plan_create",
    "bsr_plan_create_composable",
    "bsr_plan_destroy",
    "bsr_plan_workspace_bytes",
    "bsr_plan_upload",
    "bsr_plan_export",
    "bsr_run_decode",
    "bsr_run_decode_e4m3",
    "bsr_run_decode_scratch",
    "bsr_run_prefill",
    "bsr_run_prefill_masked",
    "bsr_merge_state",
    "bsr_debug_gather_rows",
    "bsr_timing_enable",
    "bsr_timing_read",
    "bsr_query_num_workers",
    "bsr_last_error",
    "bsr_version",
]

PROBE_EXPORTED = ["bsr_probe_read_pages", "bsr_probe_issue_mix", "bsr_probe_lds_read", "bsr_probe_l2_to_lds"]

_lib = None
_probe = None


def probe():
    """The probe library (raises if it was not built)."""
    global _probe
    if _probe is not None:
        return _probe
    if not os.path.exists(PROBE_PATH):
        raise RuntimeError(f"{PROBE_PATH} is missing: build it with `python -m block_sparse_paged_bsr_amd.build`")
    try:
        import torch  # noqa: F401  (one HIP runtime per process, as in lib())
    except ImportError:
        pass
    L = C.CDLL(PROBE_PATH)
    vp = C.c_void_p
    L.bsr_probe_read_pages.argtypes = [vp, vp, vp, C.c_int64, C.c_int64, C.c_int32, C.c_uint32, vp, vp]
    L.bsr_probe_read_pages.restype = C.c_int
    i32 = C.c_int32
    L.bsr_probe_issue_mix.argtypes = [i32, i32, vp, vp, vp]
    L.bsr_probe_issue_mix.restype = C.c_int
    L.bsr_probe_lds_read.argtypes = [i32, i32, i32, vp, vp, vp]
    L.bsr_probe_lds_read.restype = C.c_int
    L.bsr_probe_l2_to_lds.argtypes = [vp, i32, i32, i32, vp, vp, vp]
    L.bsr_probe_l2_to_lds.restype = C.c_int
    _probe = L
    return L


def lib():
    """The loaded library (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m block_sparse_paged_bsr_amd.build` "
            "(there is no fallback path)"
        )
    # torch's HIP runtime and the one the library links carry the same soname: load torch first,
    # so the process holds exactly one runtime (the library binds to the already-loaded copy);
    # loading the library first leaves torch's device calls on a second runtime without devices
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    L = C.CDLL(LIB_PATH)
    vp = C.c_void_p
    L.bsr_plan_create.argtypes = [C.POINTER(PlanDesc), C.POINTER(vp)]
    L.bsr_plan_create.restype = C.c_int
    L.bsr_plan_create_composable.argtypes = [C.POINTER(PlanDesc), C.c_int32, C.c_int32, C.POINTER(vp)]
    L.bsr_plan_create_composable.restype = C.c_int
    L.bsr_plan_destroy.argtypes = [vp]
    L.bsr_plan_destroy.restype = None
    L.bsr_plan_workspace_bytes.argtypes = [vp, C.POINTER(C.c_size_t)]
    L.bsr_plan_workspace_bytes.restype = C.c_int
    L.bsr_plan_upload.argtypes = [vp, vp, C.c_size_t, vp]
    L.bsr_plan_upload.restype = C.c_int
    L.bsr_plan_export.argtypes = [vp, C.POINTER(PlanView)]
    L.bsr_plan_export.restype = C.c_int
    run_args = [vp, vp, vp, vp, vp, vp, C.POINTER(C.c_float), C.c_int32, C.c_float, vp]
    L.bsr_run_decode.argtypes = run_args
    L.bsr_run_decode.restype = C.c_int
    L.bsr_run_prefill.argtypes = run_args
    L.bsr_run_prefill.restype = C.c_int
    L.bsr_run_decode_scratch.argtypes = [vp, vp, vp, vp, vp, C.POINTER(C.c_float), C.c_int32, C.c_float, vp]
    L.bsr_run_decode_scratch.restype = C.c_int
    L.bsr_run_decode_e4m3.argtypes = [vp, vp, vp, vp, vp, vp, C.POINTER(C.c_float), C.c_float, C.c_float,
                                      C.c_float, vp]
    L.bsr_run_decode_e4m3.restype = C.c_int
    L.bsr_run_prefill_masked.argtypes = [vp, vp, vp, vp, vp, vp, vp, C.POINTER(C.c_float), C.c_int32, C.c_float, vp]
    L.bsr_run_prefill_masked.restype = C.c_int
    fp = C.POINTER(C.c_float)
    L.bsr_merge_state.argtypes = [vp, fp, vp, fp, vp, fp, C.c_int64, C.c_int32, C.c_int32, C.c_int32, vp]
    L.bsr_merge_state.restype = C.c_int
    L.bsr_debug_gather_rows.argtypes = [vp, vp, vp, vp]
    L.bsr_debug_gather_rows.restype = C.c_int
    L.bsr_timing_enable.argtypes = [C.c_int32]
    L.bsr_timing_enable.restype = C.c_int
    L.bsr_timing_read.argtypes = [C.POINTER(C.c_double), i64p, C.POINTER(C.c_double), i64p]
    L.bsr_timing_read.restype = C.c_int
    L.bsr_query_num_workers.argtypes = [C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32, i32p]
    L.bsr_query_num_workers.restype = C.c_int
    L.bsr_last_error.argtypes = []
    L.bsr_last_error.restype = C.c_char_p
    L.bsr_version.argtypes = []
    L.bsr_version.restype = C.c_char_p
    _lib = L
    return L


class BsrError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def check(status):
    if status != BSR_OK:
        raise BsrError(status, lib().bsr_last_error().decode(errors="replace"))

"""Python binding of libmla_decode.so - MLA decode (DeepSeek-R1 forward_absorb)
split-K for MI355X (gfx950).

Argument marshalling only: every step of the decode runs in the HIP library.
The functions carry the names of the C ABI in include/mla_decode.h; device
buffers may be passed as torch tensors (their data pointers are used) or as
integer addresses.  There is no fallback: if the library is not built this
module raises on first use.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla_decode.so")

MLA_OK, MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED, MLA_ERR_HIP = 0, 1, 2, 3
MLA_DTYPE_BF16, MLA_DTYPE_FP8_E4M3FN, MLA_DTYPE_MXFP4 = 0, 1, 2
DTYPES = {"bf16": MLA_DTYPE_BF16, "fp8": MLA_DTYPE_FP8_E4M3FN, "mxfp4": MLA_DTYPE_MXFP4}


class mla_problem(ctypes.Structure):
    _fields_ = [("batch_size", ctypes.c_int32), ("total_q", ctypes.c_int32), ("total_kv", ctypes.c_int64),
                ("num_heads", ctypes.c_int32), ("qk_dim", ctypes.c_int32), ("v_dim", ctypes.c_int32),
                ("q_dtype", ctypes.c_int32), ("kv_dtype", ctypes.c_int32), ("sm_scale", ctypes.c_float),
                ("num_cus", ctypes.c_int32), ("max_q_len", ctypes.c_int32),
                ("logit_cap", ctypes.c_float), ("kv_paged", ctypes.c_int32)]


class mla_plan_options(ctypes.Structure):
    _fields_ = [("rows_per_split", ctypes.c_int32), ("wgs_per_cu", ctypes.c_int32), ("age_skew", ctypes.c_int32),
                ("xcd_group", ctypes.c_int32)]


class mla_plan_desc(ctypes.Structure):
    _fields_ = [("num_splits", ctypes.c_int32), ("rows_per_split", ctypes.c_int32), ("tile_rows", ctypes.c_int32),
                ("stages", ctypes.c_int32), ("partial_slots", ctypes.c_int32), ("stage2", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_int64), ("lds_bytes", ctypes.c_int32), ("num_cus", ctypes.c_int32),
                ("wgs_per_cu", ctypes.c_int32), ("query_tokens", ctypes.c_int32),
                ("paired_splits", ctypes.c_int32), ("second_rows_per_split", ctypes.c_int32),
                ("xcd_group", ctypes.c_int32), ("merge_batch", ctypes.c_int32),
                ("first_piece_table", ctypes.c_int32)]


class MlaError(RuntimeError):
    def __init__(self, status: int, what: str):
        detail = ""
        if status == MLA_ERR_HIP:
            detail = ": " + _lib_handle().mla_last_error_string().decode()
        super().__init__(f"{what} failed with {mla_status_string(status)}{detail}")
        self.status = status


_lib = None


def _lib_handle():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() (hipcc, gfx950)")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        lib.mla_decode_plan.argtypes = [ctypes.POINTER(mla_problem), ctypes.POINTER(mla_plan_options), vp,
                                        ctypes.POINTER(vp), ctypes.POINTER(sz)]
        lib.mla_decode_plan.restype = i32
        lib.mla_decode_run.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.mla_decode_run.restype = i32
        lib.mla_decode_split.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.mla_decode_split.restype = i32
        lib.mla_decode_run_paged.argtypes = [vp, vp, vp, vp, vp, i64, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.mla_decode_run_paged.restype = i32
        lib.mla_decode_split_paged.argtypes = [vp, vp, vp, vp, vp, i64, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.mla_decode_split_paged.restype = i32
        lib.mla_decode_run_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.mla_decode_run_noalloc.restype = i32
        lib.mla_decode_merge.argtypes = [vp, vp, vp, vp, vp, sz, vp]
        lib.mla_decode_merge.restype = i32
        lib.mla_decode_plan_destroy.argtypes = [vp]
        lib.mla_decode_plan_destroy.restype = None
        lib.mla_decode_plan_describe.argtypes = [vp, ctypes.POINTER(mla_plan_desc)]
        lib.mla_decode_plan_describe.restype = i32
        lib.mla_decode_plan_pieces.argtypes = [vp, vp, vp, i64, ctypes.POINTER(i64)]
        lib.mla_decode_plan_pieces.restype = i32
        lib.mla_decode_plan_merge_slots.argtypes = [vp, vp, i32, vp, i32, ctypes.POINTER(i32)]
        lib.mla_decode_plan_merge_slots.restype = i32
        lib.mla_debug_decode.argtypes = [i32, vp, vp, vp, i64, vp]
        lib.mla_debug_decode.restype = i32
        lib.mla_debug_stream_read.argtypes = [vp, i64, vp, vp]
        lib.mla_debug_stream_read.restype = i32
        lib.mla_debug_stream_ring.argtypes = [vp, i64, i32, vp, vp]
        lib.mla_debug_stream_ring.restype = i32
        lib.mla_debug_wg_trace.argtypes = [vp, i64, i32]
        lib.mla_debug_wg_trace.restype = i32
        lib.mla_status_string.argtypes = [i32]
        lib.mla_status_string.restype = ctypes.c_char_p
        lib.mla_last_error_string.argtypes = []
        lib.mla_last_error_string.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def library():
    """The loaded ctypes library (raises if it is not built)."""
    return _lib_handle()


def _addr(x) -> int | None:
    """Device/host address of a torch tensor, numpy array or integer (None stays None)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    if isinstance(x, np.ndarray):
        return x.ctypes.data
    raise TypeError(f"cannot take the address of {type(x)!r}")


def _stream(stream) -> int | None:
    if stream is None:
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream  # torch.cuda.Stream


def mla_status_string(status: int) -> str:
    return _lib_handle().mla_status_string(status).decode()


def make_problem(batch_size, total_kv, q_dtype="bf16", kv_dtype="bf16", total_q=None, num_heads=16, qk_dim=576,
                 v_dim=512, sm_scale=1.0 / 24.0, num_cus=0, max_q_len=0, logit_cap=0.0, kv_paged=0) -> mla_problem:
    return mla_problem(batch_size, batch_size if total_q is None else total_q, total_kv, num_heads, qk_dim, v_dim,
                       DTYPES.get(q_dtype, q_dtype), DTYPES.get(kv_dtype, kv_dtype), sm_scale, num_cus, max_q_len,
                       logit_cap, int(kv_paged))


class Plan:
    """Owns an mla_plan*; destroyed with the object."""

    def __init__(self, handle: int, workspace_bytes: int):
        self.handle = handle
        self.workspace_bytes = workspace_bytes

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.mla_decode_plan_destroy(self.handle)
            self.handle = None


def mla_decode_plan(problem: mla_problem, options: mla_plan_options | None = None, kv_indptr_host=None) -> Plan:
    lib = _lib_handle()
    ind = None
    if kv_indptr_host is not None:
        ind = np.ascontiguousarray(kv_indptr_host, dtype=np.int32)
    handle = ctypes.c_void_p()
    ws = ctypes.c_size_t()
    st = lib.mla_decode_plan(ctypes.byref(problem), ctypes.byref(options) if options is not None else None,
                             _addr(ind), ctypes.byref(handle), ctypes.byref(ws))
    if st != MLA_OK:
        raise MlaError(st, "mla_decode_plan")
    return Plan(handle.value, ws.value)


def mla_decode_run(plan: Plan, q, q_scale, kv, kv_scale, qo_indptr, kv_indptr, out, workspace,
                   workspace_bytes: int | None = None, stream=None) -> None:
    lib = _lib_handle()
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size() if hasattr(workspace, "numel") else 0
    st = lib.mla_decode_run(plan.handle, _addr(q), _addr(q_scale), _addr(kv), _addr(kv_scale), _addr(qo_indptr),
                            _addr(kv_indptr), _addr(out), _addr(workspace), workspace_bytes, _stream(stream))
    if st != MLA_OK:
        raise MlaError(st, "mla_decode_run")


def mla_decode_run_noalloc(plan: Plan, q, q_scale, kv, kv_scale, qo_indptr, kv_indptr, out, stream=None) -> None:
    st = _lib_handle().mla_decode_run_noalloc(plan.handle, _addr(q), _addr(q_scale), _addr(kv), _addr(kv_scale),
                                              _addr(qo_indptr), _addr(kv_indptr), _addr(out), _stream(stream))
    if st != MLA_OK:
        raise MlaError(st, "mla_decode_run_noalloc")


def mla_decode_split(plan: Plan, q, q_scale, kv, kv_scale, qo_indptr, kv_indptr, out, workspace,
                     workspace_bytes: int | None = None, stream=None) -> None:
    lib = _lib_handle()
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size() if hasattr(workspace, "numel") else 0
    st = lib.mla_decode_split(plan.handle, _addr(q), _addr(q_scale), _addr(kv), _addr(kv_scale), _addr(qo_indptr),
                              _addr(kv_indptr), _addr(out), _addr(workspace), workspace_bytes, _stream(stream))
    if st != MLA_OK:
        raise MlaError(st, "mla_decode_split")


def mla_decode_run_paged(plan: Plan, q, q_scale, kv, kv_scale, kv_rows: int, kv_indices, kv_page_indptr, qo_indptr,
                         kv_indptr, out, workspace, workspace_bytes: int | None = None, stream=None) -> None:
    lib = _lib_handle()
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size() if hasattr(workspace, "numel") else 0
    st = lib.mla_decode_run_paged(plan.handle, _addr(q), _addr(q_scale), _addr(kv), _addr(kv_scale), int(kv_rows),
                                  _addr(kv_indices), _addr(kv_page_indptr), _addr(qo_indptr), _addr(kv_indptr),
                                  _addr(out), _addr(workspace), workspace_bytes, _stream(stream))
    if st != MLA_OK:
        raise MlaError(st, "mla_decode_run_paged")


def mla_decode_split_paged(plan: Plan, q, q_scale, kv, kv_scale, kv_rows: int, kv_indices, kv_page_indptr,
                           qo_indptr, kv_indptr, out, workspace, workspace_bytes: int | None = None,
                           stream=None) -> None:
    lib = _lib_handle()
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size() if hasattr(workspace, "numel") else 0
    st = lib.mla_decode_split_paged(plan.handle, _addr(q), _addr(q_scale), _addr(kv), _addr(kv_scale), int(kv_rows),
                                    _addr(kv_indices), _addr(kv_page_indptr), _addr(qo_indptr), _addr(kv_indptr),
                                    _addr(out), _addr(workspace), workspace_bytes, _stream(stream))
    if st != MLA_OK:
        raise MlaError(st, "mla_decode_split_paged")


def mla_decode_merge(plan: Plan, qo_indptr, kv_indptr, out, workspace, workspace_bytes: int | None = None,
                     stream=None) -> None:
    lib = _lib_handle()
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size() if hasattr(workspace, "numel") else 0
    st = lib.mla_decode_merge(plan.handle, _addr(qo_indptr), _addr(kv_indptr), _addr(out), _addr(workspace),
                              workspace_bytes, _stream(stream))
    if st != MLA_OK:
        raise MlaError(st, "mla_decode_merge")


def mla_decode_plan_destroy(plan: Plan) -> None:
    if plan.handle:
        _lib_handle().mla_decode_plan_destroy(plan.handle)
        plan.handle = None


def mla_decode_plan_describe(plan: Plan) -> dict:
    d = mla_plan_desc()
    st = _lib_handle().mla_decode_plan_describe(plan.handle, ctypes.byref(d))
    if st != MLA_OK:
        raise MlaError(st, "mla_decode_plan_describe")
    return {name: getattr(d, name) for name, _ in mla_plan_desc._fields_}


def mla_decode_plan_pieces(plan: Plan, kv_indptr_host) -> np.ndarray:
    """[n, 5] int64 records (workgroup, sequence, row0, row1, slot)."""
    lib = _lib_handle()
    ind = np.ascontiguousarray(kv_indptr_host, dtype=np.int32)
    count = ctypes.c_int64()
    st = lib.mla_decode_plan_pieces(plan.handle, _addr(ind), None, 0, ctypes.byref(count))
    if st != MLA_OK:
        raise MlaError(st, "mla_decode_plan_pieces")
    rec = np.zeros((count.value, 5), dtype=np.int64)
    st = lib.mla_decode_plan_pieces(plan.handle, _addr(ind), _addr(rec), count.value, ctypes.byref(count))
    if st != MLA_OK:
        raise MlaError(st, "mla_decode_plan_pieces")
    return rec


def mla_decode_plan_merge_slots(plan: Plan, kv_indptr_host, b: int) -> list[int]:
    lib = _lib_handle()
    ind = np.ascontiguousarray(kv_indptr_host, dtype=np.int32)
    count = ctypes.c_int32()
    st = lib.mla_decode_plan_merge_slots(plan.handle, _addr(ind), b, None, 0, ctypes.byref(count))
    if st != MLA_OK:
        raise MlaError(st, "mla_decode_plan_merge_slots")
    slots = np.zeros(count.value, dtype=np.int32)
    st = lib.mla_decode_plan_merge_slots(plan.handle, _addr(ind), b, _addr(slots), count.value, ctypes.byref(count))
    if st != MLA_OK:
        raise MlaError(st, "mla_decode_plan_merge_slots")
    return slots.tolist()


def mla_debug_decode(kv_dtype, codes, scales, out, n: int, stream=None) -> None:
    st = _lib_handle().mla_debug_decode(DTYPES.get(kv_dtype, kv_dtype), _addr(codes), _addr(scales), _addr(out), n,
                                        _stream(stream))
    if st != MLA_OK:
        raise MlaError(st, "mla_debug_decode")


def mla_debug_stream_read(buf, nbytes: int, sink, stream=None) -> None:
    st = _lib_handle().mla_debug_stream_read(_addr(buf), nbytes, _addr(sink), _stream(stream))
    if st != MLA_OK:
        raise MlaError(st, "mla_debug_stream_read")


def mla_debug_stream_ring(buf, nbytes: int, wgs: int, sink, stream=None) -> None:
    st = _lib_handle().mla_debug_stream_ring(_addr(buf), nbytes, wgs, _addr(sink), _stream(stream))
    if st != MLA_OK:
        raise MlaError(st, "mla_debug_stream_ring")


def mla_debug_wg_trace(host: np.ndarray | None, clear: bool = False) -> None:
    """Copy the stage-1 workgroup timeline into `host` (uint64, 4 per workgroup)
    and/or clear it; the library must be the MLA_WG_TRACE build."""
    n = 0 if host is None else int(host.size)
    if host is not None and (host.dtype != np.uint64 or not host.flags["C_CONTIGUOUS"]):
        raise ValueError("host must be a contiguous uint64 array")
    st = _lib_handle().mla_debug_wg_trace(None if host is None else host.ctypes.data, n, 1 if clear else 0)
    if st != MLA_OK:
        raise MlaError(st, "mla_debug_wg_trace")

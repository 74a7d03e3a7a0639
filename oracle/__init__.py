"""CPU fp64 oracle for MLA decode - TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline
leg may import this package.  The GPU library (``mla_decode_split_amd``) never
imports it and shares no code with it; the two meet only in the seeded inputs
of ``synth``.

The arithmetic lives in ``mla_oracle.c`` (plain C, double precision); this
module compiles it with gcc and wraps it with ctypes.  What it computes is the
decode of the kernelbot-amd-mixed-mla submission template (submission 675627):
the docstring's forward_absorb configuration and the naive reference
``custom_kernel_bf16`` - scores over the full 576-wide row scaled by
1/sqrt(576), a softmax over the sequence's KV rows, and a weighted sum of the
rows' first 512 columns - evaluated in fp64 on exactly decoded inputs.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mla_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

DTYPES = {"bf16": 0, "fp8": 1, "mxfp4": 2}

_lib = None


class _Problem(ctypes.Structure):
    _fields_ = [("batch_size", ctypes.c_int32), ("num_heads", ctypes.c_int32), ("qk_dim", ctypes.c_int32),
                ("v_dim", ctypes.c_int32), ("q_dtype", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
                ("sm_scale", ctypes.c_double), ("logit_cap", ctypes.c_double)]


def build(force: bool = True, src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle with gcc.  No fast-math: the decode and the softmax
    must follow IEEE double arithmetic."""
    if force or not os.path.exists(out):
        tmp = out + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-std=c11", "-fno-fast-math", "-ffp-contract=off",
                               "-o", tmp, src, "-lm", "-lpthread"])
        os.replace(tmp, out)
    return out


def _bind(lib):
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    lib.oracle_e4m3fn_value.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3fn_value.restype = ctypes.c_double
    lib.oracle_e2m1_value.argtypes = [ctypes.c_uint8]
    lib.oracle_e2m1_value.restype = ctypes.c_double
    lib.oracle_e8m0_value.argtypes = [ctypes.c_uint8]
    lib.oracle_e8m0_value.restype = ctypes.c_double
    lib.oracle_bf16_value.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_value.restype = ctypes.c_double
    lib.oracle_decode_fp8.argtypes = [vp, i64, ctypes.c_float, vp]
    lib.oracle_decode_mxfp4.argtypes = [vp, vp, i64, i32, vp]
    lib.oracle_mla_decode.argtypes = [ctypes.POINTER(_Problem), vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, i32]
    lib.oracle_mla_decode.restype = i32
    lib.oracle_mla_decode_paged.argtypes = [ctypes.POINTER(_Problem), vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, i32]
    lib.oracle_mla_decode_paged.restype = i32
    lib.oracle_mla_decode_pages.argtypes = [ctypes.POINTER(_Problem), vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, i32, vp,
                                            vp, i32]
    lib.oracle_mla_decode_pages.restype = i32
    return lib


def load(path: str | None = None):
    """Load the compiled oracle (building it when missing).  With ``path`` a
    separately compiled copy is loaded instead (used by the mutation tests)."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data


def e4m3fn_value(code: int) -> float:
    return load().oracle_e4m3fn_value(code)


def e2m1_value(nibble: int) -> float:
    return load().oracle_e2m1_value(nibble)


def e8m0_value(code: int) -> float:
    return load().oracle_e8m0_value(code)


def decode_fp8(codes: np.ndarray, scale: float = 1.0) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(codes.shape, dtype=np.float64)
    load().oracle_decode_fp8(_p(codes), codes.size, float(scale), _p(out))
    return out


def decode_mxfp4(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    rows, half = packed.shape
    out = np.empty((rows, 2 * half), dtype=np.float64)
    load().oracle_decode_mxfp4(_p(packed), _p(scales), rows, 2 * half, _p(out))
    return out


def mla_decode(q, kv, qo_indptr, kv_indptr, *, q_dtype="bf16", kv_dtype="bf16", q_scale=None, kv_scale=None,
               sm_scale=1.0 / 24.0, num_heads=16, qk_dim=576, v_dim=512, seq_ids=None, threads=1, lib=None,
               logit_cap=0.0, kv_indices=None, kv_page_indptr=None, page_size=1):
    """fp64 reference output and LSE.

    q: uint16 bf16 bits or uint8 fp8 codes, shape [total_q, num_heads, qk_dim].
    kv: uint16 [total_kv, qk_dim] (bf16), uint8 [total_kv, qk_dim] (fp8) or
        uint8 [total_kv, qk_dim/2] (mxfp4 packed).
    kv_scale: fp32 scalar for fp8, uint8 [total_kv, qk_dim/32] for mxfp4.
    kv_indices: None, or int32 [kv_indptr[-1]]: KV row j of the CSR space is
        kv[kv_indices[j]] (paged KV, page size 1).
    kv_page_indptr, page_size: paged KV with pages of page_size rows:
        kv_indices lists pages, sequence b's from entry kv_page_indptr[b] on,
        and its row i is kv[kv_indices[kv_page_indptr[b] + i // page_size] *
        page_size + i % page_size].
    Returns (out [total_q, num_heads, v_dim] float64, lse [total_q, num_heads]);
    rows of sequences not in ``seq_ids`` are NaN."""
    lib = lib or load()
    q = np.ascontiguousarray(q)
    kv = np.ascontiguousarray(kv)
    qo = np.ascontiguousarray(qo_indptr, dtype=np.int32)
    kvp = np.ascontiguousarray(kv_indptr, dtype=np.int32)
    total_q = q.shape[0]
    prob = _Problem(kvp.shape[0] - 1, num_heads, qk_dim, v_dim, DTYPES[q_dtype], DTYPES[kv_dtype], float(sm_scale),
                    float(logit_cap))
    qs = None if q_scale is None else np.array([q_scale], dtype=np.float32)
    if kv_dtype == "fp8":
        ks = np.array([kv_scale], dtype=np.float32)
    elif kv_dtype == "mxfp4":
        ks = np.ascontiguousarray(kv_scale, dtype=np.uint8)
    else:
        ks = None
    ids = None if seq_ids is None else np.ascontiguousarray(seq_ids, dtype=np.int32)
    out = np.full((total_q, num_heads, v_dim), np.nan, dtype=np.float64)
    lse = np.full((total_q, num_heads), np.nan, dtype=np.float64)
    n_seq = prob.batch_size if ids is None else ids.shape[0]
    if kv_page_indptr is not None:
        ki = np.ascontiguousarray(kv_indices, dtype=np.int32)
        kpp = np.ascontiguousarray(kv_page_indptr, dtype=np.int32)
        P = int(page_size)
        lens = np.diff(kvp.astype(np.int64))
        need = kpp[:-1].astype(np.int64) + (lens + P - 1) // P
        if P < 1 or kpp.shape[0] != kvp.shape[0] or (need.size and need.max() > ki.shape[0]) or \
                (ki.size and (ki.min() < 0 or (int(ki.max()) + 1) * P > kv.shape[0])):
            raise ValueError("the page lists must lie in kv_indices and name pages inside kv")
        rc = lib.oracle_mla_decode_pages(ctypes.byref(prob), _p(q), _p(qs), _p(kv), _p(ks), _p(qo), _p(kvp), _p(ki),
                                         _p(kpp), P, _p(ids), n_seq, _p(out), _p(lse), int(threads))
    elif kv_indices is None:
        rc = lib.oracle_mla_decode(ctypes.byref(prob), _p(q), _p(qs), _p(kv), _p(ks), _p(qo), _p(kvp), _p(ids),
                                   n_seq, _p(out), _p(lse), int(threads))
    else:
        ki = np.ascontiguousarray(kv_indices, dtype=np.int32)
        if ki.shape[0] < int(kvp[-1]) or (ki.size and (ki.min() < 0 or ki.max() >= kv.shape[0])):
            raise ValueError("kv_indices must cover the CSR rows and index rows of kv")
        rc = lib.oracle_mla_decode_paged(ctypes.byref(prob), _p(q), _p(qs), _p(kv), _p(ks), _p(qo), _p(kvp), _p(ki),
                                         _p(ids), n_seq, _p(out), _p(lse), int(threads))
    if rc != 0:
        raise RuntimeError(f"oracle_mla_decode failed ({rc})")
    return out, lse


def decode_workload(w, seq_ids=None, threads=1, lib=None):
    """Oracle on a ``synth.Workload``."""
    return mla_decode(w.q, w.kv, w.qo_indptr, w.kv_indptr, q_dtype=w.q_dtype, kv_dtype=w.kv_dtype,
                      q_scale=w.q_scale, kv_scale=w.kv_scale, sm_scale=w.sm_scale, seq_ids=seq_ids,
                      threads=threads, lib=lib, logit_cap=getattr(w, "logit_cap", 0.0),
                      kv_indices=getattr(w, "kv_indices", None),
                      kv_page_indptr=getattr(w, "kv_page_indptr", None), page_size=getattr(w, "page_size", 1))

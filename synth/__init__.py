"""Seeded synthetic inputs for MLA decode (DeepSeek-R1 forward_absorb shapes).

This package only draws random numbers and encodes them into the storage
formats the decode path consumes.  It holds none of the attention arithmetic
and no decoder: the CPU oracle (``oracle``) and the GPU library
(``mla_decode_split_amd``) both read the bytes produced here, and neither
imports the other.

Shapes and formats follow the template page of the kernelbot-amd-mixed-mla
pages (docstring "Input tuple" / "Output"): q is (total_q, 16, 576), the KV
buffer is (total_kv, 1, 576) as bf16, as fp8 E4M3FN with one fp32 scale, or as
MXFP4 (total_kv, 1, 288) fp4x2 plus E8M0 scales; qo_indptr / kv_indptr are
int32 CSR offsets of length batch_size + 1.

Readings of points the pages leave open (each also listed in the design notes):
  * fp8 flavour is OCP E4M3FN (bias 7, max 448, no inf).
  * the per-tensor fp8 scale is amax / 448 computed in fp32 from a bf16 N(0,1)
    source; codes are round-to-nearest-even of clamp(x / scale, +-448).
  * MXFP4: element 2i sits in the low nibble of byte i, 2i+1 in the high
    nibble; scales are a row-major uint8 array [total_kv][18], one E8M0 byte per
    32 consecutive columns of the 576-wide row.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")

NUM_HEADS = 16
QK_DIM = 576
V_DIM = 512
SM_SCALE = 1.0 / (QK_DIM ** 0.5)

STREAM_Q = 1
STREAM_KV = 2
STREAM_LEN = 3

_lib = None


def build(force: bool = True) -> str:
    """Compile libsynth.so with gcc (host code only)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-std=c11", "-D_GNU_SOURCE", "-o", tmp, _SRC,
                               "-lm", "-lpthread"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        u64, i32, f32 = ctypes.c_uint64, ctypes.c_int, ctypes.c_float
        vp = ctypes.c_void_p
        lib.synth_normal_bf16.argtypes = [u64, u64, u64, vp, i32]
        lib.synth_amax_bf16.argtypes = [u64, u64, u64, i32]
        lib.synth_amax_bf16.restype = f32
        lib.synth_fp8_tensor.argtypes = [u64, u64, u64, vp, i32]
        lib.synth_fp8_tensor.restype = f32
        lib.synth_mxfp4_rows.argtypes = [u64, u64, u64, i32, vp, vp, i32]
        lib.synth_mxfp4_rows.restype = i32
        lib.synth_uniform_lengths.argtypes = [u64, u64, i32, i32, i32, vp]
        lib.synth_encode_e4m3fn_array.argtypes = [vp, u64, vp]
        lib.synth_encode_mxfp4_array.argtypes = [vp, u64, i32, vp, vp]
        lib.synth_bf16_from_f32.argtypes = [vp, u64, vp]
        lib.synth_stream_key.argtypes = [u64, u64]
        lib.synth_stream_key.restype = u64
        lib.synth_u64.argtypes = [u64, u64]
        lib.synth_u64.restype = u64
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


# ------------------------------------------------------------------ primitives

def normal_bf16(seed: int, stream: int, n: int, threads: int | None = None) -> np.ndarray:
    """n bf16 N(0,1) values as uint16 bit patterns."""
    out = np.empty(n, dtype=np.uint16)
    if n:
        _load().synth_normal_bf16(seed, stream, n, _ptr(out), threads or default_threads())
    return out


def fp8_tensor(seed: int, stream: int, n: int, threads: int | None = None) -> tuple[np.ndarray, np.float32]:
    """Per-tensor fp8 E4M3FN codes of n bf16 N(0,1) values, and the fp32 scale."""
    out = np.empty(n, dtype=np.uint8)
    scale = _load().synth_fp8_tensor(seed, stream, n, _ptr(out), threads or default_threads()) if n else 1.0
    return out, np.float32(scale)


def mxfp4_rows(seed: int, stream: int, rows: int, row_elems: int = QK_DIM,
               threads: int | None = None) -> tuple[np.ndarray, np.ndarray]:
    """MXFP4 rows of bf16 N(0,1) values: packed [rows, row_elems/2], scales [rows, row_elems/32]."""
    packed = np.empty((rows, row_elems // 2), dtype=np.uint8)
    scales = np.empty((rows, row_elems // 32), dtype=np.uint8)
    if rows:
        rc = _load().synth_mxfp4_rows(seed, stream, rows, row_elems, _ptr(packed), _ptr(scales),
                                      threads or default_threads())
        if rc != 0:
            raise ValueError("row_elems must be a multiple of 32")
    return packed, scales


def uniform_lengths(seed: int, stream: int, bs: int, lo: int, hi: int) -> np.ndarray:
    out = np.empty(bs, dtype=np.int32)
    if bs:
        _load().synth_uniform_lengths(seed, stream, bs, lo, hi, _ptr(out))
    return out


def encode_e4m3fn(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint8)
    _load().synth_encode_e4m3fn_array(_ptr(x), x.size, _ptr(out))
    return out


def encode_mxfp4(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """x: float array [rows, row_elems] -> (packed [rows, row_elems/2], scales [rows, row_elems/32])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, d = x.shape
    packed = np.empty((rows, d // 2), dtype=np.uint8)
    scales = np.empty((rows, d // 32), dtype=np.uint8)
    _load().synth_encode_mxfp4_array(_ptr(x), rows, d, _ptr(packed), _ptr(scales))
    return packed, scales


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 values -> bf16 bit patterns (round to nearest even)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().synth_bf16_from_f32(_ptr(x), x.size, _ptr(out))
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ------------------------------------------------------------------ workloads

@dataclass
class Workload:
    """One batch of decode inputs, host-side.  Byte arrays are ready to copy to
    the device; dtype names are "bf16", "fp8" (E4M3FN) or "mxfp4"."""
    name: str
    q_dtype: str
    kv_dtype: str
    q: np.ndarray                      # uint16 [total_q,16,576] (bf16) or uint8 (fp8)
    q_scale: np.float32 | None         # fp8 q only
    kv: np.ndarray                     # uint16 [total_kv,576] | uint8 [total_kv,576] | uint8 [total_kv,288]
    kv_scale: np.ndarray | np.float32 | None   # fp8: fp32 scalar; mxfp4: uint8 [total_kv,18]
    qo_indptr: np.ndarray
    kv_indptr: np.ndarray
    sm_scale: float = SM_SCALE
    meta: dict = field(default_factory=dict)
    logit_cap: float = 0.0             # > 0: scores soft-capped as cap * tanh(s / cap)
    kv_indices: np.ndarray | None = None  # paged KV (page size 1): CSR row j is kv[kv_indices[j]]
    kv_page_indptr: np.ndarray | None = None  # pages of page_size rows: sequence b's page list
    page_size: int = 1                         # starts at kv_indices[kv_page_indptr[b]]

    @property
    def batch_size(self) -> int:
        return int(self.kv_indptr.shape[0] - 1)

    @property
    def total_q(self) -> int:
        return int(self.q.shape[0])

    @property
    def total_kv(self) -> int:
        """Rows of the CSR space (of the KV buffer when not paged)."""
        if self.kv_page_indptr is not None:
            return int(self.kv_indptr[-1])
        return int(self.kv.shape[0]) if self.kv_indices is None else int(self.kv_indices.shape[0])

    @property
    def kv_rows(self) -> int:
        """Rows of the KV buffer."""
        return int(self.kv.shape[0])

    def kv_bytes(self) -> int:
        """Bytes of the KV cache the decode must read (rows of all sequences,
        plus MXFP4 scales)."""
        n = int(self.kv_indptr[-1] - self.kv_indptr[0])
        per_row = {"bf16": 2 * QK_DIM, "fp8": QK_DIM, "mxfp4": QK_DIM // 2 + QK_DIM // 32}[self.kv_dtype]
        return n * per_row


def make_batch(lengths, q_dtype: str, kv_dtype: str, seed: int, name: str = "custom",
               threads: int | None = None, q_lens=None) -> Workload:
    """Build a decode batch with the given KV lengths and query rows per
    sequence (``q_lens``, default one each; sequence b's rows are
    qo_indptr[b] .. qo_indptr[b+1] - 1).

    Every tensor starts from bf16 N(0,1) draws of its own stream; fp8 tensors
    are quantised per tensor (amax / 448) and MXFP4 per 32-element block."""
    lengths = np.asarray(lengths, dtype=np.int64)
    bs = int(lengths.shape[0])
    kv_indptr = np.zeros(bs + 1, dtype=np.int32)
    kv_indptr[1:] = np.cumsum(lengths).astype(np.int32)
    if q_lens is None:
        qo_indptr = np.arange(bs + 1, dtype=np.int32)
    else:
        q_lens = np.asarray(q_lens, dtype=np.int64)
        if q_lens.shape != (bs,) or (q_lens < 0).any():
            raise ValueError("q_lens: one non-negative count per sequence")
        qo_indptr = np.zeros(bs + 1, dtype=np.int32)
        qo_indptr[1:] = np.cumsum(q_lens).astype(np.int32)
    total_q = int(qo_indptr[-1])
    total_kv = int(kv_indptr[-1])
    nq = total_q * NUM_HEADS * QK_DIM
    q_scale = None
    if q_dtype == "bf16":
        q = normal_bf16(seed, STREAM_Q, nq, threads).reshape(total_q, NUM_HEADS, QK_DIM)
    elif q_dtype == "fp8":
        qc, q_scale = fp8_tensor(seed, STREAM_Q, nq, threads)
        q = qc.reshape(total_q, NUM_HEADS, QK_DIM)
    else:
        raise ValueError(q_dtype)
    if kv_dtype == "bf16":
        kv = normal_bf16(seed, STREAM_KV, total_kv * QK_DIM, threads).reshape(total_kv, QK_DIM)
        kv_scale = None
    elif kv_dtype == "fp8":
        kvc, kv_scale = fp8_tensor(seed, STREAM_KV, total_kv * QK_DIM, threads)
        kv = kvc.reshape(total_kv, QK_DIM)
    elif kv_dtype == "mxfp4":
        kv, kv_scale = mxfp4_rows(seed, STREAM_KV, total_kv, QK_DIM, threads)
    else:
        raise ValueError(kv_dtype)
    return Workload(name=name, q_dtype=q_dtype, kv_dtype=kv_dtype, q=q, q_scale=q_scale, kv=kv,
                    kv_scale=kv_scale, qo_indptr=qo_indptr, kv_indptr=kv_indptr,
                    meta={"seed": seed, "lengths": lengths, "q_lens": np.diff(qo_indptr)})


def encode_batch(q: np.ndarray, kv: np.ndarray, qo_indptr, kv_indptr, q_dtype: str, kv_dtype: str,
                 name: str = "encoded") -> Workload:
    """A batch from given values instead of draws: fp32 q [total_q, 16, 576] and
    kv [total_kv, 576] encoded into the storage formats the way make_batch
    encodes its draws - bf16 round to nearest even; fp8 per tensor with scale =
    fp32(amax) / 448 and codes RNE_E4M3(clamp(fp32(x / scale), +-448)); MXFP4
    per 32-element block (shared exponent floor(log2 amax) - 2)."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    kv = np.ascontiguousarray(kv, dtype=np.float32)
    qo = np.ascontiguousarray(qo_indptr, dtype=np.int32)
    ki = np.ascontiguousarray(kv_indptr, dtype=np.int32)

    def fp8(x):
        amax = np.float32(np.abs(x).max()) if x.size else np.float32(0)
        scale = np.float32(max(amax, np.float32(1e-12)) / np.float32(448.0))
        return encode_e4m3fn(np.clip(x / scale, -448.0, 448.0).astype(np.float32)), scale

    q_scale = kv_scale = None
    if q_dtype == "bf16":
        qc = bf16_bits(q)
    elif q_dtype == "fp8":
        qc, q_scale = fp8(q)
    else:
        raise ValueError(q_dtype)
    if kv_dtype == "bf16":
        kvc = bf16_bits(kv)
    elif kv_dtype == "fp8":
        kvc, kv_scale = fp8(kv)
    elif kv_dtype == "mxfp4":
        kvc, kv_scale = encode_mxfp4(kv)
    else:
        raise ValueError(kv_dtype)
    return Workload(name=name, q_dtype=q_dtype, kv_dtype=kv_dtype, q=qc.reshape(q.shape), q_scale=q_scale,
                    kv=kvc, kv_scale=kv_scale, qo_indptr=qo, kv_indptr=ki,
                    meta={"lengths": np.diff(ki), "q_lens": np.diff(qo)})


def page_workload(w: Workload, seed: int, spare_rows: int = 0, threads: int | None = None,
                  page_size: int = 1) -> Workload:
    """The same batch with its KV rows scattered over a larger buffer (paged
    KV).  Page size 1: a seeded random injective map sends CSR row j to
    physical row kv_indices[j] of a buffer of total_kv + spare_rows rows.
    Page size P > 1: each sequence's rows fill ceil(len / P) pages, drawn by a
    seeded random injective map from the buffer's pages (enough for the rows
    plus spare_rows); kv_indices holds the page lists back to back and
    kv_page_indptr[b] is where sequence b's begins.  Rows no sequence uses hold
    fresh draws of the same format, so a wrong index reads different data.
    Only MXFP4 scale rows move with their rows."""
    n = w.total_kv
    rng = np.random.default_rng(np.random.SeedSequence([seed, 0x9A6E]))
    kv_page_indptr = None
    if page_size == 1:
        rows = n + spare_rows
        kv_indices = rng.permutation(rows)[:n].astype(np.int32)
        dest = kv_indices.astype(np.int64)
    else:
        P = int(page_size)
        lens = np.diff(np.asarray(w.kv_indptr, dtype=np.int64))
        npages = (lens + P - 1) // P
        kv_page_indptr = np.concatenate([[0], np.cumsum(npages)]).astype(np.int32)
        total_pages = int(kv_page_indptr[-1])
        pages = total_pages + (spare_rows + P - 1) // P
        rows = pages * P
        kv_indices = rng.permutation(pages)[:total_pages].astype(np.int32)
        # destination of each CSR row: its page's first row plus its place in the page
        seq = np.repeat(np.arange(lens.shape[0]), lens)
        within = np.arange(n, dtype=np.int64) - np.asarray(w.kv_indptr, dtype=np.int64)[seq]
        dest = kv_indices[kv_page_indptr[seq] + within // P].astype(np.int64) * P + within % P
    filler = make_batch([rows], "bf16", w.kv_dtype, seed=seed + 1000003, threads=threads)
    kv = filler.kv.copy()
    kv[dest] = w.kv
    kv_scale = w.kv_scale
    if w.kv_dtype == "mxfp4":
        kv_scale = filler.kv_scale.copy()
        kv_scale[dest] = w.kv_scale
    elif w.kv_dtype == "fp8":
        # the filler was quantised with its own scale: re-encode nothing, the
        # per-tensor scale of the batch applies to every row of the buffer
        kv_scale = w.kv_scale
    out = Workload(name=w.name + "_paged", q_dtype=w.q_dtype, kv_dtype=w.kv_dtype, q=w.q, q_scale=w.q_scale, kv=kv,
                   kv_scale=kv_scale, qo_indptr=w.qo_indptr, kv_indptr=w.kv_indptr, sm_scale=w.sm_scale,
                   meta=dict(w.meta, paged_seed=seed, spare_rows=spare_rows, page_size=page_size),
                   logit_cap=w.logit_cap, kv_indices=kv_indices, kv_page_indptr=kv_page_indptr, page_size=page_size)
    return out


# The five decode workloads: (batch size, KV length or "ragged", q dtype, KV dtype, seed).
# The ragged batch draws each length uniformly from [1, 16384].
WORKLOADS = {
    "bs4_kv1024_bf16": dict(bs=4, kv_len=1024, q_dtype="bf16", kv_dtype="bf16", seed=1),
    "bs32_kv1024_fp8": dict(bs=32, kv_len=1024, q_dtype="bf16", kv_dtype="fp8", seed=2),
    "bs64_kv8192_fp8": dict(bs=64, kv_len=8192, q_dtype="bf16", kv_dtype="fp8", seed=3),
    "bs256_kv8192_a8w8": dict(bs=256, kv_len=8192, q_dtype="fp8", kv_dtype="fp8", seed=4),
    "bs128_ragged_mxfp4": dict(bs=128, kv_len="ragged", q_dtype="bf16", kv_dtype="mxfp4", seed=5),
}
RAGGED_MIN, RAGGED_MAX = 1, 16384


def workload_lengths(name: str) -> np.ndarray:
    spec = WORKLOADS[name]
    if spec["kv_len"] == "ragged":
        return uniform_lengths(spec["seed"], STREAM_LEN, spec["bs"], RAGGED_MIN, RAGGED_MAX)
    return np.full(spec["bs"], spec["kv_len"], dtype=np.int32)


def make_workload(name: str, threads: int | None = None, q_len: int = 1) -> Workload:
    """One of the named workloads; with q_len > 1 every sequence gets q_len
    query rows over the same KV (named ``<name>_q<q_len>``)."""
    spec = WORKLOADS[name]
    q_lens = None if q_len == 1 else [q_len] * spec["bs"]
    return make_batch(workload_lengths(name), spec["q_dtype"], spec["kv_dtype"], spec["seed"],
                      name=name if q_len == 1 else f"{name}_q{q_len}", threads=threads, q_lens=q_lens)

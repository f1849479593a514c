"""CPU oracle for paged MXFP4 index scoring -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product library
(``mxfp4_paged_cache_amd``) never imports it and shares no code with it.

Two independent implementations live here:

* ``mxs_oracle.c`` (plain C + OpenMP, exact arithmetic, one final fp32
  rounding), loaded through ctypes by :func:`score` and the element helpers;
* ``brute.py`` (pure Python with ``fractions.Fraction``), for tiny inputs,
  used to cross-check the C oracle.

What both compute follows the pages: MXFP4 values are e2m1 x 2^(byte-127)
with one e8m0 byte per 32 elements (aiter #7061, "Format"); a bf16 query is
rounded to e4m3 with round-to-nearest-even and saturation, an e4m3 query is
used as stored (aiter #7061, "Kernels"); the logit is sm_scale times the dot,
the block score the maximum over a page's live tokens (aiter #7061, "Format").
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmxs_oracle.so")
_SRC = os.path.join(_HERE, "mxs_oracle.c")

MXO_Q_BF16 = 1
MXO_Q_E4M3 = 2
MXO_K_MXFP4 = 0
MXO_K_E4M3 = 1
MXO_MODE_PREFILL = 0
MXO_MODE_DECODE = 1


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (no GPU involved)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall", "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd, cwd=_HERE)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Args(ctypes.Structure):
    _fields_ = [
        ("mode", ctypes.c_int),
        ("q_dtype", ctypes.c_int),
        ("q", ctypes.c_void_p),
        ("q_row_stride", ctypes.c_int64),
        ("q_head_stride", ctypes.c_int64),
        ("num_heads", ctypes.c_int),
        ("k_data", ctypes.c_void_p),
        ("data_page_stride", ctypes.c_int64),
        ("k_scale", ctypes.c_void_p),
        ("scale_page_stride", ctypes.c_int64),
        ("page_size", ctypes.c_int),
        ("num_pages", ctypes.c_int64),
        ("block_table", ctypes.c_void_p),
        ("bt_row_stride", ctypes.c_int64),
        ("bt_width", ctypes.c_int),
        ("cu_seqlens_q", ctypes.c_void_p),
        ("seq_lens", ctypes.c_void_p),
        ("prefix_lens", ctypes.c_void_p),
        ("batch", ctypes.c_int),
        ("max_seq_len", ctypes.c_int),
        ("sm_scale", ctypes.c_float),
        ("rows", ctypes.c_void_p),
        ("num_rows", ctypes.c_int),
        ("num_threads", ctypes.c_int),
        ("k_dtype", ctypes.c_int),
    ]


_lib = None


def lib():
    global _lib
    if _lib is None:
        path = _LIB_PATH if os.path.exists(_LIB_PATH) else build()
        L = ctypes.CDLL(path)
        L.mxo_e2m1_value.restype = ctypes.c_double
        L.mxo_e2m1_value.argtypes = [ctypes.c_int]
        L.mxo_e8m0_value.restype = ctypes.c_double
        L.mxo_e8m0_value.argtypes = [ctypes.c_int]
        L.mxo_e4m3_value.restype = ctypes.c_double
        L.mxo_e4m3_value.argtypes = [ctypes.c_int]
        L.mxo_bf16_to_e4m3.restype = ctypes.c_int
        L.mxo_bf16_to_e4m3.argtypes = [ctypes.c_int]
        L.mxo_round_scaled_sum.restype = ctypes.c_float
        L.mxo_round_scaled_sum.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int), ctypes.c_float]
        L.mxo_round_scaled_terms.restype = ctypes.c_float
        L.mxo_round_scaled_terms.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int), ctypes.c_int,
                                             ctypes.c_int, ctypes.c_float]
        L.mxo_score.restype = ctypes.c_int
        L.mxo_score.argtypes = [ctypes.POINTER(_Args), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.mxo_score_ex.restype = ctypes.c_int
        L.mxo_score_ex.argtypes = [ctypes.POINTER(_Args), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_void_p]
        L.mxo_total_rows.restype = ctypes.c_int
        L.mxo_total_rows.argtypes = [ctypes.POINTER(_Args)]
        _lib = L
    return _lib


# ----------------------------------------------------------------- elements

def e2m1_value(code: int) -> float:
    return lib().mxo_e2m1_value(int(code))


def e8m0_value(byte: int) -> float:
    return lib().mxo_e8m0_value(int(byte))


def e4m3_value(byte: int) -> float:
    return lib().mxo_e4m3_value(int(byte))


def bf16_to_e4m3(bits: int) -> int:
    return lib().mxo_bf16_to_e4m3(int(bits))


def bf16_to_e4m3_table() -> np.ndarray:
    """e4m3 byte for each of the 65536 bf16 bit patterns."""
    L = lib()
    return np.array([L.mxo_bf16_to_e4m3(b) for b in range(65536)], dtype=np.uint8)


def round_scaled_terms(S, ex, frac_bits: int, sm_scale: float) -> float:
    n = len(S)
    Sa = (ctypes.c_double * n)(*[float(x) for x in S])
    ea = (ctypes.c_int * n)(*[int(x) for x in ex])
    return lib().mxo_round_scaled_terms(Sa, ea, n, frac_bits, ctypes.c_float(sm_scale))


def round_scaled_sum(S, s, sm_scale: float) -> float:
    Sa = (ctypes.c_double * 4)(*[float(x) for x in S])
    sa = (ctypes.c_int * 4)(*[int(x) for x in s])
    return lib().mxo_round_scaled_sum(Sa, sa, ctypes.c_float(sm_scale))


# ----------------------------------------------------------------- scoring

@dataclass
class Result:
    logits: Optional[np.ndarray]   # [R, H, max_seq_len] fp32, -inf outside the live window
    blocks: Optional[np.ndarray]   # [R, H, NB] fp32
    mags: Optional[np.ndarray]     # [R, H, max_seq_len] float64: sum |Q_hat * K| (no sm_scale)
    rows: np.ndarray               # the query rows these outputs belong to
    block_mags: Optional[np.ndarray] = None   # [R, H, NB] float64: largest mags among a page's live tokens


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def score(*, mode: str, q: np.ndarray, q_dtype: str, k_data: np.ndarray, k_scale: Optional[np.ndarray],
          page_size: int, block_table: np.ndarray, seq_lens: np.ndarray, max_seq_len: int,
          sm_scale: float, cu_seqlens_q: Optional[np.ndarray] = None,
          prefix_lens: Optional[np.ndarray] = None, rows: Optional[np.ndarray] = None,
          want_logits: bool = True, want_blocks: bool = True, want_mags: bool = False,
          want_block_mags: bool = False,
          data_page_stride: Optional[int] = None, scale_page_stride: Optional[int] = None,
          num_pages: Optional[int] = None, num_threads: int = 0, k_dtype: str = "mxfp4") -> Result:
    """Run the C oracle on host arrays.

    ``q``: uint16 bf16 bits or uint8 e4m3 bytes, shape [rows, H, 128] with any
    element strides; ``k_data``/``k_scale``: uint8 arrays whose first axis is the
    page (page strides taken from the arrays unless given, in bytes).
    ``k_dtype``: "mxfp4" (e2m1 data [pages, P, 64] + e8m0 scales [pages, P, 4])
    or "e4m3" (data [pages, P, 128] of e4m3 bytes, unit scale; k_scale None).
    """
    if k_dtype not in ("mxfp4", "e4m3"):
        raise ValueError(k_dtype)
    q = np.asarray(q)
    if q_dtype == "bf16":
        assert q.dtype == np.uint16
        qd = MXO_Q_BF16
    elif q_dtype == "e4m3":
        assert q.dtype == np.uint8
        qd = MXO_Q_E4M3
    else:
        raise ValueError(q_dtype)
    assert q.ndim == 3 and q.shape[2] == 128 and (q.size == 0 or q.strides[2] == q.itemsize)
    H = q.shape[1]
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    B = sl.shape[0]
    a = _Args()
    a.mode = MXO_MODE_DECODE if mode == "decode" else MXO_MODE_PREFILL
    a.q_dtype = qd
    a.q = q.ctypes.data
    a.q_row_stride = q.strides[0] // q.itemsize
    a.q_head_stride = q.strides[1] // q.itemsize
    a.num_heads = H
    a.k_data = k_data.ctypes.data
    a.data_page_stride = data_page_stride if data_page_stride is not None else k_data.strides[0]
    a.k_dtype = MXO_K_E4M3 if k_dtype == "e4m3" else MXO_K_MXFP4
    if k_dtype == "mxfp4":
        a.k_scale = k_scale.ctypes.data
        a.scale_page_stride = scale_page_stride if scale_page_stride is not None else k_scale.strides[0]
    a.page_size = page_size
    a.num_pages = num_pages if num_pages is not None else k_data.shape[0]
    a.block_table = bt.ctypes.data
    a.bt_row_stride = bt.shape[1] if bt.ndim == 2 else 0
    a.bt_width = bt.shape[1]
    keep = [q, bt, sl, k_data, k_scale]
    if a.mode == MXO_MODE_PREFILL:
        cu = np.ascontiguousarray(cu_seqlens_q, dtype=np.int32)
        pl = np.ascontiguousarray(prefix_lens, dtype=np.int32)
        keep += [cu, pl]
        a.cu_seqlens_q = cu.ctypes.data
        a.prefix_lens = pl.ctypes.data
    a.seq_lens = sl.ctypes.data
    a.batch = B
    a.max_seq_len = max_seq_len
    a.sm_scale = sm_scale
    a.num_threads = num_threads
    T = lib().mxo_total_rows(ctypes.byref(a))
    if rows is None:
        rows_arr = np.arange(T, dtype=np.int32)
        a.rows = None
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int32)
        a.rows = rows_arr.ctypes.data
        a.num_rows = rows_arr.shape[0]
    R = rows_arr.shape[0]
    NB = (max_seq_len + page_size - 1) // page_size
    lg = np.empty((R, H, max_seq_len), np.float32) if want_logits else None
    bl = np.empty((R, H, NB), np.float32) if want_blocks else None
    mg = np.empty((R, H, max_seq_len), np.float64) if want_mags else None
    bm = np.empty((R, H, NB), np.float64) if want_block_mags else None
    rc = lib().mxo_score_ex(ctypes.byref(a), _ptr(lg), _ptr(bl), _ptr(mg), _ptr(bm))
    del keep
    if rc != 0:
        raise ValueError(f"oracle rejected the inputs (code {rc})")
    return Result(lg, bl, mg, rows_arr, bm)

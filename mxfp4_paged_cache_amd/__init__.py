"""Paged MXFP4 index scorer for MI355X (gfx950): Python binding of libmxscore.

Argument marshalling only: every step of the scoring runs in the HIP kernels
of ``libmxscore.so`` (C ABI in ``include/mxscore.h``). PyTorch supplies device
memory and the current stream. There is no CPU fallback: if the library is
missing or the device is not gfx950 the calls raise.

Entry points mirror the C ABI (aiter #7061, "Kernels"; ATOM #2770, "How it
works"; aiter #5518, "Summary"):

* :func:`score_prefill` -- per-page max block scores (and optionally logits)
  for request-concatenated query rows with causal + prefix masking;
* :func:`score_decode` -- one query row per request, limit = seq_len;
* :func:`score_logits` -- logits-first variant of prefill;
* :func:`select_pages` -- top-k pages per (row, head) from block scores;
* :func:`write_pages` -- quantize bf16 keys into their page slots;
* :func:`check_metadata` -- synchronous check of the device-side contract;
* :func:`attn_decode` -- paged MXFP4 attention decode over K and V caches.

The cache is an MXFP4 one (``k_data`` [pages, P, 64] e2m1 bytes and
``k_scale`` [pages, P, 4] e8m0 bytes) or, with ``k_scale=None``, an fp8 one
(``k_data`` [pages, P, 128] e4m3 bytes, unit scale: the format the MXFP4
cache replaces, aiter #7061, "Summary").

Rejected inputs raise ``ValueError`` before anything is launched.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

__all__ = ["score_prefill", "score_decode", "score_logits", "select_pages", "write_pages", "check_metadata",
           "attn_decode", "make_plan", "library_path", "lib", "MxsError"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmxscore.so")

MXS_OK, MXS_EINVAL, MXS_EDTYPE, MXS_ELAYOUT, MXS_EUNSUPPORTED, MXS_EDEVICE = 0, -1, -2, -3, -4, -5
MXS_Q_BF16, MXS_Q_E4M3 = 1, 2
MXS_K_MXFP4, MXS_K_E4M3 = 0, 1
MXS_MODE_PREFILL, MXS_MODE_DECODE, MXS_MODE_LOGITS = 1, 2, 3


class MxsError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"mxscore error {code}: {msg}")
        self.code = code


class Query(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("row_stride", ctypes.c_int64),
                ("head_stride", ctypes.c_int64), ("num_heads", ctypes.c_int32)]


class KCache(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("data_page_stride", ctypes.c_int64), ("scale", ctypes.c_void_p),
                ("scale_page_stride", ctypes.c_int64), ("page_size", ctypes.c_int32), ("k_dtype", ctypes.c_int32),
                ("num_pages", ctypes.c_int64)]


class KVView(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("data_page_stride", ctypes.c_int64), ("data_head_stride", ctypes.c_int64),
                ("scale", ctypes.c_void_p), ("scale_page_stride", ctypes.c_int64),
                ("scale_head_stride", ctypes.c_int64)]


class KVCache(ctypes.Structure):
    _fields_ = [("k", KVView), ("v", KVView), ("page_size", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("num_pages", ctypes.c_int64)]


class Out(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("row_stride", ctypes.c_int64), ("head_stride", ctypes.c_int64)]


class Batch(ctypes.Structure):
    _fields_ = [("block_table", ctypes.c_void_p), ("bt_row_stride", ctypes.c_int64), ("bt_width", ctypes.c_int32),
                ("cu_seqlens_q", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p), ("prefix_lens", ctypes.c_void_p),
                ("batch", ctypes.c_int32), ("total_rows", ctypes.c_int32), ("max_query_len", ctypes.c_int32),
                ("max_seq_len", ctypes.c_int32)]


class Plan(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "mode", "q_dtype", "page_size", "num_heads", "batch", "max_query_len", "max_seq_len", "want_logits",
        "want_blocks", "grid", "block", "slots_per_item", "pages_per_item", "slot_items", "page_items",
        "head_groups")] + [("items", ctypes.c_int64), ("kernel", ctypes.c_int32), ("k_dtype", ctypes.c_int32),
                           ("xcd_split", ctypes.c_int32)]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


_lib = None
SYMBOLS = ("mxs_plan_make", "mxs_plan_make_for", "mxs_score_prefill", "mxs_score_decode", "mxs_score_logits",
           "mxs_write_pages", "mxs_select_pages", "mxs_check_metadata", "mxs_attn_decode", "mxs_last_error",
           "mxs_version")


def library_path() -> str:
    return _LIB_PATH


def lib():
    """Load libmxscore.so (built by ``mxfp4_paged_cache_amd/build.py``); raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with `python mxfp4_paged_cache_amd/build.py`")
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.POINTER
        i32 = ctypes.c_int32
        L.mxs_plan_make.argtypes = [i32] * 11 + [P(Plan)]
        L.mxs_plan_make.restype = ctypes.c_int
        L.mxs_plan_make_for.argtypes = [i32] * 13 + [P(Plan)]
        L.mxs_plan_make_for.restype = ctypes.c_int
        for name in ("mxs_score_prefill", "mxs_score_decode", "mxs_score_logits"):
            f = getattr(L, name)
            f.argtypes = [P(Query), P(KCache), P(Batch), ctypes.c_float, P(Out), P(Out), P(Plan), ctypes.c_void_p]
            f.restype = ctypes.c_int
        i64 = ctypes.c_int64
        L.mxs_select_pages.argtypes = [i32, P(Batch), i32, i32, ctypes.c_void_p, i64, i64, i32, ctypes.c_void_p, i64,
                                       i64, ctypes.c_void_p]
        L.mxs_select_pages.restype = ctypes.c_int
        L.mxs_write_pages.argtypes = [ctypes.c_void_p, i64, i64, ctypes.c_void_p, P(KCache), ctypes.c_void_p]
        L.mxs_write_pages.restype = ctypes.c_int
        L.mxs_check_metadata.argtypes = [i32, P(KCache), P(Batch), i32, ctypes.c_void_p]
        L.mxs_check_metadata.restype = ctypes.c_int
        L.mxs_attn_decode.argtypes = [P(Query), P(KVCache), ctypes.c_void_p, i64, i32, ctypes.c_void_p, i32, i32,
                                      ctypes.c_float, ctypes.c_void_p, i64, i64, ctypes.c_void_p]
        L.mxs_attn_decode.restype = ctypes.c_int
        L.mxs_last_error.restype = ctypes.c_char_p
        L.mxs_last_error.argtypes = []
        L.mxs_version.restype = ctypes.c_char_p
        L.mxs_version.argtypes = []
        _lib = L
    return _lib


def _check(rc: int):
    if rc == MXS_OK:
        return
    msg = lib().mxs_last_error().decode()
    if rc in (MXS_EINVAL, MXS_EDTYPE, MXS_ELAYOUT):
        raise ValueError(msg)
    raise MxsError(rc, msg)


# ------------------------------------------------------------------ marshalling

_E4M3_DTYPES = tuple(d for d in (getattr(torch, "float8_e4m3fn", None), torch.uint8) if d is not None)
_DATA_DTYPES = tuple(d for d in (torch.uint8, getattr(torch, "float4_e2m1fn_x2", None)) if d is not None)
_SCALE_DTYPES = tuple(d for d in (torch.uint8, getattr(torch, "float8_e8m0fnu", None)) if d is not None)


def _query(q: torch.Tensor) -> Query:
    if not isinstance(q, torch.Tensor) or q.dim() != 3 or q.shape[2] != 128:
        raise ValueError(f"query must be a [rows, heads, 128] tensor, got {tuple(getattr(q, 'shape', ()))}")
    if q.dtype == torch.bfloat16:
        dt = MXS_Q_BF16
    elif q.dtype in _E4M3_DTYPES:
        dt = MXS_Q_E4M3
    else:
        raise ValueError(f"query dtype must be bfloat16 or float8_e4m3fn, got {q.dtype} (fp16 is refused)")
    if q.numel() > 0 and q.stride(2) != 1:     # an empty tensor's strides carry no layout
        raise ValueError("query head_dim must be contiguous")
    return Query(q.data_ptr(), dt, q.stride(0), q.stride(1), q.shape[1])


def _kcache(k_data: torch.Tensor, k_scale: Optional[torch.Tensor]) -> KCache:
    if k_scale is None:
        # fp8 index cache: [pages, page_size, 128] e4m3 bytes, unit scale, no scale view
        if k_data.dtype not in _E4M3_DTYPES:
            raise ValueError(f"an fp8 cache view must be float8_e4m3fn or uint8, got {k_data.dtype}")
        if k_data.dim() != 3 or k_data.shape[2] != 128:
            raise ValueError(f"an fp8 cache view must be [pages, page_size, 128], got {tuple(k_data.shape)}")
        if k_data.stride(2) != 1 or k_data.stride(1) != 128:
            raise ValueError("cache token rows must be contiguous (128 B of e4m3 per token)")
        P = k_data.shape[1]
        if P not in (64, 128):
            raise ValueError(f"page size must be 64 or 128, got {P}")
        return KCache(data=k_data.data_ptr(), data_page_stride=k_data.stride(0), scale=None, scale_page_stride=0,
                      page_size=P, k_dtype=MXS_K_E4M3, num_pages=k_data.shape[0])
    if k_data.dtype not in _DATA_DTYPES or k_scale.dtype not in _SCALE_DTYPES:
        raise ValueError(f"cache views must be uint8 (or fp4x2 / e8m0) tensors, got {k_data.dtype} / {k_scale.dtype}")
    if k_data.dim() != 3 or k_scale.dim() != 3:
        raise ValueError("cache views must be [pages, page_size, 64] and [pages, page_size, 4]")
    P = k_data.shape[1]
    if k_data.shape[2] != 64 or k_scale.shape[2] != 4 or k_scale.shape[1] != P:
        raise ValueError(f"narrow cache views: data {tuple(k_data.shape)}, scale {tuple(k_scale.shape)}")
    if k_data.stride(2) != 1 or k_data.stride(1) != 64 or k_scale.stride(2) != 1 or k_scale.stride(1) != 4:
        raise ValueError("cache token rows must be contiguous (64 B of data, 4 B of scales per token)")
    if k_data.shape[0] != k_scale.shape[0]:
        raise ValueError(f"data and scale views hold different page counts ({k_data.shape[0]} vs {k_scale.shape[0]})")
    if P not in (64, 128):
        raise ValueError(f"page size must be 64 or 128, got {P}")
    return KCache(data=k_data.data_ptr(), data_page_stride=k_data.stride(0), scale=k_scale.data_ptr(),
                  scale_page_stride=k_scale.stride(0), page_size=P, k_dtype=MXS_K_MXFP4, num_pages=k_data.shape[0])


def _int_vec(name: str, t: Optional[torch.Tensor], n: int) -> int:
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != torch.int32 or t.dim() != 1 or t.shape[0] < n:
        raise ValueError(f"{name} must be an int32 vector of at least {n} entries")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _table(block_table: torch.Tensor) -> Tuple[int, int, int]:
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or (
            block_table.numel() > 0 and block_table.stride(1) != 1):
        raise ValueError("block_table must be an int32 [batch, width] tensor with contiguous rows")
    return block_table.data_ptr(), block_table.stride(0), block_table.shape[1]


def _same_device(*ts):
    devs = {t.device for t in ts if t is not None}
    if len(devs) != 1:
        raise ValueError(f"all tensors must be on one device, got {sorted(str(d) for d in devs)}")
    d = devs.pop()
    if d.type != "cuda":
        raise ValueError(f"tensors must be on a GPU, got {d}")
    return d


def _out(t: Optional[torch.Tensor], rows: int, H: int, width: int, name: str) -> Out:
    if t is None:
        return Out(None, 0, 0)
    if t.dtype != torch.float32 or t.dim() != 3 or tuple(t.shape) != (rows, H, width) or (width > 0 and t.stride(2) != 1):
        raise ValueError(f"{name} must be float32 [{rows}, {H}, {width}] with a contiguous last axis, got "
                         f"{t.dtype} {tuple(t.shape)}")
    return Out(t.data_ptr(), t.stride(0), t.stride(1))


def _stream(device, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def make_plan(mode: str, q_dtype: torch.dtype, page_size: int, num_heads: int, batch: int, max_query_len: int,
              max_seq_len: int, want_logits: bool, want_blocks: bool = True, parallel_unit_num: int = 0,
              k_dtype: str = "mxfp4") -> Plan:
    """Launch plan for the current device (pure function of these host
    integers). k_dtype: "mxfp4" (e2m1 + e8m0 views) or "e4m3" (fp8 cache)."""
    m = {"prefill": MXS_MODE_PREFILL, "decode": MXS_MODE_DECODE, "logits": MXS_MODE_LOGITS}[mode]
    dt = MXS_Q_BF16 if q_dtype == torch.bfloat16 else MXS_Q_E4M3
    kd = {"mxfp4": MXS_K_MXFP4, "e4m3": MXS_K_E4M3}[k_dtype]
    p = Plan()
    _check(lib().mxs_plan_make(m, dt, kd, page_size, num_heads, batch, max_query_len, max_seq_len, int(want_logits),
                               int(want_blocks), parallel_unit_num, ctypes.byref(p)))
    return p


def _prefill_like(mode, q, k_data, k_scale, block_table, cu_seqlens_q, seq_lens, prefix_lens, max_query_len,
                  max_seq_len, sm_scale, block_scores, logits, want_blocks, want_logits, plan, stream):
    dev = _same_device(q, k_data, k_scale, block_table, cu_seqlens_q, seq_lens, prefix_lens, block_scores, logits)
    qd = _query(q)
    kc = _kcache(k_data, k_scale)
    B = seq_lens.shape[0] if isinstance(seq_lens, torch.Tensor) else 0
    T = q.shape[0]
    H = q.shape[1]
    P = kc.page_size
    NB = (max_seq_len + P - 1) // P
    btp, bts, btw = _table(block_table)
    if block_table.shape[0] < B:
        raise ValueError("block_table has fewer rows than requests")
    ba = Batch(btp, bts, btw, _int_vec("cu_seqlens_q", cu_seqlens_q, B + 1), _int_vec("seq_lens", seq_lens, B),
               _int_vec("prefix_lens", prefix_lens, B), B, T, int(max_query_len), int(max_seq_len))
    if want_blocks and block_scores is None:
        block_scores = torch.empty((T, H, NB), dtype=torch.float32, device=dev)
    if want_logits and logits is None:
        logits = torch.empty((T, H, max_seq_len), dtype=torch.float32, device=dev)
    bo = _out(block_scores, T, H, NB, "block_scores")
    lo = _out(logits, T, H, max_seq_len, "logits")
    fn = lib().mxs_score_logits if mode == "logits" else lib().mxs_score_prefill
    a, b = (lo, bo) if mode == "logits" else (bo, lo)
    with torch.cuda.device(dev):
        _check(fn(ctypes.byref(qd), ctypes.byref(kc), ctypes.byref(ba), ctypes.c_float(sm_scale), ctypes.byref(a),
                  ctypes.byref(b), ctypes.byref(plan) if plan is not None else None, _stream(dev, stream)))
    return block_scores, logits


def score_prefill(q, k_data, k_scale, block_table, cu_seqlens_q, seq_lens, prefix_lens, max_query_len: int,
                  max_seq_len: int, sm_scale: float, out: Optional[torch.Tensor] = None, logits=False,
                  plan: Optional[Plan] = None, stream=None):
    """Block scores [T, H, ceil(max_seq_len/P)] (and logits [T, H, max_seq_len] when
    ``logits`` is True or a tensor). Returns ``block_scores`` or ``(block_scores, logits)``."""
    want_lg = logits is not False and logits is not None
    lg_t = logits if isinstance(logits, torch.Tensor) else None
    bs, lg = _prefill_like("prefill", q, k_data, k_scale, block_table, cu_seqlens_q, seq_lens, prefix_lens,
                           max_query_len, max_seq_len, sm_scale, out, lg_t, True, want_lg, plan, stream)
    return (bs, lg) if want_lg else bs


def score_logits(q, k_data, k_scale, block_table, cu_seqlens_q, seq_lens, prefix_lens, max_query_len: int,
                 max_seq_len: int, sm_scale: float, out: Optional[torch.Tensor] = None, block_scores=False,
                 plan: Optional[Plan] = None, stream=None):
    """Logits [T, H, max_seq_len] (and block scores when ``block_scores`` is True or a tensor)."""
    want_bs = block_scores is not False and block_scores is not None
    bs_t = block_scores if isinstance(block_scores, torch.Tensor) else None
    bs, lg = _prefill_like("logits", q, k_data, k_scale, block_table, cu_seqlens_q, seq_lens, prefix_lens,
                           max_query_len, max_seq_len, sm_scale, bs_t, out, want_bs, True, plan, stream)
    return (lg, bs) if want_bs else lg


def score_decode(q, k_data, k_scale, block_table, seq_lens, max_seq_len: int, sm_scale: float,
                 out: Optional[torch.Tensor] = None, logits=False, plan: Optional[Plan] = None, stream=None):
    """Decode block scores [B, H, ceil(max_seq_len/P)] for one query row per request."""
    dev = _same_device(q, k_data, k_scale, block_table, seq_lens, out, logits if isinstance(logits, torch.Tensor) else None)
    qd = _query(q)
    kc = _kcache(k_data, k_scale)
    B = q.shape[0]
    H = q.shape[1]
    P = kc.page_size
    NB = (max_seq_len + P - 1) // P
    btp, bts, btw = _table(block_table)
    if block_table.shape[0] < B:
        raise ValueError("block_table has fewer rows than requests")
    ba = Batch(btp, bts, btw, None, _int_vec("seq_lens", seq_lens, B), None, B, B, 1, int(max_seq_len))
    if out is None:
        out = torch.empty((B, H, NB), dtype=torch.float32, device=dev)
    want_lg = logits is not False and logits is not None
    lg = logits if isinstance(logits, torch.Tensor) else (
        torch.empty((B, H, max_seq_len), dtype=torch.float32, device=dev) if want_lg else None)
    bo = _out(out, B, H, NB, "block_scores")
    lo = _out(lg, B, H, max_seq_len, "logits")
    with torch.cuda.device(dev):
        _check(lib().mxs_score_decode(ctypes.byref(qd), ctypes.byref(kc), ctypes.byref(ba), ctypes.c_float(sm_scale),
                                      ctypes.byref(bo), ctypes.byref(lo),
                                      ctypes.byref(plan) if plan is not None else None, _stream(dev, stream)))
    return (out, lg) if want_lg else out


def check_metadata(mode: str, k_data, k_scale, block_table, seq_lens, max_seq_len: int, cu_seqlens_q=None,
                   prefix_lens=None, max_query_len: int = 0, check_scales: bool = False, stream=None) -> None:
    """Synchronous host check of the device-side contract (request metadata,
    live block-table entries, optionally live e8m0 bytes); raises ValueError
    naming the first violation. For tests and debugging, not the hot path."""
    m = {"prefill": MXS_MODE_PREFILL, "decode": MXS_MODE_DECODE, "logits": MXS_MODE_LOGITS}[mode]
    dev = _same_device(k_data, k_scale, block_table, seq_lens, cu_seqlens_q, prefix_lens)
    kc = _kcache(k_data, k_scale)
    B = seq_lens.shape[0]
    btp, bts, btw = _table(block_table)
    if m == MXS_MODE_DECODE:
        ba = Batch(btp, bts, btw, None, _int_vec("seq_lens", seq_lens, B), None, B, B, 1, int(max_seq_len))
    else:
        total = int(cu_seqlens_q[-1].item()) if B > 0 else 0
        ba = Batch(btp, bts, btw, _int_vec("cu_seqlens_q", cu_seqlens_q, B + 1), _int_vec("seq_lens", seq_lens, B),
                   _int_vec("prefix_lens", prefix_lens, B), B, total, int(max_query_len), int(max_seq_len))
    with torch.cuda.device(dev):
        _check(lib().mxs_check_metadata(m, ctypes.byref(kc), ctypes.byref(ba), int(bool(check_scales)),
                                        _stream(dev, stream)))


def select_pages(block_scores: torch.Tensor, k: int, seq_lens, max_seq_len: int, page_size: int, cu_seqlens_q=None,
                 prefix_lens=None, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Top-k pages per (row, head) of block scores [rows, H, NB]: the tail page
    plus the best other live pages (ties to the lower index), ascending, -1
    padded -> int32 [rows, H, k]. Decode rows (one per request) when
    cu_seqlens_q is None, else prefill rows."""
    dev = _same_device(block_scores, seq_lens, cu_seqlens_q, prefix_lens, out)
    if block_scores.dtype != torch.float32 or block_scores.dim() != 3 or (
            block_scores.numel() > 0 and block_scores.stride(2) != 1):
        raise ValueError("block_scores must be float32 [rows, H, NB] with unit page stride")
    R, H, NB = block_scores.shape
    if NB * page_size < max_seq_len:
        raise ValueError("block_scores is narrower than ceil(max_seq_len / page_size) pages")
    B = seq_lens.shape[0]
    if cu_seqlens_q is None:
        mode = MXS_MODE_DECODE
        if R != B:
            raise ValueError("decode selection needs one block-score row per request")
        ba = Batch(None, 0, 0, None, _int_vec("seq_lens", seq_lens, B), None, B, B, 1, int(max_seq_len))
    else:
        mode = MXS_MODE_PREFILL
        ba = Batch(None, 0, 0, _int_vec("cu_seqlens_q", cu_seqlens_q, B + 1), _int_vec("seq_lens", seq_lens, B),
                   _int_vec("prefix_lens", prefix_lens, B), B, R, 0, int(max_seq_len))
    if out is None:
        out = torch.empty((R, H, k), dtype=torch.int32, device=dev)
    if out.dtype != torch.int32 or tuple(out.shape) != (R, H, k) or (k > 0 and out.stride(2) != 1):
        raise ValueError(f"out must be int32 [{R}, {H}, {k}] with unit stride along k")
    with torch.cuda.device(dev):
        _check(lib().mxs_select_pages(mode, ctypes.byref(ba), H, page_size, block_scores.data_ptr(),
                                      block_scores.stride(0), block_scores.stride(1), int(k), out.data_ptr(),
                                      out.stride(0), out.stride(1), _stream(dev, stream)))
    return out


def write_pages(k: torch.Tensor, slot_mapping: torch.Tensor, k_data, k_scale, stream=None) -> None:
    """Quantize bf16 keys k [N, 128] into MXFP4 page slots (slot = page * P +
    offset, -1 skips): 64 e2m1 data bytes and 4 e8m0 scale bytes per token,
    OCP MX conversion; with k_scale None, into an fp8 cache (128 e4m3 bytes
    per token, nearest even, saturating). Writes the cache views in place."""
    dev = _same_device(k, slot_mapping, k_data, k_scale)
    if k.dtype != torch.bfloat16 or k.dim() != 2 or k.shape[1] != 128 or (k.numel() > 0 and k.stride(1) != 1):
        raise ValueError("k must be bf16 [N, 128] with contiguous head_dim")
    if slot_mapping.dtype != torch.int64 or slot_mapping.dim() != 1 or not slot_mapping.is_contiguous():
        raise ValueError("slot_mapping must be a contiguous int64 vector")
    if slot_mapping.shape[0] != k.shape[0]:
        raise ValueError("slot_mapping needs one entry per key row")
    kc = _kcache(k_data, k_scale)
    with torch.cuda.device(dev):
        _check(lib().mxs_write_pages(k.data_ptr(), k.stride(0), k.shape[0], slot_mapping.data_ptr(), ctypes.byref(kc),
                                     _stream(dev, stream)))


def _kvview(data: torch.Tensor, scale: torch.Tensor, name: str) -> Tuple[KVView, Tuple[int, int, int]]:
    """[pages, kv_heads, P, 64] e2m1 bytes + [pages, kv_heads, P, 4] e8m0 bytes."""
    if data.dtype not in _DATA_DTYPES or scale.dtype not in _SCALE_DTYPES:
        raise ValueError(f"{name} views must be uint8 (or fp4x2 / e8m0) tensors")
    if data.dim() != 4 or scale.dim() != 4 or data.shape[3] != 64 or scale.shape[3] != 4 or \
            tuple(data.shape[:3]) != tuple(scale.shape[:3]):
        raise ValueError(f"{name} views must be [pages, kv_heads, P, 64] and [pages, kv_heads, P, 4], got "
                         f"{tuple(data.shape)} / {tuple(scale.shape)}")
    if data.stride(3) != 1 or data.stride(2) != 64 or scale.stride(3) != 1 or scale.stride(2) != 4:
        raise ValueError(f"{name} token rows must be contiguous (64 B of data, 4 B of scales per token)")
    return (KVView(data.data_ptr(), data.stride(0), data.stride(1), scale.data_ptr(), scale.stride(0), scale.stride(1)),
            tuple(data.shape[:3]))


def attn_decode(q: torch.Tensor, k_data, k_scale, v_data, v_scale, block_table: torch.Tensor, context_lens,
                max_context: int, scale: float, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Paged MXFP4 attention decode: q [R, Hq, 128] (bf16 or e4m3), K and V caches
    as [pages, Hkv, P, 64] + [pages, Hkv, P, 4] views, block_table [R, width],
    context_lens [R] -> bf16 out [R, Hq, 128] (zeros for rows with no token)."""
    dev = _same_device(q, k_data, k_scale, v_data, v_scale, block_table, context_lens, out)
    qd = _query(q)
    kview, kshape = _kvview(k_data, k_scale, "K")
    vview, vshape = _kvview(v_data, v_scale, "V")
    if kshape != vshape:
        raise ValueError(f"K and V caches differ in shape: {kshape} vs {vshape}")
    pages, Hkv, P = kshape
    if P not in (64, 128):
        raise ValueError(f"page size must be 64 or 128, got {P}")
    R, Hq = q.shape[0], q.shape[1]
    btp, bts, btw = _table(block_table)
    if block_table.shape[0] < R:
        raise ValueError("block_table has fewer rows than the query")
    if out is None:
        out = torch.empty((R, Hq, 128), dtype=torch.bfloat16, device=dev)
    if out.dtype != torch.bfloat16 or tuple(out.shape) != (R, Hq, 128) or (out.numel() > 0 and out.stride(2) != 1):
        raise ValueError(f"out must be bf16 [{R}, {Hq}, 128] with a contiguous last axis")
    kv = KVCache(kview, vview, P, Hkv, pages)
    with torch.cuda.device(dev):
        _check(lib().mxs_attn_decode(ctypes.byref(qd), ctypes.byref(kv), btp, bts, btw,
                                     _int_vec("context_lens", context_lens, R), R, int(max_context),
                                     ctypes.c_float(scale), out.data_ptr(), out.stride(0), out.stride(1),
                                     _stream(dev, stream)))
    return out

"""Paged MXFP4 attention decode: plain CPU definition -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the smoke check and the benchmark's CPU-baseline leg load
this module; the product path never imports it.

What it computes (ATOM #2770, "How it works" and the squashed sparse
attention commit: the selected pages' K and V are read as MXFP4 by a paged
attention decode with one query row per (token, kv head) row; aiter #7056 as
quoted there: K and V are e2m1 data plus one e8m0 scale per 32 elements along
head_dim, in data and scale views with their own page and head strides):

  K[p, hk, j, e] = e2m1(code e of token j) * 2^(scale byte e/32 - 127), and V alike
  Q_hat          = e4m3 query as stored, or bf16 rounded to e4m3 (nearest
                   even, saturating, unit scale: the scorer's query rule)
  for row r, q head h (kv head hk = h // G, G = Hq / Hkv), t < ctx[r]:
      s_t   = scale * (Q_hat[r, h] . K[page(r, t), hk, t % P])
      out   = sum_t softmax(s)_t * V[page(r, t), hk, t % P]
  rows with ctx = 0 give 0.

Everything is float64: the dot of e4m3 query and MXFP4 key values is exact
in double while a token's four scale bytes span less than about 15 binades
(beyond, its relative rounding error is of order 2^-53), the softmax
subtracts the row maximum before exponentiating, and the weighted sum is
numpy's float64 matmul. The kernel returns bf16; the comparison bound is in
the tests.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

import oracle

_E2M1 = None
_E4M3 = None


def _tables():
    global _E2M1, _E4M3
    if _E2M1 is None:
        _E2M1 = np.array([oracle.e2m1_value(c) for c in range(16)], np.float64)
        _E4M3 = np.array([oracle.e4m3_value(b) for b in range(256)], np.float64)
    return _E2M1, _E4M3


def dequant_tokens(data: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """MXFP4 tokens: data [..., 64] uint8 + scale [..., 4] uint8 -> values [..., 128] float64.
    Element 2m is the low nibble of byte m; byte k of the scale covers elements 32k..32k+31."""
    e2m1, _ = _tables()
    codes = np.stack([data & 0xF, data >> 4], axis=-1).reshape(data.shape[:-1] + (128,))
    sc = np.repeat(scale.astype(np.int64), 32, axis=-1)
    return e2m1[codes] * np.ldexp(1.0, sc - 127)


def q_hat(q_bits: np.ndarray, q_dtype: str) -> np.ndarray:
    """Query rounded as the scorer rounds it: [R, Hq, 128] float64."""
    _, e4m3 = _tables()
    if q_dtype == "e4m3":
        return e4m3[q_bits.astype(np.int64)]
    lut = np.array([oracle.bf16_to_e4m3(b) for b in range(65536)], np.int64)
    return e4m3[lut[q_bits.astype(np.int64)]]


def attn_decode(*, q: np.ndarray, q_dtype: str, k_data: np.ndarray, k_scale: np.ndarray, v_data: np.ndarray,
                v_scale: np.ndarray, block_table: np.ndarray, context_lens: np.ndarray, page_size: int,
                scale: float, rows: Optional[np.ndarray] = None, want_mag: bool = False):
    """q [R, Hq, 128] (uint16 bf16 bits or uint8 e4m3 bytes); k/v data [pages, Hkv, P, 64],
    k/v scale [pages, Hkv, P, 4] (uint8); block_table [R, width]; context_lens [R].
    Returns out [R', Hq, 128] float64 for the selected rows (all rows by default) and,
    with want_mag, mag [R', Hq, 128] = sum_t softmax(s)_t * |V_t| (the scale of the
    output's rounding error) and qk_mag [R', Hq] = max_t sum_e |Q_hat_e K_t,e| (the
    scale of a logit's rounding error)."""
    R, Hq, D = q.shape
    assert D == 128
    Hkv = k_data.shape[1]
    assert Hq % Hkv == 0
    G = Hq // Hkv
    P = page_size
    qh = q_hat(q, q_dtype)
    sel = np.arange(R) if rows is None else np.asarray(rows)
    out = np.zeros((len(sel), Hq, 128), np.float64)
    mag = np.zeros((len(sel), Hq, 128), np.float64)
    qk_mag = np.zeros((len(sel), Hq), np.float64)
    for n, r in enumerate(sel):
        ctx = int(context_lens[r])
        if ctx <= 0:
            continue
        t = np.arange(ctx)
        pages = block_table[r, t // P].astype(np.int64)
        slots = t % P
        for hk in range(Hkv):
            K = dequant_tokens(k_data[pages, hk, slots], k_scale[pages, hk, slots])     # [ctx, 128]
            V = dequant_tokens(v_data[pages, hk, slots], v_scale[pages, hk, slots])
            qg = qh[r, hk * G:(hk + 1) * G]                                          # [G, 128]
            s = scale * (qg @ K.T)                                                   # [G, ctx]
            s = s - s.max(axis=1, keepdims=True)
            w = np.exp(s)
            w = w / w.sum(axis=1, keepdims=True)
            out[n, hk * G:(hk + 1) * G] = w @ V
            if want_mag:
                mag[n, hk * G:(hk + 1) * G] = w @ np.abs(V)
                qk_mag[n, hk * G:(hk + 1) * G] = (np.abs(qg) @ np.abs(K).T).max(axis=1)
    return (out, mag, qk_mag) if want_mag else out

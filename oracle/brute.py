"""Pure-Python brute-force twin of the C oracle -- TEST INFRASTRUCTURE ONLY.

Written independently of ``mxs_oracle.c`` (no shared tables or helpers) so
that the two can check each other on tiny inputs. Everything is exact
(``fractions.Fraction``) until one final round-to-nearest-even to fp32.

Definitions followed:
* e2m1 (OCP MX element): 1 sign, 2 exponent bits with bias 1, 1 mantissa bit;
  exponent field 0 is subnormal (aiter #7061, "Format": e2m1 data).
* e8m0 scale byte b: 2^(b - 127); 255 is NaN (aiter #7061, "Format").
* e4m3fn: 1 sign, 4 exponent bits with bias 7, 3 mantissa bits, no infinity,
  S.1111.111 is NaN, largest finite 448 (ATOM #2770, write-path commit:
  unit-scale saturating e4m3 in a float8_e4m3fn tensor).
* bf16 query -> nearest e4m3 value, ties to the even code, magnitudes at or
  above 448 saturate (aiter #7061, "Kernels": bf16 Q rounded to e4m3 in-kernel).
* Row i of request b sees tokens t < min(seq_len_b, prefix_b + i + 1); a decode
  row sees t < seq_len_b (aiter #7061, "Kernels" and "Changed op tests").
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction
from typing import List, Optional, Sequence

NEG_INF = float("-inf")


def e2m1(code: int) -> Fraction:
    sign = -1 if code & 0b1000 else 1
    exp_field = (code >> 1) & 0b11
    man = code & 0b1
    if exp_field == 0:
        mag = Fraction(man, 2)                              # subnormal: m/2 * 2^(1-1)
    else:
        mag = (1 + Fraction(man, 2)) * Fraction(2) ** (exp_field - 1)
    return sign * mag


def e8m0(byte: int) -> Optional[Fraction]:
    if byte == 255:
        return None
    return Fraction(2) ** (byte - 127)


def e4m3(byte: int) -> Optional[Fraction]:
    sign = -1 if byte & 0x80 else 1
    exp_field = (byte >> 3) & 0xF
    man = byte & 0x7
    if exp_field == 0xF and man == 0x7:
        return None                                          # NaN
    if exp_field == 0:
        mag = Fraction(man, 8) * Fraction(2) ** (1 - 7)
    else:
        mag = (1 + Fraction(man, 8)) * Fraction(2) ** (exp_field - 7)
    return sign * mag


_E4M3_POS = [(c, e4m3(c)) for c in range(0x7F)]              # 0x00 .. 0x7E, all finite


def bf16_value(bits: int) -> Optional[Fraction]:
    f = struct.unpack("<f", struct.pack("<I", (bits & 0xFFFF) << 16))[0]
    if math.isnan(f):
        return None
    if math.isinf(f):
        return Fraction(10 ** 9) * (1 if f > 0 else -1)      # beyond every e4m3 magnitude
    return Fraction(f)


def bf16_to_e4m3(bits: int) -> int:
    """Nearest-value search over the finite e4m3 codes, ties to the even code."""
    sign = 0x80 if bits & 0x8000 else 0
    v = bf16_value(bits)
    if v is None:
        return sign | 0x7F
    a = abs(v)
    best_code, best_d = None, None
    for code, val in _E4M3_POS:
        d = abs(val - a)
        if best_d is None or d < best_d or (d == best_d and code % 2 == 0):
            best_code, best_d = code, d
    return sign | best_code


def round_f32(x: Fraction) -> float:
    """Round an exact rational to the nearest fp32 value, ties to even."""
    if x == 0:
        return 0.0
    neg = x < 0
    a = -x if neg else x
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    lsb_exp = max(e - 23, -149)
    scaled = a / Fraction(2) ** lsb_exp
    q, r = divmod(scaled.numerator, scaled.denominator)
    twice = 2 * r
    if twice > scaled.denominator or (twice == scaled.denominator and q % 2 == 1):
        q += 1
    val = Fraction(q) * Fraction(2) ** lsb_exp
    if val >= Fraction(2) ** 128:
        out = float("inf")
    else:
        out = float(val)                                     # exact: q has <= 24 bits
    return -out if neg else out


def decode_q(q_bits: Sequence[int], q_dtype: str) -> List[Optional[Fraction]]:
    if q_dtype == "bf16":
        return [e4m3(bf16_to_e4m3(b)) for b in q_bits]
    return [e4m3(b) for b in q_bits]


def token_k(data_page: bytes, scale_page: bytes, slot: int) -> List[Optional[Fraction]]:
    out = []
    for e in range(128):
        byte = data_page[slot * 64 + e // 2]
        code = (byte >> 4) if e % 2 else (byte & 0xF)
        s = e8m0(scale_page[slot * 4 + e // 32])
        out.append(None if s is None else e2m1(code) * s)
    return out


def token_k_e4m3(data_page: bytes, slot: int) -> List[Optional[Fraction]]:
    """fp8 index cache: 128 e4m3 bytes per token, unit scale."""
    return [e4m3(data_page[slot * 128 + e]) for e in range(128)]


def token_mag(qh: List[Fraction], data_page: bytes, scale_page: bytes, slot: int) -> Fraction:
    """M of one (query vector, token) pair: sum over the 128 elements of
    |Q_hat[e]| * |e2m1(code e)| * 2^(scale byte - 127), the magnitude of the
    terms the dot adds up (no sm_scale). Live tokens only (no NaN scale)."""
    total = Fraction(0)
    for e in range(128):
        byte = data_page[slot * 64 + e // 2]
        code = (byte >> 4) if e % 2 else (byte & 0xF)
        total += abs(qh[e]) * abs(e2m1(code)) * e8m0(scale_page[slot * 4 + e // 32])
    return total


def score(*, mode: str, q_rows, q_dtype: str, pages_data, pages_scale, page_size: int,
          block_table, seq_lens, max_seq_len: int, sm_scale: float, cu_seqlens_q=None,
          prefix_lens=None, k_dtype: str = "mxfp4"):
    """(logits, blocks) of :func:`score_mags`."""
    lg, bl, _ = score_mags(mode=mode, q_rows=q_rows, q_dtype=q_dtype, pages_data=pages_data,
                           pages_scale=pages_scale, page_size=page_size, block_table=block_table,
                           seq_lens=seq_lens, max_seq_len=max_seq_len, sm_scale=sm_scale,
                           cu_seqlens_q=cu_seqlens_q, prefix_lens=prefix_lens, k_dtype=k_dtype)
    return lg, bl


def score_mags(*, mode: str, q_rows, q_dtype: str, pages_data, pages_scale, page_size: int,
               block_table, seq_lens, max_seq_len: int, sm_scale: float, cu_seqlens_q=None,
               prefix_lens=None, k_dtype: str = "mxfp4"):
    """Brute force over every (row, head, token).

    ``q_rows[r][h]`` is a list of 128 ints (bf16 bits or e4m3 bytes);
    ``pages_data[p]``/``pages_scale[p]`` are bytes objects of P*64 / P*4 bytes
    (k_dtype "mxfp4"), or ``pages_data[p]`` holds P*128 e4m3 bytes and
    ``pages_scale`` is unused (k_dtype "e4m3").
    Returns (logits[r][h][t], blocks[r][h][j], mags[r][h][t]): logits and
    blocks as nested lists of Python floats holding fp32 values, mags as exact
    Fractions (0 for dead tokens; computed for the MXFP4 cache only).
    """
    B = len(seq_lens)
    if mode == "decode":
        rows = [(b, seq_lens[b]) for b in range(B)]
    else:
        rows = []
        for b in range(B):
            for i in range(cu_seqlens_q[b + 1] - cu_seqlens_q[b]):
                rows.append((b, min(seq_lens[b], prefix_lens[b] + i + 1)))
    nb = (max_seq_len + page_size - 1) // page_size
    s = Fraction(sm_scale)
    logits, blocks, mags = [], [], []
    for r, (b, limit) in enumerate(rows):
        limit = max(0, min(limit, max_seq_len))
        H = len(q_rows[r])
        lr = [[NEG_INF] * max_seq_len for _ in range(H)]
        br = [[NEG_INF] * nb for _ in range(H)]
        mr = [[Fraction(0)] * max_seq_len for _ in range(H)]
        qh = [decode_q(q_rows[r][h], q_dtype) for h in range(H)]
        for t in range(limit):
            page = block_table[b][t // page_size]
            if k_dtype == "e4m3":
                kv = token_k_e4m3(pages_data[page], t % page_size)
            else:
                kv = token_k(pages_data[page], pages_scale[page], t % page_size)
            for h in range(H):
                if any(v is None for v in kv) or any(v is None for v in qh[h]):
                    val = float("nan")
                else:
                    dot = sum((qh[h][e] * kv[e] for e in range(128)), Fraction(0))
                    val = round_f32(s * dot)
                lr[h][t] = val
                if k_dtype != "e4m3" and not any(v is None for v in qh[h]):
                    mr[h][t] = token_mag(qh[h], pages_data[page], pages_scale[page], t % page_size)
                j = t // page_size
                if val > br[h][j]:
                    br[h][j] = val
        logits.append(lr)
        blocks.append(br)
        mags.append(mr)
    return logits, blocks, mags

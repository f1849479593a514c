"""MXFP4 index-K writer: plain CPU definition of the quantization into pages.

TEST INFRASTRUCTURE ONLY: loaded by tests/, the smoke check and the
benchmark's CPU-baseline leg; the product path never imports it.

The pages name the writer (ATOM #2770, "Summary" and the write-path commit:
one fused kernel quantizes the index key straight into its pool page slot;
aiter #7061, "Tests": caches built with a 1x32 e2m1 quantizer) but give no
conversion rule. Reading taken: the OCP Microscaling (MX) v1.0 conversion
for FP4 E2M1 elements with an E8M0 scale per 32 consecutive elements:
  * shared exponent e = floor(log2(amax)) - 2, amax the largest magnitude in
    the block (2 is the exponent of e2m1's largest binade); the stored byte
    is e + 127, clipped to [1, 254] (an all-zero block gets byte 1, which
    keeps it inside the scorer's contract);
  * each element x becomes the e2m1 value nearest to x / 2^e, ties to the
    even code, saturated at +-6; the sign bit is kept (also for zero).
Non-finite inputs are outside the contract (parity unpinned for them).
A token t goes to slot slot_mapping[t] = page * P + offset (-1: skipped):
data bytes at page * data_page_stride + offset * 64, scale bytes at
page * scale_page_stride + offset * 4; element 2m in the low nibble of
byte m (the layout the scorer reads).

An fp8 index cache (the format the MXFP4 one replaces; aiter #7061,
"Summary": 128 B of e4m3 per token) gets each element as the nearest e4m3
value, ties to the even code, saturated at +-448, unit scale -- the rounding
the query takes (aiter #7061, "Kernels") -- at byte offset * 128 + e.
"""
from __future__ import annotations

import math

import numpy as np

_E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]   # magnitude of codes 0..7


def bf16_value(bits: int) -> float:
    """Exact value of a bf16 bit pattern."""
    return float(np.array([bits << 16], dtype=np.uint32).view(np.float32)[0])


def e2m1_code(v: float) -> int:
    """Nearest e2m1 code to v (ties to the even code), saturating at 6."""
    sign = 8 if math.copysign(1.0, v) < 0 else 0
    a = abs(v)
    best = 0
    for c in range(1, 8):
        d_best, d_c = abs(a - _E2M1[best]), abs(a - _E2M1[c])
        if d_c < d_best or (d_c == d_best and c % 2 == 0):
            best = c
    return sign | best


def quantize_block(vals) -> tuple:
    """32 exact values -> (scale byte, 32 codes)."""
    amax = max(abs(v) for v in vals)
    if amax == 0.0:
        byte = 1
    else:
        m, ex = math.frexp(amax)            # amax = m * 2^ex, m in [0.5, 1): floor(log2 amax) = ex - 1
        byte = min(254, max(1, (ex - 1) - 2 + 127))
    e = byte - 127
    return byte, [e2m1_code(math.ldexp(v, -e)) for v in vals]


def quantize_token(bits) -> tuple:
    """128 bf16 bit patterns -> (64 data bytes, 4 scale bytes)."""
    vals = [bf16_value(int(b)) for b in bits]
    data = bytearray(64)
    scales = bytearray(4)
    for k in range(4):
        byte, codes = quantize_block(vals[32 * k:32 * k + 32])
        scales[k] = byte
        for e, c in enumerate(codes):
            i = 32 * k + e
            data[i // 2] |= c << (4 * (i % 2))
    return bytes(data), bytes(scales)


def write_pages_e4m3(k_bits: np.ndarray, slot_mapping, k_data: np.ndarray, page_size: int) -> None:
    """Round k_bits [N, 128] (uint16 bf16 patterns) to e4m3 bytes into the fp8
    page view k_data [pages, P, 128] (uint8), in place; slot -1 skips."""
    from oracle import bf16_to_e4m3
    for t, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        page, off = divmod(int(slot), page_size)
        k_data[page, off, :] = [bf16_to_e4m3(int(b)) for b in k_bits[t]]


def write_pages(k_bits: np.ndarray, slot_mapping, k_data: np.ndarray, k_scale: np.ndarray, page_size: int) -> None:
    """Quantize k_bits [N, 128] (uint16 bf16 patterns) into the page views
    k_data [pages, P, 64] and k_scale [pages, P, 4] (uint8), in place."""
    for t, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        page, off = divmod(int(slot), page_size)
        d, s = quantize_token(k_bits[t])
        k_data[page, off, :] = np.frombuffer(d, dtype=np.uint8)
        k_scale[page, off, :] = np.frombuffer(s, dtype=np.uint8)

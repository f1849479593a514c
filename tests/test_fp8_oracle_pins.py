"""Pins for the oracle's fp8 (e4m3) index-cache path.

The fp8 cache is the format the MXFP4 one replaces (aiter #7061, "Summary":
128 B of e4m3 per token against 68 B; "Kernels": 16 KB per 128-token
buffer). Reading taken: K(p, j, e) = e4m3(byte e of token j), unit scale,
the same query rounding, mask, logit and block rules as the MXFP4 path.

What pins it, other than its own formula:
  * inside the e8m0 window [119, 133] every MXFP4 value is an e4m3 value
    (aiter #7061, "Format" and "Validation": the fp8 scorer judges the MXFP4
    one there), so an MXFP4 cache converted value by value to e4m3 bytes must
    score bit for bit like the MXFP4 oracle (itself pinned independently);
  * hand-worked pages (the same dots as the MXFP4 golden pages: 128 and 24);
  * closed forms at the largest magnitudes and under cancellation;
  * the pure-Python twin (Fractions) on tiny random caches over all codes;
  * planted mistakes in the twin each break a pin.
"""
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import brute
from tests.oracle_cases import SM_SCALE, random_case, run_c


def f32_bits(x) -> int:
    return struct.unpack("<I", struct.pack("<f", np.float32(x)))[0]


def bf16_bits(x: float) -> int:
    b = struct.unpack("<I", struct.pack("<f", x))[0]
    assert b & 0xFFFF == 0, x
    return b >> 16


# e4m3 code of every finite value, from the twin's own decoder
_VAL_TO_E4M3 = {}
for _b in range(256):
    _v = brute.e4m3(_b)
    if _v is not None:
        _VAL_TO_E4M3.setdefault(_v, _b)


def to_e4m3_cache(k_data: np.ndarray, k_scale: np.ndarray) -> np.ndarray:
    """MXFP4 pages [pool, P, 64] + [pool, P, 4] -> e4m3 pages [pool, P, 128] of
    the same values (every scale byte must be in [119, 133]; tokens whose
    scale is 255 become NaN bytes, as dead garbage)."""
    pool, P, _ = k_data.shape
    out = np.zeros((pool, P, 128), np.uint8)
    for p in range(pool):
        for j in range(P):
            for e in range(128):
                byte = int(k_data[p, j, e // 2])
                code = (byte >> 4) if e % 2 else (byte & 0xF)
                s = int(k_scale[p, j, e // 32])
                if s == 255:
                    out[p, j, e] = 0x7F
                    continue
                out[p, j, e] = _VAL_TO_E4M3[brute.e2m1(code) * Fraction(2) ** (s - 127)]
    return out


def run_e4m3(c, k8, **kw):
    return oracle.score(mode=kw.pop("mode", "prefill"), q=c["q"], q_dtype=kw.pop("q_dtype", "bf16"), k_data=k8,
                        k_scale=None, page_size=kw.pop("page_size"), block_table=c["block_table"],
                        seq_lens=c["seq_lens"], max_seq_len=kw.pop("max_seq_len"), sm_scale=SM_SCALE,
                        cu_seqlens_q=c.get("cu_seqlens_q"), prefix_lens=c.get("prefix_lens"), k_dtype="e4m3", **kw)


def one_page(tokens, P=64):
    """e4m3 page 0 holding the given 128-byte token rows from slot 0."""
    k8 = np.zeros((1, P, 128), np.uint8)
    for j, row in enumerate(tokens):
        k8[0, j] = row
    return k8


def single_row(q_bits, n_tokens):
    return dict(q=np.array(q_bits, np.uint16).reshape(1, 1, 128), block_table=np.zeros((1, 1), np.int32),
                seq_lens=np.array([n_tokens], np.int32), cu_seqlens_q=np.array([0, 1], np.int32),
                prefix_lens=np.array([n_tokens - 1], np.int32))


def logits_of(c, k8, n, P=64):
    return run_e4m3(c, k8, page_size=P, max_seq_len=n).logits[0, 0, :n]


# ------------------------------------------------------------------ hand-worked

def test_all_ones_page():
    # Q = 1.0 everywhere, K = e4m3 1.0 (0x38) everywhere: dot 128, logit
    # RN32(128 * RN32(1/sqrt(128))) = 0x413504F3 (the MXFP4 all-ones page).
    c = single_row([bf16_bits(1.0)] * 128, 1)
    lg = logits_of(c, one_page([[0x38] * 128]), 1)
    assert f32_bits(lg[0]) == 0x413504F3


def test_one_hot_element_order_and_token_stride():
    # Token 1 (bytes 128..255 of the page) holds element 0 = 2.0 (0x40) and
    # element 1 = 24.0 (0x5C); Q is one-hot at element 1. dot = 24, logit
    # 0x4007C3B6 (the MXFP4 one-hot page with scale 2^2). Reading element 0
    # instead gives 2; a 64-byte token stride reads token 0's zeros.
    q = [0] * 128
    q[1] = bf16_bits(1.0)
    tok1 = [0] * 128
    tok1[0], tok1[1] = 0x40, 0x5C
    c = single_row(q, 2)
    lg = logits_of(c, one_page([[0] * 128, tok1]), 2)
    assert f32_bits(lg[0]) == 0 and f32_bits(lg[1]) == 0x4007C3B6


def test_largest_magnitudes_closed_form():
    # Q = K = 448 (the largest e4m3, bf16 0x43E0, e4m3 0x7E): dot = 128 * 448^2
    # = 25,690,112, exact; logit = RN32(dot * sm_scale).
    c = single_row([0x43E0] * 128, 1)
    lg = logits_of(c, one_page([[0x7E] * 128]), 1)
    assert float(lg[0]) == brute.round_f32(Fraction(25690112) * Fraction(SM_SCALE))


def test_cancellation_closed_form():
    # Q = +-448 alternating (even +, odd -), K = 448 except K[0] = 2^-9 (the
    # smallest subnormal, 0x01): dot = 448 * 2^-9 + 63 * 448^2 - 64 * 448^2
    # = 0.875 - 200704, a small residue next to terms of 2^17.6.
    q = [0x43E0 if e % 2 == 0 else 0xC3E0 for e in range(128)]
    k = [0x7E] * 128
    k[0] = 0x01
    c = single_row(q, 1)
    lg = logits_of(c, one_page([k]), 1)
    assert float(lg[0]) == brute.round_f32((Fraction(7, 8) - 200704) * Fraction(SM_SCALE))
    # full cancellation: K[0] = 448 too -> 64 terms of +448^2 and 64 of -448^2
    k[0] = 0x7E
    assert f32_bits(logits_of(c, one_page([k]), 1)[0]) == 0
    # and with Q[127] flipped to +448: dot = 2 * 448^2
    q2 = list(q)
    q2[127] = 0x43E0
    c2 = single_row(q2, 1)
    assert float(logits_of(c2, one_page([k]), 1)[0]) == brute.round_f32(Fraction(2 * 200704) * Fraction(SM_SCALE))


# ------------------------------------------------------------------ the e4m3-exact window

@pytest.mark.parametrize("P,mode,q_dtype,seed", [(64, "prefill", "bf16", 0), (128, "prefill", "e4m3", 1),
                                                 (64, "decode", "bf16", 2), (128, "decode", "e4m3", 3)])
def test_equals_mxfp4_oracle_inside_window(P, mode, q_dtype, seed):
    rng = np.random.default_rng(100 + seed)
    if mode == "decode":
        c = random_case(rng, B=3, H=2, page_size=P, q_lens=[1, 1, 1], prefix_lens=[0, 0, 0],
                        seq_lens=[P + 5, 2 * P, 3], q_dtype=q_dtype, scale_lo=119, scale_hi=133)
    else:
        c = random_case(rng, B=2, H=2, page_size=P, q_lens=[3, 2], prefix_lens=[P - 2, 0],
                        seq_lens=[P + 1, P + 17], q_dtype=q_dtype, scale_lo=119, scale_hi=133)
    W = int(c["seq_lens"].max()) + 3
    ref = run_c(c, mode=mode, q_dtype=q_dtype, page_size=P, max_seq_len=W)
    k8 = to_e4m3_cache(c["k_data"], c["k_scale"])
    got = run_e4m3(c, k8, mode=mode, q_dtype=q_dtype, page_size=P, max_seq_len=W)
    assert np.array_equal(ref.logits.view(np.uint32), got.logits.view(np.uint32))
    assert np.array_equal(ref.blocks.view(np.uint32), got.blocks.view(np.uint32))


# ------------------------------------------------------------------ two oracles

def _random_e4m3_case(rng, P, H, seq_lens, q_lens, prefix_lens):
    npr = [(s + P - 1) // P for s in seq_lens]
    pool = sum(npr) + 1
    k8 = rng.integers(0, 256, (pool, P, 128), dtype=np.uint8)
    k8[(k8 & 0x7F) == 0x7F] = 0x7E                      # every finite code, no NaN
    bt = np.full((len(seq_lens), max(npr) + 1), -1, np.int32)
    perm = rng.permutation(pool)
    pos = 0
    for b, n in enumerate(npr):
        bt[b, :n] = perm[pos:pos + n]
        pos += n
    T = sum(q_lens)
    x = (rng.standard_normal((T, H, 128)) * 4).astype(np.float32)
    q = (x.view(np.uint32) >> 16).astype(np.uint16)
    c = dict(q=q, block_table=bt, seq_lens=np.array(seq_lens, np.int32),
             cu_seqlens_q=np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32),
             prefix_lens=np.array(prefix_lens, np.int32))
    return c, k8


@pytest.mark.parametrize("seed", range(2))
def test_c_and_python_oracles_agree(seed):
    rng = np.random.default_rng(200 + seed)
    P = 64
    c, k8 = _random_e4m3_case(rng, P, 2, [70, 9], [2, 1], [68, 8])
    W = 72
    got = run_e4m3(c, k8, page_size=P, max_seq_len=W)
    q_rows = [[list(map(int, c["q"][r, h])) for h in range(2)] for r in range(3)]
    lb, bb = brute.score(mode="prefill", q_rows=q_rows, q_dtype="bf16",
                         pages_data=[bytes(k8[p].reshape(-1)) for p in range(k8.shape[0])], pages_scale=None,
                         page_size=P, block_table=[list(map(int, r)) for r in c["block_table"]],
                         seq_lens=list(map(int, c["seq_lens"])), max_seq_len=W, sm_scale=SM_SCALE,
                         cu_seqlens_q=list(map(int, c["cu_seqlens_q"])), prefix_lens=list(map(int, c["prefix_lens"])),
                         k_dtype="e4m3")
    assert np.array_equal(got.logits.view(np.uint32), np.array(lb, np.float32).view(np.uint32))
    assert np.array_equal(got.blocks.view(np.uint32), np.array(bb, np.float32).view(np.uint32))


def test_round_scaled_terms_matches_rational():
    # the exact rounding of sums far wider than 64 bits (e4m3 x e4m3 block sums
    # are multiples of 2^-18 up to 2^22.6), against Fraction rounding
    rng = np.random.default_rng(5)
    for _ in range(400):
        n = 4
        S = [float(int(rng.integers(-(1 << 41), 1 << 41))) / (1 << 18) for _ in range(n)]
        ex = [int(rng.integers(-30, 30)) for _ in range(n)]
        sm = float(np.float32(rng.uniform(0.01, 4.0)))
        want = brute.round_f32(sum((Fraction(s) * Fraction(2) ** e for s, e in zip(S, ex)), Fraction(0)) * Fraction(sm))
        got = oracle.round_scaled_terms(S, ex, 18, sm)
        assert f32_bits(got) == f32_bits(want), (S, ex, sm)
    # near-cancelling pairs
    for _ in range(200):
        a = int(rng.integers(1 << 39, 1 << 41))
        d = int(rng.integers(-5, 6))
        S = [a / (1 << 18), -(a + d) / (1 << 18), 0.0, 0.0]
        want = brute.round_f32(Fraction(-d, 1 << 18) * Fraction(SM_SCALE))
        assert f32_bits(oracle.round_scaled_terms(S, [0] * 4, 18, SM_SCALE)) == f32_bits(want)


def test_scale_view_is_not_read():
    c = single_row([bf16_bits(1.0)] * 128, 1)
    r = run_e4m3(c, one_page([[0x38] * 128]), page_size=64, max_seq_len=1, scale_page_stride=0)
    assert f32_bits(r.logits[0, 0, 0]) == 0x413504F3


# ------------------------------------------------------------------ planted mistakes

def _hand_pins_hold_for_twin():
    q = [0] * 128
    q[1] = bf16_bits(1.0)
    tok1 = [0] * 128
    tok1[0], tok1[1] = 0x40, 0x5C
    page = bytes([0] * 128 + tok1 + [0] * 128 * 62)
    lb, _ = brute.score(mode="decode", q_rows=[[q]], q_dtype="bf16", pages_data=[page], pages_scale=None,
                        page_size=64, block_table=[[0]], seq_lens=[2], max_seq_len=2, sm_scale=SM_SCALE,
                        k_dtype="e4m3")
    ones = bytes([0x38] * 128 * 64)
    lo, _ = brute.score(mode="decode", q_rows=[[[bf16_bits(1.0)] * 128]], q_dtype="bf16", pages_data=[ones],
                        pages_scale=None, page_size=64, block_table=[[0]], seq_lens=[1], max_seq_len=1,
                        sm_scale=SM_SCALE, k_dtype="e4m3")
    return f32_bits(lb[0][0][1]) == 0x4007C3B6 and f32_bits(lb[0][0][0]) == 0 and f32_bits(lo[0][0][0]) == 0x413504F3


_ORIG_TOKEN = brute.token_k_e4m3
_ORIG_E4M3 = brute.e4m3


def _stride_64(page, slot):
    return [brute.e4m3(page[slot * 64 + e]) for e in range(128)]


def _pairs_swapped(page, slot):
    return [brute.e4m3(page[slot * 128 + (e ^ 1)]) for e in range(128)]


def _bias_8(byte):
    v = _ORIG_E4M3(byte)
    return None if v is None else v / 2


@pytest.mark.parametrize("attr,mutant", [("token_k_e4m3", _stride_64), ("token_k_e4m3", _pairs_swapped),
                                         ("e4m3", _bias_8)])
def test_planted_mistakes_are_caught(monkeypatch, attr, mutant):
    assert _hand_pins_hold_for_twin()
    monkeypatch.setattr(brute, attr, mutant)
    assert not _hand_pins_hold_for_twin()

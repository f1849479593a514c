"""Pins of the CPU oracle against facts fixed outside it (no GPU needed).

Each test names the plausible oracle mistake it would catch. Sources: aiter
#7061 "Format" and "Kernels" (value = e2m1 x 2^(byte-127), one e8m0 byte per
32 elements, bf16 Q rounded to e4m3, max over live tokens), ATOM #2770 (unit
scale saturating e4m3 query), aiter #5518 "Summary" (page strides).
"""
import math
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import brute
from tests.oracle_cases import (SM_SCALE, load_hand_pages, random_case, run_brute, run_c, single_token_case)


def bf16_bits(x: float) -> int:
    return struct.unpack("<I", struct.pack("<f", x))[0] >> 16


def f32_bits(x: float) -> int:
    return int(np.float32(x).view(np.uint32))


# ------------------------------------------------------------------ elements

def test_e2m1_codes_match_the_format(oracle_lib):
    # OCP e2m1: largest magnitude 6, smallest nonzero 0.5, bit 3 the sign.
    # Catches: a wrong magnitude table entry or sign bit.
    vals = [oracle.e2m1_value(c) for c in range(16)]
    assert vals[:8] == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert [math.copysign(1, v) for v in vals[8:]] == [-1.0] * 8
    for c in range(16):
        assert Fraction(vals[c]) == brute.e2m1(c)


def test_e4m3_decode_matches_bit_definition(oracle_lib):
    # Catches: wrong bias, wrong subnormal scale, NaN code.
    assert oracle.e4m3_value(0x7E) == 448.0
    assert oracle.e4m3_value(0x38) == 1.0
    assert oracle.e4m3_value(0x08) == 2.0 ** -6
    assert oracle.e4m3_value(0x01) == 2.0 ** -9
    assert math.isnan(oracle.e4m3_value(0x7F)) and math.isnan(oracle.e4m3_value(0xFF))
    for b in range(256):
        c = oracle.e4m3_value(b)
        p = brute.e4m3(b)
        if p is None:
            assert math.isnan(c)
        else:
            assert Fraction(c) == p, hex(b)


def test_e8m0_scale(oracle_lib):
    assert oracle.e8m0_value(127) == 1.0
    assert oracle.e8m0_value(128) == 2.0
    assert oracle.e8m0_value(0) == 2.0 ** -127
    assert math.isnan(oracle.e8m0_value(255))


@pytest.mark.parametrize("x,expect", [
    (1.0625, 1.0),            # halfway 1 / 1.125 -> even mantissa (1.0)
    (1.1875, 1.25),           # halfway 1.125 / 1.25 -> even mantissa (1.25)
    (432.0, 448.0),           # halfway 416 / 448 -> even mantissa (448)
    (447.0, 448.0),           # bf16 keeps 448 here; saturating
    (464.0, 448.0),           # beyond the largest finite value: saturate
    (500.0, 448.0),
    (float("inf"), 448.0),
    (2.0 ** -10, 0.0),        # halfway 0 / 2^-9 -> even code 0
    (1.5 * 2.0 ** -9, 2.0 ** -8),  # halfway 2^-9 / 2^-8 -> even code (2^-8)
    (2.5 * 2.0 ** -9, 2.0 ** -8),  # halfway 2^-8 / 3*2^-9 -> even code (2^-8)
    (-0.30078125, -0.3125),   # nearest, sign kept
    (-0.0, -0.0),
])
def test_e4m3_rounding_spot_values(oracle_lib, x, expect):
    # Hand-derived RNE-satfinite results. Catches: truncation instead of RNE,
    # ties away from zero, missing saturation, lost sign.
    b = bf16_bits(x)
    got = oracle.e4m3_value(oracle.bf16_to_e4m3(b))
    assert got == expect and math.copysign(1, got) == math.copysign(1, expect)


def test_e4m3_rounding_exhaustive(oracle_lib):
    # Every bf16 bit pattern: the oracle's bit-level rounding against a
    # vectorised nearest-value search (ties to the even code), written here.
    codes = np.arange(0x7F)                                     # finite non-negative codes
    vals = np.array([oracle.e4m3_value(int(c)) for c in codes])
    bits = np.arange(65536, dtype=np.uint32)
    f = (bits << 16).view(np.float32).astype(np.float64)
    a = np.abs(f)
    a_fin = np.where(np.isfinite(a), a, 1e9)
    d = np.abs(vals[None, :] - a_fin[:, None])
    dmin = d.min(axis=1, keepdims=True)
    cand = (d == dmin)
    even = cand & (codes[None, :] % 2 == 0)
    pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    pick = np.where(a_fin >= 448.0, 0x7E, pick)
    sign = np.where((bits & 0x8000) != 0, 0x80, 0)
    ref = (pick | sign).astype(np.int64)
    ref = np.where(np.isnan(f), sign | 0x7F, ref)
    got = oracle.bf16_to_e4m3_table().astype(np.int64)
    assert np.array_equal(got, ref), np.nonzero(got != ref)[0][:10]
    # and the independent pure-Python search on a spread of patterns
    for b in list(range(0, 65536, 97)) + [0x7F80, 0xFF80, 0x7FC1, 0x43E0, 0x43E8]:
        assert oracle.bf16_to_e4m3(b) == brute.bf16_to_e4m3(b), hex(b)


# ------------------------------------------------------------------ exact rounding

def test_round_scaled_sum_matches_rational(oracle_lib):
    # The oracle's 384-bit exact sum + single rounding against Fraction
    # arithmetic. Cases include wide scale spans, cancellation, ties, fp32
    # subnormal results and overflow. Catches: double rounding, lost terms,
    # a wrong sign, a wrong exponent bias.
    rng = np.random.default_rng(7)
    cases = []
    for _ in range(3000):
        S = [int(rng.integers(-(1 << 26), 1 << 26)) / 1024.0 for _ in range(4)]
        mode = rng.integers(0, 4)
        if mode == 0:
            s = [int(x) for x in rng.integers(122, 128, 4)]
        elif mode == 1:
            s = [int(x) for x in rng.integers(100, 151, 4)]
        elif mode == 2:
            s = [int(x) for x in rng.integers(1, 255, 4)]
        else:
            s = [int(rng.integers(1, 255))] * 4
            S[1] = -S[0]                                  # exact cancellation
        sm = float(np.float32(rng.uniform(0.01, 2.0)))
        cases.append((S, s, sm))
    # hand-built ties: 2^24 + 1 (tie to even: down), 2^24 + 3 (tie: up)
    cases.append(([float(1 << 14), 1.0 / 1024, 0.0, 0.0], [137, 113, 127, 127], 1.0))
    cases.append(([float(1 << 14), 3.0 / 1024, 0.0, 0.0], [137, 113, 127, 127], 1.0))
    # subnormal fp32 result and overflow
    cases.append(([1.0 / 1024, 0.0, 0.0, 0.0], [1, 1, 1, 1], 0.5))
    cases.append(([86000.0, 86000.0, 0.0, 0.0], [254, 254, 254, 254], 1.0))
    for S, s, sm in cases:
        exact = sum((Fraction(S[k]) * Fraction(2) ** (s[k] - 127) for k in range(4)), Fraction(0)) * Fraction(sm)
        ref = brute.round_f32(exact)
        got = oracle.round_scaled_sum(S, s, sm)
        assert f32_bits(got) == f32_bits(ref) or (got == 0 and ref == 0), (S, s, sm, got, ref)


# ------------------------------------------------------------------ hand-worked pages

@pytest.mark.parametrize("case", load_hand_pages(), ids=lambda c: c["name"])
def test_hand_worked_pages(oracle_lib, case):
    # Values derived by hand (tests/golden/hand_pages.txt). Catches: nibble
    # order, scale-byte to block mapping, Q rounding, sign handling.
    c = single_token_case(case["q"], case["data"], case["scales"])
    r = run_c(c, want_mags=True, want_block_mags=True)
    got = r.logits[0, 0, 0]
    assert f32_bits(got) == case["bits"], (case["name"], hex(f32_bits(got)))
    exact = Fraction(case["dot"]) * Fraction(SM_SCALE)
    assert f32_bits(brute.round_f32(exact)) == case["bits"]
    assert r.blocks[0, 0, 0] == got
    lb, bb = run_brute(c)
    assert f32_bits(lb[0][0][0]) == case["bits"]


@pytest.mark.parametrize("case", load_hand_pages(), ids=lambda c: c["name"])
def test_hand_worked_magnitudes(oracle_lib, case):
    # M = sum_e |Q_hat[e] * K[e]| worked by hand (last field of
    # tests/golden/hand_pages.txt): the size of the terms a dot adds, which
    # bounds the rounding error of any summation order and so sets how far a
    # reordered (MFMA) sum may stray. The "alternating" and "crossblock" pages
    # cancel to a zero dot with M = 128 and 528. Catches: the e8m0 factor
    # dropped from M, sm_scale applied to M, |sum| instead of a sum of
    # magnitudes, M of dead tokens, a block M that is not the page maximum.
    c = single_token_case(case["q"], case["data"], case["scales"])
    r = run_c(c, want_mags=True, want_block_mags=True)
    assert r.mags[0, 0, 0] == case["mag"], (case["name"], r.mags[0, 0, 0])
    assert r.block_mags[0, 0, 0] == case["mag"]
    assert np.all(r.mags[0, 0, 1:] == 0.0)                          # no live token there
    _, _, mb = run_brute(c, want_mags=True)
    assert mb[0][0][0] == Fraction(case["mag"])
    # |dot| <= M, with equality iff no two products have opposite signs
    assert abs(case["dot"]) <= case["mag"]


@pytest.mark.parametrize("seed,q_dtype", [(0, "bf16"), (1, "e4m3")])
def test_magnitudes_match_fraction_twin_wide_bytes(oracle_lib, seed, q_dtype):
    # C oracle's M (double) against the twin's exact Fraction M on random tiny
    # batches with all 16 codes and e8m0 bytes 100..150 (a 2^50 spread of
    # block scales: the four scaled block sums of the C oracle are added in
    # double, so allow 2^-50 relative). Block M = the largest M among the
    # page's live tokens; dead tokens and pages have M = 0.
    rng = np.random.default_rng(300 + seed)
    P = 64
    c = random_case(rng, B=2, H=2, page_size=P, q_lens=[2, 1], prefix_lens=[64, 0], seq_lens=[66, 9],
                    q_dtype=q_dtype, scale_lo=100, scale_hi=150)
    W = 70
    r = run_c(c, page_size=P, max_seq_len=W, q_dtype=q_dtype, want_mags=True, want_block_mags=True)
    lb, _, mb = run_brute(c, page_size=P, max_seq_len=W, q_dtype=q_dtype, want_mags=True)
    NB = (W + P - 1) // P
    for row in range(r.mags.shape[0]):
        for h in range(2):
            for t in range(W):
                ref = mb[row][h][t]
                got = r.mags[row, h, t]
                if ref == 0:
                    assert got == 0.0
                else:
                    assert abs(Fraction(got) - ref) <= ref * Fraction(1, 2 ** 50), (row, h, t)
                    assert np.isfinite(lb[row][h][t])
            for j in range(NB):
                seg = [mb[row][h][t] for t in range(j * P, min((j + 1) * P, W))]
                assert abs(Fraction(r.block_mags[row, h, j]) - max(seg)) <= max(seg) * Fraction(1, 2 ** 50)


def test_magnitude_scale_shift_and_bound(oracle_lib):
    # +1 on every e8m0 byte doubles every M exactly (as it doubles every dot),
    # and every finite logit satisfies |logit| <= sm_scale * M up to one fp32
    # rounding (|dot| <= M). Catches: M taken without the e8m0 factors (it
    # would not double), M scaled by sm_scale (the bound would fail).
    rng = np.random.default_rng(17)
    c = random_case(rng, B=2, H=3, page_size=128, q_lens=[3, 2], prefix_lens=[129, 7], seq_lens=[132, 9],
                    scale_lo=110, scale_hi=140, garbage_tail=False)
    r0 = run_c(c, want_mags=True)
    r1 = run_c(dict(c, k_scale=c["k_scale"] + 1), want_mags=True)
    assert np.array_equal(r1.mags, 2.0 * r0.mags)
    fin = np.isfinite(r0.logits)
    lg = r0.logits[fin].astype(np.float64)
    m = r0.mags[fin]
    assert np.all(np.abs(lg) <= SM_SCALE * m * (1 + 2.0 ** -23))
    assert np.all(m[np.abs(lg) > 0] > 0)
    assert np.all(r0.mags[~fin] == 0.0)


def test_causal_prefix_example(oracle_lib):
    # prefix 2, two query rows, seq_len 4: row 0 sees tokens {0, 1, 2},
    # row 1 sees {0, 1, 2, 3} (inclusive diagonal). Catches: off-by-one mask.
    rng = np.random.default_rng(3)
    c = random_case(rng, B=1, H=1, page_size=64, q_lens=[2], prefix_lens=[2], seq_lens=[4], garbage_tail=True)
    r = run_c(c, page_size=64, max_seq_len=4)
    live = np.isfinite(r.logits[:, 0, :])
    assert live.tolist() == [[True, True, True, False], [True, True, True, True]]


def test_causal_limit_with_prefix_near_int32_max(oracle_lib):
    # The limit min(seq_len, prefix_len + i + 1) is a statement about
    # integers: with prefix 2^31 - 2 the sum passes 2^31 - 1 from the second
    # row on, and every row still sees its whole sequence. Catches: the sum
    # taken in int32 (wraps negative and masks the row out).
    rng = np.random.default_rng(4)
    c = random_case(rng, B=1, H=2, page_size=64, q_lens=[3], prefix_lens=[2**31 - 2], seq_lens=[70])
    r = run_c(c, page_size=64, max_seq_len=80)
    live = np.isfinite(r.logits)
    assert live[:, :, :70].all() and not live[:, :, 70:].any()
    assert np.array_equal(live[:, 0, :], _live_mask(c, "prefill", 80))


# ------------------------------------------------------------------ closed forms

def test_e4m3_exact_window_is_119_to_133(oracle_lib):
    # For every e2m1 code c, e2m1(c) * 2^(b-127) is an e4m3 value iff
    # 119 <= b <= 133 (aiter #7061, "Format"). Catches: a wrong e8m0 bias or a
    # wrong e4m3 decode range in the oracle.
    e4m3_set = {oracle.e4m3_value(b) for b in range(256) if not math.isnan(oracle.e4m3_value(b))}
    ok = []
    for b in range(1, 255):
        if all(oracle.e2m1_value(c) * oracle.e8m0_value(b) in e4m3_set for c in range(16)):
            ok.append(b)
    assert ok == list(range(119, 134))


def test_e4m3_dequant_path_matches_inside_window(oracle_lib):
    # Second path (the pages' fp8 judge): inside [119, 133] dequantize K to
    # e4m3, then an e4m3 x e4m3 dot in float64 (exact: 128 products of <= 8
    # significant bits within 2^-18..2^17) must equal the MXFP4 oracle bitwise.
    rng = np.random.default_rng(11)
    c = random_case(rng, B=2, H=3, page_size=64, q_lens=[3, 2], prefix_lens=[60, 0], seq_lens=[63, 130],
                    scale_lo=119, scale_hi=133, garbage_tail=False)
    r = run_c(c, page_size=64)
    val_to_code = {}
    for b in range(256):
        v = oracle.e4m3_value(b)
        if not math.isnan(v):
            val_to_code.setdefault(v, b)
    qhat = np.vectorize(lambda b: oracle.e4m3_value(oracle.bf16_to_e4m3(int(b))))(c["q"])
    T = c["q"].shape[0]
    cu = c["cu_seqlens_q"]
    for row in range(T):
        b = int(np.searchsorted(cu, row, side="right") - 1)
        limit = min(int(c["seq_lens"][b]), int(c["prefix_lens"][b]) + row - int(cu[b]) + 1)
        for t in range(limit):
            page = c["block_table"][b, t // 64]
            d = c["k_data"][page, t % 64]
            s = c["k_scale"][page, t % 64]
            codes = np.stack([d & 0xF, d >> 4], axis=1).reshape(-1)
            kv = np.array([oracle.e2m1_value(int(cc)) for cc in codes]) * np.repeat([oracle.e8m0_value(int(x)) for x in s], 32)
            k8 = np.array([oracle.e4m3_value(val_to_code[v]) for v in kv])   # dequantized to e4m3 bytes and back
            dots = qhat[row] @ k8
            for h in range(c["q"].shape[1]):
                ref = brute.round_f32(Fraction(float(dots[h])) * Fraction(SM_SCALE))
                assert f32_bits(r.logits[row, h, t]) == f32_bits(ref)


def test_scale_byte_shift_doubles_logits(oracle_lib):
    # +1 on every e8m0 byte multiplies every dot, hence every logit, by exactly
    # 2 (aiter #7061, "Validation": the +-1 scale-byte mutation). Catches: a
    # scale applied per token instead of per block, or not at all.
    rng = np.random.default_rng(5)
    c = random_case(rng, B=2, H=2, page_size=128, q_lens=[2, 3], prefix_lens=[130, 5], seq_lens=[132, 8],
                    scale_lo=110, scale_hi=140, garbage_tail=False)
    r0 = run_c(c)
    c2 = dict(c)
    c2["k_scale"] = c["k_scale"] + 1
    r1 = run_c(c2)
    fin = np.isfinite(r0.logits)
    assert np.array_equal(fin, np.isfinite(r1.logits))
    assert np.array_equal(r1.logits[fin], r0.logits[fin] * np.float32(2.0))
    assert np.array_equal(r1.blocks[np.isfinite(r0.blocks)], r0.blocks[np.isfinite(r0.blocks)] * np.float32(2.0))


def test_small_integer_dots(oracle_lib):
    # Q in {0, +-1, +-2}, K codes in {0, +-1, +-2}, scales 2^0: every dot is an
    # integer, computed here with an int64 matrix product. Catches: a transposed
    # operand, a dropped element, a wrong head or token index.
    rng = np.random.default_rng(9)
    H, P, L = 3, 64, 150
    qv = rng.choice([0.0, 1.0, -1.0, 2.0, -2.0], size=(1, H, 128)).astype(np.float32)
    q = (qv.view(np.uint32) >> 16).astype(np.uint16)
    code_of = {0.0: 0, 1.0: 2, -1.0: 10, 2.0: 4, -2.0: 12}
    kvals = rng.choice([0.0, 1.0, -1.0, 2.0, -2.0], size=(3, P, 128))
    codes = np.vectorize(code_of.get)(kvals).astype(np.uint8)
    k_data = (codes[:, :, 0::2] | (codes[:, :, 1::2] << 4)).astype(np.uint8)
    k_scale = np.full((3, P, 4), 127, np.uint8)
    bt = np.array([[2, 0, 1]], np.int32)
    c = dict(q=q, k_data=k_data, k_scale=k_scale, block_table=bt, seq_lens=np.array([L], np.int32),
             cu_seqlens_q=np.array([0, 1], np.int32), prefix_lens=np.array([L - 1], np.int32))
    r = run_c(c, page_size=P)
    kseq = np.concatenate([kvals[p] for p in bt[0]], axis=0)[:L].astype(np.int64)
    dots = qv[0].astype(np.int64) @ kseq.T                          # [H, L]
    for h in range(H):
        for t in range(L):
            ref = brute.round_f32(Fraction(int(dots[h, t])) * Fraction(SM_SCALE))
            assert f32_bits(r.logits[0, h, t]) == f32_bits(ref)


# ------------------------------------------------------------------ masks, layouts, modes

def _live_mask(c, mode, max_seq_len):
    rows = []
    B = len(c["seq_lens"])
    if mode == "decode":
        for b in range(B):
            rows.append(min(int(c["seq_lens"][b]), max_seq_len))
    else:
        cu = c["cu_seqlens_q"]
        for b in range(B):
            for i in range(int(cu[b + 1] - cu[b])):
                rows.append(min(int(c["seq_lens"][b]), int(c["prefix_lens"][b]) + i + 1, max_seq_len))
    m = np.zeros((len(rows), max_seq_len), bool)
    for r, lim in enumerate(rows):
        m[r, :max(lim, 0)] = True
    return m


@pytest.mark.parametrize("seed", range(4))
def test_masks_brute_force_with_garbage(oracle_lib, seed):
    # Ragged batch, mid-page prefixes, a trailing empty request, garbage (NaN
    # scales) past every request's end. The oracle's -inf pattern must equal
    # the enumerated live set and no NaN may appear. Catches: dead tokens
    # leaking, window past seq_len, empty requests scored.
    rng = np.random.default_rng(100 + seed)
    P = 64
    q_lens = [3, 1, 4, 0]
    prefix = [70, 0, 125, 10]
    seq = [73, 1, 128, 10]
    c = random_case(rng, B=4, H=2, page_size=P, q_lens=q_lens, prefix_lens=prefix, seq_lens=seq)
    W = 140
    r = run_c(c, page_size=P, max_seq_len=W)
    live = _live_mask(c, "prefill", W)
    for h in range(2):
        assert np.array_equal(np.isfinite(r.logits[:, h, :]), live)
        blive = np.stack([live[:, j * P:(j + 1) * P].any(axis=1) for j in range((W + P - 1) // P)], axis=1)
        assert np.array_equal(np.isfinite(r.blocks[:, h, :]), blive)
    assert not np.isnan(r.logits).any() and not np.isnan(r.blocks).any()


def test_split_and_single_region_layouts_agree(oracle_lib):
    # Same bytes through split views and through single-region pages
    # [P x 64 B data][P x 4 B scale] with page stride 8704 (aiter #7061,
    # "Format": both layouts must agree bitwise). Catches: page stride ignored.
    rng = np.random.default_rng(21)
    P = 128
    c = random_case(rng, B=2, H=2, page_size=P, q_lens=[2, 1], prefix_lens=[200, 0], seq_lens=[202, 77])
    npg = c["k_data"].shape[0]
    region = np.zeros((npg, P * 68), np.uint8)
    region[:, :P * 64] = c["k_data"].reshape(npg, -1)
    region[:, P * 64:] = c["k_scale"].reshape(npg, -1)
    kd = np.lib.stride_tricks.as_strided(region, (npg, P, 64), (P * 68, 64, 1))
    ks = np.lib.stride_tricks.as_strided(region[:, P * 64:], (npg, P, 4), (P * 68, 4, 1))
    r0 = run_c(c)
    c1 = dict(c, k_data=kd, k_scale=ks)
    r1 = run_c(c1)
    assert r1.logits.tobytes() == r0.logits.tobytes() and r1.blocks.tobytes() == r0.blocks.tobytes()


def test_page_permutation_invariance_and_wrong_map(oracle_lib):
    # Physical page order is irrelevant once the table is remapped; a wrong
    # map must change the scores (aiter #5518, "Correctness": shuffled pages,
    # deliberately wrong page map detected).
    rng = np.random.default_rng(31)
    P = 64
    c = random_case(rng, B=2, H=2, page_size=P, q_lens=[2, 2], prefix_lens=[100, 50], seq_lens=[102, 52],
                    garbage_tail=False)
    r0 = run_c(c, page_size=P)
    npg = c["k_data"].shape[0]
    perm = rng.permutation(npg)
    inv = np.argsort(perm)
    bt = c["block_table"].copy()
    bt[bt >= 0] = inv[bt[bt >= 0]]
    c1 = dict(c, k_data=c["k_data"][perm].copy(), k_scale=c["k_scale"][perm].copy(), block_table=bt)
    r1 = run_c(c1, page_size=P)
    assert r1.logits.tobytes() == r0.logits.tobytes()
    bad = c["block_table"].copy()
    bad[0, 0], bad[0, 1] = bad[0, 1], bad[0, 0]
    r2 = run_c(dict(c, block_table=bad), page_size=P)
    assert r2.logits.tobytes() != r0.logits.tobytes()


def test_decode_equals_prefill_with_one_row(oracle_lib):
    # Decode is prefill with one row per request and prefix seq_len - 1; the
    # block score equals the max of the same row's logits per page.
    rng = np.random.default_rng(41)
    P = 128
    seq = [300, 128, 1, 0]
    c = random_case(rng, B=4, H=3, page_size=P, q_lens=[1, 1, 1, 1], prefix_lens=[s - 1 for s in seq], seq_lens=seq)
    W = 300
    rp = run_c(c, page_size=P, max_seq_len=W)
    rd = run_c(dict(c, cu_seqlens_q=None, prefix_lens=None), mode="decode", page_size=P, max_seq_len=W)
    assert rp.logits.tobytes() == rd.logits.tobytes() and rp.blocks.tobytes() == rd.blocks.tobytes()
    for j in range(rd.blocks.shape[2]):
        seg = rd.logits[:, :, j * P:(j + 1) * P]
        assert np.array_equal(seg.max(axis=2), rd.blocks[:, :, j])


def test_row_subset_matches_full(oracle_lib):
    rng = np.random.default_rng(51)
    c = random_case(rng, B=2, H=2, page_size=64, q_lens=[5, 3], prefix_lens=[60, 2], seq_lens=[65, 5])
    full = run_c(c, page_size=64)
    rows = np.array([7, 0, 4], np.int32)
    sub = run_c(c, page_size=64, rows=rows)
    assert sub.logits.tobytes() == full.logits[rows].tobytes()


@pytest.mark.parametrize("seed,q_dtype", [(0, "bf16"), (1, "e4m3"), (2, "bf16")])
def test_c_and_python_oracles_agree(oracle_lib, seed, q_dtype):
    # Two independent implementations, bitwise, on tiny random inputs with all
    # 16 codes and e8m0 bytes 100..150.
    rng = np.random.default_rng(200 + seed)
    c = random_case(rng, B=2, H=2, page_size=64, q_lens=[2, 1], prefix_lens=[64, 0], seq_lens=[66, 9],
                    q_dtype=q_dtype, scale_lo=100, scale_hi=150)
    W = 70
    r = run_c(c, page_size=64, max_seq_len=W, q_dtype=q_dtype)
    lb, bb = run_brute(c, page_size=64, max_seq_len=W, q_dtype=q_dtype)
    assert np.array(lb, np.float32).tobytes() == r.logits.tobytes()
    assert np.array(bb, np.float32).tobytes() == r.blocks.tobytes()

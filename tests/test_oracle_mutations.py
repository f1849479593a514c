"""Plant plausible mistakes in the pure-Python oracle twin and check that the
hand-worked pins reject each one (the pins are only worth something if a
wrong oracle fails them). Mirrors the mutation checks of aiter #7061
("Validation": a wrong e8m0 byte, a shifted scale byte)."""
import struct
from fractions import Fraction

import numpy as np
import pytest

from oracle import brute
from tests.oracle_cases import load_hand_pages, random_case, run_brute, single_token_case


def _bits(x):
    return struct.unpack("<I", struct.pack("<f", np.float32(x)))[0]


def _hand_pins_pass():
    for case in load_hand_pages():
        lb, _ = run_brute(single_token_case(case["q"], case["data"], case["scales"]))
        if _bits(lb[0][0][0]) != case["bits"]:
            return False
    return True


def _hand_mag_pins_pass():
    for case in load_hand_pages():
        _, _, mb = run_brute(single_token_case(case["q"], case["data"], case["scales"]), want_mags=True)
        if mb[0][0][0] != Fraction(case["mag"]):
            return False
    return True


def _swapped_nibbles(data_page, scale_page, slot):
    out = []
    for e in range(128):
        byte = data_page[slot * 64 + e // 2]
        code = (byte & 0xF) if e % 2 else (byte >> 4)
        out.append(brute.e2m1(code) * brute.e8m0(scale_page[slot * 4 + e // 32]))
    return out


def _scale_per_16(data_page, scale_page, slot):
    out = []
    for e in range(128):
        byte = data_page[slot * 64 + e // 2]
        code = (byte >> 4) if e % 2 else (byte & 0xF)
        out.append(brute.e2m1(code) * brute.e8m0(scale_page[slot * 4 + (e // 16) % 4]))
    return out


def _truncating_e4m3(bits):
    sign = 0x80 if bits & 0x8000 else 0
    a = abs(brute.bf16_value(bits))
    best = 0
    for code, val in brute._E4M3_POS:
        if val <= a:
            best = code
    return sign | best


_ORIG_E2M1 = brute.e2m1


def _unsigned_e2m1(code):
    return abs(Fraction(_ORIG_E2M1(code)))


def _bias_128(byte):
    return None if byte == 255 else Fraction(2) ** (byte - 128)


@pytest.mark.parametrize("target,replacement", [
    ("token_k", _swapped_nibbles),
    ("token_k", _scale_per_16),
    ("bf16_to_e4m3", _truncating_e4m3),
    ("e2m1", _unsigned_e2m1),
    ("e8m0", _bias_128),
])
def test_planted_mistake_is_caught(monkeypatch, target, replacement):
    assert _hand_pins_pass()
    monkeypatch.setattr(brute, target, replacement)
    assert not _hand_pins_pass(), f"planted mistake in {target} was not caught"


def test_planted_off_by_one_mask_is_caught(monkeypatch):
    rng = np.random.default_rng(3)
    c = random_case(rng, B=1, H=1, page_size=64, q_lens=[2], prefix_lens=[2], seq_lens=[4], garbage_tail=False)
    lb, _ = run_brute(c, page_size=64, max_seq_len=4)
    good = [[np.isfinite(v) for v in row[0]] for row in lb]
    assert good == [[True, True, True, False], [True, True, True, True]]
    orig = brute.score

    def exclusive_diagonal(**kw):
        kw = dict(kw)
        kw["prefix_lens"] = [p - 1 for p in kw["prefix_lens"]]
        return orig(**kw)

    monkeypatch.setattr(brute, "score", exclusive_diagonal)
    lb2, _ = run_brute(c, page_size=64, max_seq_len=4)
    assert [[np.isfinite(v) for v in row[0]] for row in lb2] != good


# Planted mistakes in the twin's M (sum_e |Q_hat[e] K[e]|): each must fail the
# hand-worked M of tests/golden/hand_pages.txt.
_ORIG_MAG = brute.token_mag
_SM = Fraction(float(np.uint32(0x3DB504F3).view(np.float32)))


def _mag_without_e8m0(qh, data_page, scale_page, slot):
    return _ORIG_MAG(qh, data_page, bytes([127]) * len(scale_page), slot)


def _mag_with_sm_scale(qh, data_page, scale_page, slot):
    return _ORIG_MAG(qh, data_page, scale_page, slot) * _SM


def _mag_of_signed_sum(qh, data_page, scale_page, slot):
    k = brute.token_k(data_page, scale_page, slot)
    return abs(sum((qh[e] * k[e] for e in range(128)), Fraction(0)))


@pytest.mark.parametrize("replacement", [_mag_without_e8m0, _mag_with_sm_scale, _mag_of_signed_sum])
def test_planted_magnitude_mistake_is_caught(monkeypatch, replacement):
    assert _hand_mag_pins_pass()
    monkeypatch.setattr(brute, "token_mag", replacement)
    assert not _hand_mag_pins_pass(), f"planted mistake {replacement.__name__} was not caught"

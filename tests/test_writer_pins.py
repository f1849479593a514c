"""Pins for the MXFP4 writer oracle (oracle/writer.py).

The rule is the OCP MX conversion (a reading: the pages give none). It is
pinned by hand-worked blocks, by properties that characterise it without
re-typing it (the scale puts amax/2^e in [4, 8); every element decodes to the
grid value nearest to it, ties to the even code), and by the scorer oracle's
own decoders reading the written page (nibble order, scale placement).
Planted mistakes must each break a pin."""
import math
import struct

import numpy as np
import pytest

import oracle
from oracle import writer


def bf16_bits(x: float) -> int:
    """bf16 pattern of x (x must be exactly representable in bf16)."""
    b = struct.unpack("<I", struct.pack("<f", x))[0]
    assert b & 0xFFFF == 0, x
    return b >> 16


def block(vals):
    return writer.quantize_block([writer.bf16_value(bf16_bits(v)) for v in vals])


def test_hand_worked_blocks():
    # amax 1 -> floor(log2) 0 -> e = -2, byte 125; 1 / 2^-2 = 4 -> code 6
    assert block([1.0] * 32) == (125, [6] * 32)
    # amax 6 -> e = 0, byte 127; exact grid values keep their codes
    assert block([6.0, -3.0, 0.5, 0.0] + [0.0] * 28) == (127, [7, 8 | 5, 1, 0] + [0] * 28)
    # ties go to the even code: 0.25->0, 0.75->1.0, 1.25->1.0, 1.75->2, 2.5->2, 3.5->4, 5->4
    b, c = block([6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0] + [0.0] * 24)
    assert b == 127 and c[:8] == [7, 0, 2, 2, 4, 4, 6, 6]
    # amax 7 (binade of 4) -> e = 0; 7 saturates to 6
    b, c = block([7.0, -7.0] + [0.0] * 30)
    assert b == 127 and c[:2] == [7, 15]
    # signed zero keeps its sign bit; a zero block gets byte 1
    b, c = block([-0.0, 0.0] + [0.0] * 30)
    assert b == 1 and c[:2] == [8, 0]
    # large and tiny magnitudes: 2^100 -> byte 225; 2^-130 clips to byte 1 and rounds to 0
    assert block([2.0 ** 100] + [0.0] * 31)[0] == 225
    b, c = block([2.0 ** -130] + [0.0] * 31)
    assert b == 1 and c[0] == 0


def _grid(e):
    return [(code, math.copysign(1.0, -1.0 if code & 8 else 1.0) * oracle.e2m1_value(code & 7) * 2.0 ** e)
            for code in range(16)]


@pytest.mark.parametrize("seed", range(12))
def test_random_blocks_satisfy_the_definition(seed):
    rng = np.random.default_rng(seed)
    scale = 2.0 ** rng.integers(-40, 40)
    x = (rng.standard_normal(32) * scale).astype(np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint32)          # truncate to bf16 patterns
    vals = [writer.bf16_value(int(b)) for b in bits]
    byte, codes = writer.quantize_block(vals)
    amax = max(abs(v) for v in vals)
    e = byte - 127
    if 1 < byte < 254:
        assert 4.0 <= amax / 2.0 ** e < 8.0
    for v, code in zip(vals, codes):
        d = oracle.e2m1_value(code) * 2.0 ** e
        dist = abs(v - d)
        for other, g in _grid(e):
            if abs(v) >= 6 * 2.0 ** e and abs(g) == 6 * 2.0 ** e and (g > 0) == (v > 0):
                continue
            assert dist <= abs(v - g) + 0.0, (v, code, other)
            if abs(v - g) == dist and other != code and (other & 7) != (code & 7):
                assert (code & 1) == 0, (v, code, other)   # ties to the even code


def test_written_page_decodes_with_the_scorer_oracle():
    # one token, element 1 = 6.0, everything else 0; element 70 = -0.5 in block 2
    bits = np.zeros(128, dtype=np.uint16)
    bits[1] = bf16_bits(6.0)
    bits[70] = bf16_bits(-0.5)
    kd = np.zeros((3, 64, 64), dtype=np.uint8)
    ks = np.zeros((3, 64, 4), dtype=np.uint8)
    writer.write_pages(bits[None], [2 * 64 + 5], kd, ks, 64)      # page 2, slot 5
    data, scale = kd[2, 5], ks[2, 5]
    # element 1: 6.0 / 2^0 -> code 7 (high nibble of byte 0); element 70: block amax 0.5 ->
    # e = -3, -0.5 / 2^-3 = -4 -> code 0xE (low nibble of byte 35)
    assert data[0] == 0x70 and data[35] == 0x0E and int(data.sum()) == 0x70 + 0x0E
    assert list(scale) == [127, 1, 124, 1]
    for i, want in [(1, 6.0), (70, -0.5), (0, 0.0)]:
        code = (data[i // 2] >> (4 * (i % 2))) & 0xF
        sgn = -1.0 if code & 8 else 1.0
        assert sgn * oracle.e2m1_value(code & 7) * oracle.e8m0_value(int(scale[i // 32])) == want
    assert kd[:2].sum() == 0 and ks[:2].sum() == 0 and kd[2, 4].sum() == 0   # nothing else written
    writer.write_pages(bits[None], [-1], kd, ks, 64)                 # slot -1 writes nothing


def _mutant_floor(vals):
    amax = max(abs(v) for v in vals)
    m, ex = math.frexp(amax) if amax else (0, 0)
    byte = min(254, max(1, (ex - 1) - 1 + 127)) if amax else 1   # exponent one too high
    e = byte - 127
    return byte, [writer.e2m1_code(math.ldexp(v, -e)) for v in vals]


_ORIG_BLOCK = writer.quantize_block


def _mutant_ties(vals):
    byte, _ = _ORIG_BLOCK(vals)
    e = byte - 127
    out = []
    for v in vals:
        a = abs(math.ldexp(v, -e))
        best = min(range(8), key=lambda c: (abs(a - writer._E2M1[c]), -c))   # ties away from zero
        out.append((8 if v < 0 else 0) | best)
    return byte, out


@pytest.mark.parametrize("mutant", [_mutant_floor, _mutant_ties])
def test_planted_mistakes_are_caught(monkeypatch, mutant):
    monkeypatch.setattr(writer, "quantize_block", mutant)
    with pytest.raises(AssertionError):
        test_hand_worked_blocks()


def test_fp8_cache_writer_hand_worked():
    # fp8 cache: each element is rounded like the query (nearest e4m3, ties to
    # even, saturating): 1.0 -> 0x38, 448 -> 0x7E, 500 -> 0x7E (saturated),
    # -0.0 -> 0x80, 1.0625 -> 0x38 (tie to even), 1.1875 -> 0x3A (tie to even);
    # element e at byte e of the token's 128-byte row.
    bits = np.zeros((2, 128), dtype=np.uint16)
    vals = [1.0, 448.0, 500.0, -0.0, 1.0625, 1.1875]
    for e, v in enumerate(vals):
        bits[1, 10 + e] = bf16_bits(v)
    kd = np.zeros((2, 64, 128), dtype=np.uint8)
    writer.write_pages_e4m3(bits, [-1, 64 + 3], kd, 64)                  # token 0 skipped; token 1 -> page 1, slot 3
    row = kd[1, 3]
    assert list(row[10:16]) == [0x38, 0x7E, 0x7E, 0x80, 0x38, 0x3A]
    assert int(row.sum()) == sum([0x38, 0x7E, 0x7E, 0x80, 0x38, 0x3A])
    assert kd[0].sum() == 0 and kd[1, :3].sum() == 0 and kd[1, 4:].sum() == 0

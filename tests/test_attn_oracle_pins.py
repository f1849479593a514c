"""Pins for the paged MXFP4 attention-decode oracle (oracle/attn.py).

Pinned by closed forms (one token, a zero query, two tokens), by an
independent dequantisation (the Fraction twin's decoders) feeding scipy's
softmax, by the grouped-query head mapping, masking and page-permutation
properties, and by planted mistakes that must each break a pin."""
import math
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import softmax

import oracle
from oracle import attn, brute

SCALE = float(np.float32(1.0 / math.sqrt(128.0)))


def bf16(x):
    b = np.array([x], np.float32).view(np.uint32)[0]
    assert b & 0xFFFF == 0, x
    return int(b >> 16)


def cache(pool, Hkv, P, rng=None, fill=None, scale_lo=122, scale_hi=127):
    """K and V views [pool, Hkv, P, 64|4]."""
    rng = rng or np.random.default_rng(0)
    kd = rng.integers(0, 256, (pool, Hkv, P, 64), dtype=np.uint8) if fill is None else np.full((pool, Hkv, P, 64), fill, np.uint8)
    vd = rng.integers(0, 256, (pool, Hkv, P, 64), dtype=np.uint8) if fill is None else np.full((pool, Hkv, P, 64), fill, np.uint8)
    ks = rng.integers(scale_lo, scale_hi + 1, (pool, Hkv, P, 4), dtype=np.uint8)
    vs = rng.integers(scale_lo, scale_hi + 1, (pool, Hkv, P, 4), dtype=np.uint8)
    return kd, ks, vd, vs


def run(q, kd, ks, vd, vs, bt, ctx, P, q_dtype="bf16", **kw):
    return attn.attn_decode(q=q, q_dtype=q_dtype, k_data=kd, k_scale=ks, v_data=vd, v_scale=vs, block_table=bt,
                            context_lens=np.asarray(ctx), page_size=P, scale=SCALE, **kw)


def brute_tokens(data, scale):
    """Independent dequantisation with the Fraction twin: [..., 64] + [..., 4] -> float [..., 128]."""
    flat_d = data.reshape(-1, 64)
    flat_s = scale.reshape(-1, 4)
    out = np.zeros((flat_d.shape[0], 128))
    for n in range(flat_d.shape[0]):
        out[n] = [float(v) for v in brute.token_k(bytes(flat_d[n]), bytes(flat_s[n]), 0)]
    return out.reshape(data.shape[:-1] + (128,))


def test_one_token_returns_its_value():
    rng = np.random.default_rng(1)
    kd, ks, vd, vs = cache(2, 1, 64, rng)
    q = (rng.standard_normal((1, 4, 128)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    out = run(q, kd, ks, vd, vs, np.array([[1, 0]], np.int32), [1], 64)
    v0 = brute_tokens(vd[1, 0, 0], vs[1, 0, 0])
    for h in range(4):
        assert np.array_equal(out[0, h], v0)


def test_zero_query_averages_the_values():
    rng = np.random.default_rng(2)
    kd, ks, vd, vs = cache(3, 1, 64, rng)
    q = np.zeros((1, 2, 128), np.uint16)
    ctx = 150
    out = run(q, kd, ks, vd, vs, np.array([[2, 0, 1]], np.int32), [ctx], 64)
    t = np.arange(ctx)
    pages = np.array([2, 0, 1])[t // 64]
    vals = brute_tokens(vd[pages, 0, t % 64], vs[pages, 0, t % 64])
    exact = [sum(Fraction(float(x)) for x in vals[:, e]) / ctx for e in range(128)]
    assert np.allclose(out[0, 0], [float(x) for x in exact], rtol=1e-13, atol=1e-13 * np.abs(vals).max())
    assert np.array_equal(out[0, 0], out[0, 1])


def test_two_tokens_closed_form():
    # Q one-hot at element 0 (1.0); K0[0] = 6 * 2^0, K1[0] = 1 * 2^0 (codes 7 and 2, scale 127):
    # s0 - s1 = 5 * SCALE; V0 = all 1.0, V1 = all -2.0 (codes 2 and 12)
    kd = np.zeros((1, 1, 64, 64), np.uint8)
    ks = np.full((1, 1, 64, 4), 127, np.uint8)
    kd[0, 0, 0, 0], kd[0, 0, 1, 0] = 0x07, 0x02
    vd = np.zeros((1, 1, 64, 64), np.uint8)
    vd[0, 0, 0, :], vd[0, 0, 1, :] = 0x22, 0xCC
    vs = np.full((1, 1, 64, 4), 127, np.uint8)
    q = np.zeros((1, 1, 128), np.uint16)
    q[0, 0, 0] = bf16(1.0)
    out = run(q, kd, ks, vd, vs, np.array([[0]], np.int32), [2], 64)
    e0, e1 = math.exp(6 * SCALE), math.exp(1 * SCALE)
    want = (e0 * 1.0 + e1 * -2.0) / (e0 + e1)
    assert np.allclose(out[0, 0], want, rtol=1e-15)


@pytest.mark.parametrize("seed,q_dtype", [(3, "bf16"), (4, "e4m3")])
def test_matches_scipy_softmax_on_independent_dequant(seed, q_dtype):
    rng = np.random.default_rng(seed)
    P, Hkv, G = 64, 2, 3
    kd, ks, vd, vs = cache(5, Hkv, P, rng)
    R = 3
    if q_dtype == "bf16":
        q = (rng.standard_normal((R, Hkv * G, 128)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    else:
        q = rng.integers(0, 256, (R, Hkv * G, 128), dtype=np.uint8)
        q[(q & 0x7F) == 0x7F] = 0x38
    bt = np.array([[4, 1, 0], [2, 3, 0], [0, 0, 0]], np.int32)
    ctx = [130, 65, 1]
    out = run(q, kd, ks, vd, vs, bt, ctx, P, q_dtype=q_dtype)
    for r in range(R):
        t = np.arange(ctx[r])
        pages = bt[r, t // P]
        for h in range(Hkv * G):
            hk = h // G
            K = brute_tokens(kd[pages, hk, t % P], ks[pages, hk, t % P])
            V = brute_tokens(vd[pages, hk, t % P], vs[pages, hk, t % P])
            bits = q[r, h]
            qv = np.array([float(brute.e4m3(brute.bf16_to_e4m3(int(b)) if q_dtype == "bf16" else int(b))) for b in bits])
            w = softmax(SCALE * (K @ qv))
            assert np.allclose(out[r, h], w @ V, rtol=1e-12, atol=1e-12 * np.abs(V).max())


def test_grouped_query_heads_use_their_kv_head():
    # Hkv = 2, G = 2: kv head 0 holds V = +1, kv head 1 holds V = -1
    kd, ks, vd, vs = cache(1, 2, 64, fill=0x00)
    vd[:, 0], vd[:, 1] = 0x22, 0xAA
    q = np.zeros((1, 4, 128), np.uint16)
    out = run(q, kd, ks, vd, vs, np.array([[0]], np.int32), [10], 64)
    assert np.all(out[0, 0:2] > 0) and np.all(out[0, 2:4] < 0)


def test_empty_rows_and_garbage_past_the_context():
    rng = np.random.default_rng(6)
    kd, ks, vd, vs = cache(2, 1, 64, rng)
    q = (rng.standard_normal((2, 2, 128)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    bt = np.array([[0, 1], [1, 0]], np.int32)
    clean = run(q, kd, ks, vd, vs, bt, [70, 0], 64)
    kd2, ks2, vd2, vs2 = kd.copy(), ks.copy(), vd.copy(), vs.copy()
    ks2[1, 0, 6:], vs2[1, 0, 6:] = 255, 255          # e8m0 NaN past token 70 of row 0
    kd2[1, 0, 6:], vd2[1, 0, 6:] = 0xFF, 0xFF
    dirty = run(q, kd2, ks2, vd2, vs2, bt, [70, 0], 64)
    assert np.array_equal(clean, dirty)
    assert np.all(clean[1] == 0.0)


def test_page_permutation_invariance():
    rng = np.random.default_rng(7)
    kd, ks, vd, vs = cache(4, 1, 64, rng)
    q = (rng.standard_normal((1, 2, 128)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    bt = np.array([[3, 0, 2]], np.int32)
    a = run(q, kd, ks, vd, vs, bt, [170], 64)
    perm = np.array([2, 3, 1, 0])                          # new page n holds old page perm[n]
    inv = np.argsort(perm)
    b = run(q, kd[perm], ks[perm], vd[perm], vs[perm], inv[bt].astype(np.int32), [170], 64)
    assert np.array_equal(a, b)


def test_large_logits_select_the_best_token():
    # scale byte 140 on K token 2 makes its logit ~ 2^13 larger: the output is its V
    kd, ks, vd, vs = cache(1, 1, 64, fill=0x22)            # K = V = 1.0 everywhere
    ks[0, 0, 2] = 140
    vd[0, 0, 2] = 0x77                                     # V = 6.0 at token 2
    vs[0, 0, 2] = 127
    q = np.full((1, 1, 128), bf16(1.0), np.uint16)
    out = run(q, kd, ks, vd, vs, np.array([[0]], np.int32), [5], 64)
    assert np.allclose(out[0, 0], 6.0, rtol=1e-12)


_ORIG_DEQ = attn.dequant_tokens


def _swapped_nibbles(data, scale):
    e2m1 = np.array([oracle.e2m1_value(c) for c in range(16)])
    codes = np.stack([data >> 4, data & 0xF], axis=-1).reshape(data.shape[:-1] + (128,))
    return e2m1[codes] * np.ldexp(1.0, np.repeat(scale.astype(np.int64), 32, axis=-1) - 127)


def _no_scale(data, scale):
    return _ORIG_DEQ(data, np.full_like(scale, 127))


@pytest.mark.parametrize("mutant", [_swapped_nibbles, _no_scale])
def test_planted_mistakes_are_caught(monkeypatch, mutant):
    monkeypatch.setattr(attn, "dequant_tokens", mutant)
    with pytest.raises(AssertionError):
        test_one_token_returns_its_value()
        test_large_logits_select_the_best_token()


def test_planted_head_mapping_is_caught(monkeypatch):
    orig = attn.attn_decode

    def wrong(**kw):
        # kv head h % Hkv instead of h // G: swap the middle heads' outputs
        out = orig(**kw)
        return out[:, [0, 2, 1, 3]]
    monkeypatch.setattr(attn, "attn_decode", wrong)
    with pytest.raises(AssertionError):
        test_grouped_query_heads_use_their_kv_head()

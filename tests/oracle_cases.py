"""Test-side helpers: build tiny hand-specified caches and run the oracles on them."""
from __future__ import annotations

import os
from typing import Dict, List

import numpy as np

import oracle
from oracle import brute

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
SM_SCALE = float(np.uint32(0x3DB504F3).view(np.float32))   # RN32(1/sqrt(128))


def parse_assign(spec: str, n: int, width: int) -> List[int]:
    """'all=X', 'i=X j=Y ...' or 'a-b=X' (hex values, index ranges inclusive) -> list of n ints."""
    out = [0] * n
    for tok in spec.split():
        k, v = tok.split("=")
        if k == "all":
            out = [int(v, 16)] * n
        elif "-" in k:
            lo, hi = (int(x) for x in k.split("-"))
            for i in range(lo, hi + 1):
                out[i] = int(v, 16)
        else:
            out[int(k)] = int(v, 16)
    for x in out:
        assert 0 <= x < (1 << width)
    return out


def load_hand_pages() -> List[Dict]:
    cases = []
    with open(os.path.join(GOLDEN, "hand_pages.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, q, data, scales, dot, bits, mag = [x.strip() for x in line.split("|")]
            cases.append(dict(name=name, q=parse_assign(q, 128, 16), data=parse_assign(data, 64, 8),
                              scales=[int(x) for x in scales.split()], dot=float(dot), bits=int(bits, 16),
                              mag=float(mag)))
    return cases


def single_token_case(q_bits: List[int], data: List[int], scales: List[int], page_size: int = 128):
    """One request, one query row, one live token in slot 0 of page 0; other slots zero."""
    P = page_size
    k_data = np.zeros((1, P, 64), np.uint8)
    k_scale = np.full((1, P, 4), 127, np.uint8)
    k_data[0, 0, :] = data
    k_scale[0, 0, :] = scales
    q = np.array(q_bits, np.uint16).reshape(1, 1, 128)
    return dict(q=q, k_data=k_data, k_scale=k_scale, block_table=np.zeros((1, 1), np.int32),
                seq_lens=np.array([1], np.int32), cu_seqlens_q=np.array([0, 1], np.int32),
                prefix_lens=np.array([0], np.int32))


def run_c(case, *, mode="prefill", q_dtype="bf16", page_size=128, max_seq_len=None, sm_scale=SM_SCALE,
          want_mags=False, **kw):
    ms = max_seq_len if max_seq_len is not None else int(np.max(case["seq_lens"])) if len(case["seq_lens"]) else 0
    return oracle.score(mode=mode, q=case["q"], q_dtype=q_dtype, k_data=case["k_data"], k_scale=case["k_scale"],
                        page_size=page_size, block_table=case["block_table"], seq_lens=case["seq_lens"],
                        max_seq_len=ms, sm_scale=sm_scale, cu_seqlens_q=case.get("cu_seqlens_q"),
                        prefix_lens=case.get("prefix_lens"), want_mags=want_mags, **kw)


def run_brute(case, *, mode="prefill", q_dtype="bf16", page_size=128, max_seq_len=None, sm_scale=SM_SCALE,
              want_mags=False):
    ms = max_seq_len if max_seq_len is not None else int(np.max(case["seq_lens"])) if len(case["seq_lens"]) else 0
    q = case["q"]
    q_rows = [[list(map(int, q[r, h])) for h in range(q.shape[1])] for r in range(q.shape[0])]
    pages_data = [bytes(case["k_data"][p].reshape(-1)) for p in range(case["k_data"].shape[0])]
    pages_scale = [bytes(case["k_scale"][p].reshape(-1)) for p in range(case["k_scale"].shape[0])]
    bt = [list(map(int, row)) for row in case["block_table"]]
    kw = dict(mode=mode, q_rows=q_rows, q_dtype=q_dtype, pages_data=pages_data, pages_scale=pages_scale,
              page_size=page_size, block_table=bt, seq_lens=list(map(int, case["seq_lens"])),
              max_seq_len=ms, sm_scale=sm_scale,
              cu_seqlens_q=None if case.get("cu_seqlens_q") is None else list(map(int, case["cu_seqlens_q"])),
              prefix_lens=None if case.get("prefix_lens") is None else list(map(int, case["prefix_lens"])))
    if want_mags:
        return brute.score_mags(**kw)
    return brute.score(**kw)


def random_case(rng: np.random.Generator, *, B: int, H: int, page_size: int, q_lens, prefix_lens, seq_lens,
                q_dtype="bf16", scale_lo=122, scale_hi=127, pool_extra=2, garbage_tail=True):
    """Small random batch. Pages past each request's live window are filled with
    garbage (e2m1 -6 and e8m0 255 = NaN) so that any leak of a dead token shows."""
    P = page_size
    npr = [(s + P - 1) // P for s in seq_lens]
    width = max(npr + [1]) + 1
    pool = sum(npr) + pool_extra
    k_data = rng.integers(0, 256, (pool, P, 64), dtype=np.uint8)
    k_scale = rng.integers(scale_lo, scale_hi + 1, (pool, P, 4), dtype=np.uint8)
    perm = rng.permutation(pool)
    bt = np.full((B, width), -1, np.int32)
    pos = 0
    for b in range(B):
        bt[b, :npr[b]] = perm[pos:pos + npr[b]]
        pos += npr[b]
        if garbage_tail and seq_lens[b] % P:
            last = bt[b, npr[b] - 1]
            k_data[last, seq_lens[b] % P:] = 0xFF
            k_scale[last, seq_lens[b] % P:] = 255
    T = int(sum(q_lens))
    if q_dtype == "bf16":
        x = rng.standard_normal((T, H, 128)).astype(np.float32)
        q = (x.view(np.uint32) >> 16).astype(np.uint16)        # truncated bf16 bits: any bf16 pattern will do
    else:
        q = rng.integers(0, 256, (T, H, 128), dtype=np.uint8)
        q[(q & 0x7F) == 0x7F] = 0x38                           # no NaN queries
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    return dict(q=q, k_data=k_data, k_scale=k_scale, block_table=bt, seq_lens=np.array(seq_lens, np.int32),
                cu_seqlens_q=cu, prefix_lens=np.array(prefix_lens, np.int32))

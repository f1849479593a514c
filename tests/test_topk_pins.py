"""Pins for the top-k page selection oracle (oracle/topk.py).

The selection is fixed by properties that determine it uniquely: the
tail page is in, the result has min(k, live) pages, every chosen page
beats (score, then lower index) every live page left out, the result is
ascending and padded with -1. The pins check those properties on seeded
random cases with many ties, plus hand-worked cases; planted mistakes in a
copy of the selection must each break one of them."""
import numpy as np
import pytest

from oracle import topk


def _beats(s, a, b):
    return s[a] > s[b] or (s[a] == s[b] and a < b)


def check_selection(scores, limits, P, k, out):
    """Raise AssertionError unless out is the selection the reading defines."""
    R, H, NB = scores.shape
    assert out.shape == (R, H, k) and out.dtype == np.int32
    for r in range(R):
        tail = (int(limits[r]) - 1) // P if limits[r] > 0 else -1
        for h in range(H):
            s = scores[r, h]
            live = set(np.nonzero(np.isfinite(s))[0].tolist())
            row = out[r, h].tolist()
            n = min(k, len(live))
            chosen, pad = row[:n], row[n:]
            assert all(x == -1 for x in pad), "padding"
            assert chosen == sorted(chosen) and len(set(chosen)) == n, "ascending, distinct"
            assert set(chosen) <= live, "only live pages"
            if tail in live and k > 0:
                assert tail in chosen, "tail page"
            left = live - set(chosen)
            for j in chosen:
                if j == tail:
                    continue
                for u in left:
                    if u != tail:
                        assert _beats(s, j, u), (r, h, j, u)


def random_case(rng, R=5, H=3, NB=12, P=64):
    # scores from a small set of values so ties are common; some pages dead
    vals = np.array([-2.0, -0.5, 0.0, 0.25, 1.0, 3.0], dtype=np.float32)
    s = vals[rng.integers(0, len(vals), (R, H, NB))]
    dead = rng.random((R, H, NB)) < 0.2
    s[dead] = -np.inf
    limits = rng.integers(0, NB * P + 1, R)
    # pages at or past a row's limit hold no visible token: -inf, as the scorer writes them
    for r in range(R):
        live_pages = -(-int(limits[r]) // P)
        s[r, :, live_pages:] = -np.inf
        if limits[r] > 0:
            s[r, :, (int(limits[r]) - 1) // P] = np.float32(rng.choice(vals))   # the tail page is live
    return s, limits


@pytest.mark.parametrize("seed", range(20))
@pytest.mark.parametrize("k", [0, 1, 2, 5, 16])
def test_random_cases_satisfy_the_definition(seed, k):
    rng = np.random.default_rng(seed)
    s, lim = random_case(rng)
    check_selection(s, lim, 64, k, topk.select_pages(s, lim, 64, k))


def test_hand_cases():
    ninf = -np.inf
    s = np.array([[[1, 5, 5, 3, ninf, 2]]], dtype=np.float32)
    lim = np.array([6 * 64 - 10])          # tail page 5
    assert topk.select_pages(s, lim, 64, 3).tolist() == [[[1, 2, 5]]]
    assert topk.select_pages(s, lim, 64, 1).tolist() == [[[5]]]
    assert topk.select_pages(s, lim, 64, 7).tolist() == [[[0, 1, 2, 3, 5, -1, -1]]]
    ties = np.array([[[2, 2, 2, 2]]], dtype=np.float32)
    assert topk.select_pages(ties, np.array([4 * 128]), 128, 2).tolist() == [[[0, 3]]]
    dead = np.full((1, 2, 3), ninf, dtype=np.float32)
    assert topk.select_pages(dead, np.array([0]), 64, 2).tolist() == [[[-1, -1], [-1, -1]]]


def test_row_limits():
    assert topk.row_limits("prefill", [4], 10, [0, 2], [2]).tolist() == [3, 4]
    assert topk.row_limits("prefill", [4, 9], 8, [0, 2, 3], [2, 8]).tolist() == [3, 4, 8]
    assert topk.row_limits("decode", [0, 5, 99], 64).tolist() == [0, 5, 64]
    # prefix_len + i + 1 past 2^31 - 1: the limit is still seq_len (integers, no wrap)
    assert topk.row_limits("prefill", [450, 12], 512, [0, 3, 5], [2**31 - 2, 10]).tolist() == [450, 450, 450, 11, 12]


def _mutant(kind):
    def sel(block_scores, limits, page_size, k):
        bs = np.asarray(block_scores, dtype=np.float32)
        R, H, NB = bs.shape
        out = np.full((R, H, k), -1, dtype=np.int32)
        for r in range(R):
            lim = int(limits[r])
            tail = (lim - 1) // page_size if lim > 0 else -1
            for h in range(H):
                s = bs[r, h]
                live = np.nonzero(np.isfinite(s))[0]
                if k == 0 or len(live) == 0:
                    continue
                others = [j for j in live if j != tail]
                if kind == "ties_high":
                    others.sort(key=lambda j: (-float(s[j]), -int(j)))
                else:
                    others.sort(key=lambda j: (-float(s[j]), int(j)))
                lead = [] if kind == "no_tail" else ([tail] if tail in set(live.tolist()) else [])
                chosen = (lead + others)[:k]
                chosen = sorted(chosen, reverse=(kind == "descending"))
                out[r, h, :len(chosen)] = chosen
        return out
    return sel


@pytest.mark.parametrize("kind", ["ties_high", "no_tail", "descending"])
def test_planted_mistakes_are_caught(kind):
    caught = False
    for seed in range(20):
        rng = np.random.default_rng(100 + seed)
        s, lim = random_case(rng)
        try:
            check_selection(s, lim, 64, 3, _mutant(kind)(s, lim, 64, 3))
        except AssertionError:
            caught = True
            break
    assert caught, kind

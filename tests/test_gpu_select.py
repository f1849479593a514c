"""GPU parity of the top-k page selection (mxs_select_pages, through the C ABI)
against the CPU definition in oracle/topk.py: page indices bit-exact."""
import numpy as np
import pytest
import torch

import mxfp4_paged_cache_amd as mx
from mxfp4_paged_cache_amd import workloads as W
from oracle import topk
from tests.gpu_helpers import gpu_inputs, run_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    mx.lib()
    yield
    torch.cuda.synchronize()


def synthetic_scores(rng, limits, H, P, NB, n_values=5):
    """Scores from a few values (many ties); -inf past each row's limit and on
    some pages before it, as the scorer would write for dead pages."""
    vals = np.linspace(-3, 3, n_values).astype(np.float32)
    R = len(limits)
    s = vals[rng.integers(0, n_values, (R, H, NB))]
    s[rng.random((R, H, NB)) < 0.1] = -np.inf
    for r in range(R):
        live = -(-int(limits[r]) // P)
        s[r, :, live:] = -np.inf
        if limits[r] > 0:
            s[r, :, (int(limits[r]) - 1) // P] = vals[rng.integers(0, n_values)]
    return s


@pytest.mark.parametrize("k", [1, 4, 13, 40])
@pytest.mark.parametrize("NB", [9, 64, 100, 700, 2100, 4096])
def test_prefill_rows_match_oracle(NB, k):
    P = 64
    rng = np.random.default_rng(NB * 7 + k)
    q_lens, prefix = [3, 0, 6, 1], [NB * P // 2, 5, NB * P - 6, 0]
    seq = [min(p + q, NB * P) for p, q in zip(prefix, q_lens)]
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    msl = NB * P
    lim = topk.row_limits("prefill", seq, msl, cu, prefix)
    s = synthetic_scores(rng, lim, 3, P, NB)
    say(f"prefill select NB={NB} k={k} rows={len(lim)}")
    got = mx.select_pages(torch.from_numpy(s).cuda(), k, torch.tensor(seq, dtype=torch.int32, device="cuda"), msl, P,
                          cu_seqlens_q=torch.from_numpy(cu).cuda(),
                          prefix_lens=torch.tensor(prefix, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), topk.select_pages(s, lim, P, k))


def test_prefix_near_int32_max():
    # rows whose prefix_len + i + 1 passes 2^31 - 1: their limit is seq_len,
    # so the tail page is the sequence's last
    P, NB, k = 64, 8, 3
    rng = np.random.default_rng(77)
    q_lens, prefix, seq = [3, 2], [2**31 - 2, 10], [450, 12]
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    msl = NB * P
    lim = topk.row_limits("prefill", seq, msl, cu, prefix)
    assert lim.tolist() == [450, 450, 450, 11, 12]
    s = synthetic_scores(rng, lim, 3, P, NB)
    say(f"prefill select with prefix 2^31 - 2, NB={NB} k={k}")
    got = mx.select_pages(torch.from_numpy(s).cuda(), k, torch.tensor(seq, dtype=torch.int32, device="cuda"), msl, P,
                          cu_seqlens_q=torch.from_numpy(cu).cuda(),
                          prefix_lens=torch.tensor(prefix, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), topk.select_pages(s, lim, P, k))


@pytest.mark.parametrize("NB,k", [(2100, 300), (4096, 600)])
def test_large_k(NB, k):
    # k above the 256 results staged in LDS: ids go straight to the output
    # row; with more than 512 candidates the search runs without compaction
    P = 64
    rng = np.random.default_rng(NB + k)
    q_lens, prefix = [2, 3], [NB * P - 2, NB * P // 3]
    seq = [min(p + q, NB * P) for p, q in zip(prefix, q_lens)]
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    msl = NB * P
    lim = topk.row_limits("prefill", seq, msl, cu, prefix)
    s = synthetic_scores(rng, lim, 2, P, NB, n_values=7)
    say(f"prefill select NB={NB} k={k} rows={len(lim)}")
    got = mx.select_pages(torch.from_numpy(s).cuda(), k, torch.tensor(seq, dtype=torch.int32, device="cuda"), msl, P,
                          cu_seqlens_q=torch.from_numpy(cu).cuda(),
                          prefix_lens=torch.tensor(prefix, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), topk.select_pages(s, lim, P, k))


@pytest.mark.parametrize("P", [64, 128])
def test_decode_rows_and_strided_views(P):
    rng = np.random.default_rng(P)
    seq = [0, 1, P, P + 1, 30 * P, 31 * P - 3]
    msl = 31 * P
    NB = 31
    lim = topk.row_limits("decode", seq, msl)
    s = synthetic_scores(rng, lim, 5, P, NB, n_values=3)
    big = torch.full((len(seq), 5, NB + 7), 7.0, device="cuda")        # padded rows: strided input view
    big[:, :, :NB] = torch.from_numpy(s).cuda()
    outv = torch.full((len(seq), 5, 16), -7, dtype=torch.int32, device="cuda")[:, :, :6]   # strided output view
    got = mx.select_pages(big[:, :, :NB], 6, torch.tensor(seq, dtype=torch.int32, device="cuda"), msl, P, out=outv)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), topk.select_pages(s, lim, P, 6))


@pytest.mark.parametrize("NB", [300, 700, 1024, 2100])
def test_live_pages_past_the_tail_and_tail_below_the_rest(NB):
    # Distinct continuous scores, finite on every page: pages past a row's
    # tail page are live (a finite score is what makes a page live), so the
    # tail is not the last live page, and the tail's own score is pushed to
    # the lowest on its row, so it is chosen only by the tail rule. Rows of
    # 300 pages are searched on the registers, longer ones through the
    # compacted candidates.
    P, H = 128, 4
    rng = np.random.default_rng(NB)
    msl = NB * P
    seq = [1, P + 5, msl // 3, msl // 2 + 17, msl - P, msl]
    lim = topk.row_limits("decode", seq, msl)
    s = rng.standard_normal((len(seq), H, NB)).astype(np.float32)
    for r, L in enumerate(lim):
        s[r, :, (int(L) - 1) // P] = -50.0
    for k in (1, 16, 64):
        say(f"decode select NB={NB} k={k}, live pages past the tail")
        got = mx.select_pages(torch.from_numpy(s).cuda(), k, torch.tensor(seq, dtype=torch.int32, device="cuda"),
                              msl, P)
        torch.cuda.synchronize()
        assert np.array_equal(got.cpu().numpy(), topk.select_pages(s, lim, P, k)), k


@pytest.mark.parametrize("NB", [600, 1024, 1500])
@pytest.mark.parametrize("k", [65, 128, 256, 257])
def test_k_above_64_continuous_scores(NB, k):
    # k above the 64 lanes: the lower bound comes from the lanes' second
    # largest scores; up to 256 results are staged in LDS, 257 go straight to
    # the output row. Continuous scores with dead pages in between, so the
    # candidates are compacted (no ties to force the register search).
    P, H = 128, 3
    rng = np.random.default_rng(NB * 3 + k)
    msl = NB * P
    seq = [P * 3 + 1, msl // 2, msl - 5, msl]
    lim = topk.row_limits("decode", seq, msl)
    s = rng.standard_normal((len(seq), H, NB)).astype(np.float32)
    s[rng.random(s.shape) < 0.05] = -np.inf
    for r, L in enumerate(lim):
        s[r, :, -(-int(L) // P):] = -np.inf
    say(f"decode select NB={NB} k={k}, continuous scores")
    got = mx.select_pages(torch.from_numpy(s).cuda(), k, torch.tensor(seq, dtype=torch.int32, device="cuda"), msl, P)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), topk.select_pages(s, lim, P, k))


def test_seeded_sweep_of_shapes_and_score_kinds():
    # 80 seeded cases: row lengths across every per-lane register count and
    # the compaction limit, k from 1 to 400, and four kinds of scores:
    # continuous, heavy ties, close values in one binade (long shared key
    # prefixes), and continuous with -inf, NaN, +inf and -0.0 mixed in
    rng = np.random.default_rng(2024)
    for case in range(80):
        NB = int(rng.choice([1, 5, 63, 64, 65, 200, 511, 512, 513, 700, 1000, 1024, 1025, 1500, 2048, 3000, 4096]))
        k = int(rng.choice([1, 2, 7, 16, 31, 63, 64, 65, 100, 128, 200, 256, 257, 400]))
        P = int(rng.choice([64, 128]))
        H, R = int(rng.integers(1, 5)), int(rng.integers(1, 6))
        kind = case % 4
        msl = NB * P
        seq = rng.integers(0, msl + 1, R)
        lim = topk.row_limits("decode", seq, msl)
        if kind == 0:
            s = rng.standard_normal((R, H, NB)).astype(np.float32)
        elif kind == 1:
            s = rng.choice(np.linspace(-2, 2, 9).astype(np.float32), (R, H, NB))
        elif kind == 2:
            s = (rng.standard_normal((R, H, NB)) * 1e-3 + 5.0).astype(np.float32)
        else:
            s = rng.standard_normal((R, H, NB)).astype(np.float32)
            s[rng.random(s.shape) < 0.3] = -np.inf
            s[rng.random(s.shape) < 0.01] = np.float32(np.nan)
            s[rng.random(s.shape) < 0.01] = np.float32(np.inf)
            s[rng.random(s.shape) < 0.05] = np.float32(-0.0)
        say(f"sweep case {case}: NB={NB} k={k} P={P} H={H} R={R} kind={kind}")
        got = mx.select_pages(torch.from_numpy(s).cuda(), k, torch.from_numpy(seq.astype(np.int32)).cuda(), msl, P)
        torch.cuda.synchronize()
        assert np.array_equal(got.cpu().numpy(), topk.select_pages(s, lim, P, k)), case


def test_many_items_per_wave_odd_head_count():
    # More (row, head) items than the grid has waves (the grid is capped at
    # 32 workgroups per CU), with 7 heads, which do not divide the grid
    # stride: each wave takes several items and the head index wraps when
    # the stride is added.
    P, NB, H, R = 64, 9, 7, 10000
    rng = np.random.default_rng(77)
    msl = NB * P
    seq = rng.integers(0, msl + 1, R)
    lim = topk.row_limits("decode", seq, msl)
    s = synthetic_scores(rng, lim, H, P, NB)
    say(f"decode select rows={R} heads={H} k=4")
    got = mx.select_pages(torch.from_numpy(s).cuda(), 4, torch.tensor(seq, dtype=torch.int32, device="cuda"), msl, P)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), topk.select_pages(s, lim, P, 4))


def test_selection_of_scorer_output():
    # the step as it follows the scorer: block scores of the 64-row prefill
    # workload (ctx 1024, 8 pages), k = 3
    wl = W.prefill_small()
    host = W.make_inputs(wl, 21, "cpu")
    dev = gpu_inputs(host)
    bs, _ = run_gpu(dev, want_logits=False)
    got = mx.select_pages(bs, 3, dev.seq_lens, wl.window, wl.page_size, cu_seqlens_q=dev.cu_seqlens_q,
                          prefix_lens=dev.prefix_lens)
    torch.cuda.synchronize()
    lim = topk.row_limits("prefill", wl.seq_lens, wl.window, host.cu_seqlens_q.numpy(), wl.prefix_lens)
    assert np.array_equal(got.cpu().numpy(), topk.select_pages(bs.cpu().numpy(), lim, wl.page_size, 3))


def test_full_size_selection_sampled_rows():
    # block scores of the 4096-row, 128K-context prefill (4096 x 64 x 1024),
    # k = 64; 12 sampled rows (all heads) against the oracle
    wl = W.prefill_long()
    dev = W.make_inputs(wl, 22, "cuda")
    bs, _ = run_gpu(dev, want_logits=False)
    got = mx.select_pages(bs, 64, dev.seq_lens, wl.window, wl.page_size, cu_seqlens_q=dev.cu_seqlens_q,
                          prefix_lens=dev.prefix_lens)
    torch.cuda.synchronize()
    lim = topk.row_limits("prefill", wl.seq_lens, wl.window, dev.cu_seqlens_q.cpu().numpy(), wl.prefix_lens)
    rows = np.array([0, 1, 777, 2048, 4094, 4095] + list(np.random.default_rng(3).integers(0, 4096, 6)))
    ref = topk.select_pages(bs[rows].cpu().numpy(), lim[rows], wl.page_size, 64)
    assert np.array_equal(got[rows].cpu().numpy(), ref)
    # every selection holds its row's tail page
    tails = (torch.from_numpy(lim).cuda() - 1) // wl.page_size
    assert bool((got == tails[:, None, None]).any(dim=2).all())


def test_signed_zeros_tie_at_the_kth_place():
    # -0.0 and +0.0 compare equal, so they tie and the lower page wins: with
    # the k-th place contested by zeros of both signs, the lowest-indexed
    # zeros are taken whatever their sign (oracle/topk.py sorts by value, then
    # by page index)
    P, NB, H = 64, 200, 4
    rng = np.random.default_rng(5)
    R = 3
    s = np.full((R, H, NB), -1.0, np.float32)
    for r in range(R):
        for h in range(H):
            s[r, h, rng.choice(NB, 6, replace=False)] = 2.0          # 6 clear winners
            z = rng.choice(NB, 12, replace=False)
            s[r, h, z] = np.where(rng.random(12) < 0.5, np.float32(-0.0), np.float32(0.0))
    seq = [NB * P] * R
    lim = topk.row_limits("decode", seq, NB * P)
    for k in (8, 10, 13):
        ref = topk.select_pages(s, lim, P, k)
        got = mx.select_pages(torch.from_numpy(s).cuda(), k, torch.tensor(seq, dtype=torch.int32, device="cuda"),
                              NB * P, P)
        torch.cuda.synchronize()
        assert np.array_equal(got.cpu().numpy(), ref), k
    say("  signed zeros at the k-th place: selections equal the oracle's")


def test_empty_window_reads_nothing_and_pads():
    # max_seq_len 0: no page is live, every row is k entries of -1, and no
    # score is read (the scores tensor has one column and starts its own
    # allocation; a read before it would land outside)
    R, H, k = 5, 3, 4
    bs = torch.full((R, H, 1), float("nan"), device="cuda")
    seq = torch.zeros(R, dtype=torch.int32, device="cuda")
    got = mx.select_pages(bs, k, seq, 0, 64)
    cu = torch.tensor([0, 2, 5], dtype=torch.int32, device="cuda")
    got_p = mx.select_pages(bs, k, torch.zeros(2, dtype=torch.int32, device="cuda"), 0, 128, cu_seqlens_q=cu,
                            prefix_lens=torch.zeros(2, dtype=torch.int32, device="cuda"))
    # the same with an empty score tensor (NULL data pointer), and a call with no rows
    got_e = mx.select_pages(torch.empty((R, H, 0), device="cuda"), k, seq, 0, 64)
    none = mx.select_pages(torch.empty((0, H, 7), device="cuda"), k, torch.zeros(0, dtype=torch.int32, device="cuda"),
                           7 * 64, 64)
    torch.cuda.synchronize()
    assert (got == -1).all() and (got_p == -1).all() and (got_e == -1).all()
    assert none.shape == (0, H, k)

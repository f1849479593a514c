"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs. Comparison rule in tests/gpu_helpers.py."""
import math

import numpy as np
import pytest
import torch

import oracle
import mxfp4_paged_cache_amd as mx
from mxfp4_paged_cache_amd import workloads as W
from tests.gpu_helpers import (compare, compare_argmax, gpu_inputs, oracle_run, run_gpu, say)

pytestmark = pytest.mark.gpu

S = W.INV_SQRT_D


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    mx.lib()   # fails loudly when the HIP library is missing
    oracle.build()
    yield
    torch.cuda.synchronize()


def check_case(wl: W.Workload, *, seed=0, min_exact=0.999, q_strided=False, want_logits=None, out_bs=0, out_lg=0,
               argmax=0):
    """HIP path against the oracle on one seeded case. out_bs / out_lg: the
    case's ceilings on block scores / logits outside 2^-20 relative; argmax:
    on differing argmax positions (see tests/gpu_helpers.py)."""
    say(f"case {wl.name} seed={seed} P={wl.page_size} H={wl.H} q={wl.q_dtype} B={wl.B} mode={wl.mode}")
    host = W.make_inputs(wl, seed, "cpu", q_strided=q_strided)
    dev = gpu_inputs(host)
    lg_on = wl.want_logits if want_logits is None else want_logits
    bs, lg = run_gpu(dev, want_logits=lg_on)
    torch.cuda.synchronize()
    ref = oracle_run(host, want_logits=True, want_blocks=True)
    if bs is not None:
        compare(bs.cpu().numpy(), ref.blocks, ref.block_mags, S, what="block scores", min_exact=min_exact,
                max_outside=out_bs)
        compare_argmax(bs.cpu().numpy(), ref.blocks, ref.block_mags, S, "block scores", max_diff=argmax)
    if lg is not None:
        compare(lg.cpu().numpy(), ref.logits, ref.mags, S, what="logits", min_exact=min_exact, max_outside=out_lg)
    return host, dev, bs, lg, ref


def test_prefill_64_rows_ctx1k():
    # 64 rows after a 960-token prefix, ctx 1024, H=64, P=128, 16-page pool:
    # logits and block scores (the small prefill workload).
    check_case(W.prefill_small(), seed=1, out_bs=5, out_lg=305)


@pytest.mark.parametrize("P", [64, 128])
@pytest.mark.parametrize("qdt", ["bf16", "e4m3"])
def test_decode_ragged(P, qdt):
    wl = W.Workload("decode_ragged", "decode", H=64, page_size=P, q_lens=[1] * 5, prefix_lens=[0] * 5,
                    seq_lens=[1000, 128, 1, 0, 300], q_dtype=qdt, want_logits=True, max_seq_len=1030)
    check_case(wl, seed=2)


# Prefill cases run twice: block scores alone (the block-score kernel) and
# with logits (the logits kernel, which also returns the block scores).
LOGITS = pytest.mark.parametrize("lg", [False, True], ids=["blocks", "logits"])


# logits outside 2^-20 relative, per (page size, heads); 0 for the others
RAGGED_LOGITS_OUTSIDE = {(64, 64): 8, (128, 64): 3}


@LOGITS
@pytest.mark.parametrize("H", [1, 2, 3, 17, 64])
@pytest.mark.parametrize("P", [64, 128])
def test_prefill_ragged_heads(H, P, lg):
    # mixed query lengths with an empty request, prefixes mid-page, heads that
    # are not a multiple of the 16-slot tile (tiles straddle rows)
    wl = W.Workload("prefill_ragged", "prefill", H=H, page_size=P, q_lens=[5, 0, 17, 1], prefix_lens=[70, 3, 100, 0],
                    seq_lens=[75, 3, 117, 1], want_logits=lg, max_seq_len=200)
    check_case(wl, seed=3 + H, out_lg=RAGGED_LOGITS_OUTSIDE.get((P, H), 0))


@LOGITS
def test_prefill_many_rows_ragged_pages(lg):
    # more than one work item along slots and pages, a window that is not a
    # multiple of the page size and limits that end mid-page
    wl = W.Workload("prefill_many_rows", "prefill", H=24, page_size=64, q_lens=[37, 70], prefix_lens=[1000, 515],
                    seq_lens=[1037, 585], want_logits=lg, max_seq_len=1100)
    check_case(wl, seed=12, out_bs=5, out_lg=212)


@LOGITS
def test_prefix_near_int32_max(lg):
    # prefix_len + i + 1 passes 2^31 - 1 from the second row of the first
    # request on; the limit min(seq_len, prefix_len + i + 1) is over the
    # integers, so those rows see their whole sequence (an int32 sum wraps
    # negative and masks them out)
    wl = W.Workload("prefill_huge_prefix", "prefill", H=16, page_size=64, q_lens=[3, 2], prefix_lens=[2**31 - 2, 5],
                    seq_lens=[70, 7], want_logits=lg, max_seq_len=80)
    check_case(wl, seed=21)


@LOGITS
def test_prefill_e4m3_query_long_rows(lg):
    wl = W.Workload("prefill_e4m3", "prefill", H=64, page_size=128, q_lens=[40], prefix_lens=[2000],
                    seq_lens=[2040], q_dtype="e4m3", want_logits=lg)
    check_case(wl, seed=4, out_bs=2, out_lg=124)


@LOGITS
def test_wide_scale_bytes(lg):
    # e8m0 bytes 100..150 (outside the e4m3-exact window [119, 133]), one per
    # (token, 32-block): block scales 2^50 apart inside one dot, where the
    # MFMA's group truncation shows on many more values
    wl = W.Workload("prefill_wide_scales", "prefill", H=64, page_size=128, q_lens=[24], prefix_lens=[700],
                    seq_lens=[724], scale_lo=100, scale_hi=150, want_logits=lg)
    check_case(wl, seed=5, min_exact=0.60, out_bs=1, out_lg=4756)


@LOGITS
def test_wide_scale_bytes_per_token(lg):
    # one e8m0 byte per token, uniform over 100..150 (the chunked-prefill
    # workload's bytes; aiter #7061, "Format": that cache is judged against an
    # fp64 computation bit for bit). A common scale per token is a power of two
    # on the whole dot, so the relative error is as for bytes 122..127.
    wl = W.Workload("prefill_wide_token_scales", "prefill", H=64, page_size=128, q_lens=[24], prefix_lens=[700],
                    seq_lens=[724], scale_lo=100, scale_hi=150, scale_mode="token", want_logits=lg)
    check_case(wl, seed=15, min_exact=0.999, out_bs=3, out_lg=122)


def _sweep_workload(rng, n):
    """One seeded shape: mode, heads, page size, query dtype, ragged and empty
    requests, limits clipped by seq_len or by the causal diagonal, a window
    past the longest sequence, both scale-byte ranges, table fills, layouts."""
    mode = ("prefill", "prefill", "logits", "decode")[int(rng.integers(4))]
    H = int(rng.choice([1, 2, 5, 16, 17, 24, 64]))
    P = int(rng.choice([64, 128]))
    B = int(rng.integers(1, 6))
    if mode == "decode":
        q_lens, prefix = [1] * B, [0] * B
        seq = [int(rng.integers(0, 1200)) for _ in range(B)]
    else:
        q_lens = [int(rng.integers(0, 41)) for _ in range(B)]
        prefix = [int(rng.integers(0, 700)) for _ in range(B)]
        seq = []
        for p_, q_ in zip(prefix, q_lens):
            kind = int(rng.integers(4))
            if kind == 2:      # seq_len below prefix + q_len: the last rows see seq_len tokens
                seq.append(max(0, p_ + q_ - int(rng.integers(1, 60))))
            elif kind == 3:    # seq_len past the diagonal of the last row
                seq.append(p_ + q_ + int(rng.integers(1, 90)))
            else:
                seq.append(p_ + q_)
    window = max(seq + [1]) + int(rng.integers(0, 3 * P))
    wide = bool(rng.random() < 0.25)
    return W.Workload(f"sweep{n}", mode, H=H, page_size=P, q_lens=q_lens, prefix_lens=prefix, seq_lens=seq,
                      q_dtype=str(rng.choice(["bf16", "e4m3"])), scale_lo=100 if wide else 122,
                      scale_hi=150 if wide else 127, want_logits=mode == "logits" or bool(rng.random() < 0.5),
                      max_seq_len=window, table_fill=str(rng.choice(["pad", "perm"])),
                      layout=str(rng.choice(["split", "region"]))), wide


def test_seeded_sweep_of_shapes():
    # 48 seeded shapes through the C ABI against the oracle. Masks, -inf
    # patterns and layouts compare exactly; every finite value lies within
    # 2^-10 * sm_scale * M, and those outside 2^-20 relative stay under 0.1%
    # of a case's finite values (1% with bytes 100..150 per 32-element block,
    # at least 4 per case); argmax positions that differ must be near ties
    # and stay under 1% of the (row, head) pairs; cases of 100 values or more
    # keep the bit-identical floor (0.99, or 0.5 with the wide bytes).
    rng = np.random.default_rng(2026)
    for n in range(48):
        wl, wide = _sweep_workload(rng, n)
        say(f"case sweep{n}: mode={wl.mode} H={wl.H} P={wl.page_size} q={wl.q_dtype} B={wl.B} q_lens={wl.q_lens} "
            f"prefix={wl.prefix_lens} seq={wl.seq_lens} window={wl.window} wide={wide} logits={wl.want_logits} "
            f"fill={wl.table_fill} layout={wl.layout}")
        host = W.make_inputs(wl, 3000 + n, "cpu")
        dev = gpu_inputs(host)
        bs, lg = run_gpu(dev)
        torch.cuda.synchronize()
        ref = oracle_run(host, want_logits=True, want_blocks=True)
        frac = 0.01 if wide else 0.001
        ceil = lambda ref_: max(4, int(frac * np.isfinite(ref_).sum()))
        # the bit-identical floor guards a statistic: cases of under 100 values go without it
        floor = lambda ref_: (0.5 if wide else 0.99) if np.isfinite(ref_).sum() >= 100 else 0.0
        if bs is not None:
            compare(bs.cpu().numpy(), ref.blocks, ref.block_mags, S, what=f"sweep{n} block scores",
                    min_exact=floor(ref.blocks), max_outside=ceil(ref.blocks))
            compare_argmax(bs.cpu().numpy(), ref.blocks, ref.block_mags, S, f"sweep{n} block scores",
                           max_diff=max(1, wl.T * wl.H // 100))
        if lg is not None:
            compare(lg.cpu().numpy(), ref.logits, ref.mags, S, what=f"sweep{n} logits",
                    min_exact=floor(ref.logits), max_outside=ceil(ref.logits))


def test_logits_shared_region_small():
    # two-slot shared region, slot 1 scored, 64-token pages, padded table rows,
    # window not a multiple of the page size
    wl = W.Workload("logits_shared_small", "logits", H=64, page_size=64, q_lens=[20, 7], prefix_lens=[480, 0],
                    seq_lens=[500, 7], want_logits=True, want_blocks=True, layout="shared", shared_first_page=5,
                    table_pad=3, max_seq_len=530)
    check_case(wl, seed=6, out_lg=78)


@LOGITS
def test_strided_query(lg):
    wl = W.Workload("prefill_strided_q", "prefill", H=16, page_size=128, q_lens=[9], prefix_lens=[250],
                    seq_lens=[259], want_logits=lg)
    check_case(wl, seed=7, q_strided=True)


def test_e4m3_conversion_exhaustive():
    # Every bf16 pattern through the real path: query element 0 = pattern,
    # K = 1.0 at element 0, scale 2^0, sm_scale 1 -> the logit is the e4m3
    # value the kernel rounded the pattern to; compare with the oracle's table.
    T, H = 1024, 64
    q = torch.zeros((T, H, 128), dtype=torch.int16)
    q[:, :, 0] = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(T, H)
    q = q.view(torch.bfloat16).cuda()
    kd = torch.zeros((1, 128, 64), dtype=torch.uint8)
    kd[0, 0, 0] = 0x02
    ks = torch.full((1, 128, 4), 127, dtype=torch.uint8)
    kd, ks = kd.cuda(), ks.cuda()
    bt = torch.zeros((1, 1), dtype=torch.int32, device="cuda")
    cu = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    sl = torch.tensor([1], dtype=torch.int32, device="cuda")
    pl = torch.tensor([0], dtype=torch.int32, device="cuda")
    bs, lg = mx.score_prefill(q, kd, ks, bt, cu, sl, pl, T, 1, 1.0, logits=True)
    got = lg[:, :, 0].reshape(-1).cpu().numpy()
    table = oracle.bf16_to_e4m3_table()
    ref = np.array([oracle.e4m3_value(int(b)) for b in table])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan].astype(np.float32))   # +0 and -0 compare equal
    say(f"  all {65536 - nan.sum()} non-NaN bf16 patterns round exactly as the oracle")


def test_cross_mode_bitwise():
    # decode == prefill with one row per request (prefix = seq_len - 1) ==
    # logits mode, element for element, and the block scores of all three
    # kernels agree bitwise; block score == max of the logits.
    seq = [700, 129, 64, 1]
    B = len(seq)
    wd = W.Workload("xm_decode", "decode", H=64, page_size=128, q_lens=[1] * B, prefix_lens=[s - 1 for s in seq],
                    seq_lens=seq, want_logits=True, max_seq_len=768)
    host = W.make_inputs(wd, 8, "cpu")
    dev = gpu_inputs(host)
    bs_d, lg_d = run_gpu(dev, want_logits=True)
    dev.wl = W.Workload("xm_prefill", "prefill", H=64, page_size=128, q_lens=[1] * B,
                        prefix_lens=[s - 1 for s in seq], seq_lens=seq, want_logits=True, max_seq_len=768)
    bs_p, lg_p = run_gpu(dev, want_logits=True)
    bs_b, _ = run_gpu(dev, want_logits=False)
    dev.wl = W.Workload("xm_logits", "logits", H=64, page_size=128, q_lens=[1] * B,
                        prefix_lens=[s - 1 for s in seq], seq_lens=seq, want_logits=True, want_blocks=True,
                        max_seq_len=768)
    bs_l, lg_l = run_gpu(dev)
    torch.cuda.synchronize()
    for a, b_, n in [(bs_d, bs_p, "decode/prefill blocks"), (bs_d, bs_l, "decode/logits blocks"),
                     (bs_d, bs_b, "decode/block-score kernel"),
                     (lg_d, lg_p, "decode/prefill logits"), (lg_d, lg_l, "decode/logits logits")]:
        assert torch.equal(a.view(torch.int32), b_.view(torch.int32)), n
    mx_of_logits = lg_d.view(B, 64, 6, 128).amax(dim=3)
    assert torch.equal(mx_of_logits, bs_d)


def test_split_and_region_layouts_bitwise():
    wl = W.Workload("region", "prefill", H=64, page_size=128, q_lens=[8, 3], prefix_lens=[300, 40],
                    seq_lens=[308, 43], want_logits=True, layout="region")
    host = W.make_inputs(wl, 9, "cpu")
    dev_region = gpu_inputs(host)
    dev_split = gpu_inputs(host)
    dev_split.k_data = host.k_data.contiguous().cuda()
    dev_split.k_scale = host.k_scale.contiguous().cuda()
    dev_split.region = None
    a = run_gpu(dev_region)
    b = run_gpu(dev_split)
    torch.cuda.synchronize()
    assert torch.equal(a[0].view(torch.int32), b[0].view(torch.int32))
    assert torch.equal(a[1].view(torch.int32), b[1].view(torch.int32))


@pytest.mark.parametrize("pad", [1, 3, 8, 13])
def test_block_scores_into_strided_unaligned_rows(pad):
    # Block-score rows starting at every 4-byte offset of a 64-byte segment
    # (output views [T, H, NB] cut out of [T, H, NB + pad] at column `pad`):
    # the block-score kernel writes each row in 64-byte-aligned segments, and
    # the result must equal the contiguous output bit for bit, with nothing
    # written outside the view; windows that end mid-segment and several
    # page chunks per row included.
    wl = W.Workload("strided_bs", "prefill", H=7, page_size=64, q_lens=[40, 3], prefix_lens=[2000, 90],
                    seq_lens=[2040, 93], max_seq_len=2100)
    host = W.make_inputs(wl, 30 + pad, "cpu")
    dev = gpu_inputs(host)
    NB = wl.NB
    ref, _ = run_gpu(dev)
    for pun in (0, 3):
        base = torch.full((wl.T, wl.H, NB + pad), 7.0, device="cuda")
        view = base[:, :, pad:]
        p = mx.make_plan("prefill", torch.bfloat16, 64, wl.H, 2, 40, 2100, False, True, pun)
        mx.score_prefill(dev.q, dev.k_data, dev.k_scale, dev.block_table, dev.cu_seqlens_q, dev.seq_lens,
                         dev.prefix_lens, 40, 2100, S, out=view, plan=p)
        torch.cuda.synchronize()
        assert torch.equal(view.contiguous().view(torch.int32), ref.view(torch.int32)), (pad, pun)
        assert bool((base[:, :, :pad] == 7.0).all()), (pad, pun)
    say(f"  pad {pad}: strided block scores equal the contiguous ones")


def test_explicit_plans_give_identical_outputs():
    wl = W.Workload("plans", "prefill", H=64, page_size=128, q_lens=[33, 12], prefix_lens=[900, 100],
                    seq_lens=[933, 112])
    host = W.make_inputs(wl, 10, "cpu")
    dev = gpu_inputs(host)
    base, _ = run_gpu(dev)
    for pun in (1, 7, 64, 1000):
        p = mx.make_plan("prefill", torch.bfloat16, 128, 64, 2, 33, 933, False, True, pun)
        other, _ = run_gpu(dev, plan=p)
        assert torch.equal(base.view(torch.int32), other.view(torch.int32)), pun
    wd = W.Workload("plans_d", "decode", H=64, page_size=64, q_lens=[1] * 3, prefix_lens=[0] * 3,
                    seq_lens=[4000, 10, 2500])
    host = W.make_inputs(wd, 11, "cpu")
    dev = gpu_inputs(host)
    base, _ = run_gpu(dev)
    for pun in (1, 5, 300):
        p = mx.make_plan("decode", torch.bfloat16, 64, 64, 3, 1, 4000, False, True, pun)
        other, _ = run_gpu(dev, plan=p)
        assert torch.equal(base.view(torch.int32), other.view(torch.int32)), pun
    wl = W.Workload("plans_l", "logits", H=20, page_size=64, q_lens=[30, 9], prefix_lens=[600, 40],
                    seq_lens=[630, 49], want_logits=True, want_blocks=True)
    host = W.make_inputs(wl, 13, "cpu")
    dev = gpu_inputs(host)
    base_bs, base_lg = run_gpu(dev)
    for pun in (1, 3, 17, 500):
        p = mx.make_plan("logits", torch.bfloat16, 64, 20, 2, 30, 630, True, True, pun)
        obs, olg = run_gpu(dev, plan=p)
        assert torch.equal(base_lg.view(torch.int32), olg.view(torch.int32)), pun
        assert torch.equal(base_bs.view(torch.int32), obs.view(torch.int32)), pun


def test_calls_with_nothing_to_write():
    # no query rows, or an empty window: the outputs are empty tensors (NULL
    # data pointers) and each call returns without launching anything
    wl = W.Workload("no_rows", "prefill", H=16, page_size=64, q_lens=[0, 0], prefix_lens=[30, 0],
                    seq_lens=[30, 5], want_logits=True, max_seq_len=64)
    d = gpu_inputs(W.make_inputs(wl, 16, "cpu"))
    bs, lg = mx.score_prefill(d.q, d.k_data, d.k_scale, d.block_tables[0], d.cu_seqlens_q, d.seq_lens, d.prefix_lens,
                              0, 64, S, logits=True)
    assert bs.shape == (0, 16, 1) and lg.shape == (0, 16, 64)
    lg2 = mx.score_logits(d.q, d.k_data, d.k_scale, d.block_tables[0], d.cu_seqlens_q, d.seq_lens, d.prefix_lens,
                          0, 64, S)
    assert lg2.shape == (0, 16, 64)
    wl = W.Workload("empty_window", "decode", H=16, page_size=64, q_lens=[1, 1], prefix_lens=[0, 0],
                    seq_lens=[0, 0], max_seq_len=0)
    d = gpu_inputs(W.make_inputs(wl, 17, "cpu"))
    bs = mx.score_decode(d.q, d.k_data, d.k_scale, d.block_tables[0], d.seq_lens, 0, S)
    torch.cuda.synchronize()
    assert bs.shape == (2, 16, 0)


def test_empty_tensors_with_zero_strides():
    # empty tensors made from numpy arrays have all-zero strides: with nothing
    # to read or write, every call takes them
    z = lambda shape, dt: torch.from_numpy(np.zeros(shape, dt)).cuda()
    q0 = z((0, 8, 128), np.int16).view(torch.bfloat16)
    kd, ks = z((3, 64, 64), np.uint8), z((3, 64, 4), np.uint8)
    bt0 = z((2, 0), np.int32)
    cu, seq, pre = (torch.tensor(v, dtype=torch.int32, device="cuda") for v in ([0, 0, 0], [10, 0], [10, 0]))
    bs, lg = mx.score_prefill(q0, kd, ks, bt0, cu, seq, pre, 0, 0, S, logits=True)
    assert bs.shape == (0, 8, 0) and lg.shape == (0, 8, 0)
    sel = mx.select_pages(z((0, 8, 0), np.float32), 4, z((0,), np.int32), 0, 64)
    assert sel.shape == (0, 8, 4)
    mx.write_pages(z((0, 128), np.int16).view(torch.bfloat16), z((0,), np.int64), kd, ks)
    torch.cuda.synchronize()


def test_larger_max_query_len_changes_nothing():
    # max_query_len only bounds the rows per request: a larger one plans more
    # (empty) slot blocks, and the outputs stay the same bits
    wl = W.Workload("mql", "prefill", H=24, page_size=64, q_lens=[19, 0, 41], prefix_lens=[300, 7, 60],
                    seq_lens=[319, 7, 101], want_logits=True)
    host = W.make_inputs(wl, 14, "cpu")
    d = gpu_inputs(host)
    outs = []
    for mql in (41, 42, 300):
        bs, lg = mx.score_prefill(d.q, d.k_data, d.k_scale, d.block_tables[0], d.cu_seqlens_q, d.seq_lens,
                                  d.prefix_lens, mql, wl.window, S, logits=True)
        lg2 = mx.score_logits(d.q, d.k_data, d.k_scale, d.block_tables[0], d.cu_seqlens_q, d.seq_lens,
                              d.prefix_lens, mql, wl.window, S)
        torch.cuda.synchronize()
        outs.append((bs.view(torch.int32).clone(), lg.view(torch.int32).clone(), lg2.view(torch.int32).clone()))
    for o in outs[1:]:
        assert all(torch.equal(a_, b_) for a_, b_ in zip(outs[0], o))
    assert torch.equal(outs[0][1], outs[0][2])


def test_graph_replay_with_poisoned_outputs():
    # Captured decode and prefill calls are replayed with outputs poisoned
    # (NaN) in between; every replay must rewrite every element (aiter #5518,
    # "Correctness": graph replay with logical outputs poisoned between replays).
    wd = W.Workload("g_decode", "decode", H=64, page_size=128, q_lens=[1] * 3, prefix_lens=[0] * 3,
                    seq_lens=[900, 5, 0], want_logits=True, max_seq_len=1024)
    wp = W.Workload("g_prefill", "prefill", H=64, page_size=128, q_lens=[6, 2], prefix_lens=[500, 0],
                    seq_lens=[506, 2], want_logits=True)
    hd, hp = W.make_inputs(wd, 12, "cpu"), W.make_inputs(wp, 13, "cpu")
    dd, dp = gpu_inputs(hd), gpu_inputs(hp)
    bs_d = torch.empty((3, 64, 8), device="cuda")
    lg_d = torch.empty((3, 64, 1024), device="cuda")
    bs_p = torch.empty((8, 64, 4), device="cuda")
    lg_p = torch.empty((8, 64, 506), device="cuda")
    pd = mx.make_plan("decode", torch.bfloat16, 128, 64, 3, 1, 1024, True, True)
    pp = mx.make_plan("prefill", torch.bfloat16, 128, 64, 2, 6, 506, True, True)

    def step():
        mx.score_decode(dd.q, dd.k_data, dd.k_scale, dd.block_table, dd.seq_lens, 1024, S, out=bs_d, logits=lg_d,
                        plan=pd)
        mx.score_prefill(dp.q, dp.k_data, dp.k_scale, dp.block_table, dp.cu_seqlens_q, dp.seq_lens, dp.prefix_lens,
                         6, 506, S, out=bs_p, logits=lg_p, plan=pp)

    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (bs_d, lg_d, bs_p, lg_p)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for t in (bs_d, lg_d, bs_p, lg_p):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, e in zip((bs_d, lg_d, bs_p, lg_p), eager):
            assert torch.equal(t.view(torch.int32), e.view(torch.int32)), rep
    say("  4 replays with poisoned outputs equal the eager result")


def test_rejections_on_gpu_tensors():
    dev = "cuda"
    q = torch.zeros((2, 4, 128), dtype=torch.bfloat16, device=dev)
    kd = torch.zeros((3, 128, 64), dtype=torch.uint8, device=dev)
    ks = torch.zeros((3, 128, 4), dtype=torch.uint8, device=dev)
    bt = torch.zeros((2, 2), dtype=torch.int32, device=dev)
    sl = torch.tensor([100, 200], dtype=torch.int32, device=dev)
    ok = mx.score_decode(q, kd, ks, bt, sl, 256, S)
    assert ok.shape == (2, 4, 2)
    with pytest.raises(ValueError):
        mx.score_decode(q.half(), kd, ks, bt, sl, 256, S)                     # fp16 query
    with pytest.raises(ValueError):
        mx.score_decode(q, kd[:, :, :32], ks, bt, sl, 256, S)                 # narrow data view
    with pytest.raises(ValueError):
        mx.score_decode(q, kd, ks[:2], bt, sl, 256, S)                        # page counts differ
    with pytest.raises(ValueError):
        mx.score_decode(q, kd, ks, bt[:, :1], sl, 256, S)                     # narrow block table
    with pytest.raises(ValueError):
        mx.score_decode(q, kd, ks, bt, torch.tensor([100, 0, 200, 0], dtype=torch.int32, device=dev)[::2], 256, S)
    big = torch.zeros((2, 4, 132), dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError):
        mx.score_decode(big[:, :, :128], kd, ks, bt, sl, 256, S)             # misaligned query rows
    with pytest.raises(ValueError):
        mx.score_decode(q, kd, ks, bt, sl, 256, float("nan"))
    cu = torch.tensor([0, 1, 2], dtype=torch.int32, device=dev)
    pl = torch.tensor([0, 0], dtype=torch.int32, device=dev)
    with pytest.raises(ValueError):
        mx.score_prefill(q, kd, ks, bt, cu, sl, pl, 1, 256, S, out=torch.empty((2, 4, 3), device=dev))
    # plans whose work decomposition was altered after planning are refused before launch
    pd = mx.make_plan("decode", torch.bfloat16, 128, 4, 2, 1, 256, False, True)
    assert mx.score_decode(q, kd, ks, bt, sl, 256, S, plan=pd).shape == (2, 4, 2)
    for field, val in (("pages_per_item", 64), ("grid", pd.grid + 1), ("page_items", pd.page_items + 1),
                       ("head_groups", 2)):
        bad = type(pd).from_buffer_copy(bytes(pd))
        setattr(bad, field, val)
        with pytest.raises(ValueError):
            mx.score_decode(q, kd, ks, bt, sl, 256, S, plan=bad)
    pp = mx.make_plan("prefill", torch.bfloat16, 128, 4, 2, 1, 256, False, True)
    for field, val in (("slots_per_item", 128), ("items", pp.items + 1), ("pages_per_item", 0)):
        bad = type(pp).from_buffer_copy(bytes(pp))
        setattr(bad, field, val)
        with pytest.raises(ValueError):
            mx.score_prefill(q, kd, ks, bt, cu, sl, pl, 1, 256, S, plan=bad)


def test_check_metadata_finds_contract_violations():
    wl = W.Workload("meta", "prefill", H=8, page_size=64, q_lens=[3, 0, 5], prefix_lens=[100, 7, 60],
                    seq_lens=[103, 7, 65], max_seq_len=160, table_pad=2)
    host = W.make_inputs(wl, 14, "cpu")
    dev = gpu_inputs(host)
    args = dict(cu_seqlens_q=dev.cu_seqlens_q, prefix_lens=dev.prefix_lens, max_query_len=5)
    mx.check_metadata("prefill", dev.k_data, dev.k_scale, dev.block_table, dev.seq_lens, 160, check_scales=True,
                      **args)
    mx.check_metadata("decode", dev.k_data, dev.k_scale, dev.block_table, dev.seq_lens, 160, check_scales=True)

    def expect(msg, **over):
        kw = dict(block_table=dev.block_table, seq_lens=dev.seq_lens, k_scale=dev.k_scale, **args)
        kw.update(over)
        with pytest.raises(ValueError, match=msg):
            mx.check_metadata("prefill", dev.k_data, kw.pop("k_scale"), kw.pop("block_table"), kw.pop("seq_lens"), 160,
                              check_scales=True, **kw)

    bt = dev.block_table.clone()
    bt[2, 1] = host.k_data.shape[0]          # live page of request 2 out of range
    expect("outside", block_table=bt)
    bt = dev.block_table.clone()
    bt[0, 1] = -1                            # request 0 sees tokens 0..102: page 1 is live
    expect("outside", block_table=bt)
    bt = dev.block_table.clone()
    bt[0, 2] = -1                            # page 2 of request 0 holds no live token: padding is fine
    mx.check_metadata("prefill", dev.k_data, dev.k_scale, bt, dev.seq_lens, 160, **args)
    expect("seq_lens", seq_lens=torch.tensor([103, 7, 200], dtype=torch.int32, device="cuda"))
    expect("decreases", cu_seqlens_q=torch.tensor([0, 3, 2, 8], dtype=torch.int32, device="cuda"))
    expect("max_query_len", max_query_len=4)
    ks = dev.k_scale.clone()
    page = int(dev.block_table[2, 0])
    ks[page, 5, 1] = 0                       # live token 5 of request 2
    expect("e8m0", k_scale=ks)
    ks = dev.k_scale.clone()
    ks[page, 63, 3] = 255                    # token 63 of request 2 (limit 65): live
    expect("e8m0", k_scale=ks)
    ks = dev.k_scale.clone()
    page1 = int(dev.block_table[2, 1])
    ks[page1, 1, 0] = 255                    # token 65 of request 2: dead, garbage allowed
    mx.check_metadata("prefill", dev.k_data, ks, dev.block_table, dev.seq_lens, 160, check_scales=True, **args)


# ------------------------------------------------------------------ boundary pages past 2 GiB and 4 GiB

# values outside 2^-20 relative per (boundary, view): (block scores, logits)
STRADDLE_OUTSIDE = {(1 << 31, "data"): (0, 12), (1 << 31, "scale"): (1, 17), (1 << 32, "data"): (0, 20),
                    (1 << 32, "scale"): (1, 19)}


@pytest.mark.parametrize("view", ["data", "scale"])
@pytest.mark.parametrize("boundary", [1 << 31, 1 << 32], ids=["2GiB", "4GiB"])
def test_pages_straddling_2gib_and_4gib(boundary, view):
    # One uint8 region holds two-slot page blocks (17408 B at P = 128); the
    # data and scale views start at nonzero slot offsets chosen so that one
    # live page's data (view "data") or scales (view "scale") straddle byte
    # offset 2^31 or 2^32 of the region. The same bytes copied into a dense
    # split pool must give bitwise-equal scores in all three kernels, and both
    # must match the oracle (aiter #5518, "Correctness": 2 GiB and 4 GiB
    # boundaries, dense against shared pool bit-identical).
    P, H = 128, 64
    S_blk = 2 * P * 68
    r = boundary % S_blk
    if view == "data":
        od = (r - 32 * P) % S_blk          # boundary falls on byte 32 P of a page's data (token 64)
        os_ = od + 64 * P                  # scales right after the data in the slot
    else:
        os_ = (r - 2 * P) % S_blk + S_blk  # boundary falls on byte 2 P of a page's scales (token 64)
        od = os_ - 64 * P
    assert od > 0 and os_ > 0
    p_x = (boundary - (od if view == "data" else os_)) // S_blk
    lo_v, hi_v = (od + p_x * S_blk, od + p_x * S_blk + 64 * P) if view == "data" else \
        (os_ + p_x * S_blk, os_ + p_x * S_blk + 4 * P)
    assert lo_v < boundary < hi_v
    npool = p_x + 4
    say(f"case straddle {view} at {boundary}: page {p_x}, view bytes [{lo_v}, {hi_v})")
    region = torch.empty(os_ + npool * S_blk + 4 * P, dtype=torch.uint8, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(4242 + (boundary >> 31) + (view == "scale"))
    region.random_(0, 256, generator=g)
    kd = torch.as_strided(region, (npool, P, 64), (S_blk, 64, 1), od)
    ks = torch.as_strided(region, (npool, P, 4), (S_blk, 4, 1), os_)
    ks.copy_(torch.randint(122, 128, ks.shape, generator=g, device="cuda", dtype=torch.uint8))
    # requests: the straddling page sits mid-context, last, and first
    seq = [600, 300, 129]
    rng = np.random.default_rng(boundary % 1000 + len(view))
    others = [int(x) for x in rng.choice(np.arange(npool - 1), 16, replace=False) if int(x) != p_x]
    rows = [[others[0], p_x, others[1], others[2], others[3]], [others[4], others[5], p_x], [p_x, others[6]]]
    NB = (max(seq) + P - 1) // P
    bt = torch.full((3, NB + 1), -1, dtype=torch.int32)
    for b, row in enumerate(rows):
        bt[b, :len(row)] = torch.tensor(row, dtype=torch.int32)
    bt = bt.cuda()
    used = sorted({p for row in rows for p in row})
    remap = {p: i for i, p in enumerate(used)}
    idx = torch.tensor(used, dtype=torch.long, device="cuda")
    kd_dense, ks_dense = kd.index_select(0, idx).contiguous(), ks.index_select(0, idx).contiguous()
    bt_dense = torch.full_like(bt, -1)
    for b, row in enumerate(rows):
        bt_dense[b, :len(row)] = torch.tensor([remap[p] for p in row], dtype=torch.int32)
    q_lens = [4, 3, 2]
    prefix = [s_ - q for s_, q in zip(seq, q_lens)]
    g2 = torch.Generator(device="cuda")
    g2.manual_seed(77)
    q = torch.randn((sum(q_lens), H, 128), generator=g2, device="cuda").to(torch.bfloat16)
    qd = torch.randn((3, H, 128), generator=g2, device="cuda").to(torch.bfloat16)
    cu = torch.tensor([0, 4, 7, 9], dtype=torch.int32, device="cuda")
    sl = torch.tensor(seq, dtype=torch.int32, device="cuda")
    pl = torch.tensor(prefix, dtype=torch.int32, device="cuda")
    W_ = max(seq)
    outs = {}
    for name, (kdv, ksv, btv) in {"shared": (kd, ks, bt), "dense": (kd_dense, ks_dense, bt_dense)}.items():
        o = {}
        o["decode"] = mx.score_decode(qd, kdv, ksv, btv, sl, W_, S)
        o["prefill"] = mx.score_prefill(q, kdv, ksv, btv, cu, sl, pl, 4, W_, S)
        o["logits"] = mx.score_logits(q, kdv, ksv, btv, cu, sl, pl, 4, W_, S)
        outs[name] = o
    torch.cuda.synchronize()
    for k in ("decode", "prefill", "logits"):
        assert torch.equal(outs["shared"][k].view(torch.int32), outs["dense"][k].view(torch.int32)), k
    # and the dense copy against the oracle
    kdh, ksh, bth = kd_dense.cpu().numpy(), ks_dense.cpu().numpy(), bt_dense.cpu().numpy()
    qn = q.cpu().view(torch.int16).numpy().view(np.uint16)
    ref = oracle.score(mode="prefill", q=qn, q_dtype="bf16", k_data=kdh, k_scale=ksh, page_size=P, block_table=bth,
                       seq_lens=np.array(seq, np.int32), max_seq_len=W_, sm_scale=S, cu_seqlens_q=cu.cpu().numpy(),
                       prefix_lens=np.array(prefix, np.int32), want_mags=True, want_block_mags=True)
    out_bs, out_lg = STRADDLE_OUTSIDE[(boundary, view)]
    compare(outs["shared"]["prefill"].cpu().numpy(), ref.blocks, ref.block_mags, S, what="straddling block scores",
            max_outside=out_bs, min_exact=0.999)
    compare(outs["shared"]["logits"].cpu().numpy(), ref.logits, ref.mags, S, what="straddling logits",
            max_outside=out_lg, min_exact=0.999)
    qdn = qd.cpu().view(torch.int16).numpy().view(np.uint16)
    refd = oracle.score(mode="decode", q=qdn, q_dtype="bf16", k_data=kdh, k_scale=ksh, page_size=P, block_table=bth,
                        seq_lens=np.array(seq, np.int32), max_seq_len=W_, sm_scale=S, want_logits=False,
                        want_block_mags=True)
    compare(outs["shared"]["decode"].cpu().numpy(), refd.blocks, refd.block_mags, S,
            what="straddling decode block scores", max_outside=0, min_exact=0.999)
    del region, kd, ks
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ full-size workloads (sampled oracle)

def _limits(wl: W.Workload) -> torch.Tensor:
    return torch.tensor(wl.limits(), dtype=torch.int64)


def _check_block_mask_full(bs: torch.Tensor, wl: W.Workload):
    lim = _limits(wl).to(bs.device)
    live_pages = (lim + wl.page_size - 1) // wl.page_size
    j = torch.arange(bs.shape[2], device=bs.device)
    expect_fin = (j[None, :] < live_pages[:, None])[:, None, :].expand_as(bs)
    assert not torch.isnan(bs).any()
    assert torch.equal(torch.isfinite(bs), expect_fin)
    assert torch.equal(torch.isneginf(bs), ~expect_fin)


def _sample_rows(wl: W.Workload, extra: int, seed: int):
    """The first and last rows, the rows whose limit crosses into a new page
    (up to 8), and `extra` seeded random rows."""
    T = wl.T
    rng = np.random.default_rng(seed)
    rows = {0, T - 1}
    lim = wl.limits()
    P = wl.page_size
    crossing = [r for r in range(1, T) if lim[r] // P != lim[r - 1] // P]
    rows |= set(crossing[:4]) | set(crossing[-4:])
    rows |= set(int(x) for x in rng.choice(T, size=min(extra, T), replace=False))
    return np.array(sorted(rows), np.int32)


def _full_blocks_case(wl: W.Workload, seed: int, rows, *, out_bs: int, argmax: int, min_exact: float):
    say(f"case {wl.name}: generating inputs on the GPU")
    inp = W.make_inputs(wl, seed, "cuda")
    bs, _ = run_gpu(inp)
    torch.cuda.synchronize()
    _check_block_mask_full(bs, wl)
    say(f"  {len(rows)} rows through the oracle")
    ref = oracle_run(inp, rows=rows, want_logits=False, compact=True)
    got = bs[torch.as_tensor(rows, dtype=torch.long, device="cuda")].cpu().numpy()
    compare(got, ref.blocks, ref.block_mags, S, what=f"{wl.name} block scores ({len(rows)} rows)",
            min_exact=min_exact, max_outside=out_bs)
    compare_argmax(got, ref.blocks, ref.block_mags, S, f"{wl.name} block scores", max_diff=argmax)
    del bs, inp
    torch.cuda.empty_cache()


def test_full_decode_b64_ctx128k():
    # every one of the 64 requests, every head and page
    wl = W.decode_b64_128k()
    _full_blocks_case(wl, 20, np.arange(64, dtype=np.int32), out_bs=628, argmax=0, min_exact=0.999)


def test_full_prefill_q4096_ctx128k_e4m3():
    wl = W.prefill_long()
    _full_blocks_case(wl, 21, _sample_rows(wl, 64, 21), out_bs=491, argmax=0, min_exact=0.999)


def test_full_chunked_prefill_32k_per_token_scales():
    # the chunked-prefill workload as stated: one e8m0 byte per token in 100..150
    wl = W.prefill_chunk()
    assert wl.scale_mode == "token"
    _full_blocks_case(wl, 22, _sample_rows(wl, 64, 22), out_bs=309, argmax=0, min_exact=0.999)


def test_full_chunked_prefill_32k_block_scales():
    # the same shape with a byte per (token, 32-block) in 100..150
    wl = W.prefill_chunk_block_scales()
    _full_blocks_case(wl, 24, _sample_rows(wl, 16, 24), out_bs=36, argmax=0, min_exact=0.60)


def test_full_logits_shared_pool_past_4p6gb():
    # all 1024 rows, every head and token, in chunks of 128 rows
    wl = W.logits_shared_pool()
    say(f"case {wl.name}: generating the 4.6 GB shared region on the GPU")
    inp = W.make_inputs(wl, 23, "cuda")
    first = int(inp.block_table[inp.block_table >= 0].min()) * inp.k_data.stride(0) + inp.k_data.storage_offset()
    assert first >= 4_608_000_000
    _, lg = run_gpu(inp)
    torch.cuda.synchronize()
    lim = _limits(wl).cuda()
    t = torch.arange(wl.window, device="cuda")
    expect_fin = (t[None, :] < lim[:, None])[:, None, :].expand_as(lg)
    assert not torch.isnan(lg).any()
    assert torch.equal(torch.isfinite(lg), expect_fin)
    total_out = 0
    for r0 in range(0, wl.T, 128):
        rows = np.arange(r0, r0 + 128, dtype=np.int32)
        ref = oracle_run(inp, rows=rows, want_logits=True, want_blocks=False, compact=True)
        got = lg[r0:r0 + 128].cpu().numpy()
        st = compare(got, ref.logits, ref.mags, S, what=f"logits past 4.608e9 B, rows {r0}..{r0 + 127}",
                     min_exact=0.999, max_outside=10 ** 9)
        total_out += st.outside
        del ref, got
    say(f"  logits past 4.608e9 B: {total_out} values outside 2^-20 relative over all 1024 rows")
    assert total_out <= 30746, f"{total_out} logits outside 2^-20 relative, ceiling 30746"
    del lg, inp
    torch.cuda.empty_cache()

"""GPU parity of the MXFP4 writer (mxs_write_pages, through the C ABI) against
oracle/writer.py: every byte of the cache views, written slots and untouched
ones alike."""
import numpy as np
import pytest
import torch

import mxfp4_paged_cache_amd as mx
from mxfp4_paged_cache_amd import workloads as W
from oracle import writer
from tests.gpu_helpers import compare, oracle_run, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    mx.lib()
    yield
    torch.cuda.synchronize()


def make_keys(rng, n):
    """bf16 keys: N(0,1) rows at per-token magnitudes 2^-60..2^60, with zero
    blocks, signed zeros, grid midpoints (exact ties) and saturating values."""
    x = rng.standard_normal((n, 128)).astype(np.float32)
    x *= (2.0 ** rng.integers(-60, 60, (n, 1))).astype(np.float32)
    x[rng.random(n) < 0.1, 32:64] = 0.0
    x[rng.random(n) < 0.1, 0] = -0.0
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.0, -2.5, -0.75], dtype=np.float32)
    for t in range(0, n, 7):                                   # a block of exact midpoints at scale 2^e
        e = int(rng.integers(-20, 20))
        blk = rng.choice(ties, 32).astype(np.float32) * np.float32(2.0 ** e)
        blk[0] = np.float32(6.0 * 2.0 ** e)                     # amax in [4, 8) * 2^e keeps the scale at e
        x[t, 64:96] = blk
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)          # exact bf16 patterns (truncation)
    # subnormal bf16 blocks (magnitudes 2^-133 .. 2^-127): the scale clips to 2^-126
    for t in range(3, n, 50):
        bits[t, 96:128] = rng.integers(1, 0x80, 32).astype(np.uint16) | (rng.integers(0, 2, 32) << 15).astype(np.uint16)
    return bits


@pytest.mark.parametrize("P,layout", [(64, "split"), (128, "split"), (128, "region")])
def test_writer_matches_oracle_bytewise(P, layout):
    rng = np.random.default_rng(P + len(layout))
    n, pages = 900, 20
    bits = make_keys(rng, n)
    slots = rng.permutation(pages * P)[:n].astype(np.int64)
    slots[rng.random(n) < 0.05] = -1                            # skipped tokens
    slots[:3] = [pages * P, pages * P + 5, 10 ** 12]            # past the pool: skipped by the kernel
    if layout == "split":
        kd = np.full((pages, P, 64), 0xA5, dtype=np.uint8)
        ks = np.full((pages, P, 4), 0x5A, dtype=np.uint8)
        gd, gs = torch.from_numpy(kd.copy()).cuda(), torch.from_numpy(ks.copy()).cuda()
        mx.write_pages(torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16),
                       torch.from_numpy(slots).cuda(), gd, gs)
    else:
        region = torch.full((pages * P * 68,), 0xA5, dtype=torch.uint8, device="cuda")
        gd = torch.as_strided(region, (pages, P, 64), (P * 68, 64, 1), 0)
        gs = torch.as_strided(region, (pages, P, 4), (P * 68, 4, 1), P * 64)
        kd = np.ascontiguousarray(gd.cpu().numpy())
        ks = np.ascontiguousarray(gs.cpu().numpy())
        mx.write_pages(torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16),
                       torch.from_numpy(slots).cuda(), gd, gs)
    torch.cuda.synchronize()
    say(f"writer P={P} {layout}: {int((slots >= 0).sum())} tokens")
    writer.write_pages(bits, np.where(slots < pages * P, slots, -1), kd, ks, P)
    assert np.array_equal(gd.cpu().numpy(), kd)
    assert np.array_equal(gs.cpu().numpy(), ks)


def test_strided_keys_and_rejections():
    rng = np.random.default_rng(5)
    bits = make_keys(rng, 40)
    big = torch.zeros((40, 256), dtype=torch.int16, device="cuda")
    big[:, :128] = torch.from_numpy(bits.view(np.int16)).cuda()
    kd = torch.zeros((4, 64, 64), dtype=torch.uint8, device="cuda")
    ks = torch.zeros((4, 64, 4), dtype=torch.uint8, device="cuda")
    slots = torch.arange(40, dtype=torch.int64, device="cuda") * 3
    mx.write_pages(big.view(torch.bfloat16)[:, :128], slots, kd, ks)
    hd, hs = np.zeros((4, 64, 64), np.uint8), np.zeros((4, 64, 4), np.uint8)
    writer.write_pages(bits, slots.cpu().numpy(), hd, hs, 64)
    torch.cuda.synchronize()
    assert np.array_equal(kd.cpu().numpy(), hd) and np.array_equal(ks.cpu().numpy(), hs)
    with pytest.raises(ValueError):
        mx.write_pages(big.view(torch.bfloat16)[:, :128], slots.int(), kd, ks)          # int32 slots
    with pytest.raises(ValueError):
        mx.write_pages(big.view(torch.bfloat16)[:, 1:129], slots, kd, ks)               # misaligned rows


def test_write_then_score():
    # the writer feeds the scorer: pages written from bf16 keys, then scored
    # (prefill, 24 rows after a prefix of 1000) against the scorer oracle
    rng = np.random.default_rng(9)
    P, H, ctx, q = 128, 16, 1024, 24
    wl = W.Workload("write_score", "prefill", H=H, page_size=P, q_lens=[q], prefix_lens=[ctx - q],
                    seq_lens=[ctx], want_logits=True, pool_pages=8)
    host = W.make_inputs(wl, 31, "cpu")
    keys = (rng.standard_normal((ctx, 128)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    bt = host.block_table[0].numpy()
    slots = np.array([int(bt[t // P]) * P + t % P for t in range(ctx)], dtype=np.int64)
    kd = torch.zeros_like(host.k_data).cuda()
    ks = torch.zeros_like(host.k_scale).cuda()
    mx.write_pages(torch.from_numpy(keys.view(np.int16)).cuda().view(torch.bfloat16), torch.from_numpy(slots).cuda(),
                   kd, ks)
    hd, hs = np.zeros(tuple(kd.shape), np.uint8), np.zeros(tuple(ks.shape), np.uint8)
    writer.write_pages(keys, slots, hd, hs, P)
    torch.cuda.synchronize()
    assert np.array_equal(kd.cpu().numpy(), hd) and np.array_equal(ks.cpu().numpy(), hs)
    host.k_data, host.k_scale = torch.from_numpy(hd), torch.from_numpy(hs)
    bs, lg = mx.score_prefill(host.q.cuda(), kd, ks, host.block_table.cuda(), host.cu_seqlens_q.cuda(),
                              host.seq_lens.cuda(), host.prefix_lens.cuda(), q, ctx, W.INV_SQRT_D, logits=True)
    ref = oracle_run(host, want_logits=True, want_blocks=True)
    compare(lg.cpu().numpy(), ref.logits, ref.mags, W.INV_SQRT_D, what="logits of written pages", min_exact=0.99,
            max_outside=47)
    compare(bs.cpu().numpy(), ref.blocks, ref.block_mags, W.INV_SQRT_D, what="block scores of written pages",
            min_exact=0.99, max_outside=1)

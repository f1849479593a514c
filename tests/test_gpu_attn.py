"""GPU parity of the paged MXFP4 attention decode (mxs_attn_decode, through
the C ABI) against oracle/attn.py.

Bound per output element, from the kernel's arithmetic: the probabilities
are rounded to bf16 (relative 2^-9) and normalised by the sum of the rounded
values, so each weight is within about 2^-8 of the exact softmax weight,
relative; a logit carries the block-scaled MFMA's error, at most
2^-10 * scale * sum_e |Q_hat_e K_e| (the scorers' bound), which moves a
weight by at most twice that, relative; the normalised output is rounded
once to bf16 (2^-9). With a 2x margin on the rounding terms:
    |gpu - ref| <= (2^-7 + 2 * dS) * sum_t w_t |V_t| + 2^-8 * |ref|,
    dS = 2^-10 * scale * max_t sum_e |Q_hat_e K_t,e|.
As the scorers' bit-identical floor does, a percentile guard keeps the bound
from hiding a drift: the 99th percentile of |gpu - ref| / sum_t w_t |V_t| must
stay below 2^-8 (the bf16 rounding of the weights).
"""
import math

import numpy as np
import pytest
import torch

import mxfp4_paged_cache_amd as mx
from mxfp4_paged_cache_amd import workloads as W
from oracle import attn
from tests.gpu_helpers import say

pytestmark = pytest.mark.gpu

SCALE = float(np.float32(1.0 / math.sqrt(128.0)))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    mx.lib()
    yield
    torch.cuda.synchronize()


def make_case(seed, *, R, Hkv, G, P, ctx, q_dtype="bf16", extra_pages=3, scale_lo=122, scale_hi=127):
    rng = np.random.default_rng(seed)
    npr = [(c + P - 1) // P for c in ctx]
    pool = sum(npr) + extra_pages
    kd = rng.integers(0, 256, (pool, Hkv, P, 64), dtype=np.uint8)
    vd = rng.integers(0, 256, (pool, Hkv, P, 64), dtype=np.uint8)
    ks = rng.integers(scale_lo, scale_hi + 1, (pool, Hkv, P, 4), dtype=np.uint8)
    vs = rng.integers(scale_lo, scale_hi + 1, (pool, Hkv, P, 4), dtype=np.uint8)
    perm = rng.permutation(pool)
    width = max(npr + [1]) + 2
    bt = np.full((R, width), -1, np.int32)
    pos = 0
    for r in range(R):
        bt[r, :npr[r]] = perm[pos:pos + npr[r]]
        pos += npr[r]
        if ctx[r] % P:                                   # garbage past the context: e2m1 -6, e8m0 NaN
            last = bt[r, npr[r] - 1]
            for arr, val in ((kd, 0xFF), (vd, 0xFF), (ks, 255), (vs, 255)):
                arr[last, :, ctx[r] % P:] = val
    Hq = Hkv * G
    if q_dtype == "bf16":
        x = rng.standard_normal((R, Hq, 128)).astype(np.float32)
        q = (x.view(np.uint32) >> 16).astype(np.uint16)
    else:                                                 # N(0, 1) stored as e4m3 (the writer's main query)
        x = torch.from_numpy(rng.standard_normal((R, Hq, 128)).astype(np.float32))
        q = x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return dict(q=q, kd=kd, ks=ks, vd=vd, vs=vs, bt=bt, ctx=np.array(ctx, np.int32), P=P, q_dtype=q_dtype)


def to_gpu(c):
    q = torch.from_numpy(c["q"].view(np.int16) if c["q_dtype"] == "bf16" else c["q"]).cuda()
    q = q.view(torch.bfloat16) if c["q_dtype"] == "bf16" else q.view(torch.float8_e4m3fn)
    t = {k: torch.from_numpy(c[k]).cuda() for k in ("kd", "ks", "vd", "vs", "bt", "ctx")}
    return q, t


def compare(gpu: np.ndarray, ref: np.ndarray, mag: np.ndarray, qk_mag: np.ndarray, what: str):
    assert gpu.shape == ref.shape
    assert np.isfinite(gpu).all(), f"{what}: non-finite output"
    err = np.abs(gpu - ref)
    ds = 2.0 ** -10 * SCALE * qk_mag[:, :, None]
    tol = (2.0 ** -7 + 2 * ds) * mag + 2.0 ** -8 * np.abs(ref)
    bad = err > tol
    if bad.any():
        k = np.unravel_index(np.argmax(err - tol), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {err.size} outside the bound; worst at {k}: "
                             f"gpu={gpu[k]!r} ref={ref[k]!r} mag={mag[k]!r}")
    live = mag > 0
    rel = err[live] / mag[live]
    p99 = float(np.quantile(rel, 0.99)) if rel.size else 0.0
    say(f"  {what}: {err.size} values, err/mag max {rel.max() if rel.size else 0:.3g}, p99 {p99:.3g}, "
        f"mean {rel.mean() if rel.size else 0:.3g}")
    assert p99 <= 2.0 ** -8, f"{what}: 99th percentile of err/mag {p99:.3g} above 2^-8"


def run_case(c, *, rows=None, max_context=None, out=None):
    q, t = to_gpu(c)
    mc = int(c["ctx"].max()) if max_context is None else max_context
    o = mx.attn_decode(q, t["kd"], t["ks"], t["vd"], t["vs"], t["bt"], t["ctx"], mc, SCALE, out=out)
    torch.cuda.synchronize()
    ref, mag, qkm = attn.attn_decode(q=c["q"], q_dtype=c["q_dtype"], k_data=c["kd"], k_scale=c["ks"],
                                     v_data=c["vd"], v_scale=c["vs"], block_table=c["bt"],
                                     context_lens=np.minimum(c["ctx"], mc), page_size=c["P"], scale=SCALE, rows=rows,
                                     want_mag=True)
    got = o.float().cpu().numpy()
    if rows is not None:
        got = got[rows]
    return got, ref, mag, qkm


CTX = [0, 1, 63, 64, 65, 127, 129, 300, 700, 513]


@pytest.mark.parametrize("P", [64, 128])
@pytest.mark.parametrize("q_dtype", ["bf16", "e4m3"])
@pytest.mark.parametrize("Hkv,G", [(1, 16), (2, 4), (3, 1)])
def test_attn_matches_oracle(P, q_dtype, Hkv, G):
    say(f"attn P={P} q={q_dtype} Hkv={Hkv} G={G}")
    c = make_case(100 + P + 7 * G + Hkv, R=len(CTX), Hkv=Hkv, G=G, P=P, ctx=CTX, q_dtype=q_dtype)
    got, ref, mag, qkm = run_case(c)
    compare(got, ref, mag, qkm, "attention output")
    assert np.all(got[0] == 0.0)                         # a row with no token gives zeros


def test_attn_seeded_sweep_of_shapes():
    # 24 seeded shapes: rows, kv heads, query heads per kv head (1..16), page
    # size, query dtype, contexts from 0 to past a page boundary and long ones,
    # both scale-byte ranges, and max_context below the longest context
    rng = np.random.default_rng(2028)
    for n in range(24):
        P = int(rng.choice([64, 128]))
        R = int(rng.integers(1, 41))
        Hkv = int(rng.integers(1, 5))
        G = int(rng.choice([1, 2, 3, 5, 8, 16]))
        edges = [0, 1, P - 1, P, P + 1]
        ctx = [int(rng.choice(edges)) if rng.random() < 0.3 else int(rng.integers(0, 1500)) for _ in range(R)]
        wide = bool(rng.random() < 0.25)
        q_dtype = str(rng.choice(["bf16", "e4m3"]))
        clamp = bool(rng.random() < 0.25) and max(ctx) > 1
        mc = int(rng.integers(1, max(ctx))) if clamp else None
        say(f"attn sweep{n}: P={P} R={R} Hkv={Hkv} G={G} q={q_dtype} wide={wide} max_context={mc} ctx={ctx}")
        c = make_case(5000 + n, R=R, Hkv=Hkv, G=G, P=P, ctx=ctx, q_dtype=q_dtype,
                      scale_lo=100 if wide else 122, scale_hi=150 if wide else 127)
        got, ref, mag, qkm = run_case(c, max_context=mc)
        compare(got, ref, mag, qkm, f"attn sweep{n}")
        live = np.minimum(c["ctx"], mc if mc is not None else c["ctx"].max()) > 0
        assert np.all(got[~live] == 0.0)                 # rows with no live token give zeros


def test_attn_wide_scales_and_single_token_rows():
    # e8m0 bytes 100..150: one live token returns its V (bf16-exact), wide scales elsewhere
    c = make_case(7, R=4, Hkv=1, G=8, P=128, ctx=[1, 1, 260, 1000], scale_lo=100, scale_hi=150)
    got, ref, mag, qkm = run_case(c)
    compare(got, ref, mag, qkm, "attention output, wide scales")
    assert np.array_equal(got[:2], ref[:2])              # softmax over one token: exactly V


def test_attn_clamps_to_max_context_and_strided_output():
    c = make_case(8, R=3, Hkv=2, G=2, P=64, ctx=[300, 40, 200])
    full = torch.full((3, 4, 256), 7.0, dtype=torch.bfloat16, device="cuda")
    got, ref, mag, qkm = run_case(c, max_context=130, out=full[:, :, :128])
    compare(got, ref, mag, qkm, "attention output, clamped context")
    assert torch.all(full[:, :, 128:] == 7.0)            # nothing written outside the view


def test_attn_rejections():
    c = make_case(9, R=2, Hkv=2, G=2, P=64, ctx=[10, 20])
    q, t = to_gpu(c)
    with pytest.raises(ValueError):                      # 3 query heads over 2 kv heads
        mx.attn_decode(q[:, :3], t["kd"], t["ks"], t["vd"], t["vs"], t["bt"], t["ctx"], 20, SCALE)
    big = torch.zeros((2, 34, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mx.MxsError):                     # 17 query heads per kv head
        mx.attn_decode(big, t["kd"], t["ks"], t["vd"], t["vs"], t["bt"], t["ctx"], 20, SCALE)
    with pytest.raises(ValueError):                      # block table narrower than max_context
        mx.attn_decode(q, t["kd"], t["ks"], t["vd"], t["vs"], t["bt"][:, :1], t["ctx"], 200, SCALE)


def test_full_attention_workload_sampled_rows():
    # the benchmark's workload and launch: 2048 rows x 16 query heads (e4m3), 2048 tokens each
    wl = W.attn_decode_sparse()
    say(f"case {wl.name}: generating inputs on the GPU")
    inp = W.make_inputs(wl, 31, "cuda")
    out = mx.attn_decode(inp.q, inp.k_data, inp.k_scale, inp.extras["v_data"], inp.extras["v_scale"],
                         inp.block_table, inp.seq_lens, wl.window, SCALE)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    rows = np.array([0, 1, 1023, 2047], np.int64)
    bt = inp.block_table.cpu().numpy()[rows]
    used = np.unique(bt[bt >= 0])
    idx = torch.as_tensor(used, dtype=torch.long, device="cuda")
    host = [t.index_select(0, idx).cpu().numpy() for t in (inp.k_data, inp.k_scale, inp.extras["v_data"],
                                                            inp.extras["v_scale"])]
    remap = np.full(int(bt.max()) + 1, -1, np.int64)
    remap[used] = np.arange(len(used))
    bt = np.where(bt >= 0, remap[np.maximum(bt, 0)], -1).astype(np.int32)
    q = inp.q.cpu()[rows].view(torch.uint8).numpy()
    ref, mag, qkm = attn.attn_decode(q=q, q_dtype="e4m3", k_data=host[0], k_scale=host[1], v_data=host[2],
                                     v_scale=host[3], block_table=bt, context_lens=inp.seq_lens.cpu().numpy()[rows],
                                     page_size=wl.page_size, scale=SCALE, want_mag=True)
    compare(out.float().cpu().numpy()[rows], ref, mag, qkm, "attention workload (4 sampled rows)")
    del out, inp
    torch.cuda.empty_cache()


def test_sparse_pipeline_graph_replay_with_poisoned_outputs():
    # decode scores over an fp8 index cache -> top-k pages of head 0 -> the
    # selected pages' K and V through the attention decode, captured in one
    # HIP graph; outputs are poisoned (NaN / -7) before every replay, and
    # every replay must give the eager result bit for bit
    P, B, k = 128, 4, 8
    wl = W.Workload("g_sparse", "decode", H=64, page_size=P, q_lens=[1] * B, prefix_lens=[0] * B,
                    seq_lens=[3000, 700, 129, 2000], k_dtype="e4m3", max_seq_len=3072)
    dev = W.make_inputs(wl, 44, "cuda")
    NB = wl.NB
    pool = dev.k_data.shape[0]
    rng = np.random.default_rng(45)
    kv = [torch.from_numpy(a).cuda() for a in (rng.integers(0, 256, (pool, 1, P, 64), dtype=np.uint8),
                                                 rng.integers(122, 128, (pool, 1, P, 4), dtype=np.uint8),
                                                 rng.integers(0, 256, (pool, 1, P, 64), dtype=np.uint8),
                                                 rng.integers(122, 128, (pool, 1, P, 4), dtype=np.uint8))]
    qa = torch.randn((B, 16, 128), device="cuda").to(torch.bfloat16)
    bs = torch.empty((B, 64, NB), device="cuda")
    sel = torch.empty((B, 64, k), dtype=torch.int32, device="cuda")
    out = torch.empty((B, 16, 128), dtype=torch.bfloat16, device="cuda")
    plan = mx.make_plan("decode", torch.bfloat16, P, 64, B, 1, wl.window, False, True, k_dtype="e4m3")
    seq = dev.seq_lens
    tail_tokens = ((seq - 1) % P + 1).to(torch.int32)

    def step():
        mx.score_decode(dev.q, dev.k_data, None, dev.block_table, seq, wl.window, SCALE, out=bs, plan=plan)
        mx.select_pages(bs, k, seq, wl.window, P, out=sel)
        s0 = sel[:, 0, :]
        live = s0 >= 0
        table = torch.where(live, dev.block_table.gather(1, s0.clamp(min=0).long()), -1).to(torch.int32)
        ctx = ((live.sum(1).to(torch.int32) - 1) * P + tail_tokens).to(torch.int32)
        mx.attn_decode(qa, kv[0], kv[1], kv[2], kv[3], table.contiguous(), ctx.contiguous(), k * P, SCALE, out=out)

    step()
    torch.cuda.synchronize()
    eager = [bs.clone(), sel.clone(), out.clone()]
    assert torch.isfinite(out.float()).all()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        bs.fill_(float("nan"))
        sel.fill_(-7)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bs.view(torch.int32), eager[0].view(torch.int32)), rep
        assert torch.equal(sel, eager[1]), rep
        assert torch.equal(out.view(torch.int16), eager[2].view(torch.int16)), rep
    say("  3 replays of score -> select -> attention with poisoned outputs equal the eager run")

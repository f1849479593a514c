"""Seeded synthetic inputs for paged MXFP4 index scoring.

This module holds no arithmetic of the scoring method: it only draws random
bytes and values and lays them out. Both the HIP path and the CPU oracle are
fed from it, so it must stay free of decoding, rounding rules or scoring.

Recipe (the pages' scorer benchmarks use random K data with e8m0 bytes in
[122, 127] and Q drawn per row; aiter #7061, "Performance"):
* Q: N(0, 1) fp32 draws cast by torch to bf16, or to float8_e4m3fn where a
  workload hands the query over as e4m3;
* K data: uniform random bytes, so both e2m1 codes of a byte are uniform over
  all 16 codes;
* K scales: uniform random e8m0 bytes in [lo, hi], one per (token, 32-element
  block), or one per token repeated over its four blocks (scale_mode "token",
  the chunked-prefill workload's per-token bytes);
* fp8 cache (k_dtype "e4m3", the format the MXFP4 one replaces): 128 bytes
  per token drawn uniformly over the 254 finite e4m3 codes, no scale view;
* block table: distinct pages drawn without replacement from a larger pool, so
  the gather is a real random gather;
* cu_seqlens_q / seq_lens / prefix_lens: as the workload states;
* attention decode (attn_group > 0): K and V caches [pages, kv heads, P, 64]
  + [pages, kv heads, P, 4], bytes drawn as for the index cache.

Streams: one torch.Generator per field, seeded with (seed, field id), so a
field can be regenerated without the others.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import torch

D = 128                    # head dim: 64 B of e2m1 data + 4 e8m0 bytes per token
SLOT_DATA_BYTES = 64
SLOT_SCALE_BYTES = 4

F_Q, F_KDATA, F_KSCALE, F_TABLE, F_POISON = range(5)


@dataclass
class Workload:
    name: str
    mode: str                       # "prefill" | "decode" | "logits"
    H: int
    page_size: int
    q_lens: List[int]               # per request (decode: all 1)
    prefix_lens: List[int]
    seq_lens: List[int]
    q_dtype: str = "bf16"           # "bf16" | "e4m3"
    scale_lo: int = 122
    scale_hi: int = 127
    scale_mode: str = "block"       # "block": a byte per (token, 32-block); "token": one byte per token
    pool_pages: int = 0             # 0 -> exactly the pages the requests need
    want_logits: bool = False
    want_blocks: bool = True
    layout: str = "split"           # "split" | "region" | "shared"
    shared_first_page: int = 0      # physical id of the first used page ("shared")
    table_pad: int = 0              # extra -1 entries per block-table row
    table_width: int = 0            # minimum block-table width
    table_fill: str = "pad"         # entries past a request's pages: "pad" (-1) or "perm" (more distinct pages)
    max_seq_len: Optional[int] = None
    tables: int = 1                 # disjoint block tables (benchmark rotation)
    select_k: int = 0               # > 0: the workload is top-k page selection over this prefill's block scores
    write_tokens: int = 0           # > 0: the workload is writing this many bf16 keys into page slots
    k_dtype: str = "mxfp4"          # "mxfp4" (e2m1 + e8m0 views) | "e4m3" (fp8 cache, 128 B per token)
    attn_group: int = 0             # > 0: paged attention decode; H kv heads with this many query heads each
    note: str = ""

    @property
    def B(self) -> int:
        return len(self.seq_lens)

    @property
    def T(self) -> int:
        return sum(self.q_lens)

    @property
    def window(self) -> int:
        return self.max_seq_len if self.max_seq_len is not None else max(self.seq_lens, default=0)

    @property
    def NB(self) -> int:
        return (self.window + self.page_size - 1) // self.page_size

    def limits(self) -> List[int]:
        """Live-token count per query row, in row order."""
        out = []
        for b in range(self.B):
            for i in range(self.q_lens[b]):
                if self.mode == "decode":
                    lim = self.seq_lens[b]
                else:
                    lim = min(self.seq_lens[b], self.prefix_lens[b] + i + 1)
                out.append(max(0, min(lim, self.window)))
        return out

    def live_triples(self) -> int:
        return sum(self.limits()) * self.H

    def pages_per_request(self) -> List[int]:
        return [(s + self.page_size - 1) // self.page_size for s in self.seq_lens]


def _gen(seed: int, fid: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1000003 + fid * 7919 + 17)
    return g


@dataclass
class Inputs:
    wl: Workload
    q: torch.Tensor                 # [T, H, 128] bf16 or float8_e4m3fn (may be a strided view)
    k_data: torch.Tensor            # uint8 view [pages, P, 64] (fp8 cache: [pages, P, 128])
    k_scale: Optional[torch.Tensor]  # uint8 view [pages, P, 4] (fp8 cache: None)
    block_tables: List[torch.Tensor]  # int32 [B, width], one per rotation
    cu_seqlens_q: torch.Tensor      # int32 [B+1]
    seq_lens: torch.Tensor          # int32 [B]
    prefix_lens: torch.Tensor       # int32 [B]
    region: Optional[torch.Tensor] = None   # backing uint8 region for "region"/"shared"
    extras: dict = field(default_factory=dict)

    @property
    def block_table(self) -> torch.Tensor:
        return self.block_tables[0]


def make_q(wl: Workload, seed: int, device="cpu", q_strided: bool = False) -> torch.Tensor:
    g = _gen(seed, F_Q, device)
    T = wl.T
    heads = wl.H * wl.attn_group if wl.attn_group else wl.H
    x = torch.randn((T, heads, D), generator=g, device=device, dtype=torch.float32)
    dt = torch.bfloat16 if wl.q_dtype == "bf16" else torch.float8_e4m3fn
    if not q_strided:
        return x.to(dt)
    # strided rows: every row padded by 64 extra elements, heads padded by 128
    big = torch.zeros((T, heads, 2 * D), device=device, dtype=dt)
    big[:, :, :D] = x.to(dt)
    return big[:, :, :D]


def make_inputs(wl: Workload, seed: int = 0, device="cpu", q_strided: bool = False) -> Inputs:
    P = wl.page_size
    npr = wl.pages_per_request()
    need = sum(npr)
    width = max(max(npr, default=0), wl.NB, wl.table_width) + wl.table_pad
    per_table = need if wl.table_fill == "pad" else wl.B * width
    pool = max(1, wl.pool_pages, per_table * wl.tables)   # the scorers take pools of one page or more
    if wl.layout == "shared":
        pool = max(pool, wl.shared_first_page + per_table * wl.tables)

    gd = _gen(seed, F_KDATA, device)
    gs = _gen(seed, F_KSCALE, device)
    gt = _gen(seed, F_TABLE, "cpu")

    region = None
    fp8 = wl.k_dtype == "e4m3"
    tb = 128 if fp8 else SLOT_DATA_BYTES     # data bytes per token
    sb = 0 if fp8 else SLOT_SCALE_BYTES      # scale bytes per token

    def scale_bytes(shape):
        # shape [..., 4]: one draw per block, or one per token repeated over its 4 blocks
        if wl.scale_mode == "token":
            one = torch.randint(wl.scale_lo, wl.scale_hi + 1, tuple(shape[:-1]) + (1,), generator=gs, device=device,
                                dtype=torch.uint8)
            return one.expand(*shape).contiguous()
        return torch.randint(wl.scale_lo, wl.scale_hi + 1, tuple(shape), generator=gs, device=device,
                             dtype=torch.uint8)

    def data_bytes(shape):
        if not fp8:
            return torch.randint(0, 256, shape, generator=gd, device=device, dtype=torch.uint8)
        # uniform over the 254 finite e4m3 codes: skip 0x7F (and 0xFF, never drawn)
        u = torch.randint(0, 254, shape, generator=gd, device=device, dtype=torch.uint8)
        return u + (u >= 0x7F).to(torch.uint8)

    if wl.attn_group:
        # paged K and V caches with kv heads: [pool, H, P, 64] data + [pool, H, P, 4] scales each
        k_data = torch.randint(0, 256, (pool, wl.H, P, SLOT_DATA_BYTES), generator=gd, device=device, dtype=torch.uint8)
        k_scale = torch.randint(wl.scale_lo, wl.scale_hi + 1, (pool, wl.H, P, SLOT_SCALE_BYTES), generator=gs,
                                device=device, dtype=torch.uint8)
        v_data = torch.randint(0, 256, (pool, wl.H, P, SLOT_DATA_BYTES), generator=gd, device=device, dtype=torch.uint8)
        v_scale = torch.randint(wl.scale_lo, wl.scale_hi + 1, (pool, wl.H, P, SLOT_SCALE_BYTES), generator=gs,
                                device=device, dtype=torch.uint8)
    elif wl.layout == "split":
        k_data = data_bytes((pool, P, tb))
        k_scale = None if fp8 else scale_bytes((pool, P, SLOT_SCALE_BYTES))
    else:
        # One uint8 region. "region": page = [P x 64 B data][P x 4 B scale].
        # "shared": page block = two layer slots of that shape; slot 1 is scored,
        # every byte outside the scored pages is 0xFF (e2m1 -6, e8m0 NaN).
        slot = P * (tb + sb)
        stride = slot if wl.layout == "region" else 2 * slot
        off = 0 if wl.layout == "region" else slot
        region = torch.full((pool * stride,), 0xFF, device=device, dtype=torch.uint8)
        view = region.view(pool, stride)
        lo = wl.shared_first_page if wl.layout == "shared" else 0
        hi = pool
        nused = hi - lo
        view[lo:hi, off:off + P * tb] = data_bytes((nused, P * tb))
        k_data = torch.as_strided(region, (pool, P, tb), (stride, tb, 1), off)
        k_scale = None
        if not fp8:
            scale_part = scale_bytes((nused, P, SLOT_SCALE_BYTES)).reshape(nused, P * SLOT_SCALE_BYTES)
            view[lo:hi, off + P * tb:off + slot] = scale_part
            k_scale = torch.as_strided(region, (pool, P, SLOT_SCALE_BYTES), (stride, SLOT_SCALE_BYTES, 1),
                                       off + P * tb)

    # block tables: distinct pages; rotations use disjoint page sets
    lo = wl.shared_first_page if wl.layout == "shared" else 0
    perm = torch.randperm(pool - lo, generator=gt)[: per_table * wl.tables] + lo
    tables = []
    for r in range(wl.tables):
        bt = torch.full((wl.B, width), -1, dtype=torch.int32)
        chunk = perm[r * per_table:(r + 1) * per_table]
        pos = 0
        for b in range(wl.B):
            n = npr[b] if wl.table_fill == "pad" else width
            bt[b, :n] = chunk[pos:pos + n].to(torch.int32)
            pos += n
        tables.append(bt.to(device))

    cu = [0]
    for ql in wl.q_lens:
        cu.append(cu[-1] + ql)
    extras = {"v_data": v_data, "v_scale": v_scale} if wl.attn_group else {}
    return Inputs(
        extras=extras,
        wl=wl,
        q=make_q(wl, seed, device, q_strided),
        k_data=k_data,
        k_scale=k_scale,
        block_tables=tables,
        cu_seqlens_q=torch.tensor(cu, dtype=torch.int32, device=device),
        seq_lens=torch.tensor(wl.seq_lens, dtype=torch.int32, device=device),
        prefix_lens=torch.tensor(wl.prefix_lens, dtype=torch.int32, device=device),
        region=region,
    )


# ---------------------------------------------------------------- workloads

INV_SQRT_D = float(torch.tensor(1.0 / math.sqrt(D), dtype=torch.float32))   # RN32(1/sqrt(128))


def prefill_small() -> Workload:
    """64 query rows after a 960-token prefix, context 1024, 16-page pool, logits + block scores."""
    return Workload("prefill_q64_ctx1k", "prefill", H=64, page_size=128, q_lens=[64], prefix_lens=[960],
                    seq_lens=[1024], pool_pages=16, want_logits=True, table_width=16, table_fill="perm")


def decode_b64_128k(tables: int = 1) -> Workload:
    """B=64 decode rows, context 131072 (1024 pages each), pages drawn from a 300k-page pool."""
    return Workload("decode_b64_ctx128k", "decode", H=64, page_size=128, q_lens=[1] * 64,
                    prefix_lens=[131071] * 64, seq_lens=[131072] * 64, pool_pages=300_000, tables=tables)


def prefill_long() -> Workload:
    """4096 query rows after a 126976-token prefix (context 131072), e4m3 Q given directly."""
    return Workload("prefill_q4096_ctx128k", "prefill", H=64, page_size=128, q_lens=[4096], prefix_lens=[126976],
                    seq_lens=[131072], q_dtype="e4m3", pool_pages=300_000)


def prefill_chunk() -> Workload:
    """32768-row chunk after a 100000-token prefix (context 132768), one e8m0 byte per token, uniform in 100..150."""
    return Workload("prefill_chunk32k_ctx132768", "prefill", H=64, page_size=128, q_lens=[32768],
                    prefix_lens=[100000], seq_lens=[132768], scale_lo=100, scale_hi=150, scale_mode="token",
                    pool_pages=300_000)


def prefill_chunk_block_scales() -> Workload:
    """The chunked prefill with an e8m0 byte drawn per (token, 32-element block) instead of per token."""
    wl = prefill_chunk()
    wl.name = "prefill_chunk32k_ctx132768_blockscales"
    wl.scale_mode = "block"
    return wl


def logits_shared_pool() -> Workload:
    """Logits mode, 64-token pages in a shared two-slot region past byte offset 4.608e9, B=8 x 128 rows, ctx 8192."""
    return Workload("logits_b8_q128_ctx8k_shared", "logits", H=64, page_size=64, q_lens=[128] * 8,
                    prefix_lens=[8064] * 8, seq_lens=[8192] * 8, want_logits=True, want_blocks=False,
                    layout="shared", shared_first_page=529_412, table_pad=8)


def select_after_prefill_long() -> Workload:
    """Top-64 page selection over the block scores of the 4096-row, 128K-context prefill (4096 x 64 x 1024)."""
    wl = prefill_long()
    wl.name = "select_k64_q4096_ctx128k"
    wl.select_k = 64
    return wl


def write_1m_tokens() -> Workload:
    """Writing 1,048,576 bf16 keys (8192 whole 128-token pages in random page order) into a 300k-page pool."""
    return Workload("write_1m_tokens_p128", "prefill", H=1, page_size=128, q_lens=[1], prefix_lens=[0],
                    seq_lens=[1], pool_pages=300_000, write_tokens=1 << 20)


def attn_decode_sparse() -> Workload:
    """Paged MXFP4 attention decode: 2048 rows (one kv head, 16 query heads each, e4m3 query), 2048 live
    tokens per row (16 selected 128-token pages), K and V pages drawn from a 300k-page pool."""
    return Workload("attn_decode_r2048_ctx2048_g16", "decode", H=1, page_size=128, q_lens=[1] * 2048,
                    prefix_lens=[2047] * 2048, seq_lens=[2048] * 2048, q_dtype="e4m3", pool_pages=300_000,
                    attn_group=16)


def decode_b64_128k_fp8() -> Workload:
    """The decode workload over an fp8 (e4m3, 128 B per token) index cache: the format the MXFP4 one replaces."""
    wl = decode_b64_128k()
    wl.name = "decode_b64_ctx128k_fp8cache"
    wl.k_dtype = "e4m3"
    return wl


def prefill_long_fp8() -> Workload:
    """The 4096-row, 128K-context prefill over an fp8 index cache."""
    wl = prefill_long()
    wl.name = "prefill_q4096_ctx128k_fp8cache"
    wl.k_dtype = "e4m3"
    return wl


def write_1m_tokens_fp8() -> Workload:
    """Writing 1,048,576 bf16 keys into an fp8 index cache (128 e4m3 bytes per token)."""
    wl = write_1m_tokens()
    wl.name = "write_1m_tokens_p128_fp8cache"
    wl.k_dtype = "e4m3"
    return wl


CONFIGS = {
    1: prefill_small,
    2: decode_b64_128k,
    3: prefill_long,
    4: prefill_chunk,
    5: logits_shared_pool,
    6: select_after_prefill_long,
    7: write_1m_tokens,
    8: decode_b64_128k_fp8,
    9: prefill_long_fp8,
    10: write_1m_tokens_fp8,
    11: attn_decode_sparse,
    12: prefill_chunk_block_scales,
}

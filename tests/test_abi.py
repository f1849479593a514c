"""C-ABI checks that need no GPU: the library loads, exports what the header
declares, validates arguments before any device work, and plans purely from
host integers (aiter #5518, decode auto-CTA: host-known buckets, graph-stable).
"""
import ctypes
import os
import re

import pytest

import mxfp4_paged_cache_amd as mx
from mxfp4_paged_cache_amd import build as mxbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxscore.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(mx.library_path()):
        mxbuild.build(force=True)
    return mx.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mxs_[a-z_]+)\s*\(", text)))


def test_header_and_library_agree(L):
    names = declared_functions()
    assert set(names) == set(mx.SYMBOLS)
    for n in names:
        assert hasattr(L, n), f"{n} declared in mxscore.h but not exported"


def test_exports_are_c_symbols():
    out = os.popen(f"nm -D --defined-only {mx.library_path()}").read()
    for n in declared_functions():
        assert re.search(rf"\bT {n}$", out, re.M), n


def test_version(L):
    assert b"gfx950" in L.mxs_version()


# ------------------------------------------------------------------ validation

FAKE = 0x7F0000000000   # 16-byte aligned, never dereferenced: every case below fails validation first


def valid_args(mode=mx.MXS_MODE_PREFILL):
    q = mx.Query(FAKE, mx.MXS_Q_BF16, 64 * 128, 128, 64)
    k = mx.KCache(data=FAKE + 0x100000, data_page_stride=8704, scale=FAKE + 0x100000 + 8192, scale_page_stride=8704,
                  page_size=128, k_dtype=mx.MXS_K_MXFP4, num_pages=16)
    b = mx.Batch(FAKE + 0x200000, 16, 16, FAKE + 0x300000, FAKE + 0x300100, FAKE + 0x300200, 1, 64, 64, 1024)
    bs = mx.Out(FAKE + 0x400000, 64 * 8, 8)
    lg = mx.Out(None, 0, 0)
    return q, k, b, bs, lg


def call(L, q, k, b, bs, lg, sm=0.0883883, fn="mxs_score_prefill"):
    f = getattr(L, fn)
    return f(ctypes.byref(q), ctypes.byref(k), ctypes.byref(b), ctypes.c_float(sm), ctypes.byref(bs),
             ctypes.byref(lg), None, None)


CASES = [
    ("fp16 query dtype", lambda q, k, b, bs, lg: setattr(q, "dtype", 3), mx.MXS_EDTYPE),
    ("zero heads", lambda q, k, b, bs, lg: setattr(q, "num_heads", 0), mx.MXS_EINVAL),
    ("page size 32", lambda q, k, b, bs, lg: setattr(k, "page_size", 32), mx.MXS_ELAYOUT),
    ("misaligned query rows", lambda q, k, b, bs, lg: setattr(q, "row_stride", 64 * 128 + 4), mx.MXS_ELAYOUT),
    ("misaligned query base", lambda q, k, b, bs, lg: setattr(q, "ptr", FAKE + 8), mx.MXS_ELAYOUT),
    ("narrow data view", lambda q, k, b, bs, lg: setattr(k, "data_page_stride", 4096), mx.MXS_ELAYOUT),
    ("narrow scale view", lambda q, k, b, bs, lg: setattr(k, "scale_page_stride", 256), mx.MXS_ELAYOUT),
    ("misaligned data view", lambda q, k, b, bs, lg: setattr(k, "data", FAKE + 0x100004), mx.MXS_ELAYOUT),
    ("misaligned scale view", lambda q, k, b, bs, lg: setattr(k, "scale", FAKE + 0x100002), mx.MXS_ELAYOUT),
    ("no pages", lambda q, k, b, bs, lg: setattr(k, "num_pages", 0), mx.MXS_EINVAL),
    ("narrow block table", lambda q, k, b, bs, lg: setattr(b, "bt_width", 7), mx.MXS_ELAYOUT),
    ("null block table", lambda q, k, b, bs, lg: setattr(b, "block_table", None), mx.MXS_EINVAL),
    ("null seq_lens", lambda q, k, b, bs, lg: setattr(b, "seq_lens", None), mx.MXS_EINVAL),
    ("null prefix_lens", lambda q, k, b, bs, lg: setattr(b, "prefix_lens", None), mx.MXS_EINVAL),
    ("negative batch", lambda q, k, b, bs, lg: setattr(b, "batch", -1), mx.MXS_EINVAL),
    ("no block_scores", lambda q, k, b, bs, lg: setattr(bs, "ptr", None), mx.MXS_EINVAL),
    ("narrow output rows", lambda q, k, b, bs, lg: setattr(bs, "head_stride", 4), mx.MXS_ELAYOUT),
    ("misaligned output", lambda q, k, b, bs, lg: setattr(bs, "ptr", FAKE + 0x400002), mx.MXS_ELAYOUT),
    ("null query", lambda q, k, b, bs, lg: setattr(q, "ptr", None), mx.MXS_EINVAL),
    ("unknown cache dtype", lambda q, k, b, bs, lg: setattr(k, "k_dtype", 2), mx.MXS_EDTYPE),
    ("null scale view (MXFP4)", lambda q, k, b, bs, lg: setattr(k, "scale", None), mx.MXS_EINVAL),
    # an fp8 cache needs 128 bytes per token: the 8704-byte MXFP4 page stride is too narrow
    ("narrow fp8 data view", lambda q, k, b, bs, lg: setattr(k, "k_dtype", mx.MXS_K_E4M3), mx.MXS_ELAYOUT),
    # page-rounded token indices must stay within int32
    ("window above 2^31 - 256", lambda q, k, b, bs, lg: setattr(b, "max_seq_len", 2**31 - 255), mx.MXS_EINVAL),
]


@pytest.mark.parametrize("name,mutate,code", CASES, ids=[c[0] for c in CASES])
def test_rejections_before_device_work(L, name, mutate, code):
    q, k, b, bs, lg = valid_args()
    mutate(q, k, b, bs, lg)
    assert call(L, q, k, b, bs, lg) == code, L.mxs_last_error()
    assert L.mxs_last_error()


@pytest.mark.parametrize("sm", [0.0, -1.0, float("nan"), float("inf")])
def test_rejects_bad_sm_scale(L, sm):
    q, k, b, bs, lg = valid_args()
    assert call(L, q, k, b, bs, lg, sm=sm) == mx.MXS_EINVAL


def test_empty_problems_accept_null_outputs(L):
    # no rows (an empty tensor's data pointer is NULL) or an empty window:
    # nothing to write, so the required output may be NULL; with rows it may not
    for field, decode_empty in (("total_rows", False), ("max_seq_len", True), ("batch", True)):
        q, k, b, bs, lg = valid_args()
        setattr(b, field, 0)
        bs.ptr = None
        assert call(L, q, k, b, bs, lg) == mx.MXS_OK, (field, L.mxs_last_error())
        # decode rows are the requests: total_rows = 0 leaves one row to score
        want = mx.MXS_OK if decode_empty else mx.MXS_EINVAL
        assert call(L, q, k, b, bs, lg, fn="mxs_score_decode") == want, (field, L.mxs_last_error())
    q, k, b, bs, lg = valid_args()
    bs.ptr = None
    assert call(L, q, k, b, bs, lg) == mx.MXS_EINVAL


def test_logits_mode_needs_logits(L):
    q, k, b, bs, lg = valid_args()
    assert call(L, q, k, b, lg, bs, fn="mxs_score_logits") == mx.MXS_EINVAL


def test_empty_problem_is_a_no_op(L):
    # nothing to write: returns OK without touching any pointer or the device
    q, k, b, bs, lg = valid_args()
    b.total_rows = 0
    assert call(L, q, k, b, bs, lg) == mx.MXS_OK
    q, k, b, bs, lg = valid_args()
    b.max_seq_len = 0
    assert call(L, q, k, b, bs, lg) == mx.MXS_OK


def test_no_device_is_reported():
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a HIP device is visible; this case only runs without one")
    L = mx.lib()
    q, k, b, bs, lg = valid_args()
    assert call(L, q, k, b, bs, lg) == mx.MXS_EUNSUPPORTED


def test_fp8_cache_needs_no_scale_view():
    # an fp8 cache with 128 B per token and no scale view passes every host
    # check (without a device the call then stops at the device query)
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a HIP device is visible; this case only runs without one")
    L = mx.lib()
    q, k, b, bs, lg = valid_args()
    k.k_dtype = mx.MXS_K_E4M3
    k.scale = None
    k.scale_page_stride = 0
    k.data_page_stride = 128 * 128
    assert call(L, q, k, b, bs, lg) == mx.MXS_EUNSUPPORTED
    k.data_page_stride = 128 * 128 + 8                                   # not a multiple of 16
    assert call(L, q, k, b, bs, lg) == mx.MXS_ELAYOUT


# ------------------------------------------------------------------ planning

def plan_for(L, mode, *, H=64, P=128, B=64, mql=1, msl=131072, lg=0, bs=1, pun=0, cus=256, occ=3, dt=mx.MXS_Q_BF16,
             kd=mx.MXS_K_MXFP4):
    p = mx.Plan()
    rc = L.mxs_plan_make_for(mode, dt, kd, P, H, B, mql, msl, lg, bs, pun, cus, occ, ctypes.byref(p))
    return rc, p


def test_plan_records_the_cache_dtype(L):
    for kd in (mx.MXS_K_MXFP4, mx.MXS_K_E4M3):
        for mode, kw in [(mx.MXS_MODE_DECODE, {}), (mx.MXS_MODE_PREFILL, dict(B=1, mql=4096))]:
            rc, p = plan_for(L, mode, kd=kd, **kw)
            assert rc == 0 and p.k_dtype == kd


def test_plan_is_pure(L):
    for mode, kw in [(mx.MXS_MODE_DECODE, {}), (mx.MXS_MODE_PREFILL, dict(B=1, mql=4096)),
                     (mx.MXS_MODE_LOGITS, dict(B=8, mql=128, msl=8192, P=64, lg=1, bs=0))]:
        rc1, p1 = plan_for(L, mode, **kw)
        rc2, p2 = plan_for(L, mode, **kw)
        assert rc1 == rc2 == 0
        assert bytes(p1) == bytes(p2)


def test_decode_plan_covers_every_page_once(L):
    for B, msl, occ in [(64, 131072, 3), (1, 8192, 3), (4, 1000, 2), (3, 0, 1)]:
        rc, p = plan_for(L, mx.MXS_MODE_DECODE, B=B, msl=msl, occ=occ)
        assert rc == 0
        NB = (msl + 127) // 128
        assert 1 <= p.pages_per_item <= 32
        assert p.page_items * p.pages_per_item >= NB
        # chunks come in fours (one workgroup = four chunks of one request);
        # only the surplus of that rounding may be empty
        assert p.page_items % 4 == 0
        nonempty = -(-max(NB, 1) // p.pages_per_item)
        assert p.page_items - nonempty < 4
        assert p.items == B * p.head_groups * p.page_items
        assert p.grid * 4 == p.items


def test_decode_with_logits_plans_the_logits_kernel(L):
    # a decode request is one query row: with logits it runs on the logits
    # kernel (64 query slots per item), block scores alone on the decode kernel
    for B, H, msl in [(64, 64, 131072), (5, 64, 1030), (3, 4, 256)]:
        rc, p = plan_for(L, mx.MXS_MODE_DECODE, B=B, H=H, msl=msl, lg=1)
        assert rc == 0
        assert p.kernel == 3 and p.max_query_len == 1
        assert p.slot_items * p.slots_per_item >= H
        assert p.page_items * p.pages_per_item >= (msl + 127) // 128
        assert p.items == B * p.slot_items * p.page_items
        rc, p0 = plan_for(L, mx.MXS_MODE_DECODE, B=B, H=H, msl=msl, lg=0)
        assert rc == 0 and p0.kernel == 1


def test_prefill_plan_covers_every_slot(L):
    for B, mql, H, msl in [(1, 4096, 64, 131072), (1, 32768, 64, 132768), (3, 17, 2, 300), (8, 128, 64, 8192)]:
        rc, p = plan_for(L, mx.MXS_MODE_PREFILL, B=B, mql=mql, H=H, msl=msl)
        assert rc == 0
        assert p.slot_items * p.slots_per_item >= mql * H
        assert p.page_items * p.pages_per_item >= (msl + 127) // 128
        assert p.items == B * p.slot_items * p.page_items
        assert 1 <= p.grid <= max(p.items, 1)


def test_parallel_unit_override(L):
    rc, p = plan_for(L, mx.MXS_MODE_PREFILL, B=1, mql=4096, pun=100)
    assert rc == 0 and p.grid == 100
    rc, p = plan_for(L, mx.MXS_MODE_DECODE, pun=512)
    assert rc == 0 and abs(p.grid - 512) <= 64


def test_plan_rejections(L):
    assert plan_for(L, 9)[0] == mx.MXS_EINVAL
    assert plan_for(L, mx.MXS_MODE_DECODE, P=32)[0] == mx.MXS_ELAYOUT
    assert plan_for(L, mx.MXS_MODE_DECODE, dt=5)[0] == mx.MXS_EDTYPE
    assert plan_for(L, mx.MXS_MODE_DECODE, kd=7)[0] == mx.MXS_EDTYPE
    assert plan_for(L, mx.MXS_MODE_DECODE, H=0)[0] == mx.MXS_EINVAL
    assert plan_for(L, mx.MXS_MODE_LOGITS, lg=0)[0] == mx.MXS_EINVAL
    assert plan_for(L, mx.MXS_MODE_DECODE, msl=2**31 - 255)[0] == mx.MXS_EINVAL
    assert plan_for(L, mx.MXS_MODE_DECODE, msl=2**31 - 256)[0] == mx.MXS_OK     # the largest window planned


def test_check_metadata_rejections_before_any_copy(L):
    q, k, b, bs, lg = valid_args()
    assert L.mxs_check_metadata(9, ctypes.byref(k), ctypes.byref(b), 0, None) == mx.MXS_EINVAL
    assert L.mxs_check_metadata(mx.MXS_MODE_PREFILL, None, ctypes.byref(b), 0, None) == mx.MXS_EINVAL
    bad = mx.KCache.from_buffer_copy(bytes(k))
    bad.page_size = 32
    assert L.mxs_check_metadata(mx.MXS_MODE_PREFILL, ctypes.byref(bad), ctypes.byref(b), 0, None) == mx.MXS_ELAYOUT
    empty = mx.Batch.from_buffer_copy(bytes(b))
    empty.batch = 0
    assert L.mxs_check_metadata(mx.MXS_MODE_DECODE, ctypes.byref(k), ctypes.byref(empty), 1, None) == mx.MXS_OK
    nulls = mx.Batch.from_buffer_copy(bytes(b))
    nulls.seq_lens = None
    assert L.mxs_check_metadata(mx.MXS_MODE_DECODE, ctypes.byref(k), ctypes.byref(nulls), 0, None) == mx.MXS_EINVAL
    assert b"NULL" in L.mxs_last_error()
    wide = mx.Batch.from_buffer_copy(bytes(b))
    wide.max_seq_len = 2**31 - 255
    assert L.mxs_check_metadata(mx.MXS_MODE_PREFILL, ctypes.byref(k), ctypes.byref(wide), 0, None) == mx.MXS_EINVAL
    assert b"limit" in L.mxs_last_error()


def test_select_pages_rejections_before_device_work(L):
    q, k, b, bs, lg = valid_args()
    sel = lambda mode, bt, H, P, kk, rs=64 * 8, hs=8, prs=64 * 4, phs=4: L.mxs_select_pages(
        mode, ctypes.byref(bt) if bt is not None else None, H, P, FAKE, rs, hs, kk, FAKE + 0x10000, prs, phs, None)
    assert sel(mx.MXS_MODE_PREFILL, None, 64, 128, 4) == mx.MXS_EINVAL
    assert sel(7, b, 64, 128, 4) == mx.MXS_EINVAL
    assert sel(mx.MXS_MODE_PREFILL, b, 64, 96, 4) == mx.MXS_ELAYOUT
    assert sel(mx.MXS_MODE_PREFILL, b, 0, 128, 4) == mx.MXS_EINVAL
    assert sel(mx.MXS_MODE_PREFILL, b, 64, 128, -1) == mx.MXS_EINVAL
    assert sel(mx.MXS_MODE_PREFILL, b, 64, 128, 0) == mx.MXS_OK                      # nothing to write
    assert sel(mx.MXS_MODE_PREFILL, b, 64, 128, 4, hs=4) == mx.MXS_ELAYOUT            # narrow score rows
    assert sel(mx.MXS_MODE_PREFILL, b, 64, 128, 4, phs=2) == mx.MXS_ELAYOUT           # narrow output rows
    wide = mx.Batch.from_buffer_copy(bytes(b))
    wide.max_seq_len = 128 * 4097
    assert sel(mx.MXS_MODE_PREFILL, wide, 64, 128, 4, rs=64 * 4097, hs=4097) == mx.MXS_EUNSUPPORTED
    wide.max_seq_len = 2**31 - 255
    assert sel(mx.MXS_MODE_PREFILL, wide, 64, 128, 4) == mx.MXS_EINVAL
    # an empty window reads no score: a NULL score tensor is taken (up to the device check)
    empty = mx.Batch.from_buffer_copy(bytes(b))
    empty.max_seq_len = 0
    rc = L.mxs_select_pages(mx.MXS_MODE_PREFILL, ctypes.byref(empty), 64, 128, None, 0, 0, 4, FAKE + 0x10000, 64 * 4,
                            4, None)
    assert rc != mx.MXS_EINVAL or b"NULL" not in L.mxs_last_error(), L.mxs_last_error()
    assert L.mxs_select_pages(mx.MXS_MODE_PREFILL, ctypes.byref(b), 64, 128, None, 64 * 8, 8, 4, FAKE + 0x10000,
                              64 * 4, 4, None) == mx.MXS_EINVAL                          # scores needed when NB > 0


def test_write_pages_rejections_before_device_work(L):
    q, k, b, bs, lg = valid_args()
    w = lambda kp, rs, n, slots, kc: L.mxs_write_pages(kp, rs, n, slots, ctypes.byref(kc) if kc else None, None)
    assert w(FAKE, 128, 4, FAKE + 0x1000, None) == mx.MXS_EINVAL
    assert w(FAKE, 128, -1, FAKE + 0x1000, k) == mx.MXS_EINVAL
    assert w(FAKE, 128, 0, None, k) == mx.MXS_OK                          # nothing to write
    assert w(None, 128, 4, FAKE + 0x1000, k) == mx.MXS_EINVAL
    assert w(FAKE + 8, 128, 4, FAKE + 0x1000, k) == mx.MXS_ELAYOUT          # misaligned key rows
    assert w(FAKE, 100, 4, FAKE + 0x1000, k) == mx.MXS_ELAYOUT              # row stride < 128
    assert w(FAKE, 128, 4, FAKE + 0x1004, k) == mx.MXS_ELAYOUT              # misaligned slot_mapping
    bad = mx.KCache.from_buffer_copy(bytes(k))
    bad.data_page_stride = 100
    assert w(FAKE, 128, 4, FAKE + 0x1000, bad) == mx.MXS_ELAYOUT
    bad = mx.KCache.from_buffer_copy(bytes(k))
    bad.k_dtype = 5
    assert w(FAKE, 128, 4, FAKE + 0x1000, bad) == mx.MXS_EDTYPE
    fp8 = mx.KCache.from_buffer_copy(bytes(k))
    fp8.k_dtype = mx.MXS_K_E4M3                                          # 8704 B < 128 tokens x 128 B
    assert w(FAKE, 128, 4, FAKE + 0x1000, fp8) == mx.MXS_ELAYOUT


def test_python_layer_rejects_cpu_tensors():
    import torch
    q = torch.zeros((1, 1, 128), dtype=torch.bfloat16)
    kd = torch.zeros((1, 128, 64), dtype=torch.uint8)
    ks = torch.zeros((1, 128, 4), dtype=torch.uint8)
    bt = torch.zeros((1, 1), dtype=torch.int32)
    sl = torch.ones(1, dtype=torch.int32)
    with pytest.raises(ValueError):
        mx.score_decode(q, kd, ks, bt, sl, 128, 0.1)


def test_python_layer_fp8_cache_views():
    import torch
    # an fp8 cache is a [pages, P, 128] e4m3 (or uint8) view with no scale view
    k8 = torch.zeros((2, 64, 128), dtype=torch.uint8)
    kc = mx._kcache(k8, None)
    assert kc.k_dtype == mx.MXS_K_E4M3 and kc.page_size == 64 and kc.num_pages == 2 and kc.data_page_stride == 8192
    assert not kc.scale
    kc = mx._kcache(torch.zeros((3, 128, 64), dtype=torch.uint8), torch.zeros((3, 128, 4), dtype=torch.uint8))
    assert kc.k_dtype == mx.MXS_K_MXFP4 and kc.num_pages == 3
    with pytest.raises(ValueError):
        mx._kcache(torch.zeros((2, 64, 64), dtype=torch.uint8), None)            # MXFP4-shaped data, no scales
    with pytest.raises(ValueError):
        mx._kcache(torch.zeros((2, 64, 128), dtype=torch.bfloat16), None)         # not a byte view
    with pytest.raises(ValueError):
        mx._kcache(torch.zeros((2, 64, 256), dtype=torch.uint8)[:, :, :128], None)   # token rows not contiguous


# ------------------------------------------------------------------ attention decode

def attn_args():
    q = mx.Query(FAKE, mx.MXS_Q_E4M3, 16 * 128, 128, 16)
    kview = mx.KVView(FAKE + 0x100000, 8704, 8704, FAKE + 0x100000 + 8192, 8704, 8704)
    vview = mx.KVView(FAKE + 0x900000, 8704, 8704, FAKE + 0x900000 + 8192, 8704, 8704)
    kv = mx.KVCache(kview, vview, 128, 1, 100)
    return q, kv


def attn_call(L, q, kv, *, bt=FAKE + 0x2000000, bts=16, btw=16, ctx=FAKE + 0x3000000, R=8, maxc=2048, scale=0.088,
              out=FAKE + 0x4000000, ors=16 * 128, ohs=128):
    return L.mxs_attn_decode(ctypes.byref(q), ctypes.byref(kv), bt, bts, btw, ctx, R, maxc, ctypes.c_float(scale), out,
                             ors, ohs, None)


def test_attn_decode_rejections_before_device_work(L):
    q, kv = attn_args()
    assert attn_call(L, q, kv, R=0) == mx.MXS_OK                                        # nothing to do
    cases = [
        ("fp16 query", lambda q, kv: setattr(q, "dtype", 3), {}, mx.MXS_EDTYPE),
        ("page size 32", lambda q, kv: setattr(kv, "page_size", 32), {}, mx.MXS_ELAYOUT),
        ("heads not a multiple of kv heads", lambda q, kv: setattr(kv, "num_kv_heads", 3), {}, mx.MXS_EINVAL),
        ("17 query heads per kv head", lambda q, kv: setattr(q, "num_heads", 17), {}, mx.MXS_EUNSUPPORTED),
        ("zero scale", lambda q, kv: None, {"scale": 0.0}, mx.MXS_EINVAL),
        ("misaligned K data", lambda q, kv: setattr(kv.k, "data", FAKE + 0x100008), {}, mx.MXS_ELAYOUT),
        ("null V scale", lambda q, kv: setattr(kv.v, "scale", None), {}, mx.MXS_EINVAL),
        ("narrow K page stride", lambda q, kv: setattr(kv.k, "data_page_stride", 4096), {}, mx.MXS_ELAYOUT),
        ("narrow block table", lambda q, kv: None, {"btw": 15}, mx.MXS_ELAYOUT),
        ("null context lengths", lambda q, kv: None, {"ctx": None}, mx.MXS_EINVAL),
        ("narrow output rows", lambda q, kv: None, {"ors": 128}, mx.MXS_ELAYOUT),
        ("null output", lambda q, kv: None, {"out": None}, mx.MXS_EINVAL),
        ("misaligned query", lambda q, kv: setattr(q, "ptr", FAKE + 8), {}, mx.MXS_ELAYOUT),
        ("context above 2^31 - 256", lambda q, kv: None, {"maxc": 2**31 - 255, "btw": 2**24}, mx.MXS_EINVAL),
    ]
    for name, mutate, kw, code in cases:
        q, kv = attn_args()
        mutate(q, kv)
        assert attn_call(L, q, kv, **kw) == code, (name, L.mxs_last_error())
    import torch
    if torch.cuda.device_count() == 0:
        q, kv = attn_args()
        assert attn_call(L, q, kv) == mx.MXS_EUNSUPPORTED                               # valid: stops at the device

"""Benchmark of the paged MXFP4 index scorer on one MI355X.

Default run: the five scorer workloads, each with inputs resident in HBM
before any timing starts:
  1 prefill_q64_ctx1k          64 query rows after a 960-token prefix, logits
                               + block scores, 16-page pool;
  2 decode_b64_ctx128k         B = 64 decode rows, context 131072, pages drawn
                               from a 300k-page pool (2.6 GB);
  3 prefill_q4096_ctx128k      4096 rows after prefix 126976, e4m3 query;
  4 prefill_chunk32k_ctx132768 32768 rows after prefix 100000, one e8m0 byte
                               per token in 100..150 (the headline: the largest);
  5 logits_b8_q128_ctx8k_shared per-head logits, 64-token pages in a shared
                               two-slot pool past byte 4.608e9.
H = 64, D = 128, bf16 query ~ N(0, 1) unless stated, e2m1 codes uniform,
e8m0 bytes uniform in [122, 127] unless stated. Workloads beyond the smallest
rotate four disjoint block tables between steps so consecutive calls read
different pages.

Timing (the pages' method: graph replay, medians, two rounds with the order
reversed): per workload W untimed warmup steps, then K steps captured once in
a HIP graph; each round replays every workload's graph R times, the second
round in reverse workload order; HIP events on the replay stream bracket
each replay, so a step's time is its kernel's average launch duration. The
reported time is the median over all replays of both rounds.

Prints one JSON line (stdout): the headline workload's figures at the top
level (throughput = live scored (row x head x token) triples per second,
us/call, achieved HBM GB/s and scaled-MFMA rate, the roofline of its kernel,
the CPU oracle's rate on a bounded sample) and the same record for every
workload under "workloads".

HBM traffic: `--copy-probe` adds a plain 1 GiB float32 negation (reads and
writes 2^30 bytes) ahead of the warmup, so that one `rocprofv3 --pmc
FETCH_SIZE` run and one `--pmc WRITE_SIZE` run see the scorer and a kernel
of known size; `--pmc-summary DB...` turns the two runs' databases into a
traffic file (counter readings scaled by known bytes / copy reading), which
the roofline picks up while the kernel sources still hash the same.

--config N runs one workload instead (profiling): 1-5 as above, 6: top-64
page selection over the block scores of config 3, 7: writing 2^20 bf16 keys
into MXFP4 page slots; 8, 9, 10: configs 2, 3 and 7 over an fp8 (e4m3, 128 B
per token) index cache, the format the MXFP4 one replaces; 11: paged MXFP4
attention decode, 2048 rows x 16 query heads over 2048 tokens of K and V;
12: config 4 with an e8m0 byte per (token, 32-element block).
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0            # MI355X HBM3E
MFMA_FP8_PEAK_TFLOPS = 5000.0     # dense fp8 rate; the fp4 x fp8 scaled MFMA issues at this rate
MFMA_FP4_PEAK_TFLOPS = 10100.0    # dense fp4 x fp4, for reference


COPY_PROBE_BYTES = 1 << 30        # bytes read (and written) by the --copy-probe kernel
PROFILES = os.path.join(ROOT, "profiles")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_name(wl) -> str:
    """The kernel a workload runs: decode, the block-score kernel, the logits
    kernel (every call that writes logits) or the page selection."""
    if wl.select_k:
        return "k_select"
    if wl.write_tokens:
        return "k_write"
    if wl.attn_group:
        return "k_attn"
    if wl.mode == "logits" or wl.want_logits:
        return "k_logits"
    return "k_decode" if wl.mode == "decode" else "k_prefill"


def kernel_source_hash(kernel: str) -> str:
    """Hash of everything one kernel is compiled and launched from: its own
    device source, the shared headers, the planner that sets its launch shape
    and the build flags (a change to another kernel leaves it as it was)."""
    pkg = os.path.join(ROOT, "mxfp4_paged_cache_amd")
    own = os.path.join(pkg, "csrc", "mxs_" + kernel[len("k_"):] + ".hip")
    if not os.path.exists(own):
        raise RuntimeError(f"no device source for kernel {kernel}")
    files = ([own] + sorted(glob.glob(os.path.join(pkg, "csrc", "*.h"))) +
             [os.path.join(pkg, "csrc", "mxs_api.cpp"), os.path.join(pkg, "build.py"),
              os.path.join(ROOT, "include", "mxscore.h")])
    h = hashlib.sha256()
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_path(wl) -> str:
    return os.path.join(PROFILES, f"{kernel_name(wl)}_{wl.name}_traffic.json")


def pmc_summary(dbs):
    """Per-dispatch averages of FETCH_SIZE / WRITE_SIZE (KiB) for the scorer and
    the copy probe, from rocprofv3 databases; returns the traffic record."""
    import sqlite3
    acc = {}
    for db in dbs:
        con = sqlite3.connect(db)
        per = {}
        for name, disp, val, kname in con.execute(
                "select counter_name, dispatch_id, value, kernel_name from counters_collection"):
            kind = "copy" if "neg" in kname else next(
                (k for k in ("k_decode", "k_prefill", "k_logits", "k_select", "k_write", "k_attn") if k in kname), None)
            if kind is None:
                continue
            per.setdefault((name, kind), {}).setdefault(disp, 0.0)
            per[(name, kind)][disp] += val
        for key, d in per.items():
            acc[key] = sum(d.values()) / len(d)
    out = {}
    for counter, field in (("FETCH_SIZE", "read"), ("WRITE_SIZE", "write")):
        copy = acc.get((counter, "copy"))
        for k in ("k_decode", "k_prefill", "k_logits", "k_select", "k_write", "k_attn"):
            v = acc.get((counter, k))
            if v is None or not copy:
                continue
            factor = COPY_PROBE_BYTES / (copy * 1024.0)
            out.setdefault(k, {})[field] = {"counter_kib_per_dispatch": v, "copy_probe_kib": copy,
                                            "scale": factor, "bytes": v * 1024.0 * factor}
    return out


def path_dtype(wl) -> str:
    """The arithmetic type the measured path computes in."""
    if wl.attn_group:
        return "e2m1 x e4m3 -> f32; bf16 x bf16 -> f32; bf16 out"
    if wl.write_tokens:
        return "bf16 -> e4m3" if wl.k_dtype == "e4m3" else "bf16 -> e2m1 + e8m0"
    if wl.select_k:
        return "f32"
    return "e4m3 x e4m3 -> f32" if wl.k_dtype == "e4m3" else "e2m1 x e4m3 -> f32"


def algorithmic_bytes(wl, inp) -> int:
    """Bytes a call must move at minimum: every live page once (data + scales),
    the query rows, the block-table entries of live pages, and every output
    element written once."""
    token_bytes = 128 if wl.k_dtype == "e4m3" else 68     # fp8 cache: 128 e4m3 bytes; MXFP4: 64 + 4
    if wl.write_tokens:
        # the writer reads each bf16 key (256 B) and its slot (8 B) and writes one cache token
        return wl.write_tokens * (256 + 8 + token_bytes)
    if wl.select_k:
        # the selection reads every block score and writes k page ids per (row, head)
        return wl.T * wl.H * (wl.NB + wl.select_k) * 4 + (wl.B * 3 + 1) * 4
    P = wl.page_size
    if wl.attn_group:
        # K and V of every live page (68 B per token each, per kv head), the query, the bf16
        # output, the live table entries and the context lengths
        pages = sum((min(s, wl.window) + P - 1) // P for s in wl.seq_lens)
        hq = wl.H * wl.attn_group
        qb = 2 if wl.q_dtype == "bf16" else 1
        return pages * P * 136 * wl.H + wl.T * hq * 128 * (qb + 2) + pages * 4 + wl.B * 4
    pages = sum((min(s, wl.window) + P - 1) // P for s in wl.seq_lens)
    kbytes = pages * P * token_bytes
    qbytes = wl.T * wl.H * 128 * (2 if wl.q_dtype == "bf16" else 1)
    table = pages * 4
    out = 0
    if wl.want_blocks:
        out += wl.T * wl.H * wl.NB * 4
    if wl.want_logits:
        out += wl.T * wl.H * wl.window * 4
    meta = (wl.B * 3 + 1) * 4
    return kbytes + qbytes + table + out + meta


SUITE = (1, 2, 3, 4, 5)            # the default run: the five scorer workloads
HEADLINE = 4                        # the largest one carries the top-level line


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


class Case:
    """One workload on the GPU: inputs resident in HBM, its plan and outputs,
    and the K timed steps captured once in a HIP graph."""

    def __init__(self, cfg: int, args, dev):
        import torch
        import mxfp4_paged_cache_amd as mx
        from mxfp4_paged_cache_amd import workloads as W
        self.cfg = cfg
        wl = W.CONFIGS[cfg]()
        # consecutive calls read disjoint page sets (the decode pool is larger
        # than the 256 MB last-level cache; the prefill pages are not, and are
        # rotated all the same)
        if wl.mode == "decode" or wl.T * wl.H > 64 * 64:
            wl.tables = 4
        self.wl = wl
        log(f"workload {wl.name}: generating inputs on the GPU")
        t0 = time.time()
        inp = W.make_inputs(wl, args.seed, dev)
        torch.cuda.synchronize()
        log(f"inputs ready in {time.time() - t0:.1f}s")
        self.inp = inp
        T, H, P = wl.T, wl.H, wl.page_size
        NB, Wd = wl.NB, wl.window
        S = W.INV_SQRT_D
        bs = torch.empty((T, H, NB), dtype=torch.float32, device=dev) if (wl.want_blocks and not wl.attn_group) else None
        lg = torch.empty((T, H, Wd), dtype=torch.float32, device=dev) if wl.want_logits else None
        self.bs, self.lg = bs, lg
        plan = None
        if not wl.attn_group:
            plan = mx.make_plan(wl.mode, inp.q.dtype, P, H, wl.B, max(wl.q_lens), Wd, wl.want_logits, wl.want_blocks,
                                k_dtype=wl.k_dtype)
            log(f"plan: {plan.as_dict()}")
        self.plan = plan
        ao = torch.empty((T, H * wl.attn_group, 128), dtype=torch.bfloat16, device=dev) if wl.attn_group else None
        sel = None
        if wl.select_k:
            # the selection's input: this prefill's block scores, computed once before timing
            mx.score_prefill(inp.q, inp.k_data, inp.k_scale, inp.block_tables[0], inp.cu_seqlens_q, inp.seq_lens,
                             inp.prefix_lens, max(wl.q_lens), Wd, S, out=bs, plan=plan)
            sel = torch.empty((T, H, wl.select_k), dtype=torch.int32, device=dev)
        wk = wslots = None
        if wl.write_tokens:
            # keys N(0,1) in bf16; whole pages in a seeded random page order
            g = torch.Generator(device=dev)
            g.manual_seed(args.seed * 1000003 + 77)
            wk = torch.randn((wl.write_tokens, 128), generator=g, device=dev).to(torch.bfloat16)
            npages = wl.write_tokens // P
            pages = torch.randperm(wl.pool_pages, generator=g, device=dev)[:npages]
            wslots = (pages[:, None] * P + torch.arange(P, device=dev)[None, :]).reshape(-1).to(torch.int64)
        self.wk, self.wslots = wk, wslots

        def call(i):
            bt = inp.block_tables[i % len(inp.block_tables)]
            if wl.attn_group:
                mx.attn_decode(inp.q, inp.k_data, inp.k_scale, inp.extras["v_data"], inp.extras["v_scale"], bt,
                               inp.seq_lens, Wd, S, out=ao)
            elif wl.write_tokens:
                mx.write_pages(wk, wslots, inp.k_data, inp.k_scale)
            elif wl.select_k:
                mx.select_pages(bs, wl.select_k, inp.seq_lens, Wd, P, cu_seqlens_q=inp.cu_seqlens_q,
                                prefix_lens=inp.prefix_lens, out=sel)
            elif wl.mode == "decode":
                mx.score_decode(inp.q, inp.k_data, inp.k_scale, bt, inp.seq_lens, Wd, S, out=bs,
                                logits=lg if lg is not None else False, plan=plan)
            elif wl.mode == "logits":
                mx.score_logits(inp.q, inp.k_data, inp.k_scale, bt, inp.cu_seqlens_q, inp.seq_lens, inp.prefix_lens,
                                max(wl.q_lens), Wd, S, out=lg, block_scores=bs if bs is not None else False, plan=plan)
            else:
                mx.score_prefill(inp.q, inp.k_data, inp.k_scale, bt, inp.cu_seqlens_q, inp.seq_lens, inp.prefix_lens,
                                 max(wl.q_lens), Wd, S, out=bs, logits=lg if lg is not None else False, plan=plan)
        self.call = call
        self.graph = None
        self.replay_ms = {}            # round -> [ms per step of each replay]

    def warm_and_capture(self, warmup: int, steps: int, eager: bool, dev):
        import torch
        for i in range(warmup):
            self.call(i)
        torch.cuda.synchronize()
        if eager:
            return
        # capture the K timed steps once (side stream warm-up first, as capture requires)
        side = torch.cuda.Stream(dev)
        side.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(side):
            self.call(0)
        torch.cuda.current_stream(dev).wait_stream(side)
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            for i in range(steps):
                self.call(i)
        torch.cuda.synchronize()

    def time_replays(self, rnd: int, replays: int, steps: int, dev):
        """`replays` timed runs of the K steps (a graph replay, or K eager
        launches), each between two HIP events on the stream the kernels run
        on; per-step times (ms) go to self.replay_ms[rnd]."""
        import torch
        stream = torch.cuda.current_stream(dev)   # the launches (or the replay) run on this stream
        out = self.replay_ms.setdefault(rnd, [])
        for _ in range(replays):
            ev0 = torch.cuda.Event(enable_timing=True)
            ev1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            ev0.record(stream)
            if self.graph is not None:
                self.graph.replay()
            else:
                for i in range(steps):
                    self.call(i)
            ev1.record(stream)
            torch.cuda.synchronize()
            out.append(ev0.elapsed_time(ev1) / steps)   # one kernel launch per step

    def record(self, args, with_cpu: bool):
        """The workload's measurement record (the median over every replay of
        both rounds; each round's median alongside)."""
        import numpy as np
        wl, inp = self.wl, self.inp
        allms = [m for r in sorted(self.replay_ms) for m in self.replay_ms[r]]
        ms = float(np.median(allms))
        # live (row, query head, token) triples; attention counts every query head of every kv head
        triples = wl.live_triples() * (wl.attn_group or 1)
        # throughput: scored (row, head, token) triples/s; the selection consumes (row, head, page) block scores
        units = wl.write_tokens if wl.write_tokens else (wl.T * wl.H * wl.NB if wl.select_k else triples)
        value = units / (ms / 1e3)
        abytes = algorithmic_bytes(wl, inp)
        flops = (4.0 if wl.attn_group else 2.0) * 128 * triples   # attention: Q.K and P.V
        gbps = abytes / (ms / 1e3) / 1e9
        tflops = flops / (ms / 1e3) / 1e12
        hbm_bound = (wl.mode in ("decode", "logits") or (wl.T * wl.H <= 64 * 64) or bool(wl.select_k) or
                     bool(wl.write_tokens))
        traffic = None
        tpath = args.traffic or traffic_path(wl)
        if os.path.exists(tpath):
            with open(tpath) as f:
                tr = json.load(f)
            # counters taken on other kernel code no longer describe this kernel
            if tr.get("workload") == wl.name and tr.get("source_hash") == kernel_source_hash(kernel_name(wl)):
                traffic = tr.get("bytes_per_launch")
        if hbm_bound:
            roof = {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": traffic}
        else:
            roof = {"bound": "mfma", "achieved": round(tflops, 1), "peak": MFMA_FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(tflops / MFMA_FP8_PEAK_TFLOPS, 4), "traffic": traffic}
        cpu = None
        if with_cpu:
            if wl.attn_group:
                cpu = cpu_baseline_attn(wl, inp, args.cpu_sample)
            elif wl.write_tokens:
                cpu = cpu_baseline_write(wl, self.wk, self.wslots, args.cpu_sample)
            elif wl.select_k:
                cpu = cpu_baseline_select(wl, self.bs, inp, args.cpu_sample)
            else:
                cpu = cpu_baseline(wl, inp, args.cpu_sample, args.cpu_seconds)
        return {
            "value": value,
            "unit": "tokens/s" if wl.write_tokens else (
                "(row\u00d7head\u00d7page)/s" if wl.select_k else "(row\u00d7head\u00d7token)/s"),
            "ms_per_step": ms,
            "us_per_call": ms * 1e3,
            "timing": {"stat": "median of every replay of both rounds", "replays": len(allms),
                       "steps_per_replay": args.steps,
                       "graph": self.graph is not None,
                       "round_median_us": {str(r): round(float(np.median(v)) * 1e3, 3)
                                           for r, v in sorted(self.replay_ms.items())},
                       "min_us": round(min(allms) * 1e3, 3), "max_us": round(max(allms) * 1e3, 3)},
            "dtype": path_dtype(wl),
            "config": workload_config(wl, inp),
            "hbm_gbps": round(gbps, 1),
            "mfma_tflops": None if (wl.select_k or wl.write_tokens) else round(tflops, 2),
            "mfma_util_fp8_rate": None if (wl.select_k or wl.write_tokens or wl.attn_group) else round(
                tflops / MFMA_FP8_PEAK_TFLOPS, 4),
            "algorithmic_bytes": abytes,
            "live_triples": None if (wl.select_k or wl.write_tokens) else triples,
            "roofline": roof,
            "cpu_baseline": cpu,
            "kernel": kernel_name(wl),
        }


def workload_config(wl, inp) -> dict:
    return {"workload": wl.name, "batch": wl.B, "query_rows": wl.T, "heads": wl.H, "head_dim": 128,
            "page_size": wl.page_size, "context": max(wl.seq_lens), "q_dtype": wl.q_dtype, "cache": wl.k_dtype,
            "e8m0_range": [wl.scale_lo, wl.scale_hi],
            **({"e8m0_per": "token" if wl.scale_mode == "token" else "32-element block"}
               if wl.k_dtype == "mxfp4" else {}),
            "outputs": "attention" if wl.attn_group else (("block_scores" if wl.want_blocks else "") +
                                                          ("+logits" if wl.want_logits else "")),
            "rotating_tables": len(inp.block_tables),
            **({"select_k": wl.select_k} if wl.select_k else {}),
            **({"write_tokens": wl.write_tokens} if wl.write_tokens else {}),
            **({"query_heads_per_kv_head": wl.attn_group} if wl.attn_group else {})}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20, help="steps per timed replay (K)")
    ap.add_argument("--warmup", type=int, default=5, help="untimed warmup steps per workload (W)")
    ap.add_argument("--replays", type=int, default=5, help="timed replays per workload per round")
    ap.add_argument("--rounds", type=int, default=2, help="rounds of replays; every other round in reverse order")
    ap.add_argument("--config", type=int, default=0,
                    help="one workload (1-12) instead of the five scorer workloads (profiling runs)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=0, help="rows the oracle scores for the CPU baseline")
    ap.add_argument("--cpu-seconds", type=float, default=6.0, help="oracle work per CPU-baseline sample")
    ap.add_argument("--traffic", type=str, default="", help="traffic file (default: the one under profiles/)")
    ap.add_argument("--eager", action="store_true", help="time plain launches instead of a graph replay")
    ap.add_argument("--copy-probe", action="store_true", help="run a 1 GiB copy kernel first (counter calibration)")
    ap.add_argument("--pmc-summary", nargs="+", default=None, metavar="DB",
                    help="summarize rocprofv3 --pmc databases into a traffic record and exit")
    args = ap.parse_args()

    if args.pmc_summary:
        from mxfp4_paged_cache_amd import workloads as W
        wl = W.CONFIGS[args.config or HEADLINE]()
        rec = pmc_summary(args.pmc_summary).get(kernel_name(wl), {})
        rec = {"workload": wl.name, "kernel": kernel_name(wl), "source_hash": kernel_source_hash(kernel_name(wl)),
               "copy_probe_bytes": COPY_PROBE_BYTES, **rec}
        if "read" in rec and "write" in rec:
            rec["bytes_per_launch"] = rec["read"]["bytes"] + rec["write"]["bytes"]
        print(json.dumps(rec, indent=1))
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported. The scorer needs no "
              f"collective: every output element depends on one query vector and one token's K, so requests, "
              f"heads or context pages split across GPUs with no exchange step", file=sys.stderr)
        sys.exit(2)

    import torch

    import mxfp4_paged_cache_amd as mx

    if not os.path.exists(mx.library_path()):
        from mxfp4_paged_cache_amd import build as mxbuild
        mxbuild.build(force=True)
    mx.lib()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    cfgs = (args.config,) if args.config else SUITE
    head = args.config or HEADLINE
    cases = {c: Case(c, args, dev) for c in cfgs}

    if args.copy_probe:
        src = torch.ones(COPY_PROBE_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(2):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    for c in cfgs:
        cases[c].warm_and_capture(args.warmup, args.steps, args.eager, dev)
    wall0 = time.perf_counter()
    for rnd in range(args.rounds):
        order = cfgs if rnd % 2 == 0 else tuple(reversed(cfgs))
        for c in order:
            cases[c].time_replays(rnd, args.replays, args.steps, dev)
        log(f"round {rnd}: " + ", ".join(f"{cases[c].wl.name} {cases[c].replay_ms[rnd][-1] * 1e3:.1f} us"
                                          for c in cfgs))
    wall = time.perf_counter() - wall0

    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or os.cpu_count() or 1
    recs = {}
    for c in cfgs:
        recs[c] = cases[c].record(args, not args.no_cpu_baseline)
        log(f"{cases[c].wl.name}: {recs[c]['us_per_call']:.1f} us, roofline {recs[c]['roofline']['frac']}")
    top = recs[head]
    line = {
        "metric": "\u00b5s/call and scored (row\u00d7head\u00d7token)/s; HBM GB/s + scaled-MFMA util vs peak",
        "value": top["value"],
        "unit": top["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": top["ms_per_step"],
        "us_per_call": top["us_per_call"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": top["dtype"],
        "data": "synthetic",
        "config": top["config"],
        "hbm_gbps": top["hbm_gbps"],
        "mfma_tflops": top["mfma_tflops"],
        "mfma_util_fp8_rate": top["mfma_util_fp8_rate"],
        "algorithmic_bytes": top["algorithmic_bytes"],
        "live_triples": top["live_triples"],
        "roofline": top["roofline"],
        "cpu_baseline": top["cpu_baseline"],
        "timing": top["timing"],
        "kernel": top["kernel"],
        "host": {"cpu_model": cpu_model(), "threads": threads},
        "wall_s_timed": round(wall, 3),
        "workloads": {cases[c].wl.name: recs[c] for c in cfgs},
    }
    print(json.dumps(line), flush=True)


def cpu_baseline_write(wl, wk, wslots, sample_tokens: int):
    """The writer oracle (test infrastructure, pure Python, one core) on a
    bounded sample of the keys; reported as tokens/s."""
    import numpy as np
    import torch
    from oracle import writer
    n = sample_tokens or 8192
    bits = wk[:n].view(torch.int16).cpu().numpy().view(np.uint16)
    P = wl.page_size
    if wl.k_dtype == "e4m3":
        kd = np.zeros((n // P + 1, P, 128), np.uint8)
        t0 = time.perf_counter()
        writer.write_pages_e4m3(bits, np.arange(n), kd, P)
    else:
        kd = np.zeros((n // P + 1, P, 64), np.uint8)
        ks = np.zeros((n // P + 1, P, 4), np.uint8)
        t0 = time.perf_counter()
        writer.write_pages(bits, np.arange(n), kd, ks, P)
    dt = time.perf_counter() - t0
    return {"value": n / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} of {wl.write_tokens} keys, {dt:.2f} s"}


def cpu_baseline_attn(wl, inp, sample_rows: int):
    """The attention oracle (test infrastructure, numpy float64) on a bounded
    sample of rows; reported as (row, query head, token) triples/s."""
    import numpy as np
    import torch
    from oracle import attn
    n = sample_rows or wl.T   # ~0.13 s per 32 rows of 2048 tokens x 16 heads: every row is ~8 s
    rows = np.sort(np.random.default_rng(1234).choice(wl.T, size=min(n, wl.T), replace=False))
    bt = inp.block_tables[0].cpu().numpy()[rows]
    used = np.unique(bt[bt >= 0])
    idx = torch.as_tensor(used, dtype=torch.long, device=inp.k_data.device)
    host = [t.index_select(0, idx).cpu().numpy() for t in (inp.k_data, inp.k_scale, inp.extras["v_data"],
                                                            inp.extras["v_scale"])]
    remap = np.full(int(bt.max()) + 1, -1, np.int64)
    remap[used] = np.arange(len(used))
    bt = np.where(bt >= 0, remap[np.maximum(bt, 0)], -1).astype(np.int32)
    qc = inp.q.cpu()[rows]
    q = qc.view(torch.int16).numpy().view(np.uint16) if qc.dtype == torch.bfloat16 else qc.view(torch.uint8).numpy()
    ctx = inp.seq_lens.cpu().numpy()[rows]
    t0 = time.perf_counter()
    attn.attn_decode(q=q, q_dtype=wl.q_dtype, k_data=host[0], k_scale=host[1], v_data=host[2], v_scale=host[3],
                     block_table=bt, context_lens=ctx, page_size=wl.page_size, scale=float(np.float32(1 / np.sqrt(128))))
    dt = time.perf_counter() - t0
    trip = int(ctx.sum()) * wl.H * wl.attn_group
    return {"value": trip / dt, "unit": "(row\u00d7head\u00d7token)/s", "cores": 1, "kind": "oracle",
            "sample": f"{len(rows)} of {wl.T} rows ({trip} live triples), {dt:.2f} s"}


def cpu_baseline_select(wl, bs, inp, sample_rows: int):
    """The selection oracle (test infrastructure, pure Python, one core) on a
    bounded sample of rows; reported as (row, head, page) scores/s."""
    import numpy as np
    from oracle import topk
    # ~5 s of the pure-Python oracle (about 4.5e6 scores/s on one core)
    n_rows = sample_rows or max(1, int(5 * 4.5e6) // (wl.H * wl.NB))
    rows = np.sort(np.random.default_rng(1234).choice(wl.T, size=min(n_rows, wl.T), replace=False))
    lim = topk.row_limits("prefill", wl.seq_lens, wl.window, inp.cu_seqlens_q.cpu().numpy(), wl.prefix_lens)
    scores = bs[rows].cpu().numpy()
    t0 = time.perf_counter()
    topk.select_pages(scores, lim[rows], wl.page_size, wl.select_k)
    dt = time.perf_counter() - t0
    n = len(rows) * wl.H * wl.NB
    return {"value": n / dt, "unit": "(row\u00d7head\u00d7page)/s", "cores": 1, "kind": "oracle",
            "sample": f"{len(rows)} of {wl.T} rows, all heads and pages ({n} block scores), {dt:.2f} s"}


def cpu_baseline(wl, inp, sample_rows: int, seconds: float = 6.0):
    """The oracle (test infrastructure, untuned) on a bounded sample of the same
    workload, timed on this host's cores; reported as triples/s."""
    import numpy as np
    import torch
    import oracle

    oracle.build()
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or os.cpu_count() or 1
    T = wl.T
    if sample_rows <= 0:
        # about `seconds` of oracle work: ~7e6 live triples per core-second
        # measured for this oracle (~6.7e8 triples in 6 s on 16 cores)
        per_row = max(1, (sum(wl.limits()) * wl.H) // max(T, 1))
        budget = int(7e6 * threads * seconds)
        sample_rows = max(1, min(T, budget // per_row))
    rng = np.random.default_rng(1234)
    rows = np.sort(rng.choice(T, size=min(sample_rows, T), replace=False)).astype(np.int32)
    lim = wl.limits()
    sample_triples = int(sum(lim[r] for r in rows)) * wl.H
    # host copies of exactly the pages the sampled requests use (page order is irrelevant)
    mode = "decode" if wl.mode == "decode" else "prefill"
    bt = inp.block_tables[0].cpu().numpy()
    cu = inp.cu_seqlens_q.cpu().numpy()
    reqs = rows if mode == "decode" else np.unique(np.searchsorted(cu, rows, side="right") - 1)
    keep = np.zeros(bt.shape[0], bool)
    keep[reqs] = True
    bt = np.where(keep[:, None], bt, -1)
    used = np.unique(bt[bt >= 0])
    idx = torch.as_tensor(used, dtype=torch.long, device=inp.k_data.device)
    kd = inp.k_data.index_select(0, idx).cpu().numpy()
    ks = inp.k_scale.index_select(0, idx).cpu().numpy() if inp.k_scale is not None else None
    remap = np.full(int(bt.max()) + 1, -1, np.int64)
    remap[used] = np.arange(len(used))
    bt = np.where(bt >= 0, remap[np.maximum(bt, 0)], -1).astype(np.int32)
    qc = inp.q.cpu()
    q = qc.view(torch.int16).numpy().view(np.uint16) if qc.dtype == torch.bfloat16 else qc.view(torch.uint8).numpy()
    t0 = time.perf_counter()
    oracle.score(mode=mode, q=q, q_dtype=wl.q_dtype, k_data=kd, k_scale=ks, page_size=wl.page_size, block_table=bt,
                 seq_lens=inp.seq_lens.cpu().numpy(), max_seq_len=wl.window, sm_scale=float(np.float32(1 / np.sqrt(128))),
                 cu_seqlens_q=cu, prefix_lens=inp.prefix_lens.cpu().numpy(), rows=rows,
                 want_logits=wl.want_logits, want_blocks=wl.want_blocks, num_threads=threads, k_dtype=wl.k_dtype)
    dt = time.perf_counter() - t0
    return {"value": sample_triples / dt, "unit": "(row\u00d7head\u00d7token)/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{len(rows)} of {T} query rows ({sample_triples} live triples, all heads and pages of "
                      f"those rows), {dt:.2f} s"}


if __name__ == "__main__":
    main()

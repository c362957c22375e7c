"""Benchmark of the MSA hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

Headline workload: flat causal prefill, 2 x 8192 tokens, 16 q heads / 2 KV
heads, head_dim 128, topk 16, with the full pipeline per step: proxy score
(2 indexer heads) -> top-K block select -> sparse attention with LSE.  The
metric is selected-block attention TFLOP/s: FLOPs counted over the keys each
query actually attends (4 * head_dim per key and query head), divided by the
step time.  Inputs are seeded synthetic tensors resident in HBM before timing.
Without --workload the line also carries, under "configs", the other four
MSA workloads (the 1 x 1024 prefill and the three paged decodes), each with
its time, throughput, roofline fraction and oracle baseline.

The decode workloads (--workload paged_decode_...) report KV GB/s over the
K/V blocks actually gathered, timed cold: a 1 GiB read evicts L2 and MALL
before every step, outside the timed events.  --workload
qsa_indexed_1x8192_h12kv1_d256_w2048 times the QSA indexed forward,
qsa_bitmap_1x8192_h12kv1_d256_causal_q25 the QSA bitmap forward.  --graph
(decode workloads) adds the same step replayed as one HIP graph
(graph_ms_per_step); --temperature-lse TAU (prefill workloads) also returns
the temperature LSE (accumulated by the same prefill kernel);
--kv-format fp8 (prefill workloads) stores K/V as fp8 E4M3.

Per-stage times come from HIP events recorded on the stream the kernels run
on.  One JSON line is printed.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E

DEFAULT_WORKLOAD = "flat_prefill_2x8192_h16kv2_top16_pipeline"


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None,
                    help="time this workload alone (default: the 2 x 8192 prefill pipeline as "
                         "the headline line, with every other MSA workload under 'configs')")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kv-format", choices=("bf16", "fp8"), default="bf16",
                    help="prefill workloads: K/V stored as bf16 (default) or fp8 E4M3 (the "
                         "same values cast; proxy and attention read fp8)")
    ap.add_argument("--temperature-lse", type=float, default=None, metavar="TAU",
                    help="prefill workloads: also return the temperature LSE with this scale")
    ap.add_argument("--graph", action="store_true",
                    help="decode workloads: also time the whole step replayed as one HIP graph")
    ap.add_argument("--cpu-sample-rows", type=int, default=16384)
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run plain copies of BYTES bytes (profiler counter scaling)")
    ap.add_argument("--traffic-from", default=None, metavar="DIR",
                    help="no GPU: write profiles/traffic.json from rocprofv3 --pmc FETCH_SIZE / "
                         "WRITE_SIZE runs under DIR (pmc_<counter>_<workload>/ and "
                         "pmc_<counter>_copy/ for a 1 GiB copy)")
    return ap.parse_args()


def _events(n):
    import torch
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


TRAFFIC_SOURCE = ("stored: profiles/traffic.json, rocprofv3 FETCH_SIZE + WRITE_SIZE per launch "
                  "(copy-calibrated), used only while the kernel sources hash as when taken; "
                  "not measured in this run")


def _traffic_for(kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    ent = data.get(kernel)
    if not ent:
        return None
    h = hashlib.sha256()
    for name in ent["sources"]:
        with open(os.path.join(ROOT, "block_sparse_top_msa_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return ent["bytes_per_launch"] if h.hexdigest()[:16] == ent.get("sources_sha256_16") else None


# kernel -> the sources its machine code is built from (the stored traffic
# is used only while they hash as they did when the counters were taken)
TRAFFIC_KERNELS = {
    "msa_prefill_kernel": ["prefill.hip", "async_lds.hpp", "common.hpp", "tile_union.hpp",
                           "internal.hpp"],
    "msa_decode_kernel": ["decode.hip", "async_lds.hpp", "common.hpp", "tile_union.hpp",
                          "internal.hpp"],
    "msa_qsa_kernel": ["qsa.hip", "async_lds.hpp", "common.hpp", "internal.hpp"],
}


def write_traffic(src_dir: str, copy_bytes: int = 1 << 30):
    """profiles/traffic.json from rocprofv3 counter CSVs: per workload, the
    roofline kernel's FETCH_SIZE and WRITE_SIZE (KiB per dispatch, averaged),
    each scaled by the factor that makes a plain copy of copy_bytes read and
    write copy_bytes."""
    import collections
    import csv
    import glob
    import hashlib

    def pmc(counter, tag):
        files = glob.glob(os.path.join(src_dir, f"pmc_{counter}_{tag}", "**",
                                       "*counter_collection.csv"), recursive=True)
        acc = collections.defaultdict(list)
        for f in files:
            for r in csv.DictReader(open(f)):
                acc[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        return acc

    def mean(v):
        return sum(v) / len(v)

    cf = pmc("FETCH_SIZE", "copy")
    cw = pmc("WRITE_SIZE", "copy")
    kf = [v for k, v in cf.items() if "copyBuffer" in k][0]
    kw = [v for k, v in cw.items() if "copyBuffer" in k][0]
    fs = copy_bytes / 1024 / mean(kf)
    ws = copy_bytes / 1024 / mean(kw)
    out = {"_about": "HBM bytes per launch from rocprofv3 FETCH_SIZE and WRITE_SIZE (KiB per "
                     "dispatch), each scaled by the factor that makes a plain 1 GiB device copy "
                     "read 1 GiB and write 1 GiB; valid only while the listed kernel sources "
                     "hash to sources_sha256_16; written by bench.py --traffic-from"}
    for d in sorted(glob.glob(os.path.join(src_dir, "pmc_FETCH_SIZE_*"))):
        wl = os.path.basename(d)[len("pmc_FETCH_SIZE_"):]
        if wl == "copy":
            continue
        f, w = pmc("FETCH_SIZE", wl), pmc("WRITE_SIZE", wl)
        for kern, srcs in TRAFFIC_KERNELS.items():
            names = [k for k in f if kern + "<" in k or kern + "(" in k]
            if not names:
                continue
            fk = mean(sum((f[k] for k in names), []))
            wk = mean(sum((w[k] for k in names), []))
            h = hashlib.sha256()
            for n in srcs:
                with open(os.path.join(ROOT, "block_sparse_top_msa_amd", "csrc", n), "rb") as fh:
                    h.update(fh.read())
            out[f"{kern}:{wl}"] = {"sources": srcs, "sources_sha256_16": h.hexdigest()[:16],
                                   "fetch_kib": round(fk, 1), "write_kib": round(wk, 1),
                                   "fetch_scale": round(fs, 5), "write_scale": round(ws, 5),
                                   "bytes_per_launch": int(round((fk * fs + wk * ws) * 1024))}
    with open(os.path.join(ROOT, "profiles", "traffic.json"), "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))


def calibrate_copy(nbytes: int, reps: int):
    """Plain device-to-device copies of a known size, for scaling the HBM
    byte counters of a profiler run (each copy reads and writes nbytes)."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "reps": reps}), flush=True)


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle on a bounded sample of the same workload
# ---------------------------------------------------------------------------

def cpu_baseline_prefill(p, rows_n):
    import torch
    import oracle
    from block_sparse_top_msa_amd import accounting
    cores = len(os.sched_getaffinity(0))
    torch.set_num_threads(cores)
    pc = p.to("cpu")
    total = pc.total_q
    step = max(1, total // rows_n)
    rows = list(range(step - 1, total, step))[:rows_n]
    pipeline = pc.proxy_q is not None
    t0 = time.perf_counter()
    if pipeline:
        s = oracle.proxy_score(pc.proxy_q, pc.k, pc.cu_seqlens_q, cu_seqlens_k=pc.cu_seqlens_k,
                               causal=True, max_k_tiles=pc.max_k_tiles, rows=rows,
                               kv_format=pc.kv_dtype)
        q2k = oracle.topk_select(s.float(), pc.topk, pc.num_kv_heads, rows=rows)
    else:
        q2k = pc.q2k
    oracle.sparse_attention(pc.q, pc.k, pc.v, q2k, pc.cu_seqlens_q,
                            cu_seqlens_k=pc.cu_seqlens_k, causal=True, rows=rows,
                            kv_format=pc.kv_dtype)
    dt = time.perf_counter() - t0
    lens = pc.cu_seqlens_k[1:] - pc.cu_seqlens_k[:-1]
    keys = accounting.attended_keys(q2k, pc.cu_seqlens_q, lens, causal=True)[:, rows]
    flops = int(keys.sum()) * (pc.num_qo_heads // pc.num_kv_heads) * 4 * pc.head_dim
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{len(rows)} of {total} query rows (every {step}th), all "
                      f"{pc.num_qo_heads} heads: fp64 "
                      f"{'proxy + top-K + attention' if pipeline else 'attention'}, {dt:.1f} s"}


def cpu_baseline_decode(p, rows_n, fmt):
    import torch
    import oracle
    from block_sparse_top_msa_amd import accounting
    cores = len(os.sched_getaffinity(0))
    torch.set_num_threads(cores)
    per = p.total_q // p.batch
    reqs = list(range(0, p.batch, max(1, p.batch // max(1, rows_n // per))))[:max(1, rows_n // per)]
    rows = [b * per + t for b in reqs for t in range(per)]
    t0 = time.perf_counter()
    if p.q2k is None:
        # full pipeline: the oracle selects the blocks for the sampled rows itself
        s = oracle.proxy_score(p.q, p.k, p.cu_seqlens_q.cpu(), page_table=p.page_table.cpu(),
                               seqused_k=p.seqused_k.cpu(), causal=True,
                               max_k_tiles=p.max_k_tiles, reduce_heads=p.reduce_heads,
                               kv_format=fmt, rows=rows)
        q2k = oracle.topk_select(s.float(), p.topk, p.num_kv_heads, rows=rows)
        what = "fp64 proxy + top-K + attention"
    else:
        q2k = p.q2k.cpu()
        what = "fp64 attention over their selected pages"
    oracle.sparse_attention(p.q, p.k, p.v, q2k, p.cu_seqlens_q.cpu(), page_table=p.page_table.cpu(),
                            seqused_k=p.seqused_k.cpu(), causal=True, kv_format=fmt,
                            k_scale=p.k_scale, v_scale=p.v_scale,
                            k_global_scale=p.k_global_scale, v_global_scale=p.v_global_scale,
                            rows=rows)
    dt = time.perf_counter() - t0
    sub = torch.zeros_like(q2k).fill_(-1)
    sub[:, rows] = q2k[:, rows]
    nbytes = accounting.decode_kv_bytes(sub, p.cu_seqlens_q.cpu(), p.seqused_k.cpu(), fmt,
                                        p.max_k_tiles)
    return {"value": round(nbytes / dt / 1e9, 6), "unit": "GB/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{len(reqs)} of {p.batch} requests ({len(rows)} query rows): "
                      f"{what}, {dt:.1f} s"}


# ---------------------------------------------------------------------------
# GPU runs
# ---------------------------------------------------------------------------

def bench_prefill_pipeline(args, msa, synth, torch):
    from block_sparse_top_msa_amd import accounting
    p = synth.workload(args.workload, device="cuda")
    if args.kv_format == "fp8":
        p.k, p.v = p.k.to(torch.float8_e4m3fn), p.v.to(torch.float8_e4m3fn)
        p.kv_dtype = synth.KV_FP8
    T, B = p.max_k_tiles, p.batch
    mq = max(p.q_lens)
    # a workload without proxy heads comes with its q2k: the step is the
    # attention alone
    pipeline = p.proxy_q is not None
    if pipeline:
        scores = torch.empty(p.proxy_q.shape[1], T, p.total_q, dtype=torch.float32,
                             device="cuda")
        q2k = torch.empty(p.num_kv_heads, p.total_q, p.topk, dtype=torch.int32, device="cuda")
    else:
        q2k = p.q2k
    out = torch.empty_like(p.q)
    lse = torch.empty(p.total_q, p.num_qo_heads, dtype=torch.float32, device="cuda")
    temp = args.temperature_lse is not None
    lse_t = torch.empty_like(lse) if temp else None

    def step(ev=None):
        if ev: ev[0].record()
        if pipeline:
            msa.proxy_score(p.proxy_q, p.k, p.cu_seqlens_q, p.cu_seqlens_k, causal=True,
                            max_seqlen_q=mq, max_k_tiles=T, output=scores)
        if ev: ev[1].record()
        if pipeline:
            msa.topk_select(scores, p.topk, p.num_kv_heads, out=q2k)
        if ev: ev[2].record()
        msa.sparse_attention(p.q, p.k, p.v, q2k, p.cu_seqlens_q, p.cu_seqlens_k, causal=True,
                             return_softmax_lse=True, max_seqlen_q=mq, max_k_tiles=T,
                             out=out, lse=lse, return_temperature_lse=temp,
                             lse_temperature_scale=args.temperature_lse or 1.0, lse_t=lse_t)
        if ev: ev[3].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    lens = p.cu_seqlens_k[1:] - p.cu_seqlens_k[:-1]
    flops = accounting.attention_flops(q2k, p.cu_seqlens_q, lens, p.num_qo_heads)
    pflops = accounting.proxy_flops(p.cu_seqlens_q, lens, p.proxy_q.shape[1]) if pipeline else 0
    # MFMA work the tile kernel executes (whole 32-row slots over union blocks)
    exe_flops = accounting.prefill_executed_flops(
        q2k, p.cu_seqlens_q, lens, p.num_qo_heads,
        accounting.prefill_tile_tokens(p.num_qo_heads, p.num_kv_heads, p.topk))

    evs = [_events(4) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    st = [sum(e[i].elapsed_time(e[i + 1]) for e in evs) / args.steps for i in range(3)]
    ms_step = wall * 1e3 / args.steps
    attn_ms = st[2]
    achieved = flops / (attn_ms * 1e-3) / 1e12
    res = {
        "metric": "selected-block attention TFLOP/s",
        "value": round(flops / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "ms_per_step": round(ms_step, 4),
        "dtype": "bf16" if args.kv_format == "bf16" else "fp8_e4m3->bf16",
        "config": {"workload": p.name, "batch": B, "seq_len": mq, "num_qo_heads": p.num_qo_heads,
                   "num_kv_heads": p.num_kv_heads, "head_dim": p.head_dim, "topk": p.topk,
                   "proxy_heads": p.proxy_q.shape[1] if pipeline else 0, "causal": True,
                   **({"kv_format": "fp8_e4m3"} if args.kv_format == "fp8" else {}),
                   **({"temperature_lse": args.temperature_lse} if temp else {})},
        "stages_ms": ({"proxy_score": round(st[0], 4), "topk_select": round(st[1], 4),
                       "sparse_attention": round(st[2], 4)} if pipeline
                      else {"sparse_attention": round(st[2], 4)}),
        "work": {"attention_flops": flops, "proxy_flops": pflops,
                 "proxy_tflops": round(pflops / (st[0] * 1e-3) / 1e12, 3) if pipeline else None},
        "roofline": {"kernel": ("msa_stage16_kernel + msa_prefill_kernel<8,1>"
                                if args.kv_format == "fp8" else "msa_prefill_kernel<8,1>"),
                     "bound": "mfma",
                     "achieved": round(achieved, 3), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": (None if temp or args.kv_format == "fp8"
                                 else _traffic_for("msa_prefill_kernel:" + p.name)),
                     "executed": {
                         "flops": exe_flops,
                         "tflops": round(exe_flops / (attn_ms * 1e-3) / 1e12, 3),
                         "frac": round(exe_flops / (attn_ms * 1e-3) / 1e12
                                       / MFMA_BF16_PEAK_TFLOPS, 4),
                         "selected_share": round(flops / exe_flops, 4) if exe_flops else None,
                         "what": "MFMA FLOPs of the tile kernel: every 32-row slot x union "
                                 "block it computes (S^T and O^T += V^T P^T), counted on the "
                                 "host from q2k; diagnostic, not the metric"}},
    }
    return res, p


def _graph_decode_ms(args, p, scrub32, sink, torch):
    """The same cold decode step (proxy and top-K included when the workload
    has them) captured once and replayed as one HIP graph: ms per step."""
    from block_sparse_top_msa_amd.graph import DecodeGraph
    g = DecodeGraph(p.q, p.k, p.v, p.cu_seqlens_q, max_seqlen_q=max(p.q_lens),
                    max_k_tiles=p.max_k_tiles, topk=p.topk, page_table=p.page_table,
                    seqused_k=p.seqused_k, q2k=p.q2k, reduce_heads=p.reduce_heads,
                    k_scale=p.k_scale, v_scale=p.v_scale, k_global_scale=p.k_global_scale,
                    v_global_scale=p.v_global_scale, warmup=max(1, args.warmup))
    evs = [_events(2) for _ in range(args.steps)]
    for k in range(args.steps):
        torch.sum(scrub32, dim=0, out=sink)
        evs[k][0].record()
        g.replay()
        evs[k][1].record()
    torch.cuda.synchronize()
    return round(sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps, 4)


def bench_decode(args, msa, synth, torch):
    from block_sparse_top_msa_amd import accounting
    p = synth.workload(args.workload, device="cuda")
    fmt = p.kv_dtype
    T, B = p.max_k_tiles, p.batch
    mq = max(p.q_lens)
    out = torch.empty_like(p.q)
    lse = torch.empty(p.total_q, p.num_qo_heads, dtype=torch.float32, device="cuda")
    pipeline = p.q2k is None
    ws = q2k = None
    if pipeline:
        # proxy -> head reduce -> top-K in one call (the running top-K)
        q2k = torch.empty(p.num_kv_heads, p.total_q, p.topk, dtype=torch.int32, device="cuda")
        ws = msa.Workspace(msa.proxy_topk_workspace_size(
            p.q, p.k, p.cu_seqlens_q, topk=p.topk, page_table=p.page_table,
            seqused_k=p.seqused_k, causal=True, max_seqlen_q=mq, max_k_tiles=T,
            reduce_heads=p.reduce_heads), "cuda")
    else:
        q2k = p.q2k
    scrub32 = torch.zeros(1 << 28, dtype=torch.int32, device="cuda")

    def step(ev=None):
        if ev: ev[0].record()
        if pipeline:
            msa.proxy_topk(p.q, p.k, p.cu_seqlens_q, topk=p.topk, page_table=p.page_table,
                           seqused_k=p.seqused_k, causal=True, max_seqlen_q=mq, max_k_tiles=T,
                           reduce_heads=p.reduce_heads, out=q2k, workspace=ws)
        if ev: ev[1].record()
        if ev: ev[2].record()
        msa.sparse_attention(p.q, p.k, p.v, q2k, p.cu_seqlens_q, causal=True,
                             page_table=p.page_table, seqused_k=p.seqused_k,
                             return_softmax_lse=True, k_scale=p.k_scale, v_scale=p.v_scale,
                             k_global_scale=p.k_global_scale, v_global_scale=p.v_global_scale,
                             max_seqlen_q=mq, max_k_tiles=T, out=out, lse=lse)
        if ev: ev[3].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    nbytes = accounting.decode_kv_bytes(q2k, p.cu_seqlens_q, p.seqused_k, fmt, T)
    evs = [_events(4) for _ in range(args.steps)]
    sink = torch.empty((), dtype=torch.int64, device="cuda")
    for k in range(args.steps):
        # evict L2 and MALL before every step (cold K/V): a 1 GiB read leaves
        # the caches full of clean lines, so the step pays no writeback of a
        # previous kernel's dirty data
        torch.sum(scrub32, dim=0, out=sink)
        step(evs[k])
    torch.cuda.synchronize()
    st = [sum(e[i].elapsed_time(e[i + 1]) for e in evs) / args.steps for i in range(3)]
    # without the proxy and top-K stages a step is the attention call alone
    ms_step = sum(st) if pipeline else st[2]
    gbs = nbytes / (st[2] * 1e-3) / 1e9
    res = {
        "metric": "KV GB/s",
        "value": round(gbs, 3),
        "unit": "GB/s",
        "ms_per_step": round(ms_step, 4),
        "tokens_per_s": round(p.total_q / (ms_step * 1e-3), 1),
        "dtype": {"bf16": "bf16", "fp8_e4m3": "fp8_e4m3->bf16", "e2m1x2": "e2m1->bf16"}[fmt],
        "config": {"workload": p.name, "batch": B, "seqlen_q": mq, "num_qo_heads": p.num_qo_heads,
                   "num_kv_heads": p.num_kv_heads, "head_dim": p.head_dim, "topk": p.topk,
                   "kv_format": fmt, "cold_cache": True},
        "stages_ms": ({"proxy_topk": round(st[0], 4), "sparse_attention": round(st[2], 4)}
                      if pipeline else {"sparse_attention": round(st[2], 4)}),
        "work": {"kv_bytes": nbytes},
        **({"graph_ms_per_step": _graph_decode_ms(args, p, scrub32, sink, torch)}
           if args.graph else {}),
        "roofline": {"kernel": "msa_decode_kernel", "bound": "hbm",
                     "achieved": round(gbs, 3), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": _traffic_for("msa_decode_kernel:" + p.name)},
    }
    return res, p


def _qsa_keys(p):
    """Attended (query, key) pairs of a QSA problem: listed entries >= 0, or
    the tokens (< Tk) of every selected 4-token block."""
    if p.bitmap is None:
        return int((p.indices >= 0).sum())
    tk = p.k.shape[0]
    sel = p.bitmap != 0
    keys = 4 * int(sel.sum())
    if tk % 4:
        keys -= (4 - tk % 4) * int(sel[:, -1].sum())
    return keys


def bench_qsa(args, msa, synth, torch):
    """QSA forward (qsa page, indexed or bitmap API): selected-token attention
    TFLOP/s, FLOPs counted as 4 * head_dim per (query head, attended key)."""
    bitmap = args.workload == synth.QSA_BITMAP_WORKLOAD
    p = synth.qsa_bitmap_workload(device="cuda") if bitmap else synth.qsa_workload(device="cuda")
    T, hq, d = p.q.shape
    out = torch.empty_like(p.q)
    out_f32 = torch.empty(T, hq, d, dtype=torch.float32, device="cuda")
    lse = torch.empty(hq, T, dtype=torch.float32, device="cuda")
    keys = _qsa_keys(p)
    flops = 4 * d * hq * keys
    from block_sparse_top_msa_amd import accounting
    exe_flops, exe_shared, exe_token = accounting.qsa_executed(
        hq, p.k.shape[1], indices=None if bitmap else p.indices,
        bitmap=p.bitmap if bitmap else None, num_kv_tokens=p.k.shape[0], head_dim=d)

    def step():
        if bitmap:
            msa.qsa_bitmap_forward(p.q, p.k, p.v, p.bitmap, out=out, out_f32=out_f32, lse=lse)
        else:
            msa.qsa_indexed_forward(p.q, p.k, p.v, p.indices, out=out, out_f32=out_f32, lse=lse)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [_events(2) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for k in range(args.steps):
        evs[k][0].record()
        step()
        evs[k][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    ms_step = wall * 1e3 / args.steps
    achieved = flops / (kern_ms * 1e-3) / 1e12
    res = {
        "metric": "selected-token attention TFLOP/s",
        "value": round(flops / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "ms_per_step": round(ms_step, 4),
        "dtype": "bf16",
        "config": {"workload": p.name, "total_q": T, "num_qo_heads": hq,
                   "num_kv_heads": p.k.shape[1], "head_dim": d,
                   **({"num_blocks": p.bitmap.shape[1]} if bitmap else
                      {"width": p.indices.shape[1]})},
        "stages_ms": {("qsa_bitmap_forward" if bitmap else "qsa_indexed_forward"): round(kern_ms, 4)},
        "work": {"attention_flops": flops, "attended_keys": keys},
        "roofline": {"kernel": "msa_qsa_kernel", "bound": "mfma",
                     "achieved": round(achieved, 3), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": _traffic_for("msa_qsa_kernel:" + p.name),
                     "executed": {
                         "flops": exe_flops,
                         "tflops": round(exe_flops / (kern_ms * 1e-3) / 1e12, 3),
                         "frac": round(exe_flops / (kern_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                         "selected_share": round(flops / exe_flops, 4) if exe_flops else None,
                         "tiles_shared": exe_shared, "tiles_per_token": exe_token,
                         "what": "MFMA FLOPs of the QSA kernel: each shared-key tile's live 16-row "
                                 "slots over its whole key union, each per-token tile's tokens over "
                                 "their own chunks, counted on the host; diagnostic, not the metric"}},
    }
    return res, p


def cpu_baseline_qsa(p, rows_n):
    import torch
    import oracle
    import synth
    cores = len(os.sched_getaffinity(0))
    torch.set_num_threads(cores)
    pc = p.to("cpu")
    T, hq, d = pc.q.shape
    step = max(1, T // rows_n)
    rows = list(range(step - 1, T, step))[:rows_n]
    t0 = time.perf_counter()
    if pc.bitmap is None:
        oracle.qsa_indexed_attention(pc.q[rows], pc.k, pc.v, pc.indices[rows])
    else:
        oracle.qsa_bitmap_attention(pc.q[rows], pc.k, pc.v, pc.bitmap[rows])
    dt = time.perf_counter() - t0
    sub = synth.QsaProblem("rows", pc.q[rows], pc.k, pc.v,
                           None if pc.indices is None else pc.indices[rows], [len(rows)],
                           None if pc.bitmap is None else pc.bitmap[rows])
    keys = _qsa_keys(sub)
    return {"value": round(4 * d * hq * keys / dt / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{len(rows)} of {T} query rows (every {step}th), all {hq} heads: "
                      f"fp64 {'bitmap' if pc.bitmap is not None else 'indexed'} attention, "
                      f"{dt:.1f} s"}


def main():
    args = _args()
    if args.traffic_from:
        write_traffic(args.traffic_from)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the MSA hot path here runs on a single MI355X and "
              f"has no multi-GPU path (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    import torch
    import block_sparse_top_msa_amd as msa
    import synth
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy, args.steps)
        return
    single = args.workload is not None
    if not single:
        args.workload = DEFAULT_WORKLOAD
    res, cpu = run_workload(args, msa, synth, torch)
    line = {
        "metric": res["metric"], "value": res["value"], "unit": res["unit"], "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": res["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": res["dtype"], "data": "synthetic (seeded, generated on the GPU)",
        "config": res["config"],
    }
    for k in ("tokens_per_s", "stages_ms", "graph_ms_per_step", "work"):
        if k in res:
            line[k] = res[k]
    line["roofline"] = res["roofline"]
    line["cpu_baseline"] = cpu
    if not single:
        # the other MSA workloads, each timed as in its own --workload run
        # (decode cold), with its roofline fraction and oracle baseline
        line["configs"] = {}
        for name in synth.WORKLOADS:
            if name == DEFAULT_WORKLOAD:
                continue
            args.workload = name
            r, c = run_workload(args, msa, synth, torch)
            ent = {"metric": r["metric"], "value": r["value"], "unit": r["unit"],
                   "ms_per_step": r["ms_per_step"], "dtype": r["dtype"]}
            for k in ("tokens_per_s", "stages_ms", "work"):
                if k in r:
                    ent[k] = r[k]
            ent["roofline"] = r["roofline"]
            ent["cpu_baseline"] = c
            line["configs"][name] = ent
            torch.cuda.empty_cache()
    print(json.dumps(line), flush=True)


def run_workload(args, msa, synth, torch):
    """(result, cpu baseline) of args.workload."""
    if args.workload in (synth.QSA_WORKLOAD, synth.QSA_BITMAP_WORKLOAD):
        res, p = bench_qsa(args, msa, synth, torch)
        cpu = None if args.no_cpu_baseline else cpu_baseline_qsa(p, 512)
    elif args.workload.startswith("flat_prefill"):
        res, p = bench_prefill_pipeline(args, msa, synth, torch)
        cpu = None if args.no_cpu_baseline else cpu_baseline_prefill(p, args.cpu_sample_rows)
    else:
        res, p = bench_decode(args, msa, synth, torch)
        cpu = None if args.no_cpu_baseline else cpu_baseline_decode(p, p.total_q, p.kv_dtype)
    rf = res["roofline"]
    rf["traffic_source"] = TRAFFIC_SOURCE if rf.get("traffic") is not None else None
    del p
    return res, cpu


if __name__ == "__main__":
    main()

"""Benchmark of the ragged paged attention hot path on one MI355X.

A step is one rpa_forward call with the step's new keys/values: KV-cache
update (scatter), device planning, attention and split merge, over one batch of
synthetic input resident in HBM.  Default workload: bf16 decode (256
sequences, kv_len ~ U{512..4096}, page_size 16, 32 q heads, 8 kv heads,
head_dim 128).  Prints ONE JSON line.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "ragged paged attn: decode KV GB/s + prefill TFLOP/s, % of HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
ELEM = {"f32": 4, "bf16": 2, "fp8": 1}


def work_counts(w, split=False):
    """Algorithmic work of one step.

    kv_bytes: every KV token some query of a sequence can see is read once
    per sequence, 2 * Hkv * D * elem bytes per token (K and V of all heads).
    flops: 4 * D per visible (query, key, q head) triple (2D for q.k, 2D for p.v).
    With split=True also returns the share of each attention kernel: the KV
    bytes of the sequences the row kernel serves (q_len 1, or all of them for
    f32, which has no prefill kernel) and the FLOPs of the prefill tiles.
    """
    kvb = 0
    pairs = 0
    row_kvb = 0
    pf_pairs = 0
    has_prefill_kernel = w.q_dtype == "bf16"
    tok_bytes = 2 * w.num_kv_heads * w.head_dim * ELEM[w.cache_dtype]
    W = w.sliding_window
    for s in range(w.num_seqs):
        q_len = int(w.query_start_loc[s + 1] - w.query_start_loc[s])
        kv = int(w.kv_lens[s])
        ctx = kv - q_len
        if q_len == 0:
            continue
        lo = max(0, ctx - W + 1) if W else 0
        kvb += (kv - lo) * tok_bytes
        t = np.arange(q_len, dtype=np.int64)
        vis = ctx + t + 1
        if W:
            vis = np.minimum(vis, W)
        pairs += int(vis.sum())
        if has_prefill_kernel and q_len >= 2:
            pf_pairs += int(vis.sum())
        else:
            row_kvb += (kv - lo) * tok_bytes
    flops = 4 * w.head_dim * pairs * w.num_q_heads
    if split:
        return kvb, flops, row_kvb, 4 * w.head_dim * pf_pairs * w.num_q_heads
    return kvb, flops


def cpu_baseline(w, budget_s=15.0, min_s=10.0, max_passes=8):
    """The oracle as it stands, timed on the host on a bounded sample of the
    same workload: whole sequences drawn in a fixed order until ~budget_s of
    CPU work (passes over the batch repeat while under min_s); reported in the
    metric's unit scaled by the sample's share."""
    import threadpoolctl

    from oracle import rpa_oracle as O
    from tests.helpers import bits, compact_pages

    rng = np.random.default_rng(0)
    order = rng.permutation(w.num_seqs)
    q_bits = bits(w.queries, w.q_dtype)
    k_bits = bits(w.keys, w.kv_in_dtype)
    v_bits = bits(w.values, w.kv_in_dtype)
    sink = None if w.attention_sink is None else w.attention_sink.cpu().numpy()
    done, t_used, kvb, flops = 0, 0.0, 0, 0
    tok_bytes = 2 * w.num_kv_heads * w.head_dim * ELEM[w.cache_dtype]
    threads = threadpoolctl.threadpool_info()
    nthreads = max([t.get("num_threads", 1) for t in threads] + [1])
    schedule = [int(s) for _ in range(max_passes) for s in order]
    for i, s in enumerate(schedule):
        if i > 0 and i % len(order) == 0 and t_used >= min_s:
            break                     # a whole pass done and enough CPU time
        sub_cache, sub_bt = compact_pages(w, [s])
        q0, ql, ctx, kvl = O.seq_bounds(w.query_start_loc, w.kv_lens, s)
        pps = w.pages_per_seq
        t0 = time.perf_counter()
        cache = O.update_kv_cache(sub_cache, k_bits[q0:q0 + ql], v_bits[q0:q0 + ql],
                                  np.array([kvl], np.int32), sub_bt[s * pps:(s + 1) * pps],
                                  np.array([0, ql], np.int32), np.array([0, 0, 1], np.int32),
                                  page_size=w.page_size, pages_per_seq=pps,
                                  kv_in_dtype=w.kv_in_dtype, cache_dtype=w.cache_dtype,
                                  k_scale=w.k_scale, v_scale=w.v_scale)
        k, v = O.gather_kv(cache, 0, kvl, sub_bt[s * pps:(s + 1) * pps], page_size=w.page_size,
                           pages_per_seq=pps, head_dim=w.head_dim, cache_dtype=w.cache_dtype,
                           k_scale=w.k_scale, v_scale=w.v_scale)
        q = O.to_f64(q_bits[q0:q0 + ql], w.q_dtype)
        O.attend_sequence(q, k, v, ctx, softmax_scale=w.softmax_scale,
                          sliding_window=w.sliding_window, logits_soft_cap=w.logits_soft_cap,
                          q_scale=w.q_scale, sink=sink)
        t_used += time.perf_counter() - t0
        lo = max(0, ctx - w.sliding_window + 1) if w.sliding_window else 0
        kvb += (kvl - lo) * tok_bytes
        vis = ctx + np.arange(ql) + 1
        if w.sliding_window:
            vis = np.minimum(vis, w.sliding_window)
        flops += 4 * w.head_dim * int(vis.sum()) * w.num_q_heads
        done += 1
        if t_used >= budget_s:
            break
    return dict(seconds=t_used, seqs=done, kv_bytes=kvb, flops=flops, threads=nthreads)


KERNEL_SOURCES = {  # kernel -> sources whose hash identifies a counter summary
    "decode": ["decode.hip", "merge.h", "device_common.h", "rpa_internal.h"],
    "prefill": ["prefill.hip", "merge.h", "device_common.h", "rpa_internal.h"],
}
KERNEL_SYMBOL = {"decode": "row_kernel", "prefill": "prefill_kernel"}


def source_hash(kernel):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "ragged_paged_kv_scatter_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_file(workload):
    return os.path.join(ROOT, "profiles", f"traffic_{workload}.json")


def read_counter_csv(path):
    """{dispatch_id: (kernel_name, {counter: summed value})} from a rocprofv3
    counter_collection.csv (values summed over the counter's instances)."""
    import csv
    out = {}
    with open(path) as fh:
        for r in csv.DictReader(fh):
            d = out.setdefault(r["Dispatch_Id"], (r["Kernel_Name"], {}))
            d[1][r["Counter_Name"]] = d[1].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return out


def summarize_counters(workload, kernel, fetch_csv, write_csv, copy_bytes):
    """HBM traffic of one launch of `kernel` from a FETCH_SIZE run and a
    WRITE_SIZE run (KiB per dispatch), each scaled by what the same counter
    reads for the calibration copy of `copy_bytes` (read once, written once)."""
    sym = KERNEL_SYMBOL[kernel]
    res = {}
    for name, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        disp = read_counter_csv(path)
        copies = [c[name] for k, c in disp.values() if "copy" in k.lower() and name in c]
        ours = [c[name] for k, c in disp.values() if sym in k and name in c]
        if not copies or not ours:
            raise SystemExit(f"no copy or {sym} dispatch with {name} in {path}")
        copy_kib = max(copies)
        factor = copy_bytes / (copy_kib * 1024.0)
        res[name] = dict(kernel_kib=sum(ours) / len(ours), dispatches=len(ours),
                         copy_kib=copy_kib, factor=factor,
                         bytes=sum(ours) / len(ours) * 1024.0 * factor)
    out = dict(workload=workload, kernel=kernel, source_hash=source_hash(kernel),
               copy_bytes=copy_bytes, fetch=res["FETCH_SIZE"], write=res["WRITE_SIZE"],
               traffic_bytes=res["FETCH_SIZE"]["bytes"] + res["WRITE_SIZE"]["bytes"])
    with open(traffic_file(workload), "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))


def bench_reshape_and_cache(args, w, dev):
    """One step = rpa_slot_mapping + rpa_reshape_and_cache of the workload's new
    tokens into split K / V caches ([num_pages, page_size, Hkv, Dpad] each).
    Algorithmic bytes: the new K and V rows read once and stored once."""
    import torch

    import ragged_paged_kv_scatter_amd as rpa
    from oracle import rpa_oracle as O
    from tests.helpers import bits

    meta = {k: torch.from_numpy(np.ascontiguousarray(getattr(w, k))).to(dev)
            for k in ("kv_lens", "block_tables", "query_start_loc", "distribution")}
    kc = w.kv_cache[:, :, 0::2, :].contiguous()
    vc = w.kv_cache[:, :, 1::2, :].contiguous()
    slots = torch.empty(w.total_tokens, dtype=torch.int64, device=dev)

    def step():
        rpa.rpa_slot_mapping(meta["kv_lens"], meta["block_tables"], meta["query_start_loc"],
                             meta["distribution"], page_size=w.page_size,
                             total_tokens=w.total_tokens, out=slots)
        rpa.rpa_reshape_and_cache(w.keys, w.values, kc, vc, slots, k_scale=w.k_scale,
                                  v_scale=w.v_scale)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    rpa.profile_enable(True)
    rpa.profile_read()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    rpa.profile_enable(False)
    kstats = rpa.profile_read()
    ms = (t1 - t0) * 1e3 / args.steps
    n_valid = int(w.query_start_loc[w.num_seqs])
    in_b = 2 * n_valid * w.num_kv_heads * w.head_dim * ELEM[w.kv_in_dtype]
    out_b = 2 * n_valid * w.num_kv_heads * w.head_dim_padded * ELEM[w.cache_dtype]
    nbytes = in_b + out_b
    n, kms = kstats.get("reshape_and_cache", (1, 0.0))
    kavg = kms / max(n, 1)
    achieved = nbytes / (kavg * 1e-3) / 1e9
    line = {
        "metric": "slot-mapping KV store GB/s (new K/V read + split-cache rows written)",
        "value": nbytes / (ms * 1e-3) / 1e9, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.cache_dtype, "data": "synthetic",
        "config": {"workload": w.name, "op": "reshape_and_cache", "token_rows": n_valid,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                   "kv_in_dtype": w.kv_in_dtype, "cache_dtype": w.cache_dtype,
                   "bytes": nbytes, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "reshape_and_cache", "kernel_avg_ms": kavg},
        "kernels_ms": {k: v[1] / max(v[0], 1) for k, v in kstats.items()},
    }
    if not args.no_cpu_baseline:
        kb, vb = bits(w.keys, w.kv_in_dtype), bits(w.values, w.kv_in_dtype)
        kcb, vcb = bits(kc, w.cache_dtype), bits(vc, w.cache_dtype)
        sl = O.slot_mapping(w.kv_lens, w.block_tables, w.query_start_loc, w.distribution,
                            page_size=w.page_size, pages_per_seq=w.pages_per_seq,
                            total_tokens=w.total_tokens)
        rows = min(n_valid, 4096)
        t0 = time.perf_counter()
        O.reshape_and_cache(kcb, vcb, kb[:rows], vb[:rows], sl[:rows], kv_in_dtype=w.kv_in_dtype,
                            cache_dtype=w.cache_dtype, k_scale=w.k_scale, v_scale=w.v_scale)
        secs = time.perf_counter() - t0
        line["cpu_baseline"] = dict(value=nbytes * rows / n_valid / secs / 1e9, unit="GB/s",
                                    cores=1, kind="oracle",
                                    sample=f"{rows} of {n_valid} token rows, {secs:.1f} s on "
                                           "the host (cache copies included)")
    print(json.dumps(line), flush=True)


def graph_timing(args, step, dev, work, decode_like, unit):
    """The same step captured once in a HIP graph and replayed: the launches
    without the host's per-call work (rpa_forward's checks and its three
    launch calls)."""
    import torch

    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    value = work / (ms * 1e-3) / (1e9 if decode_like else 1e12)
    return dict(ms_per_step=ms, value=value, unit=unit)


def bench_copy_blocks(args, w, dev, num_blocks=8192, num_pairs=2048):
    """One step = rpa_copy_blocks of num_pairs (source, destination) block pairs
    in one layer's K and V caches of num_blocks blocks [page_size, Hkv, Dpad].
    Algorithmic bytes: every copied block read once and written once."""
    import torch

    import ragged_paged_kv_scatter_amd as rpa
    from oracle import rpa_oracle as O

    dt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}[w.cache_dtype]
    shape = (num_blocks, w.page_size, w.num_kv_heads, w.head_dim_padded)
    kc = torch.zeros(shape, dtype=dt, device=dev)
    vc = torch.zeros(shape, dtype=dt, device=dev)
    rng = np.random.default_rng(0)
    perm = rng.permutation(num_blocks)
    pairs_np = np.stack([perm[:num_pairs], perm[num_pairs:2 * num_pairs]], 1).astype(np.int64)
    pairs = torch.from_numpy(pairs_np).to(dev)

    def step():
        rpa.rpa_copy_blocks([kc], [vc], pairs)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    rpa.profile_enable(True)
    rpa.profile_read()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    rpa.profile_enable(False)
    kstats = rpa.profile_read()
    ms = (t1 - t0) * 1e3 / args.steps
    block = kc[0].numel() * kc.element_size()
    nbytes = 2 * 2 * num_pairs * block            # K and V planes, read + write
    n, kms = kstats.get("copy_blocks", (1, 0.0))
    kavg = kms / max(n, 1)
    achieved = nbytes / (kavg * 1e-3) / 1e9
    line = {
        "metric": "block copy GB/s (copied K/V blocks read + written)",
        "value": nbytes / (ms * 1e-3) / 1e9, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.cache_dtype, "data": "synthetic",
        "config": {"workload": w.name, "op": "copy_blocks", "num_blocks": num_blocks,
                   "pairs": num_pairs, "block_bytes": block, "bytes": nbytes,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None, "kernel": "copy_blocks",
                     "kernel_avg_ms": kavg},
        "kernels_ms": {k: v[1] / max(v[0], 1) for k, v in kstats.items()},
    }
    if not args.no_cpu_baseline:
        host = np.zeros((num_blocks,) + shape[1:], dtype=np.uint8 if dt == torch.uint8 else
                        (np.uint16 if dt == torch.bfloat16 else np.uint32))
        t0 = time.perf_counter()
        O.copy_blocks([host, host], pairs_np)
        secs = time.perf_counter() - t0
        line["cpu_baseline"] = dict(value=nbytes / secs / 1e9, unit="GB/s", cores=1,
                                    kind="oracle",
                                    sample=f"all {num_pairs} pairs of both planes, {secs:.1f} s "
                                           "on the host (whole-cache copies included)")
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode_bf16")
    ap.add_argument("--op", default="forward",
                    choices=["forward", "reshape_and_cache", "copy_blocks"],
                    help="forward: the whole step (default); reshape_and_cache: the update's "
                         "slot-mapping form into split K/V caches, at the workload's token "
                         "count; copy_blocks: 2048 block copies in 8192-block split caches of "
                         "the workload's block shape")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip timing the step replayed from a captured HIP graph")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run one device copy of this size first (counter calibration)")
    ap.add_argument("--summarize-counters", nargs=3, metavar=("KERNEL", "FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic_<workload>.json from two rocprofv3 --pmc runs")
    args = ap.parse_args()
    if args.summarize_counters:
        k, f, wcsv = args.summarize_counters
        summarize_counters(args.workload, k, f, wcsv, args.calib_copy_mib * 2 ** 20)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the path needs no "
              "collective and shards by kv head or by sequence with no exchange.", file=sys.stderr)
        sys.exit(2)

    import torch

    import ragged_paged_kv_scatter_amd as rpa
    from ragged_paged_kv_scatter_amd import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = W.make(args.workload, device=dev)
    if args.op == "reshape_and_cache":
        bench_reshape_and_cache(args, w, dev)
        return
    if args.op == "copy_blocks":
        bench_copy_blocks(args, w, dev)
        return
    meta = {k: torch.from_numpy(np.ascontiguousarray(getattr(w, k))).to(dev)
            for k in ("kv_lens", "block_tables", "query_start_loc", "distribution")}
    out = torch.empty(w.queries.shape, dtype=w.queries.dtype, device=dev)
    opts = w.options()
    ws_bytes = rpa.rpa_workspace_bytes(
        rpa._desc(w.queries, rpa._dtype(w.keys), w.kv_cache, meta["kv_lens"],
                  meta["block_tables"]),
        rpa._options(**opts, chunk_prefill_size=None, num_kv_pages_per_block=None,
                     num_queries_per_block=None, vmem_limit_bytes=None))
    workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

    def step():
        rpa.rpa_forward(w.queries, w.keys, w.values, w.kv_cache, meta["kv_lens"],
                        meta["block_tables"], meta["query_start_loc"], meta["distribution"],
                        w.attention_sink, out=out, workspace=workspace, **opts)

    if args.calib_copy_mib:
        src = torch.ones(args.calib_copy_mib * 2 ** 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    rpa.profile_enable(True)
    rpa.profile_read()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    rpa.profile_enable(False)
    kstats = rpa.profile_read()
    ms = (t1 - t0) * 1e3 / args.steps

    kvb, flops, row_kvb, pf_flops = work_counts(w, split=True)
    decode_like = args.workload != "prefill_bf16"   # prefill reports TFLOP/s, the rest KV GB/s
    if decode_like:
        value, unit = kvb / (ms * 1e-3) / 1e9, "GB/s"
    else:
        value, unit = flops / (ms * 1e-3) / 1e12, "TFLOP/s"
    # dominant kernel: of the two attention kernels, the one with the larger
    # summed time among those with work in this batch (on the side-stream path
    # a kernel with no work still spans the other's run while it waits for
    # slots, so it is not a candidate); its roofline is priced on its own
    # algorithmic work: the row kernel's KV bytes, the prefill tiles' FLOPs
    cands = {k: v for k, v in kstats.items()
             if (k == "decode" and row_kvb > 0) or (k == "prefill" and pf_flops > 0)}
    dom = max(cands.items(), key=lambda kv: kv[1][1]) if cands else ("none", (1, 0.0))
    dom_name, (dom_n, dom_ms) = dom
    dom_avg_ms = dom_ms / max(dom_n, 1)
    if dom_name == "prefill":
        achieved = pf_flops / (dom_avg_ms * 1e-3) / 1e12
        roof = dict(bound="mfma", achieved=achieved, peak=BF16_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=achieved / BF16_PEAK_TFLOPS, traffic=None)
    else:
        achieved = row_kvb / (dom_avg_ms * 1e-3) / 1e9
        roof = dict(bound="hbm", achieved=achieved, peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=achieved / HBM_PEAK_GBS, traffic=None)
    roof["kernel"] = dom_name
    roof["kernel_avg_ms"] = dom_avg_ms
    # HBM traffic per launch from a committed counter summary, only while the
    # kernel's sources are the ones the counters were taken on
    tf = traffic_file(w.name)
    if os.path.exists(tf) and dom_name in KERNEL_SOURCES:
        with open(tf) as fh:
            t = json.load(fh)
        if t.get("kernel") == dom_name and t.get("source_hash") == source_hash(dom_name):
            roof["traffic"] = t["traffic_bytes"]

    line = {
        "metric": METRIC, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.q_dtype, "data": "synthetic",
        "config": {"workload": w.name, "num_seqs": w.num_seqs, "total_tokens": w.total_tokens,
                   "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim, "page_size": w.page_size,
                   "cache_dtype": w.cache_dtype, "kv_bytes": kvb, "flops": flops,
                   "parallelism": "single GPU"},
        "roofline": roof,
        "kernels_ms": {k: v[1] / max(v[0], 1) for k, v in kstats.items()},
    }
    if not args.no_graph:
        try:
            line["graph"] = graph_timing(args, step, dev, kvb if decode_like else flops,
                                         decode_like, unit)
        except Exception as e:  # reported, never fatal: `value` is the eager step
            line["graph"] = dict(error=str(e)[:200])
    if not args.no_cpu_baseline:
        cb = cpu_baseline(w, args.cpu_budget)
        if unit == "GB/s":
            cv = cb["kv_bytes"] / cb["seconds"] / 1e9
        else:
            cv = cb["flops"] / cb["seconds"] / 1e12
        line["cpu_baseline"] = dict(
            value=cv, unit=unit, cores=cb["threads"], kind="oracle",
            sample=f"{cb['seqs']} sequence evaluations over a {w.num_seqs}-sequence batch "
                   f"(update + gather + float64 attention), {cb['seconds']:.1f} s on the host")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

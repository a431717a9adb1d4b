"""Benchmark of the ragged paged attention hot path on one MI355X.

A step is one rpa_forward call with the step's new keys/values: KV-cache
update (scatter), device planning, attention and split merge, over one batch of
synthetic input resident in HBM.  The default run prints ONE JSON line whose
`value` is the bf16 decode workload's KV GB/s (256 sequences, kv_len
~ U{512..4096}, page_size 16, 32 q heads, 8 kv heads, head_dim 128) and whose
nested `prefill` object is the bf16 long-prefill workload's TFLOP/s (2 x 8192
tokens, no context, causal, 64 q heads, 8 kv heads, head_dim 128, page_size
128): the two halves of the metric.

Timing protocol: W untimed warm-up steps; then K timed steps, each preceded
by a 1 GiB write that evicts L2 and the 256 MB MALL, each bracketed by
hipEvents on the step's stream (profiling off); the whole loop sits between
two device synchronisations.  Per-kernel times come from a second, profiled
pass of K steps (the library's events around each launch).  Probes of the
GPU (HBM read / copy streams, a dense bf16 MFMA burn with its shader clock,
VALU issue rates) give measured ceilings beside the published peaks.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--op OP] [--no-cpu-baseline]
"""
import argparse
import contextlib
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
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense fp8 MFMA
# Long-prefill workloads report TFLOP/s; the others KV GB/s.
PREFILL_WORKLOADS = ("prefill_bf16", "prefill_fp8q")
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
    has_prefill_kernel = w.q_dtype in ("bf16", "fp8")
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


def update_bytes(w):
    """HBM bytes of the cache update: the valid new rows' K and V read in the
    input dtype and written as whole cache rows (D elements, pad lanes zeroed
    up to Dpad) in the cache dtype."""
    n_tok = int(np.asarray(w.query_start_loc)[w.num_seqs])
    in_sz, c_sz = ELEM[w.kv_in_dtype], ELEM[w.cache_dtype]
    return n_tok * 2 * w.num_kv_heads * (w.head_dim * in_sz + w.head_dim_padded * c_sz)


def cpu_info():
    """Host CPU model and logical CPU count (where the oracle baseline runs)."""
    model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count()
    return dict(model=model, cpu_count=os.cpu_count(), affinity=affinity)


def cpu_baseline(w, budget_s=10.0, threads=None, row_block=64, metric="kv"):
    """The oracle as it stands, timed on the host on a bounded sample of the
    same workload, with BLAS limited to `threads` (None: as configured).

    The sample walks the sequences in a fixed random order; each sequence is
    updated (its new tokens scattered into a compact copy of its pages) and
    gathered once, then its query rows are attended to in blocks of
    `row_block` in a fixed random order, until `budget_s` seconds of oracle
    time.  metric "kv": KV bytes of the sequences done whole / time (decode);
    "flops": 4 D FLOPs per visible (query, key, q head) of the rows done / time.
    """
    import threadpoolctl

    from oracle import rpa_oracle as O
    from tests.helpers import bits, compact_pages

    limits = threadpoolctl.threadpool_limits(limits=threads) if threads else \
        contextlib.nullcontext()
    with limits:
        info = threadpoolctl.threadpool_info()
        used = max([t.get("num_threads", 1) for t in info] + [1])
        rng = np.random.default_rng(0)
        q_bits = bits(w.queries, w.q_dtype)
        k_bits = bits(w.keys, w.kv_in_dtype)
        v_bits = bits(w.values, w.kv_in_dtype)
        sink = None if w.attention_sink is None else w.attention_sink.cpu().numpy()
        tok_bytes = 2 * w.num_kv_heads * w.head_dim * ELEM[w.cache_dtype]
        pps = w.pages_per_seq
        t_used, kvb, flops, rows_done, seqs_done = 0.0, 0, 0, 0, 0
        for s in rng.permutation(w.num_seqs):
            s = int(s)
            q0, ql, ctx, kvl = O.seq_bounds(w.query_start_loc, w.kv_lens, s)
            if ql == 0:
                continue
            sub_cache, sub_bt = compact_pages(w, [s])
            t0 = time.perf_counter()
            cache = O.update_kv_cache(sub_cache, k_bits[q0:q0 + ql], v_bits[q0:q0 + ql],
                                      np.array([kvl], np.int32), sub_bt[s * pps:(s + 1) * pps],
                                      np.array([0, ql], np.int32), np.array([0, 0, 1], np.int32),
                                      page_size=w.page_size, pages_per_seq=pps,
                                      kv_in_dtype=w.kv_in_dtype, cache_dtype=w.cache_dtype,
                                      k_scale=w.k_scale, v_scale=w.v_scale)
            k, v = O.gather_kv(cache, 0, kvl, sub_bt[s * pps:(s + 1) * pps],
                               page_size=w.page_size, pages_per_seq=pps, head_dim=w.head_dim,
                               cache_dtype=w.cache_dtype, k_scale=w.k_scale, v_scale=w.v_scale)
            t_used += time.perf_counter() - t0
            blocks = list(range(0, ql, row_block))
            whole = True
            for b in rng.permutation(len(blocks)):
                t_lo = blocks[int(b)]
                n = min(row_block, ql - t_lo)
                q = O.to_f64(q_bits[q0 + t_lo:q0 + t_lo + n], w.q_dtype)
                t0 = time.perf_counter()
                O.attend_sequence(q, k, v, ctx + t_lo, softmax_scale=w.softmax_scale,
                                  sliding_window=w.sliding_window,
                                  logits_soft_cap=w.logits_soft_cap, q_scale=w.q_scale,
                                  sink=sink)
                t_used += time.perf_counter() - t0
                vis = ctx + t_lo + np.arange(n) + 1
                if w.sliding_window:
                    vis = np.minimum(vis, w.sliding_window)
                flops += 4 * w.head_dim * int(vis.sum()) * w.num_q_heads
                rows_done += n
                if t_used >= budget_s:
                    whole = n + t_lo == ql and len(blocks) == 1
                    break
            if whole:
                lo = max(0, ctx - w.sliding_window + 1) if w.sliding_window else 0
                kvb += (kvl - lo) * tok_bytes
                seqs_done += 1
            if t_used >= budget_s:
                break
    value = (kvb / t_used / 1e9) if metric == "kv" else (flops / t_used / 1e12)
    return dict(value=value, seconds=t_used, rows=rows_done, seqs=seqs_done, threads=used)


def cpu_baseline_entry(w, budget_s, metric, unit):
    """cpu_baseline at all of BLAS's threads and at one thread."""
    host = cpu_info()
    runs = {}
    for label, threads in (("all", None), ("one", 1)):
        progress(f"{w.name}: oracle baseline, {label} thread(s)")
        runs[label] = cpu_baseline(w, budget_s, threads=threads, metric=metric)
    a, o = runs["all"], runs["one"]
    what = "sequences" if metric == "kv" else "query-row blocks of 64"
    return dict(value=a["value"], unit=unit, cores=a["threads"], kind="oracle",
                sample=f"{a['seqs']} sequences / {a['rows']} query rows of the {w.num_seqs}-"
                       f"sequence batch ({what}, update + gather + float64 attention), "
                       f"{a['seconds']:.1f} s of oracle time on the host",
                one_thread=dict(value=o["value"], cores=o["threads"], seconds=o["seconds"],
                                seqs=o["seqs"], rows=o["rows"]),
                host_cpu=host["model"], host_cpu_count=host["cpu_count"],
                host_cpu_affinity=host["affinity"])


KERNEL_SOURCES = {  # kernel -> sources whose hash identifies a counter summary
    "decode": ["decode.hip", "merge.h", "device_common.h", "rpa_internal.h"],
    "prefill": ["prefill.hip", "merge.h", "device_common.h", "rpa_internal.h"],
}
# kernel -> the symbols whose dispatches make up one launch of it; the first
# is dispatched once per step (prefill_kernel is, and the two-group kernel
# runs after it on bf16 batches, one of the two taking the tiles)
KERNEL_SYMBOL = {"decode": ("row_kernel",), "prefill": ("prefill_kernel", "prefill_pair_kernel")}


def strip_timeline(text):
    """The source without the wave-timeline instrumentation: the blocks under
    `#ifdef RPA_WAVE_TIMELINE` (to their matching #endif) and the RPA_TL_*
    statements, which expand to nothing unless that macro is defined."""
    import re
    out, depth = [], 0
    for line in text.split("\n"):
        d = line.strip()
        if depth:
            if d.startswith("#if"):
                depth += 1
            elif d.startswith("#endif"):
                depth -= 1
            continue
        if d == "#ifdef RPA_WAVE_TIMELINE":
            depth = 1
            continue
        out.append(line)
    return re.sub(r"RPA_TL_\w+\([^()]*\);", " ", "\n".join(out))


def source_hash(kernel):
    """Hash of the kernel's sources with comments, blank space and the
    wave-timeline instrumentation removed, so that a counter summary stays
    valid across edits that leave the product build's code unchanged."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "ragged_paged_kv_scatter_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        text = strip_timeline(text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def traffic_file(workload, kernel):
    return os.path.join(ROOT, "profiles", f"traffic_{workload}_{kernel}.json")


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
    reads for the calibration copy of `copy_bytes` (read once, written once).
    The flush writes between timed steps are dispatches of their own and are
    not counted."""
    syms = KERNEL_SYMBOL[kernel]
    res = {}
    for name, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        disp = read_counter_csv(path)
        copies = [c[name] for k, c in disp.values()
                  if "copy" in k.lower() and "probe" not in k.lower() and name in c]
        ours = [c[name] for k, c in disp.values() if any(s in k for s in syms) and name in c]
        launches = sum(1 for k, c in disp.values() if syms[0] in k and name in c)
        if not copies or not ours or not launches:
            raise SystemExit(f"no copy or {syms[0]} dispatch with {name} in {path}")
        copy_kib = max(copies)
        factor = copy_bytes / (copy_kib * 1024.0)
        res[name] = dict(kernel_kib=sum(ours) / launches, dispatches=len(ours),
                         launches=launches, copy_kib=copy_kib, factor=factor,
                         bytes=sum(ours) / launches * 1024.0 * factor)
    out = dict(workload=workload, kernel=kernel, source_hash=source_hash(kernel),
               copy_bytes=copy_bytes, fetch=res["FETCH_SIZE"], write=res["WRITE_SIZE"],
               traffic_bytes=res["FETCH_SIZE"]["bytes"] + res["WRITE_SIZE"]["bytes"])
    with open(traffic_file(workload, kernel), "w") as fh:
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


FLUSH_BYTES = 1 << 30   # written before every timed step: evicts L2 (4 MB / XCD) and the 256 MB MALL


class Flusher:
    """A 1 GiB device buffer written (one fill kernel) before each timed step."""

    def __init__(self, dev):
        import torch
        self.buf = torch.empty(FLUSH_BYTES // 4, dtype=torch.int32, device=dev)
        self.k = 0

    def __call__(self):
        self.k += 1
        self.buf.fill_(self.k)


def progress(msg):
    """A progress line on stderr (the JSON line alone goes to stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def timed_steps(step, steps, flush):
    """K steps, each after a cache flush, each bracketed by events on the
    current stream (rpa_forward joins all of its work back into it); returns
    (per-step ms list, wall ms per step including the flushes)."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in evs:
        flush()
        a.record()
        step()
        b.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    return [a.elapsed_time(b) for a, b in evs], wall


def back_to_back(step, steps):
    """K steps back to back between two synchronisations (no flush)."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def timeline_summary(a):
    """Per-wave stamps (rows of start, first step, end, steps << 32 | XCC_ID
    << 16 | HW_ID; 100 MHz ticks) -> where the waves of one launch start and
    end, how each CU's workgroups end, and the mean end per XCD (us)."""
    a = a[a[:, 0] > 0]
    if len(a) == 0:
        return {"waves": 0}
    t0, t1, t2 = (a[:, i].astype(np.int64) for i in range(3))
    base = int(t0.min())
    steps = (a[:, 3] >> 32).astype(np.int64)
    hw = (a[:, 3] & 0xFFFF).astype(np.int64)
    xcc = ((a[:, 3] >> 16) & 0xF).astype(np.int64)
    # HW_ID: wave slot 3:0, SIMD 5:4, CU 11:8, shader array 12, shader engine 15:13
    cu = xcc * 1000 + ((hw >> 13) & 7) * 100 + ((hw >> 12) & 1) * 16 + ((hw >> 8) & 0xF)
    slot = hw & 0xF
    us = lambda v: float(v) / 100.0
    q = lambda v: [round(us(np.percentile(v, x)), 2) for x in (0, 10, 50, 90, 100)]
    end = t2 - base
    cu_last, cu_spread = [], []
    for c in np.unique(cu):
        m = cu == c
        cu_last.append(end[m].max())
        by_slot = [end[m & (slot == s)].mean() for s in np.unique(slot[m])]
        cu_spread.append(max(by_slot) - min(by_slot))
    return {
        "waves": int(len(a)), "cus": int(len(cu_last)),
        "start_us": q(t0 - base), "first_step_end_us": q(t1 - base), "end_us": q(end),
        "steps": [int(steps.min()), int(np.median(steps)), int(steps.max())],
        "cu_last_end_us": q(np.array(cu_last)), "cu_mean_last_end_us": round(us(np.mean(cu_last)), 2),
        "cu_slot_spread_us": q(np.array(cu_spread)),
        "xcd_mean_end_us": [round(us(end[xcc == x].mean()), 1) for x in range(8) if (xcc == x).any()],
    }


PF_PHASES = ("issue", "qk", "pv", "tail")


def pf_timeline_summary(a):
    """Per-wave prefill kernel counts (rows of total, copy-wait and
    barrier-wait shader clocks, steps, then the issue / q.k / p.v / tail
    parts of the steps) -> how the waves' time splits: the means over waves
    of each share of the wave's time and of the clocks per pipeline step."""
    a = a[a[:, 3] > 0].astype(np.float64)
    if len(a) == 0:
        return {"waves": 0}
    tot, vm, bar, steps = a[:, 0], a[:, 1], a[:, 2], a[:, 3]
    out = {
        "waves": int(len(a)), "steps": [int(steps.min()), int(np.median(steps)), int(steps.max())],
        "total_clk": [round(float(np.percentile(tot, x))) for x in (0, 50, 100)],
        "copy_wait_share": round(float((vm / tot).mean()), 4),
        "barrier_wait_share": round(float((bar / tot).mean()), 4),
        "clk_per_step": round(float((tot / steps).mean()), 1),
        "copy_wait_clk_per_step": round(float((vm / steps).mean()), 1),
        "barrier_wait_clk_per_step": round(float((bar / steps).mean()), 1),
    }
    for i, name in enumerate(PF_PHASES):
        out[f"{name}_clk_per_step"] = round(float((a[:, 4 + i] / steps).mean()), 1)
    return out


PP_PARTS = ("pre_qk", "qk", "group_b_barrier", "pv", "tail", "unit_end")


def pp_timeline_summary(a):
    """Per-wave counts of the two-group prefill kernel (rows of total clocks,
    steps, then clocks in: step start -> q.k (group A's barrier and copies,
    the rescale), q.k, group B's mid-step barrier, p.v, the row max / sum
    tail, and unit set-up / end) -> means per step over the waves of each
    group (waves 0-3 and 4-7 of each workgroup)."""
    out = {}
    for gname, sel in (("group_a", lambda w: (w % 8) < 4), ("group_b", lambda w: (w % 8) >= 4)):
        idx = np.array([i for i in range(len(a)) if sel(i)], dtype=np.int64)
        r = a[idx]
        r = r[r[:, 1] > 0].astype(np.float64)
        if len(r) == 0:
            out[gname] = {"waves": 0}
            continue
        steps = r[:, 1]
        d = {"waves": int(len(r)), "clk_per_step": round(float((r[:, 0] / steps).mean()), 1)}
        for i, name in enumerate(PP_PARTS):
            d[f"{name}_clk_per_step"] = round(float((r[:, 2 + i] / steps).mean()), 1)
        out[gname] = d
    return out


def bench_timeline(args, w, dev):
    """The row kernels' per-wave clock stamps and the prefill kernel's per-wave
    wait counts (librpa_timeline.so) over a few flushed steps of the workload:
    one JSON line per launch."""
    import ctypes

    import torch

    import ragged_paged_kv_scatter_amd as rpa
    from ragged_paged_kv_scatter_amd import _lib

    lib = _lib.load()
    words, pwords = 8192 * 4, 8192 * 8
    buf = (ctypes.c_ulonglong * words)()
    pbuf = (ctypes.c_ulonglong * pwords)()
    meta = {k: torch.from_numpy(np.ascontiguousarray(getattr(w, k))).to(dev)
            for k in ("kv_lens", "block_tables", "query_start_loc", "distribution")}
    out = torch.empty(w.queries.shape, dtype=rpa.out_dtype_for(w.queries.dtype), device=dev)
    opts = w.options()
    flush = Flusher(dev)

    def step():
        rpa.rpa_forward(w.queries, w.keys, w.values, w.kv_cache, meta["kv_lens"],
                        meta["block_tables"], meta["query_start_loc"], meta["distribution"],
                        w.attention_sink, out=out, **opts)

    for _ in range(max(args.warmup, 1)):
        step()
    torch.cuda.synchronize()
    for rep in range(min(args.steps, 5)):
        if lib.rpa_timeline_clear() != 0 or lib.rpa_pf_timeline_clear() != 0:
            raise SystemExit("timeline clear failed")
        flush()
        torch.cuda.synchronize()
        step()
        torch.cuda.synchronize()
        if lib.rpa_timeline_read(buf, words) != 0:
            raise SystemExit("rpa_timeline_read failed")
        a = np.frombuffer(buf, dtype=np.uint64).reshape(-1, 4).copy()
        if lib.rpa_pf_timeline_read(pbuf, pwords) != 0:
            raise SystemExit("rpa_pf_timeline_read failed")
        b = np.frombuffer(pbuf, dtype=np.uint64).reshape(-1, 8).copy()
        if lib.rpa_pp_timeline_read(pbuf, pwords) != 0:
            raise SystemExit("rpa_pp_timeline_read failed")
        c = np.frombuffer(pbuf, dtype=np.uint64).reshape(-1, 8).copy()
        print(json.dumps({"metric": "row kernel wave timeline", "workload": w.name, "launch": rep,
                          **timeline_summary(a), "prefill": pf_timeline_summary(b),
                          "prefill_pair": pp_timeline_summary(c)}), flush=True)


def probe_ceilings(dev, full=False):
    """Measured ceilings of this GPU from librpa_probes.so: HBM streaming read
    and copy (GB/s), dense bf16 MFMA (TFLOP/s) with the shader clock it runs
    at, v_exp_f32 / v_rcp_f32 / v_fma_f32 issue rates (lane-ops/s), LDS read,
    transposed read and write rates and the L2 -> LDS copy rate (bytes per CU
    and clock, and TB/s over the chip).  full (bench.py --op probes) adds the
    MFMA rates beside VALU work and fed from LDS, and LDS reads beside
    copies."""
    import ctypes

    import torch

    from ragged_paged_kv_scatter_amd import _probes

    lib = _probes.load()
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    reps = 5

    def time_it(launch, n=reps):
        launch()                                   # warm-up
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        best = float("inf")
        for _ in range(n):
            a.record()
            launch()
            b.record()
            b.synchronize()
            best = min(best, a.elapsed_time(b))
        return best

    out = {}
    nbytes = 2 << 30
    src = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    half = nbytes // 2
    dst = torch.empty(half // 4, dtype=torch.int32, device=dev)
    # streaming rates depend on the grid: the best of 1 to 4 workgroups per CU
    # (2 to 3 read fastest here, about 7 TB/s; 16 per CU reads about 6 TB/s)
    read_ms, copy_ms = [], []
    for per_cu in (1, 2, 3, 4):
        blocks = cus * per_cu
        sink = torch.empty(blocks * 256, dtype=torch.int32, device=dev)
        read_ms.append(time_it(lambda: _probes.check(lib.rpa_probe_read(
            ctypes.c_void_p(src.data_ptr()), nbytes // 16, ctypes.c_void_p(sink.data_ptr()),
            blocks, stream), "read probe")))
        copy_ms.append(time_it(lambda: _probes.check(lib.rpa_probe_copy(
            ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), half // 16, blocks,
            stream), "copy probe")))
    out["hbm_read_gbs"] = nbytes / (min(read_ms) * 1e-3) / 1e9
    out["hbm_copy_gbs"] = 2 * half / (min(copy_ms) * 1e-3) / 1e9
    del src, dst, sink
    # MFMA: 2 workgroups (8 waves) per CU, 4 chains per wave
    mblocks, iters = cus * 2, 20000
    msink = torch.empty(mblocks * 256 * 16, dtype=torch.float32, device=dev)
    clocks = torch.zeros(mblocks * 4 * 2, dtype=torch.int64, device=dev)
    ms = time_it(lambda: _probes.check(lib.rpa_probe_mfma(
        ctypes.c_void_p(msink.data_ptr()), ctypes.c_void_p(clocks.data_ptr()), iters, mblocks,
        stream), "mfma probe"))
    flops = mblocks * 4 * 4 * iters * 32 * 32 * 16 * 2
    out["mfma_bf16_tflops"] = flops / (ms * 1e-3) / 1e12
    c = clocks.view(-1, 2).double()
    ok = c[:, 1] > 0
    out["shader_clock_ghz_mfma"] = float((c[ok, 0] / c[ok, 1]).mean() * 0.1)
    # MFMA beside 0..4 VALU pairs per MFMA (fma + exp, or two fma), at 2
    # waves per SIMD (the prefill kernel's residency) and at 1, where a wave's
    # VALU work can only run under its own MFMAs
    for per_cu in ((2, 1) if full else ()):
        xb = cus * per_cu
        xflops = xb * 4 * 4 * iters * 32 * 32 * 16 * 2
        # accumulators in AGPRs (rpa_probe_mix) and in VGPRs, the attention
        # kernels' form (rpa_probe_mix_vgpr_acc)
        cases = [(fn, acc, exp_, nv)
                 for fn, acc in ((lib.rpa_probe_mix, ""), (lib.rpa_probe_mix_vgpr_acc, "_vgpr_acc"))
                 for exp_ in (1, 0) for nv in (0, 1, 2, 4) if nv or exp_]
        for fn, acc, exp_, nv in cases:
            ms = time_it(lambda: _probes.check(fn(
                ctypes.c_void_p(msink.data_ptr()), ctypes.c_void_p(clocks.data_ptr()), nv, exp_,
                iters, xb, stream), "mix probe"))
            tag = f"mfma_w{4 * per_cu}_with_{nv}_{'fma_exp' if exp_ else 'fma_fma'}{acc}"
            out[f"{tag}_tflops"] = xflops / (ms * 1e-3) / 1e12
            c = clocks.view(-1, 2)[: xb * 4].double()
            ok = c[:, 1] > 0
            out[f"{tag}_clock_ghz"] = float((c[ok, 0] / c[ok, 1]).mean() * 0.1)
    # MFMA fed from LDS in the prefill kernel's patterns, 2 workgroups per CU
    # (2 waves per SIMD) and 1 (a wave alone on its SIMD)
    for per_cu in ((2, 1) if full else ()):
        lb = cus * per_cu
        for name, mode in _probes.LDS_MFMA_MODES.items():
            liters = iters // 4
            ms = time_it(lambda: _probes.check(lib.rpa_probe_lds_mfma(
                ctypes.c_void_p(msink.data_ptr()), ctypes.c_void_p(clocks.data_ptr()), mode,
                liters, lb, stream), "lds mfma probe"))
            lflops = lb * 4 * 16 * liters * 32 * 32 * 16 * 2
            tag = f"mfma_{name}" + ("" if per_cu == 2 else "_w4")
            out[f"{tag}_tflops"] = lflops / (ms * 1e-3) / 1e12
            c = clocks.view(-1, 2)[: lb * 4].double()
            ok = c[:, 1] > 0
            out[f"{tag}_clock_ghz"] = float((c[ok, 0] / c[ok, 1]).mean() * 0.1)
    # VALU: 8 workgroups (32 waves) per CU, 8 chains per lane
    vblocks, viters = cus * 8, 4096
    vsink = torch.empty(vblocks * 256 * 8, dtype=torch.float32, device=dev)
    for name, op in _probes.VALU_OPS.items():
        ms = time_it(lambda: _probes.check(lib.rpa_probe_valu(
            ctypes.c_void_p(vsink.data_ptr()), op, viters, vblocks, stream), "valu probe"))
        out[f"{name}_per_s"] = vblocks * 256 * 8 * viters / (ms * 1e-3)

    def clock_hz(clk):
        c = clk.view(-1, 2).double()
        ok = c[:, 1] > 0
        return float((c[ok, 0] / c[ok, 1]).mean()) * 1e8

    # LDS: 2 workgroups (8 waves, the prefill kernel's residency) and 4 per CU;
    # bytes per CU and shader clock, and the chip's total rate
    for per_cu in (2, 4):
        lblocks, liters = cus * per_cu, 4000
        lsink = torch.empty(lblocks * 256, dtype=torch.int32, device=dev)
        lclk = torch.zeros(lblocks * 4 * 2, dtype=torch.int64, device=dev)
        for name, (op, nb) in _probes.LDS_OPS.items():
            ms = time_it(lambda: _probes.check(lib.rpa_probe_lds(
                ctypes.c_void_p(lsink.data_ptr()), ctypes.c_void_p(lclk.data_ptr()), op, liters,
                lblocks, stream), "lds probe"))
            nbytes_l = lblocks * 4 * liters * 8 * nb
            out[f"lds_{name}_w{4 * per_cu}_bytes_per_cu_clk"] = (
                nbytes_l / (ms * 1e-3) / (clock_hz(lclk) * cus))
            out[f"lds_{name}_w{4 * per_cu}_tbs"] = nbytes_l / (ms * 1e-3) / 1e12
    # global -> LDS copies from a 2 MiB window (L2-resident on every XCD), at
    # the prefill kernel's 8 waves per CU and at 16
    window = 2 << 20
    dsrc = torch.ones(window // 4, dtype=torch.int32, device=dev)
    for per_cu in (2, 4):
        dblocks, diters = cus * per_cu, 2000
        dsink = torch.empty(dblocks * 256, dtype=torch.int32, device=dev)
        dclk = torch.zeros(dblocks * 4 * 2, dtype=torch.int64, device=dev)
        ms = time_it(lambda: _probes.check(lib.rpa_probe_dma(
            ctypes.c_void_p(dsrc.data_ptr()), window, ctypes.c_void_p(dsink.data_ptr()),
            ctypes.c_void_p(dclk.data_ptr()), diters, dblocks, stream), "dma probe"))
        nbytes_d = dblocks * 4 * diters * 8192
        out[f"l2_to_lds_w{4 * per_cu}_bytes_per_cu_clk"] = (
            nbytes_d / (ms * 1e-3) / (clock_hz(dclk) * cus))
        out[f"l2_to_lds_w{4 * per_cu}_tbs"] = nbytes_d / (ms * 1e-3) / 1e12
    # LDS reads (2 waves per workgroup) beside copies (the other 2), 2
    # workgroups per CU, 2 ms per run: rates of each alone and side by side,
    # bytes per CU and shader clock
    xblocks, ticks = cus * 2, 200000
    xsink = torch.empty(xblocks * 256, dtype=torch.int32, device=dev)
    xcnt = torch.zeros(xblocks * 4 * 2, dtype=torch.int64, device=dev)
    modes = ((1, "reads_alone"), (2, "copies_alone"), (3, "side_by_side")) if full else ()
    for mode, tag in modes:
        _probes.check(lib.rpa_probe_lds_dma(
            ctypes.c_void_p(dsrc.data_ptr()), window, ctypes.c_void_p(xsink.data_ptr()),
            ctypes.c_void_p(xcnt.data_ptr()), mode, ticks, xblocks, stream), "lds+dma probe")
        torch.cuda.synchronize()
        c = xcnt.view(xblocks, 4, 2).double()
        for kind, waves in (("read", slice(0, 2)), ("copy", slice(2, 4))):
            r = c[:, waves, 0]
            if float(r.sum()) == 0:
                continue
            cyc = float(c[:, waves, 1].mean())
            out[f"lds_{kind}_{tag}_bytes_per_cu_clk"] = float(r.sum()) * 8192 / cyc / cus
    torch.cuda.synchronize()
    return out


def measure_forward(args, w, dev, flush, ceilings, with_graph=True):
    """One workload's measurement: timed steps (flushed, events, profiling
    off), a profiled pass for per-kernel times, the dominant kernel's
    roofline, and optionally a HIP-graph replay timing.  Returns the dict of
    the workload's JSON fields."""
    import torch

    import ragged_paged_kv_scatter_amd as rpa

    meta = {k: torch.from_numpy(np.ascontiguousarray(getattr(w, k))).to(dev)
            for k in ("kv_lens", "block_tables", "query_start_loc", "distribution")}
    out = torch.empty(w.queries.shape, dtype=rpa.out_dtype_for(w.queries.dtype), device=dev)
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

    progress(f"{w.name}: warm-up")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    rpa.profile_enable(False)
    progress(f"{w.name}: {args.steps} timed steps")
    step_ms, wall_ms = timed_steps(step, args.steps, flush)
    ms = float(np.mean(step_ms))
    nf_ms = back_to_back(step, args.steps)
    # the two halves on their own: attention over the updated cache (no new
    # keys / values), and the update by itself
    def attn_step():
        rpa.rpa_forward(w.queries, None, None, w.kv_cache, meta["kv_lens"],
                        meta["block_tables"], meta["query_start_loc"], meta["distribution"],
                        w.attention_sink, out=out, workspace=workspace, **opts)

    def update_step():
        rpa.rpa_update_kv_cache(w.keys, w.values, w.kv_cache, meta["kv_lens"],
                                meta["block_tables"], meta["query_start_loc"],
                                meta["distribution"], k_scale=w.k_scale, v_scale=w.v_scale,
                                queries_dtype=w.queries.dtype)

    ao_ms = up_ms = None
    if not getattr(args, "no_halves", False):
        progress(f"{w.name}: attention-only and update-only steps")
        for _ in range(max(args.warmup, 1)):
            attn_step()
            update_step()
        ao_ms = float(np.mean(timed_steps(attn_step, args.steps, flush)[0]))
        up_ms = float(np.mean(timed_steps(update_step, args.steps, flush)[0]))
    # per-kernel times: a second pass with the library's launch events
    rpa.profile_enable(True)
    rpa.profile_read()
    timed_steps(step, args.steps, flush)
    rpa.profile_enable(False)
    kstats = rpa.profile_read()

    kvb, flops, row_kvb, pf_flops = work_counts(w, split=True)
    decode_like = w.name not in PREFILL_WORKLOADS
    work = kvb if decode_like else flops
    scale = 1e9 if decode_like else 1e12
    unit = "GB/s" if decode_like else "TFLOP/s"
    value = work / (ms * 1e-3) / scale
    # dominant kernel: of the two attention kernels, the one with the larger
    # summed time among those with work in this batch (on the side-stream path
    # a kernel with no work still spans the other's run while it waits for
    # slots, so it is not a candidate); its roofline is priced on its own
    # algorithmic work: the row kernel's KV bytes, the prefill tiles' FLOPs
    cands = {k: v for k, v in kstats.items()
             if (k == "decode" and row_kvb > 0) or (k == "prefill" and pf_flops > 0)}
    dom_name, (dom_n, dom_ms) = max(cands.items(), key=lambda kv: kv[1][1]) if cands else \
        ("none", (1, 0.0))
    dom_avg_ms = dom_ms / max(dom_n, 1)
    if dom_name == "prefill":
        achieved = pf_flops / (dom_avg_ms * 1e-3) / 1e12
        # e4m3 queries: q.k on fp8 MFMA, p.v on bf16 MFMA (half the FLOPs each)
        peak = FP8_PEAK_TFLOPS if w.q_dtype == "fp8" else BF16_PEAK_TFLOPS
        roof = dict(bound="mfma", achieved=achieved, peak=peak, unit="TFLOP/s",
                    frac=achieved / peak, traffic=None)
        if w.q_dtype == "fp8":
            mixed = 1.0 / (0.5 / FP8_PEAK_TFLOPS + 0.5 / BF16_PEAK_TFLOPS)
            roof["peak_fp8_qk_bf16_pv"] = mixed
            roof["frac_of_fp8_qk_bf16_pv"] = achieved / mixed
        meas = ceilings.get("mfma_bf16_tflops") if ceilings else None
    else:
        achieved = row_kvb / (dom_avg_ms * 1e-3) / 1e9
        roof = dict(bound="hbm", achieved=achieved, peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=achieved / HBM_PEAK_GBS, traffic=None)
        meas = ceilings.get("hbm_read_gbs") if ceilings else None
    roof["kernel"] = dom_name
    roof["kernel_avg_ms"] = dom_avg_ms
    if meas:
        roof["measured_ceiling"] = meas
        roof["frac_of_measured"] = achieved / meas
    # HBM traffic per launch from a committed counter summary, only while the
    # kernel's sources are the ones the counters were taken on
    tf = traffic_file(w.name, dom_name)
    if os.path.exists(tf) and dom_name in KERNEL_SOURCES:
        with open(tf) as fh:
            t = json.load(fh)
        if t.get("kernel") == dom_name and t.get("source_hash") == source_hash(dom_name):
            roof["traffic"] = t["traffic_bytes"]
    res = {
        "value": value, "unit": unit, "ms_per_step": ms,
        "ms_per_step_min": float(np.min(step_ms)),
        "wall_ms_per_step_with_flush": wall_ms,
        "no_flush": {"ms_per_step": nf_ms, "value": work / (nf_ms * 1e-3) / scale},
        "dtype": w.q_dtype,
        "config": {"workload": w.name, "num_seqs": w.num_seqs, "total_tokens": w.total_tokens,
                   "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim, "page_size": w.page_size,
                   "cache_dtype": w.cache_dtype, "kv_bytes": kvb, "flops": flops,
                   "parallelism": "single GPU"},
        "roofline": roof,
        "kernels_ms": {k: v[1] / max(v[0], 1) for k, v in kstats.items()},
        # batches with prefill tiles run the two attention kernels on two
        # streams: a kernel's event span then also covers its wait for CUs
        # that the other stream's kernel holds
        "kernels_on_two_streams": bool(w.total_tokens > w.max_num_seqs),
    }
    if ao_ms is not None:
        res["attention_only"] = {"ms_per_step": ao_ms, "value": work / (ao_ms * 1e-3) / scale,
                                 "unit": unit}
        res["update_only"] = {"ms_per_step": up_ms, "bytes": update_bytes(w),
                              "GB/s": update_bytes(w) / (up_ms * 1e-3) / 1e9}
    if ceilings and pf_flops > 0 and "prefill" in kstats:
        # VALU roof of the prefill kernel: its transcendental count at the
        # measured issue rates (one exp2 per visible logit; with a soft cap
        # also an exp2 and a reciprocal for tanh)
        n_logit = pf_flops / (4 * w.head_dim)
        t_tr = n_logit / ceilings["exp_per_s"]
        if w.logits_soft_cap:
            t_tr += n_logit / ceilings["exp_per_s"] + n_logit / ceilings["rcp_per_s"]
        pk = kstats["prefill"][1] / max(kstats["prefill"][0], 1)
        res["valu_roof"] = {"logits": n_logit,
                            "transcendentals_per_logit": 3 if w.logits_soft_cap else 1,
                            "t_transcendental_ms": t_tr * 1e3,
                            "share_of_prefill_kernel": t_tr * 1e3 / pk if pk else None}
    progress(f"{w.name}: {ms:.4f} ms per step, kernels {res['kernels_ms']}")
    if with_graph and not args.no_graph:
        try:
            res["graph"] = graph_timing(args, step, dev, work, decode_like, unit)
        except Exception as e:  # reported, never fatal: `value` is the eager step
            res["graph"] = dict(error=str(e)[:200])
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_entry(w, args.cpu_budget,
                                                 "kv" if decode_like else "flops", unit)
    del workspace, out
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode_bf16")
    ap.add_argument("--op", default="forward",
                    choices=["forward", "reshape_and_cache", "copy_blocks", "probes", "timeline"],
                    help="forward: the whole step (default; with the default workload the line "
                         "also carries the long-prefill measurement); reshape_and_cache: the "
                         "update's slot-mapping form into split K/V caches, at the workload's "
                         "token count; copy_blocks: 2048 block copies in 8192-block split "
                         "caches of the workload's block shape; probes: the measured ceilings "
                         "(HBM read / copy, bf16 MFMA and shader clock, VALU issue rates); "
                         "timeline: the row kernels' per-wave clock stamps over a few steps "
                         "(needs librpa_timeline.so)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip timing the step replayed from a captured HIP graph")
    ap.add_argument("--no-prefill", action="store_true",
                    help="default workload only: skip the nested long-prefill measurement")
    ap.add_argument("--no-probes", action="store_true", help="skip the probe ceilings")
    ap.add_argument("--no-halves", action="store_true",
                    help="skip the attention-only and update-only timings (counter runs: "
                         "every dispatch of a kernel is then one of the whole step)")
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of oracle time per CPU-baseline run (two runs per workload)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run one device copy of this size first (counter calibration)")
    ap.add_argument("--summarize-counters", nargs=3, metavar=("KERNEL", "FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic_<workload>_<kernel>.json from two rocprofv3 "
                         "--pmc runs")
    args = ap.parse_args()
    if args.summarize_counters:
        k, f, wcsv = args.summarize_counters
        summarize_counters(args.workload, k, f, wcsv, args.calib_copy_mib * 2 ** 20)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the path needs no "
              "collective and shards by kv head or by sequence with no exchange.", file=sys.stderr)
        sys.exit(2)

    if args.op == "timeline":
        # the measurement build, loaded in place of librpa.so
        from ragged_paged_kv_scatter_amd import _lib
        from ragged_paged_kv_scatter_amd.build import TIMELINE_LIB
        _lib.LIB_PATH = TIMELINE_LIB

    import torch

    from ragged_paged_kv_scatter_amd import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.op == "probes":
        line = {"metric": "GPU ceilings (probes)", "n_gpus": 1, "data": "synthetic",
                "ceilings": probe_ceilings(dev, full=True)}
        print(json.dumps(line), flush=True)
        return
    if args.calib_copy_mib:
        src = torch.ones(args.calib_copy_mib * 2 ** 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.op == "timeline":
        bench_timeline(args, W.make(args.workload, device=dev), dev)
        return
    if args.op in ("reshape_and_cache", "copy_blocks"):
        w = W.make(args.workload, device=dev)
        if args.op == "reshape_and_cache":
            bench_reshape_and_cache(args, w, dev)
        else:
            bench_copy_blocks(args, w, dev)
        return
    if not args.no_probes:
        progress("probes")
    ceilings = None if args.no_probes else probe_ceilings(dev)
    flush = Flusher(dev)
    w = W.make(args.workload, device=dev)
    res = measure_forward(args, w, dev, flush, ceilings)
    del w
    torch.cuda.empty_cache()
    line = {"metric": METRIC, "value": res.pop("value"), "unit": res.pop("unit"), "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": res.pop("ms_per_step"),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": res.pop("dtype"), "data": "synthetic"}
    line.update(res)
    if args.workload == "decode_bf16" and not args.no_prefill:
        wp = W.make("prefill_bf16", device=dev)
        pf = measure_forward(args, wp, dev, flush, ceilings)
        pf["metric"] = "ragged paged attn: long prefill TFLOP/s, % of bf16 MFMA roofline"
        line["prefill"] = pf
        del wp
    if ceilings:
        line["ceilings"] = ceilings
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

"""The algorithmic work bench.py prices its rooflines on, checked on the CPU
against closed forms: the tiny batch by hand, causal prefill pair counts, the
window's cap on visible keys, and the split between the two attention
kernels (row kernel: q_len 1 sequences, or all of them for f32; prefill
kernel: the rest)."""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from ragged_paged_kv_scatter_amd import workloads as W  # noqa: E402


def test_tiny_batch_by_hand():
    # q {1,1,5}, kv {9,17,5}: visible pairs 9 + 17 + (1+2+3+4+5) = 41; 4 q heads, D 64
    w = W.make("tiny_fp32")
    kvb, flops, row_kvb, pf_flops = bench.work_counts(w, split=True)
    tok = 2 * 2 * 64 * 4                          # K+V of 2 kv heads, D 64, f32
    assert kvb == (9 + 17 + 5) * tok
    assert flops == 4 * 64 * 41 * 4
    assert row_kvb == kvb and pf_flops == 0       # f32: every row to the row kernel


def test_long_prefill_closed_form():
    w = W.make("prefill_bf16")
    kvb, flops, row_kvb, pf_flops = bench.work_counts(w, split=True)
    n = 8192
    assert flops == 2 * 64 * (n * (n + 1) // 2) * 4 * 128
    assert kvb == 2 * n * 2 * 8 * 128 * 2
    assert row_kvb == 0 and pf_flops == flops


def test_split_partitions_the_step():
    for name in ("decode_bf16", "mixed_bf16", "fp8_full"):
        w = W.make(name, small=True)
        kvb, flops, row_kvb, pf_flops = bench.work_counts(w, split=True)
        q = np.diff(np.asarray(w.query_start_loc))[:w.num_seqs]
        assert 0 <= row_kvb <= kvb and 0 <= pf_flops <= flops
        if (q >= 2).any():
            assert pf_flops > 0
        else:
            assert pf_flops == 0 and row_kvb == kvb
        if (q == 1).any():
            assert row_kvb > 0


def test_window_caps_visible_keys():
    # one decode row with kv 5000 and window 4096 sees 4096 keys
    w = W.build("win", q_lens=[1], kv_lens=[5000], distribution=(1, 0, 0), num_q_heads=8,
                num_kv_heads=1, head_dim=64, page_size=32, q_dtype="bf16", kv_in_dtype="bf16",
                cache_dtype="fp8", softmax_scale=0.125, seed=3, sliding_window=4096,
                k_scale=0.05, v_scale=0.05, rng=np.random.default_rng(3))
    kvb, flops = bench.work_counts(w)
    assert kvb == 4096 * 2 * 1 * 64 * 1
    assert flops == 4 * 64 * 4096 * 8


def test_more_than_one_gpu_is_refused():
    # the path needs no collective; bench.py measures one GPU and says so
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout.strip() == ""


def test_cpu_baseline_fields():
    """The oracle baseline on a tiny batch: positive rate, sequences done
    whole, and the one-thread run really limited to one BLAS thread."""
    w = W.make("tiny_fp32")
    a = bench.cpu_baseline(w, budget_s=0.01)
    assert a["value"] > 0 and a["seqs"] >= 1 and a["rows"] >= 1
    one = bench.cpu_baseline(w, budget_s=0.01, threads=1)
    assert one["threads"] == 1
    p = W.make("prefill_bf16", small=True)
    f = bench.cpu_baseline(p, budget_s=0.01, metric="flops")
    assert f["value"] > 0 and f["rows"] >= 1
    info = bench.cpu_info()
    assert info["cpu_count"] >= 1


def test_update_bytes_closed_form():
    # tiny batch: 7 new tokens, 2 kv heads, D = Dpad = 64, f32 in and out:
    # K and V read (64 x 4 bytes each) and written (64 x 4 bytes each)
    w = W.make("tiny_fp32")
    assert bench.update_bytes(w) == 7 * 2 * 2 * (64 * 4 + 64 * 4)
    # fp8 batch: bf16 keys / values in, e4m3 rows out
    f = W.make("fp8_full", small=True)
    n = int(np.asarray(f.query_start_loc)[f.num_seqs])
    assert bench.update_bytes(f) == n * 2 * 8 * (64 * 2 + 64 * 1)


def test_timeline_summary_by_hand():
    # two CUs (CU ids 0 and 1 of XCD 0), two workgroup slots each; stamps in
    # 100 MHz ticks: every wave starts at 1000, ends 100 us (10000 ticks) or
    # 200 us later depending on its slot
    rows = []
    for cu in (0, 1):
        for slot in (0, 1):
            for _ in range(4):
                hw = (cu << 8) | slot
                end = 1000 + (10000 if slot == 0 else 20000) + cu * 100
                rows.append([1000, 1500, end, (5 << 32) | (0 << 16) | hw])
    rows.append([0, 0, 0, 0])                      # an empty record is skipped
    s = bench.timeline_summary(np.array(rows, dtype=np.uint64))
    assert s["waves"] == 16 and s["cus"] == 2
    assert s["start_us"] == [0.0] * 5
    assert s["end_us"][0] == 100.0 and s["end_us"][-1] == 201.0
    assert s["cu_last_end_us"][0] == 200.0 and s["cu_last_end_us"][-1] == 201.0
    assert s["cu_slot_spread_us"] == [100.0] * 5
    assert s["steps"] == [5, 5, 5]
    assert s["xcd_mean_end_us"] == [150.5]


def test_strip_timeline_removes_only_the_instrumentation():
    src = ("int a;\n#ifdef RPA_WAVE_TIMELINE\n#if X\nint b;\n#endif\nint c;\n#else\n"
           "#define RPA_TL_STEP()\n#endif\nvoid f() {\n  RPA_TL_BEGIN();\n  g();\n"
           "  RPA_TL_END(ch);\n}\n#ifdef OTHER\nint d;\n#endif\n")
    out = " ".join(bench.strip_timeline(src).split())
    assert out == "int a; void f() { g(); } #ifdef OTHER int d; #endif"



def test_pf_timeline_summary_by_hand():
    # two waves: 1000 clocks over 10 steps with 100 waiting on copies and 200
    # at barriers; 3000 clocks over 20 steps with 300 and 900; one empty record
    # (the step parts: issue 50 / q.k 400 / p.v 300 / tail 100 clocks per step
    # on the first wave, twice that on the second)
    a = np.array([[1000, 100, 200, 10, 500, 4000, 3000, 1000],
                  [3000, 300, 900, 20, 2000, 16000, 12000, 4000],
                  [0, 0, 0, 0, 0, 0, 0, 0]], dtype=np.uint64)
    s = bench.pf_timeline_summary(a)
    assert s["issue_clk_per_step"] == 75.0 and s["qk_clk_per_step"] == 600.0
    assert s["pv_clk_per_step"] == 450.0 and s["tail_clk_per_step"] == 150.0
    assert s["waves"] == 2 and s["steps"] == [10, 15, 20]
    assert s["total_clk"] == [1000, 2000, 3000]
    assert s["copy_wait_share"] == 0.1 and s["barrier_wait_share"] == 0.25
    assert s["clk_per_step"] == 125.0
    assert s["copy_wait_clk_per_step"] == 12.5 and s["barrier_wait_clk_per_step"] == 32.5


def test_counter_summary_sums_a_launchs_dispatches(tmp_path, monkeypatch):
    # two steps: each a prefill_kernel dispatch (exits at once, 1 KiB) and a
    # prefill_pair_kernel dispatch (99 KiB), plus a calibration copy of 2 KiB
    # read for 1 MiB copied; split over two instances per counter
    rows = ["Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value"]
    disp = [(1, "copy_kernel", 2.0), (2, "rpa::prefill_kernel<...>", 1.0),
            (3, "rpa::prefill_pair_kernel<...>", 99.0), (4, "rpa::prefill_kernel<...>", 1.0),
            (5, "rpa::prefill_pair_kernel<...>", 99.0), (6, "rpa::row_kernel<...>", 7.0)]
    for name in ("FETCH_SIZE", "WRITE_SIZE"):
        with open(tmp_path / f"{name}.csv", "w") as fh:
            fh.write("\n".join(rows + [f"{i},{k},{name},{v / 2}\n{i},{k},{name},{v / 2}"
                                       for i, k, v in disp]) + "\n")
    monkeypatch.setattr(bench, "traffic_file", lambda w, k: str(tmp_path / "out.json"))
    bench.summarize_counters("prefill_bf16", "prefill", str(tmp_path / "FETCH_SIZE.csv"),
                             str(tmp_path / "WRITE_SIZE.csv"), 1 << 20)
    import json
    with open(tmp_path / "out.json") as fh:
        out = json.load(fh)
    # per launch: (1 + 99) KiB scaled by 1 MiB / 2 KiB
    assert out["fetch"]["launches"] == 2 and out["fetch"]["dispatches"] == 4
    assert out["fetch"]["bytes"] == 100 * 1024 * 512
    assert out["traffic_bytes"] == 2 * 100 * 1024 * 512


def test_committed_traffic_summaries_match_the_kernel_sources():
    """Every committed HBM-traffic summary (profiles/traffic_*.json) was taken
    from the kernel sources as they stand: the bench only reports traffic whose
    source hash matches, and a stale summary would silently drop it."""
    import glob
    import json
    paths = sorted(glob.glob(os.path.join(ROOT, "profiles", "traffic_*.json")))
    assert paths
    for path in paths:
        with open(path) as fh:
            t = json.load(fh)
        assert t["kernel"] in bench.KERNEL_SOURCES, path
        assert t["source_hash"] == bench.source_hash(t["kernel"]), path
        assert t["traffic_bytes"] > 0 and t["fetch"]["launches"] > 0, path

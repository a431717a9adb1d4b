"""rpa_forward captured in a HIP graph: every replay, with eager work between
replays, gives the eager call's output and cache bit for bit (the kernels
take no atomics and record no memset, so a replay is the same launches on
the same buffers)."""
import numpy as np
import pytest
import torch

import ragged_paged_kv_scatter_amd as rpa
from ragged_paged_kv_scatter_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["tiny_fp32", "decode_bf16", "mixed_bf16", "fp8_full"])
def test_graph_replays_match_eager(name):
    print(f"\n[case] graph {name}", flush=True)
    w = W.make(name, device="cuda", small=True)
    meta = {k: torch.from_numpy(np.ascontiguousarray(getattr(w, k))).cuda()
            for k in ("kv_lens", "block_tables", "query_start_loc", "distribution")}
    opts = w.options()
    ws_bytes = rpa.rpa_workspace_bytes(
        rpa._desc(w.queries, rpa._dtype(w.keys), w.kv_cache, meta["kv_lens"],
                  meta["block_tables"]),
        rpa._options(**opts, chunk_prefill_size=None, num_kv_pages_per_block=None,
                     num_queries_per_block=None, vmem_limit_bytes=None))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    cache0 = w.kv_cache.clone()

    def call(out):
        rpa.rpa_forward(w.queries, w.keys, w.values, w.kv_cache, meta["kv_lens"],
                        meta["block_tables"], meta["query_start_loc"], meta["distribution"],
                        w.attention_sink, out=out, workspace=ws, **opts)

    out_e = torch.full(w.queries.shape, float("nan"), dtype=w.queries.dtype, device="cuda")
    call(out_e)
    torch.cuda.synchronize()
    cache_e = w.kv_cache.clone()

    out_g = torch.empty_like(out_e)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):            # warm-up off the capture
        call(out_g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out_g)
    for rep in range(3):
        w.kv_cache.copy_(cache0)             # eager work between replays
        out_g.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        n_valid = int(w.query_start_loc[w.num_seqs])
        assert torch.equal(out_g[:n_valid].view(torch.uint8), out_e[:n_valid].view(torch.uint8)), rep
        assert torch.equal(w.kv_cache.view(torch.uint8), cache_e.view(torch.uint8)), rep


def test_capture_beside_eager_call_on_another_stream():
    """While one stream captures a batch with prefill tiles (whose prefill
    kernel forks onto a side stream), an eager call with prefill tiles from a
    second stream runs inside the capture window.  Side streams belong to
    their caller's stream, so the eager call neither joins the capture nor
    waits on it: its output is the plain eager result, and every replay of the
    graph reproduces the captured call's eager result."""
    print("\n[case] capture beside another stream", flush=True)
    jobs = []
    for seed in (1302, 1303):
        w = W.make("mixed_bf16", device="cuda", small=True, seed=seed)
        meta = {k: torch.from_numpy(np.ascontiguousarray(getattr(w, k))).cuda()
                for k in ("kv_lens", "block_tables", "query_start_loc", "distribution")}
        ws = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
        jobs.append((w, meta, ws, w.kv_cache.clone()))

    def call(j, out):
        w, meta, ws, _ = jobs[j]
        rpa.rpa_forward(w.queries, w.keys, w.values, w.kv_cache, meta["kv_lens"],
                        meta["block_tables"], meta["query_start_loc"], meta["distribution"],
                        w.attention_sink, out=out, workspace=ws, **w.options())

    ref = []
    for j in range(2):
        out = torch.full(jobs[j][0].queries.shape, float("nan"), dtype=torch.bfloat16,
                         device="cuda")
        call(j, out)
        torch.cuda.synchronize()
        ref.append((out.clone(), jobs[j][0].kv_cache.clone()))
        jobs[j][0].kv_cache.copy_(jobs[j][3])
    torch.cuda.synchronize()
    out_g = torch.full_like(ref[0][0], float("nan"))
    out_o = torch.full_like(ref[1][0], float("nan"))
    other = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, capture_error_mode="relaxed"):
        call(0, out_g)
        with torch.cuda.stream(other):
            call(1, out_o)
    other.synchronize()
    n1 = int(jobs[1][0].query_start_loc[jobs[1][0].num_seqs])
    assert torch.equal(out_o[:n1].view(torch.uint8), ref[1][0][:n1].view(torch.uint8))
    assert torch.equal(jobs[1][0].kv_cache.view(torch.uint8), ref[1][1].view(torch.uint8))
    n0 = int(jobs[0][0].query_start_loc[jobs[0][0].num_seqs])
    for rep in range(3):
        jobs[0][0].kv_cache.copy_(jobs[0][3])
        out_g.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g[:n0].view(torch.uint8), ref[0][0][:n0].view(torch.uint8)), rep
        assert torch.equal(jobs[0][0].kv_cache.view(torch.uint8), ref[0][1].view(torch.uint8)), rep

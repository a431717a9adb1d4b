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

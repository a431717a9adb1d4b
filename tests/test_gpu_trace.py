"""RPA_TRACE=1: rpa_forward writes its trace to stderr, the same lines the
host-side rpa_trace_format gives for these sizes, and a last line with the
plan the device made, read back from the workspace."""
import os
import re

import numpy as np
import pytest
import torch

import ragged_paged_kv_scatter_amd as rpa
from ragged_paged_kv_scatter_amd import workloads as W
from tests.helpers import gpu_forward

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["decode_bf16", "mixed_bf16"])
def test_trace_lines_and_plan(name, capfd, monkeypatch):
    print(f"\n[case] trace {name}", flush=True)
    w = W.make(name, device="cuda", small=True)
    monkeypatch.setenv("RPA_TRACE", "1")
    gpu_forward(w)
    torch.cuda.synchronize()
    monkeypatch.setenv("RPA_TRACE", "0")
    gpu_forward(w)                        # "0" switches it off
    torch.cuda.synchronize()
    err = capfd.readouterr().err
    lines = [l for l in err.splitlines() if l.startswith("[rpa] ")]
    print("\n".join(lines), flush=True)
    kv = {k: torch.from_numpy(np.ascontiguousarray(getattr(w, k))).cuda()
          for k in ("kv_lens", "block_tables")}
    d = rpa._desc(w.queries, rpa._dtype(w.keys), w.kv_cache, kv["kv_lens"], kv["block_tables"])
    o = rpa._options(**w.options(), chunk_prefill_size=None, num_kv_pages_per_block=None,
                     num_queries_per_block=None, vmem_limit_bytes=None)
    dry = rpa.rpa_trace_format(d, o, with_update=True).strip().splitlines()
    strip = lambda l: re.sub(r" stream=\S+", "", l)
    assert [strip(l) for l in lines[:-1]] == [strip(l) for l in dry]
    assert lines[-1].startswith("[rpa] plan ")
    plan = dict(f.split("=") for f in lines[-1].split()[2:])
    q_lens = w.q_lens()
    assert int(plan["num_seqs"]) == w.num_seqs
    assert int(plan["rows"]) == int((q_lens == 1).sum())
    assert int(plan["prefill_items"]) == int(sum(-(-int(q) // 128) for q in q_lens if q >= 2))
    assert int(plan["items"]) >= int(plan["rows"]) and int(plan["chunks"]) >= 1

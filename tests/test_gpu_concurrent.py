"""rpa_forward from two host threads at once, each on its own stream with its
own workspace.  Batches with prefill tiles fork the prefill kernel onto the
side stream of their caller's stream, so the two threads' calls use separate
side streams; this checks that interleaved calls still order every call's
work on its own stream: each thread's outputs equal the serial run's bit for
bit (the kernels are deterministic for a fixed plan)."""
import threading

import numpy as np
import pytest
import torch

import ragged_paged_kv_scatter_amd as rpa
from ragged_paged_kv_scatter_amd import workloads as W

pytestmark = pytest.mark.gpu


def _setup(name, seed):
    w = W.make(name, device="cuda", small=True, seed=seed)
    meta = {k: torch.from_numpy(np.ascontiguousarray(getattr(w, k))).cuda()
            for k in ("kv_lens", "block_tables", "query_start_loc", "distribution")}
    return w, meta


def _call(w, meta, out, ws, cache):
    rpa.rpa_forward(w.queries, w.keys, w.values, cache, meta["kv_lens"], meta["block_tables"],
                    meta["query_start_loc"], meta["distribution"], w.attention_sink, out=out,
                    workspace=ws, **w.options())


@pytest.mark.parametrize("profile", [False, True])
@pytest.mark.parametrize("names", [("mixed_bf16", "fp8_full"), ("mixed_bf16", "mixed_bf16")])
def test_two_threads_match_serial(names, profile):
    """With profiling on, each thread's launches are bracketed by its own
    events: every launch of both threads is recorded once, with a positive
    duration."""
    print(f"\n[case] concurrent {names} profile={profile}", flush=True)
    jobs = [_setup(n, seed=900 + i) for i, n in enumerate(names)]
    cache0 = [w.kv_cache.clone() for w, _ in jobs]
    ref = []
    for (w, meta), c0 in zip(jobs, cache0):          # serial reference
        cache = c0.clone()
        out = torch.full(w.queries.shape, float("nan"), dtype=w.queries.dtype, device="cuda")
        _call(w, meta, out, None, cache)
        torch.cuda.synchronize()
        ref.append((out.clone(), cache.clone()))

    reps = 6
    results = [None, None]
    errors = []

    def worker(i):
        try:
            w, meta = jobs[i]
            stream = torch.cuda.Stream()
            outs = []
            with torch.cuda.stream(stream):
                ws = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
                for _ in range(reps):
                    cache = cache0[i].clone()
                    out = torch.full(w.queries.shape, float("nan"), dtype=w.queries.dtype,
                                     device="cuda")
                    _call(w, meta, out, ws, cache)
                    outs.append((out, cache))
            stream.synchronize()
            results[i] = outs
        except Exception as e:  # reported below
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    if profile:
        rpa.profile_enable(True)
        rpa.profile_read()
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not errors, errors
    if profile:
        torch.cuda.synchronize()
        rpa.profile_enable(False)
        stats = rpa.profile_read()
        print(f"[profile] {stats}", flush=True)
        # four launches per call with prefill tiles: plan+scatter, prefill, decode, merge
        for k in ("plan+scatter", "prefill", "decode", "merge"):
            n, ms = stats[k]
            assert n == 2 * reps, (k, n)
            assert ms > 0.0, k
    for i, (w, _) in enumerate(jobs):
        n = int(w.query_start_loc[w.num_seqs])
        for out, cache in results[i]:
            assert torch.equal(out[:n].view(torch.uint8), ref[i][0][:n].view(torch.uint8))
            assert torch.equal(cache.view(torch.uint8), ref[i][1].view(torch.uint8))

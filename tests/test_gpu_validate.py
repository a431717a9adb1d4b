"""rpa_validate_metadata: the device check of the metadata preconditions
(include/rpa.h) against a plain restatement of those preconditions in Python,
bit for bit, on valid batches, on each planted violation, and on random
corruptions of the metadata values (array sizes unchanged, so every read the
kernels make stays inside the arrays)."""
import numpy as np
import pytest
import torch

import ragged_paged_kv_scatter_amd as rpa
from ragged_paged_kv_scatter_amd import workloads as W

pytestmark = pytest.mark.gpu


def expected_bits(kv_lens, bt, qsl, dist, T, pps, ps, num_pages):
    """The preconditions written out: the status word a correct check returns."""
    bits = 0
    max_num_seqs = len(kv_lens)
    total = int(dist[0]) + int(dist[1]) + int(dist[2])
    if min(int(d) for d in dist) < 0 or total > max_num_seqs:
        bits |= rpa.META_DISTRIBUTION
    n = min(max(total, 0), max_num_seqs)
    if qsl[0] != 0 or qsl[n] > T:
        bits |= rpa.META_QSL
    slots = set()
    for s in range(n):
        q0, q1, kv = int(qsl[s]), int(qsl[s + 1]), int(kv_lens[s])
        if q1 < q0:
            bits |= rpa.META_QSL
        q_len = q1 - q0
        bad_len = q_len > kv or kv < 0 or kv > pps * ps
        if bad_len:
            bits |= rpa.META_LENS
        kv_c = min(max(kv, 0), pps * ps)
        row = bt[s * pps:(s + 1) * pps]
        bad_bt = any(not (0 <= int(row[i]) < num_pages) for i in range(-(-kv_c // ps)))
        if bad_bt:
            bits |= rpa.META_BLOCK_TABLE
    # the slots of the new tokens, token by token as the update writes them
    end = min(int(qsl[n]), T) if n else 0
    for t in range(max(end, 0)):
        s = _bisect(qsl, n, t)
        q0, q1, kv = int(qsl[s]), int(qsl[s + 1]), int(kv_lens[s])
        if not (q0 <= t < q1) or (q1 - q0) > kv or kv > pps * ps:
            continue
        pos = kv - (q1 - q0) + (t - q0)
        pg = int(bt[s * pps + pos // ps])
        if not (0 <= pg < num_pages):
            continue
        slot = pg * ps + pos % ps
        if slot in slots:
            bits |= rpa.META_SLOTS
        slots.add(slot)
    # no written slot may hold a context key (positions below kv_len - q_len)
    for s in range(n):
        q0, q1, kv = int(qsl[s]), int(qsl[s + 1]), int(kv_lens[s])
        if q1 < q0 or (q1 - q0) > kv or kv < 0 or kv > pps * ps:
            continue
        for pos in range(kv - (q1 - q0)):
            pg = int(bt[s * pps + pos // ps])
            if 0 <= pg < num_pages and pg * ps + pos % ps in slots:
                bits |= rpa.META_WRITE_IN_CONTEXT
                break
    return bits


def _bisect(qsl, n, t):
    lo, hi = 0, n - 1                     # last s with qsl[s] <= t, as the device searches
    while lo < hi:
        mid = (lo + hi + 1) >> 1
        if qsl[mid] <= t:
            lo = mid
        else:
            hi = mid - 1
    return lo


def run_check(w, kv_lens, bt, qsl, dist):
    dev = "cuda"
    t = {k: torch.from_numpy(np.ascontiguousarray(v, dtype=np.int32)).to(dev)
         for k, v in (("kv", kv_lens), ("bt", bt), ("qsl", qsl), ("dist", dist))}
    status = rpa.rpa_validate_metadata(w.queries, w.kv_cache, t["kv"], t["bt"], t["qsl"],
                                       t["dist"], kv_in_dtype=rpa._dtype(w.keys))
    return int(status.item())


def meta(w):
    return (np.array(w.kv_lens, np.int32).copy(), np.array(w.block_tables, np.int32).copy(),
            np.array(w.query_start_loc, np.int32).copy(), np.array(w.distribution, np.int32).copy())


def sizes(w):
    return dict(T=w.queries.shape[0], pps=w.pages_per_seq, ps=w.page_size,
                num_pages=w.kv_cache.shape[0])


@pytest.mark.parametrize("name", ["tiny_fp32", "decode_bf16", "mixed_bf16", "prefill_bf16",
                                  "fp8_full"])
def test_valid_batches_pass(name):
    print(f"\n[case] validate {name}", flush=True)
    w = W.make(name, device="cuda", small=True)
    kv, bt, qsl, dist = meta(w)
    assert expected_bits(kv, bt, qsl, dist, **sizes(w)) == 0
    assert run_check(w, kv, bt, qsl, dist) == 0


def _plant(w, kind):
    kv, bt, qsl, dist = meta(w)
    n = int(dist.sum())
    qlen = np.diff(qsl[:n + 1])
    pre = int(np.argmax(qlen))                        # the longest query of the batch
    if kind == "qsl_start":
        qsl[0] = 1
    elif kind == "qsl_order":
        qsl[pre + 1] = qsl[pre] - 1
    elif kind == "qsl_past_tokens":
        qsl[n] = w.queries.shape[0] + 1
    elif kind == "q_longer_than_kv":
        kv[pre] = qlen[pre] - 1
    elif kind == "kv_past_table":
        kv[0] = w.pages_per_seq * w.page_size + 1
    elif kind == "block_entry_out_of_pool":
        bt[pre * w.pages_per_seq] = w.kv_cache.shape[0]
    elif kind == "block_entry_negative":
        bt[pre * w.pages_per_seq] = -3
    elif kind == "shared_slot":
        # the longest query's last two pages -> one page: two new tokens per offset collide
        s, ps = pre, w.page_size
        last = (int(kv[s]) - 1) // ps
        bt[s * w.pages_per_seq + last] = bt[s * w.pages_per_seq + last - 1]
    elif kind == "written_slot_in_context":
        # the longest query's first new-token page becomes the first context
        # page of another sequence that has context
        s, ps = pre, w.page_size
        ctx = int(kv[s]) - int(qlen[s])
        other = next(o for o in range(n) if o != s and int(kv[o]) - int(qlen[o]) > 0)
        bt[other * w.pages_per_seq] = bt[s * w.pages_per_seq + ctx // ps]
    elif kind == "distribution_negative":
        dist[1] = -1
        dist[2] += 1
    elif kind == "distribution_past_max":
        dist[2] = len(kv) + 5
    else:
        raise KeyError(kind)
    return kv, bt, qsl, dist


KINDS = {"qsl_start": rpa.META_QSL, "qsl_order": rpa.META_QSL,
         "qsl_past_tokens": rpa.META_QSL, "q_longer_than_kv": rpa.META_LENS,
         "kv_past_table": rpa.META_LENS, "block_entry_out_of_pool": rpa.META_BLOCK_TABLE,
         "block_entry_negative": rpa.META_BLOCK_TABLE, "shared_slot": rpa.META_SLOTS,
         "distribution_negative": rpa.META_DISTRIBUTION,
         "distribution_past_max": rpa.META_DISTRIBUTION,
         "written_slot_in_context": rpa.META_WRITE_IN_CONTEXT}


@pytest.mark.parametrize("kind", list(KINDS))
def test_planted_violation_is_reported(kind):
    print(f"\n[case] validate planted {kind}", flush=True)
    w = W.make("mixed_bf16", device="cuda", small=True)
    kv, bt, qsl, dist = _plant(w, kind)
    want = expected_bits(kv, bt, qsl, dist, **sizes(w))
    assert want & KINDS[kind], "the planted case must violate its precondition"
    got = run_check(w, kv, bt, qsl, dist)
    print(f"[{kind}] status={got:#x} expected={want:#x}", flush=True)
    assert got == want


def test_random_corruptions_match_the_preconditions():
    """Random values written into random metadata entries (sizes unchanged):
    the device status equals the restated preconditions on every trial."""
    print("\n[case] validate random corruptions", flush=True)
    w = W.make("mixed_bf16", device="cuda", small=True)
    rng = np.random.default_rng(424242)
    P = w.kv_cache.shape[0]
    seen = 0
    for trial in range(40):
        kv, bt, qsl, dist = meta(w)
        for _ in range(int(rng.integers(1, 4))):
            which = int(rng.integers(0, 4))
            if which == 0:
                kv[rng.integers(0, len(kv))] = int(rng.integers(-5, w.pages_per_seq * w.page_size + 40))
            elif which == 1:
                bt[rng.integers(0, len(bt))] = int(rng.integers(-2, P + 3))
            elif which == 2:
                qsl[rng.integers(0, len(qsl))] = int(rng.integers(-3, w.queries.shape[0] + 8))
            else:
                dist[rng.integers(0, 3)] = int(rng.integers(-2, len(kv) + 3))
        want = expected_bits(kv, bt, qsl, dist, **sizes(w))
        got = run_check(w, kv, bt, qsl, dist)
        assert got == want, (trial, got, want)
        seen |= want
    print(f"[random] union of reported bits {seen:#x}", flush=True)

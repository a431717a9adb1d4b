"""GPU parity at the extremes of the row kernel's plan.  The planner cuts the
visible key ranges of all decode rows, as one stream, into equal chunks (one
per resident wave and kv head); these cases push that cut to its ends:
  * one very long decode row, cut into over a thousand pieces whose split
    partials the merge combines;
  * thousands of tiny rows, so that a chunk walks many rows' pieces (with the
    planner's per-sequence tables in LDS, and past that cache's size);
  * the f32 path, where every row of a prefill chunk goes to the row kernel
    and the causal rows of one sequence share chunks;
  * thousands of short prefill sequences between decode rows, so that the
    planner's prefill tiles span several blocks of sequences and one block
    holds more tiles than the planner has threads;
  * long rows cut into hundreds of pieces, which a whole wave writes and a
    whole workgroup merges: with sinks, soft cap and an e4m3 cache in the
    prefill kernel's merge; in the stand-alone merge kernel (f32); and beside
    a prefill chunk on the side stream.
Each compares rpa_forward with the oracle to the dtype's tolerance and the
updated cache bit for bit."""
import math

import numpy as np
import pytest
import torch

from ragged_paged_kv_scatter_amd import workloads as W
from tests.helpers import bits, check_output, gpu_forward, oracle_forward, poison_unused

pytestmark = pytest.mark.gpu


def _case(label, seed, device="cuda"):
    rng = np.random.default_rng(seed)
    common = dict(softmax_scale=0.0, seed=seed, device=device, rng=rng)
    if label == "one_long_row":
        # 200000 keys in one decode row next to a short one; Hkv 1 gives the
        # most chunks per kv head
        q_lens, kv_lens = [1, 1], [200_000, int(rng.integers(100, 400))]
        args = dict(num_q_heads=8, num_kv_heads=1, head_dim=64, page_size=16,
                    q_dtype="bf16", kv_in_dtype="bf16", cache_dtype="bf16", distribution=(2, 0, 0))
    elif label in ("tiny_rows_3000", "tiny_rows_4500"):
        n = 3000 if label == "tiny_rows_3000" else 4500
        q_lens = [1] * n
        kv_lens = [int(x) for x in rng.integers(1, 41, size=n)]
        args = dict(num_q_heads=4, num_kv_heads=2, head_dim=128, page_size=16,
                    q_dtype="bf16", kv_in_dtype="bf16", cache_dtype="bf16", distribution=(n, 0, 0))
    elif label == "many_prefill_seqs":
        # 2300 sequences, every fourth a decode row, the rest prefill chunks
        # of 2..300 tokens (1 to 3 tiles) after up to 40 cached tokens
        n = 2300
        q_lens, kv_lens = [], []
        for i in range(n):
            if i % 4 == 0:
                q_lens.append(1)
                kv_lens.append(int(rng.integers(1, 61)))
            else:
                q = int(rng.integers(2, 301))
                q_lens.append(q)
                kv_lens.append(q + int(rng.integers(0, 41)))
        args = dict(num_q_heads=4, num_kv_heads=2, head_dim=64, page_size=16,
                    q_dtype="bf16", kv_in_dtype="bf16", cache_dtype="bf16", distribution=(0, 0, n))
    elif label == "long_row_sink_fp8":
        q_lens, kv_lens = [1, 1], [120_000, int(rng.integers(100, 400))]
        args = dict(num_q_heads=16, num_kv_heads=2, head_dim=64, page_size=32, q_dtype="bf16",
                    kv_in_dtype="bf16", cache_dtype="fp8", distribution=(2, 0, 0),
                    logits_soft_cap=30.0, with_sink=True, k_scale=0.05, v_scale=0.05)
    elif label == "long_row_f32":
        q_lens, kv_lens = [1, 1], [60_000, int(rng.integers(100, 400))]
        args = dict(num_q_heads=4, num_kv_heads=1, head_dim=64, page_size=16, q_dtype="f32",
                    kv_in_dtype="f32", cache_dtype="f32", distribution=(2, 0, 0), with_sink=True)
    elif label == "long_row_beside_prefill":
        q_lens, kv_lens = [1, 300], [100_000, 500]
        args = dict(num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16, q_dtype="bf16",
                    kv_in_dtype="bf16", cache_dtype="bf16", distribution=(1, 1, 0))
    elif label == "f32_prefill_rows":
        q_lens, kv_lens = [300, 1, 5], [5000, 3000, 5]
        args = dict(num_q_heads=4, num_kv_heads=2, head_dim=64, page_size=32,
                    q_dtype="f32", kv_in_dtype="f32", cache_dtype="f32", distribution=(1, 2, 0))
    else:
        raise KeyError(label)
    common["softmax_scale"] = 1 / math.sqrt(args["head_dim"])
    return W.build(label, q_lens=q_lens, kv_lens=kv_lens, **args, **common)


def _workspace(w):
    import ragged_paged_kv_scatter_amd as rpa
    kv_t = torch.from_numpy(np.ascontiguousarray(w.kv_lens)).cuda()
    bt_t = torch.from_numpy(np.ascontiguousarray(w.block_tables)).cuda()
    nbytes = rpa.rpa_workspace_bytes(
        rpa._desc(w.queries, rpa._dtype(w.keys), w.kv_cache, kv_t, bt_t),
        rpa._options(**w.options(), chunk_prefill_size=None, num_kv_pages_per_block=None,
                     num_queries_per_block=None, vmem_limit_bytes=None))
    return torch.zeros(nbytes, dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("label", ["one_long_row", "tiny_rows_3000", "tiny_rows_4500",
                                   "many_prefill_seqs", "long_row_sink_fp8", "long_row_f32",
                                   "long_row_beside_prefill", "f32_prefill_rows"])
def test_plan_extremes_match_oracle(label):
    print(f"\n[case] plan {label}", flush=True)
    w = _case(label, seed=9100 + len(label))
    poison_unused(w)
    before = bits(w.kv_cache, w.cache_dtype)
    ref, ref_cache = oracle_forward(w, cache_bits=before)
    ws = _workspace(w)
    out = gpu_forward(w, workspace=ws)
    torch.cuda.synchronize()
    if label.startswith("long_row"):
        # the long row alone is cut into more than 64 pieces: written by its
        # whole wave and merged by a whole workgroup
        n_items = int(ws[:64].view(torch.int32)[2])
        print(f"[{label}] items={n_items}", flush=True)
        assert n_items > 64 + 2
    np.testing.assert_array_equal(bits(w.kv_cache, w.cache_dtype), ref_cache)
    n_valid = int(w.query_start_loc[w.num_seqs])
    check_output(label, w, out, ref, np.arange(n_valid))


# PlanHeader field order: num_seqs, n_rows, n_items, split, n_merge_rows,
# n_pf_items, row_next, pf_next, n_chunks, co_run
_CO_RUN = 9


def _mode_case(label, seed):
    rng = np.random.default_rng(seed)
    args = dict(num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16, q_dtype="bf16",
                kv_in_dtype="bf16", cache_dtype="bf16", softmax_scale=1 / math.sqrt(128),
                seed=seed, device="cuda", rng=rng)
    if label == "decode_heavy":        # rows' HBM time exceeds the tile's MFMA time
        q_lens = [1] * 32 + [64]
        kv_lens = [int(x) for x in rng.integers(1500, 2500, size=32)] + [164]
        dist = (32, 1, 0)
    elif label == "prefill_heavy":     # one long chunk next to two short decode rows
        q_lens, kv_lens, dist = [1, 1, 512], [50, 60, 1512], (2, 1, 0)
    elif label == "one_stream":        # tokens <= sequences: prefill tile on the caller's stream
        q_lens, kv_lens, dist = [1, 1, 0, 3, 0, 0], [700, 90, 40, 300, 5, 1], (2, 4, 0)
    else:
        raise KeyError(label)
    return W.build(label, q_lens=q_lens, kv_lens=kv_lens, distribution=dist, **args)


@pytest.mark.parametrize("label,co_run", [("decode_heavy", 1), ("prefill_heavy", 0),
                                          ("one_stream", 0)])
def test_side_by_side_modes_match_oracle(label, co_run):
    """Batches with prefill tiles fork the prefill kernel onto a side stream;
    the planner runs it beside the row kernel (each on half of every CU) only
    when the rows' HBM time is at least the tiles' MFMA time.  Every mode
    gives the oracle's output and cache."""
    import ragged_paged_kv_scatter_amd as rpa
    print(f"\n[case] plan mode {label}", flush=True)
    w = _mode_case(label, seed=9300 + len(label))
    poison_unused(w)
    before = bits(w.kv_cache, w.cache_dtype)
    ref, ref_cache = oracle_forward(w, cache_bits=before)
    kv_t = torch.from_numpy(np.ascontiguousarray(w.kv_lens)).cuda()
    bt_t = torch.from_numpy(np.ascontiguousarray(w.block_tables)).cuda()
    nbytes = rpa.rpa_workspace_bytes(
        rpa._desc(w.queries, rpa._dtype(w.keys), w.kv_cache, kv_t, bt_t),
        rpa._options(**w.options(), chunk_prefill_size=None, num_kv_pages_per_block=None,
                     num_queries_per_block=None, vmem_limit_bytes=None))
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    out = gpu_forward(w, workspace=ws)
    torch.cuda.synchronize()
    hdr = ws[:64].view(torch.int32).cpu().numpy()
    assert hdr[5] > 0, "the batch has prefill tiles"
    assert hdr[_CO_RUN] == co_run
    np.testing.assert_array_equal(bits(w.kv_cache, w.cache_dtype), ref_cache)
    n_valid = int(w.query_start_loc[w.num_seqs])
    print(f"[{label}] co_run={hdr[_CO_RUN]}", flush=True)
    check_output(label, w, out, ref, np.arange(n_valid))

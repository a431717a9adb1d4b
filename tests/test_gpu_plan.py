"""GPU parity at the extremes of the row kernel's plan.  The planner cuts the
visible key ranges of all decode rows, as one stream, into equal chunks (one
per resident wave and kv head); these cases push that cut to its ends:
  * one very long decode row, cut into over a thousand pieces whose split
    partials the merge combines;
  * thousands of tiny rows, so that a chunk walks many rows' pieces (with the
    planner's per-sequence tables in LDS, and past that cache's size);
  * the f32 path, where every row of a prefill chunk goes to the row kernel
    and the causal rows of one sequence share chunks.
Each compares rpa_forward with the oracle to the dtype's tolerance and the
updated cache bit for bit."""
import math

import numpy as np
import pytest
import torch

from ragged_paged_kv_scatter_amd import workloads as W
from tests.helpers import bits, gpu_forward, oracle_forward, poison_unused, tolerance

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
    elif label == "f32_prefill_rows":
        q_lens, kv_lens = [300, 1, 5], [5000, 3000, 5]
        args = dict(num_q_heads=4, num_kv_heads=2, head_dim=64, page_size=32,
                    q_dtype="f32", kv_in_dtype="f32", cache_dtype="f32", distribution=(1, 2, 0))
    else:
        raise KeyError(label)
    common["softmax_scale"] = 1 / math.sqrt(args["head_dim"])
    return W.build(label, q_lens=q_lens, kv_lens=kv_lens, **args, **common)


@pytest.mark.parametrize("label", ["one_long_row", "tiny_rows_3000", "tiny_rows_4500",
                                   "f32_prefill_rows"])
def test_plan_extremes_match_oracle(label):
    print(f"\n[case] plan {label}", flush=True)
    w = _case(label, seed=9100 + len(label))
    poison_unused(w)
    before = bits(w.kv_cache, w.cache_dtype)
    ref, ref_cache = oracle_forward(w, cache_bits=before)
    out = gpu_forward(w)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(w.kv_cache, w.cache_dtype), ref_cache)
    n_valid = int(w.query_start_loc[w.num_seqs])
    o = out[:n_valid].double().cpu().numpy()
    err = np.abs(o - ref[:n_valid]).max()
    print(f"[{label}] max_abs={err:.3e} tol={tolerance(w):.0e}", flush=True)
    assert err <= tolerance(w)

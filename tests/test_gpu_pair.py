"""GPU parity of the two-group prefill kernel (bf16 queries over a bf16 cache,
even GQA group): batches of prefill chunks only, which the planner never runs
beside rows, so the two-group kernel takes every tile.  The cases reach its
edges: tiles whose last waves have no query rows (in both groups), keys that
all come from the new rows (no context) or mostly from the cache, page
tables longer than one pass of the workgroup's fill, sliding window, soft
cap, sink, zero and negative scales, head_dim 64 and 128, group sizes 2 to
16, and the update on or off.  Each case compares rpa_forward with the oracle
on NaN-poisoned caches, to the bf16 tolerance, and the cache bit for bit."""
import math

import numpy as np
import pytest
import torch

from ragged_paged_kv_scatter_amd import workloads as W
from tests.helpers import bits, check_output, gpu_forward, oracle_forward, poison_unused

pytestmark = pytest.mark.gpu

# label: (D, Hq, Hkv, page_size, window, cap, sink, scale, q_lens, contexts, update)
CASES = {
    "d128_g2_ps16": (128, 4, 2, 16, 0, 0.0, False, None, [2, 33, 128, 129, 300],
                     [0, 70, 5, 400, 90], True),
    "d64_g8_ps32_cap_window_sink": (64, 16, 2, 32, 75, 12.0, True, None, [64, 97, 250],
                                    [30, 0, 600], True),
    "d128_g4_ps64_zero_scale": (128, 8, 2, 64, 0, 0.0, False, 0.0, [40, 200], [100, 0], True),
    "d128_g4_ps16_negative_scale": (128, 8, 2, 16, 0, 0.0, True, -0.05, [17, 140], [300, 20],
                                    True),
    "d128_g16_hkv1_ps128_window": (128, 16, 1, 128, 150, 0.0, False, None, [300, 1],
                                   [900, 50], True),
    "d64_g2_ps16_long_table": (64, 4, 2, 16, 0, 0.0, False, None, [130, 70], [9000, 3000],
                               True),
    "d128_g8_no_context": (128, 16, 2, 64, 0, 0.0, True, None, [700, 256], [0, 0], True),
    "d128_g8_cache_only": (128, 16, 2, 32, 0, 5.0, False, None, [96, 300], [500, 80], False),
}


def make_case(label, seed):
    D, hq, hkv, ps, win, cap, sink, scale, q_lens, ctx, update = CASES[label]
    # a q_len of 1 would be a decode row: keep the batch prefill-only
    q_lens = [max(q, 2) for q in q_lens]
    rng = np.random.default_rng(seed)
    w = W.build(label, q_lens=q_lens, kv_lens=[q + c for q, c in zip(q_lens, ctx)],
                distribution=(0, len(q_lens), 0), num_q_heads=hq, num_kv_heads=hkv,
                head_dim=D, head_dim_padded=D, page_size=ps, q_dtype="bf16", kv_in_dtype="bf16",
                cache_dtype="bf16", softmax_scale=1 / math.sqrt(D) if scale is None else scale,
                seed=seed, sliding_window=win, logits_soft_cap=cap, with_sink=sink,
                device="cuda", rng=rng)
    return w, update


@pytest.mark.parametrize("label", list(CASES))
def test_pair_kernel_matches_oracle(label):
    print(f"\n[case] pair {label}", flush=True)
    w, update = make_case(label, seed=9400 + list(CASES).index(label))
    poison_unused(w, include_written=update)
    before = bits(w.kv_cache, w.cache_dtype)
    ref, ref_cache = oracle_forward(w, cache_bits=before, update=update)
    out = gpu_forward(w, update=update)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(w.kv_cache, w.cache_dtype), ref_cache)
    n_valid = int(w.query_start_loc[w.num_seqs])
    check_output(f"pair {label}", w, out, ref, np.arange(n_valid))
    assert torch.isnan(out[n_valid:].float()).all()

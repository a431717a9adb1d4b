"""GPU parity on seeded random batches: every case draws a supported dtype
triple, head_dim (with or without lane padding), group size, page size,
sliding window, soft cap, sink, scales (softmax scale now and then zero or
negative) and a batch of decode rows, prefill chunks over contexts and the
odd empty query, in random order, with and without the update.  Each case
compares rpa_forward with the oracle on NaN-poisoned caches, to the dtype's
tolerance, and the updated cache bit for bit; rows past the batch stay NaN.
The draws are fixed by the case's seed, so a failure names a reproducible
batch."""
import math

import numpy as np
import pytest
import torch

from ragged_paged_kv_scatter_amd import workloads as W
from tests.helpers import bits, check_output, gpu_forward, oracle_forward, poison_unused

pytestmark = pytest.mark.gpu

TRIPLES = [("f32", "f32", "f32"), ("bf16", "bf16", "bf16"), ("bf16", "bf16", "fp8"),
           ("bf16", "fp8", "fp8"), ("fp8", "bf16", "fp8"), ("fp8", "fp8", "fp8")]
ELEM = {"f32": 4, "bf16": 2, "fp8": 1}


def draw_case(seed, device="cuda"):
    rng = np.random.default_rng(seed)
    qd, kd, cd = TRIPLES[int(rng.integers(len(TRIPLES)))]
    D = int(rng.choice([64, 128]))
    Dpad = D + (16 if rng.random() < 0.2 else 0)          # multiple of 16 elements
    hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 4, 8, 16]))
    while hkv * G > 64:
        G //= 2
    ps = int(rng.choice([16, 32, 64, 128]))
    window = int(rng.integers(1, 400)) if rng.random() < 0.4 else 0
    cap = float(rng.uniform(1.0, 50.0)) if rng.random() < 0.4 else 0.0
    sink = bool(rng.random() < 0.4)
    r = rng.random()
    scale = 0.0 if r < 0.05 else (-float(rng.uniform(0.01, 0.2)) if r < 0.1 else 1 / math.sqrt(D))
    fp8 = cd == "fp8"
    q_scale = float(rng.uniform(0.02, 0.1)) if qd == "fp8" else (0.5 if rng.random() < 0.1 else 0.0)
    k_scale = float(rng.uniform(0.02, 0.2)) if fp8 else 0.0
    v_scale = float(rng.uniform(0.02, 0.2)) if fp8 else 0.0
    n = int(rng.integers(1, 11))
    q_lens, kv_lens = [], []
    for _ in range(n):
        u = rng.random()
        if u < 0.55:
            q = 1
        elif u < 0.6:
            q = 0
        else:
            q = int(rng.integers(2, 160))
        ctx = int(rng.integers(0, 600)) if rng.random() < 0.8 else int(rng.integers(600, 2500))
        if q == 0 and ctx == 0:
            ctx = 1
        q_lens.append(q)
        kv_lens.append(ctx + q)
    n_dec = sum(1 for q in q_lens if q == 1)
    w = W.build(f"rand{seed}", q_lens=q_lens, kv_lens=kv_lens, distribution=(n_dec, n - n_dec, 0),
                num_q_heads=hkv * G, num_kv_heads=hkv, head_dim=D, head_dim_padded=Dpad,
                page_size=ps, q_dtype=qd, kv_in_dtype=kd, cache_dtype=cd, softmax_scale=scale,
                seed=seed, sliding_window=window, logits_soft_cap=cap, q_scale=q_scale,
                k_scale=k_scale, v_scale=v_scale, with_sink=sink,
                extra_seqs=int(rng.integers(0, 2)), extra_tokens=int(rng.integers(0, 3)),
                device=device, rng=rng)
    update = bool(rng.random() < 0.8)
    desc = (f"{qd}/{kd}/{cd} D{D}/{Dpad} Hkv{hkv} G{G} ps{ps} W{window} cap{cap:.1f} "
            f"sink{int(sink)} scale{scale:.3f} q_lens{q_lens} kv_lens{kv_lens} update{int(update)}")
    return w, update, desc


@pytest.mark.parametrize("seed", list(range(9100, 9200)))
def test_random_batch_matches_oracle(seed):
    w, update, desc = draw_case(seed)
    print(f"\n[case] random {seed}: {desc}", flush=True)
    poison_unused(w, include_written=update)
    before = bits(w.kv_cache, w.cache_dtype)
    ref, ref_cache = oracle_forward(w, cache_bits=before, update=update)
    out = gpu_forward(w, update=update)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(w.kv_cache, w.cache_dtype), ref_cache)
    n_valid = int(w.query_start_loc[w.num_seqs])
    check_output(f"random {seed}", w, out, ref, np.arange(n_valid))
    assert torch.isnan(out[n_valid:].float()).all()

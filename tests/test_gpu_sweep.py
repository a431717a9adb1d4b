"""GPU parity over a sweep of shapes and options the named workloads do not
reach: every supported dtype triple, head_dim 64 / 128 (with and without lane
padding), group sizes 1 to 16, page sizes 16 to 128, sliding window, soft cap,
sink and q / k / v scales, on batches mixing decode rows, prefill chunks of
awkward lengths, a zero-length query and long contexts that split.  Each case
compares rpa_forward with the oracle on NaN-poisoned caches, to the dtype's
tolerance, and the updated cache bit for bit."""
import math

import numpy as np
import pytest
import torch

from ragged_paged_kv_scatter_amd import workloads as W
from tests.helpers import bits, check_output, gpu_forward, oracle_forward, poison_unused

pytestmark = pytest.mark.gpu

# label: (q, kv_in, cache, D, Dpad, Hq, Hkv, page_size, window, cap, sink, (q, k, v) scales)
CASES = {
    "f32_g1_d64_ps16": ("f32", "f32", "f32", 64, 64, 2, 2, 16, 0, 0.0, False, (0, 0, 0)),
    "f32_g16_d128_ps32_window_sink": ("f32", "f32", "f32", 128, 128, 16, 1, 32, 40, 0.0, True,
                                      (0, 0, 0)),
    "bf16_g1_d128_ps64": ("bf16", "bf16", "bf16", 128, 128, 4, 4, 64, 0, 0.0, False, (0, 0, 0)),
    "bf16_g2_d64_ps128_cap": ("bf16", "bf16", "bf16", 64, 64, 4, 2, 128, 0, 5.0, False,
                              (0, 0, 0)),
    "bf16_g8_d128_ps16_all": ("bf16", "bf16", "bf16", 128, 128, 16, 2, 16, 64, 8.0, True,
                              (0, 0, 0)),
    "bf16_g16_d64_ps32_padded": ("bf16", "bf16", "bf16", 64, 96, 16, 1, 32, 0, 0.0, True,
                                 (0, 0, 0)),
    "bf16_g4_d128_qscale": ("bf16", "bf16", "bf16", 128, 128, 8, 2, 16, 0, 0.0, False,
                            (0.5, 0, 0)),
    "fp8_g4_d128_ps16_scales": ("bf16", "bf16", "fp8", 128, 128, 8, 2, 16, 0, 0.0, False,
                                (0, 0.07, 0.03)),
    "fp8_g8_d64_ps64_window_cap": ("bf16", "bf16", "fp8", 64, 64, 16, 2, 64, 50, 10.0, True,
                                   (0, 0.05, 0.05)),
    "fp8in_g2_d128_ps32": ("bf16", "fp8", "fp8", 128, 128, 4, 2, 32, 0, 0.0, False,
                           (0, 0.1, 0.2)),
    # e4m3 queries (q_scale dequantises them) over an e4m3 cache
    "fp8q_g8_d128_ps32_all": ("fp8", "bf16", "fp8", 128, 128, 16, 2, 32, 100, 20.0, True,
                              (0.05, 0.05, 0.05)),
    "fp8q_g2_d64_ps16": ("fp8", "fp8", "fp8", 64, 64, 4, 2, 16, 0, 0.0, False,
                         (0.05, 0.1, 0.2)),
    "fp8q_g16_d64_ps64_padded_cap": ("fp8", "bf16", "fp8", 64, 80, 16, 1, 64, 0, 5.0, False,
                                     (0.03, 0.05, 0.05)),
    "fp8q_g4_d128_ps128_window_sink": ("fp8", "bf16", "fp8", 128, 128, 8, 2, 128, 37, 0.0, True,
                                       (0.02, 0.04, 0.06)),
    "fp8q_g1_d128_ps16": ("fp8", "fp8", "fp8", 128, 128, 2, 2, 16, 0, 0.0, False,
                          (0.05, 0.05, 0.05)),
    # kv heads a multiple of 4 with G >= 8: the MFMA row kernel's shared
    # 4-head loads (the long row crosses 64-page windows at page_size 16)
    "bf16_g8_d128_hkv4_ps16_sh": ("bf16", "bf16", "bf16", 128, 128, 32, 4, 16, 0, 0.0, False,
                                  (0, 0, 0)),
    "bf16_g16_d64_hkv4_ps128_sh": ("bf16", "bf16", "bf16", 64, 64, 64, 4, 128, 0, 0.0, True,
                                   (0, 0, 0)),
    "fp8_g16_d64_hkv4_window_sink_sh": ("bf16", "bf16", "fp8", 64, 64, 64, 4, 16, 200, 0.0, True,
                                        (0, 0.05, 0.05)),
    "fp8q_g8_d64_hkv8_cap_sh": ("fp8", "bf16", "fp8", 64, 64, 64, 8, 64, 0, 10.0, False,
                                (0.05, 0.05, 0.05)),
    "fp8_g8_d128_hkv8_sh": ("bf16", "fp8", "fp8", 128, 128, 64, 8, 32, 0, 0.0, False,
                            (0, 0.1, 0.1)),
}


def make_case(label, seed, device="cuda"):
    (qd, kd, cd, D, dp, hq, hkv, ps, win, cap, sink, (qs, ks, vs)) = CASES[label]
    rng = np.random.default_rng(seed)
    # decode rows (one with a long context, split into several KV ranges), a
    # zero-length query, then prefill chunks of awkward lengths over contexts
    dec_kv = [int(rng.integers(1, 300)), 1400, int(rng.integers(300, 700))]
    q_lens = [1, 1, 1, 0]
    kv_lens = dec_kv + [int(rng.integers(1, 60))]
    for q in (2, 17, 130, 257):
        q_lens.append(q)
        kv_lens.append(q + int(rng.integers(0, 300)))
    return W.build(label, q_lens=q_lens, kv_lens=kv_lens, distribution=(3, 5, 0),
                   num_q_heads=hq, num_kv_heads=hkv, head_dim=D, head_dim_padded=dp,
                   page_size=ps, q_dtype=qd, kv_in_dtype=kd, cache_dtype=cd,
                   softmax_scale=1 / math.sqrt(D), seed=seed, sliding_window=win,
                   logits_soft_cap=cap, q_scale=qs, k_scale=ks, v_scale=vs, with_sink=sink,
                   extra_seqs=1, extra_tokens=2, device=device, rng=rng)


@pytest.mark.parametrize("label", list(CASES))
def test_sweep_case_matches_oracle(label):
    print(f"\n[case] sweep {label}", flush=True)
    w = make_case(label, seed=7000 + list(CASES).index(label))
    poison_unused(w)
    before = bits(w.kv_cache, w.cache_dtype)
    ref, ref_cache = oracle_forward(w, cache_bits=before)
    out = gpu_forward(w)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(w.kv_cache, w.cache_dtype), ref_cache)
    n_valid = int(w.query_start_loc[w.num_seqs])
    check_output(label, w, out, ref, np.arange(n_valid))
    assert torch.isnan(out[n_valid:].float()).all()


# Soft cap at head_dim 64 over the range of x = s * scale / cap: deep in the
# saturated part of tanh, around its bend, and in its near-linear part.
CAP_CASES = {
    "saturated": (1.0, 1.0),         # (cap, softmax_scale): |x| ~ 8
    "bend": (30.0, 1.0),             # x ~ N(0, 0.27)
    "linear": (30.0, 0.125),         # x ~ N(0, 0.03)
}


@pytest.mark.parametrize("cache", ["bf16", "fp8"])
@pytest.mark.parametrize("label", list(CAP_CASES))
def test_soft_cap_paths_d64(label, cache):
    print(f"\n[case] soft cap {label} {cache}", flush=True)
    cap, scale = CAP_CASES[label]
    seed = 7300 + list(CAP_CASES).index(label) + (10 if cache == "fp8" else 0)
    rng = np.random.default_rng(seed)
    q_lens = [1, 1, 90, 200]
    kv_lens = [int(rng.integers(50, 400)), 700, 90 + int(rng.integers(0, 200)), 350]
    scales = (0.05, 0.05) if cache == "fp8" else (0.0, 0.0)
    w = W.build(label, q_lens=q_lens, kv_lens=kv_lens, distribution=(2, 2, 0), num_q_heads=16,
                num_kv_heads=2, head_dim=64, page_size=32, q_dtype="bf16", kv_in_dtype="bf16",
                cache_dtype=cache, softmax_scale=scale, seed=seed, logits_soft_cap=cap,
                k_scale=scales[0], v_scale=scales[1], device="cuda", rng=rng)
    poison_unused(w)
    before = bits(w.kv_cache, w.cache_dtype)
    ref, ref_cache = oracle_forward(w, cache_bits=before)
    out = gpu_forward(w)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(w.kv_cache, w.cache_dtype), ref_cache)
    n_valid = int(w.query_start_loc[w.num_seqs])
    check_output(f"cap {label} {cache}", w, out, ref, np.arange(n_valid))


# Non-positive softmax scales (any finite scale is accepted): 0 gives every
# visible key equal weight, a negative scale inverts the ranking.  Each case
# has decode rows and causal prefill chunks, so the row kernels (VALU for
# G = 2 / 4, MFMA for G = 8) and the prefill kernel's masked diagonal blocks
# all see the scale.
SCALE_CASES = {
    # label: (q, cache, D, Hq, Hkv, page_size, cap, window, sink)
    "f32_g2": ("f32", "f32", 64, 4, 2, 16, 0.0, 0, False),
    "bf16_g4": ("bf16", "bf16", 128, 8, 2, 32, 0.0, 0, True),
    "bf16_g8_cap": ("bf16", "bf16", 64, 16, 2, 16, 5.0, 40, False),
    "fp8_g8": ("bf16", "fp8", 64, 16, 2, 32, 0.0, 0, False),
    "fp8_g4_cap": ("bf16", "fp8", 128, 8, 2, 64, 8.0, 0, True),
    "fp8q_g8": ("fp8", "fp8", 128, 16, 2, 32, 0.0, 0, False),
    "fp8q_g2_cap": ("fp8", "fp8", 64, 4, 2, 16, 4.0, 0, True),
}


@pytest.mark.parametrize("scale", [0.0, -0.09])
@pytest.mark.parametrize("label", list(SCALE_CASES))
def test_nonpositive_softmax_scale(label, scale):
    print(f"\n[case] scale {scale} {label}", flush=True)
    qd, cd, D, hq, hkv, ps, cap, win, sink = SCALE_CASES[label]
    seed = 7400 + list(SCALE_CASES).index(label) + (50 if scale else 0)
    rng = np.random.default_rng(seed)
    q_lens = [1, 1, 1, 70, 129]
    kv_lens = [int(rng.integers(2, 200)), 900, int(rng.integers(200, 500)),
               70 + int(rng.integers(0, 100)), 129]
    scales = (0.05, 0.05) if cd == "fp8" else (0.0, 0.0)
    w = W.build(label, q_lens=q_lens, kv_lens=kv_lens, distribution=(3, 2, 0),
                num_q_heads=hq, num_kv_heads=hkv, head_dim=D, page_size=ps, q_dtype=qd,
                kv_in_dtype=qd, cache_dtype=cd, softmax_scale=scale, seed=seed,
                logits_soft_cap=cap, sliding_window=win, with_sink=sink, k_scale=scales[0],
                v_scale=scales[1], device="cuda", rng=rng)
    poison_unused(w)
    before = bits(w.kv_cache, w.cache_dtype)
    ref, ref_cache = oracle_forward(w, cache_bits=before)
    out = gpu_forward(w)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(w.kv_cache, w.cache_dtype), ref_cache)
    n_valid = int(w.query_start_loc[w.num_seqs])
    check_output(f"scale {scale} {label}", w, out, ref, np.arange(n_valid))

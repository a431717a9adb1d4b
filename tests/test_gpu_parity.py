"""GPU parity: rpa_forward / rpa_update_kv_cache through the C ABI vs the CPU
oracle on the same seeded inputs.

* KV cache: bit-exact (every written slot equals the oracle's encoding,
  every other byte unchanged).
* Attention output: max abs error within 1e-5 (fp32), 2e-2 (bf16),
  6e-2 (fp8 KV); rows past qsl[num_seqs] untouched.
Unused cache slots are NaN-poisoned, so any read outside a visible range
shows up as NaN in the output."""
import numpy as np
import pytest
import torch

from oracle import rpa_oracle as O
from ragged_paged_kv_scatter_amd import workloads as W
from tests.helpers import (bits, check_output, compact_pages, gpu_forward, oracle_forward,
                           poison_unused)

pytestmark = pytest.mark.gpu
NAMES = ["tiny_fp32", "decode_bf16", "mixed_bf16", "prefill_bf16", "fp8_full", "long_decode_bf16",
         "prefill_fp8q", "mixed_fp8q"]


@pytest.mark.parametrize("name", NAMES)
def test_small_workloads_match_oracle(name):
    print(f"\n[case] small {name}", flush=True)
    w = W.make(name, device="cuda", small=True, extra_seqs=2, extra_tokens=3)
    poison_unused(w)
    before = bits(w.kv_cache, w.cache_dtype)
    ref, ref_cache = oracle_forward(w, cache_bits=before)
    out = gpu_forward(w)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(w.kv_cache, w.cache_dtype), ref_cache)
    n_valid = int(w.query_start_loc[w.num_seqs])
    check_output(name, w, out, ref, np.arange(n_valid))
    assert torch.isnan(out[n_valid:].float()).all()


@pytest.mark.parametrize("name", NAMES)
def test_attention_only_over_updated_cache(name):
    """keys = values = NULL: attention over a cache already holding the step's
    tokens gives the same rows as the fused call."""
    print(f"\n[case] attention-only {name}", flush=True)
    w = W.make(name, device="cuda", small=True)
    poison_unused(w, include_written=False)
    before = bits(w.kv_cache, w.cache_dtype)
    ref, _ = oracle_forward(w, cache_bits=before, update=False)
    out = gpu_forward(w, update=False)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(w.kv_cache, w.cache_dtype), before)
    n_valid = int(w.query_start_loc[w.num_seqs])
    check_output(name, w, out, ref, np.arange(n_valid))


def _sub_workload(w, seqs, cache_bits, bt_compact):
    """The sampled sequences as a batch of their own (renumbered 0..k-1, their
    query rows gathered, block table on the compact pool) -- test-side
    plumbing so the oracle only touches those sequences."""
    pps = w.pages_per_seq
    rows, qsl, kvl, bt = [], [0], [], []
    for s in seqs:
        q0, ql, _, kv = O.seq_bounds(w.query_start_loc, w.kv_lens, s)
        rows.append(np.arange(q0, q0 + ql))
        qsl.append(qsl[-1] + ql)
        kvl.append(kv)
        bt.append(bt_compact[s * pps:(s + 1) * pps])
    rows = np.concatenate(rows).astype(np.int64)
    return dict(rows=rows, qsl=np.array(qsl, np.int32), kv_lens=np.array(kvl, np.int32),
                bt=np.concatenate(bt).astype(np.int32),
                dist=np.array([0, 0, len(seqs)], np.int32), cache=cache_bits)


def _written_pages(w):
    """The pages holding the slots the update writes, and a block table
    renumbered onto that compact pool in the entries that cover the new
    tokens (the only entries the update reads; the others are 0)."""
    pps, ps = w.pages_per_seq, w.page_size
    bt = np.zeros_like(w.block_tables)
    pages, index = [], {}
    for s in range(w.num_seqs):
        _, ql, ctx, kvl = O.seq_bounds(w.query_start_loc, w.kv_lens, s)
        if ql == 0:
            continue
        for i in range(ctx // ps, (kvl - 1) // ps + 1):
            p = int(w.block_tables[s * pps + i])
            if p not in index:
                index[p] = len(pages)
                pages.append(p)
            bt[s * pps + i] = index[p]
    return np.array(pages, dtype=np.int64), bt


def _full_check(w, n_sample_seqs, rows_per_seq, seed):
    rng = np.random.default_rng(seed)
    n = w.num_seqs
    seqs = sorted(set(rng.choice(n, size=min(n_sample_seqs, n), replace=False).tolist()) |
                  {int(np.argmax(w.kv_lens[:n])), n - 1})
    written = O.written_slots(w.kv_lens, w.block_tables, w.query_start_loc, w.distribution,
                              page_size=w.page_size, pages_per_seq=w.pages_per_seq,
                              num_pages=w.num_pages)
    written_t = torch.from_numpy(written.reshape(-1)).to(w.kv_cache.device)
    cache_before_dev = w.kv_cache.clone()
    sub_cache, sub_bt = compact_pages(w, seqs)
    wpages, wbt = _written_pages(w)
    wpages_t = torch.from_numpy(wpages).to(w.kv_cache.device)
    written_before = bits(cache_before_dev.index_select(0, wpages_t), w.cache_dtype)
    out = gpu_forward(w)
    torch.cuda.synchronize()
    # 1) cache bytes outside the written slots unchanged (whole pool, on device)
    rows_a = w.kv_cache.view(w.num_pages * w.page_size, -1).view(torch.uint8)
    rows_b = cache_before_dev.view(w.num_pages * w.page_size, -1).view(torch.uint8)
    assert torch.equal(rows_a[~written_t], rows_b[~written_t])
    del cache_before_dev, rows_b
    # 2) every written slot, bit for bit: the oracle's update of the whole
    #    batch applied to the pages that hold written slots
    exp_written = O.update_kv_cache(written_before, bits(w.keys, w.kv_in_dtype),
                                    bits(w.values, w.kv_in_dtype), w.kv_lens, wbt,
                                    w.query_start_loc, w.distribution, page_size=w.page_size,
                                    pages_per_seq=w.pages_per_seq, kv_in_dtype=w.kv_in_dtype,
                                    cache_dtype=w.cache_dtype, k_scale=w.k_scale,
                                    v_scale=w.v_scale)
    np.testing.assert_array_equal(bits(w.kv_cache.index_select(0, wpages_t), w.cache_dtype),
                                  exp_written)
    print(f"[cache] {int(written.sum())} written slots on {len(wpages)} pages bit-exact",
          flush=True)
    del exp_written, written_before
    # 3) sampled sequences through the oracle, as a batch of their own
    sw = _sub_workload(w, seqs, sub_cache, sub_bt)
    q_bits = bits(w.queries, w.q_dtype)[sw["rows"]]
    k_bits = bits(w.keys, w.kv_in_dtype)[sw["rows"]]
    v_bits = bits(w.values, w.kv_in_dtype)[sw["rows"]]
    exp_cache = O.update_kv_cache(sw["cache"], k_bits, v_bits, sw["kv_lens"], sw["bt"],
                                  sw["qsl"], sw["dist"], page_size=w.page_size,
                                  pages_per_seq=w.pages_per_seq, kv_in_dtype=w.kv_in_dtype,
                                  cache_dtype=w.cache_dtype, k_scale=w.k_scale,
                                  v_scale=w.v_scale)
    sink = None if w.attention_sink is None else w.attention_sink.cpu().numpy()
    ref = np.full(tuple(w.queries.shape), np.nan)
    checked = []
    for i, s in enumerate(seqs):
        q0s, ql, ctx, kvl = O.seq_bounds(sw["qsl"], sw["kv_lens"], i)
        k, v = O.gather_kv(exp_cache, i, kvl, sw["bt"], page_size=w.page_size,
                           pages_per_seq=w.pages_per_seq, head_dim=w.head_dim,
                           cache_dtype=w.cache_dtype, k_scale=w.k_scale, v_scale=w.v_scale)
        ts = np.arange(ql) if ql <= rows_per_seq else np.unique(
            np.concatenate([[0, ql - 1], rng.choice(ql, rows_per_seq, replace=False)]))
        for t in ts:
            q = O.to_f64(q_bits[q0s + t:q0s + t + 1], w.q_dtype)
            orig = int(sw["rows"][q0s + t])
            ref[orig] = O.attend_sequence(q, k, v, ctx + t, softmax_scale=w.softmax_scale,
                                          sliding_window=w.sliding_window,
                                          logits_soft_cap=w.logits_soft_cap, q_scale=w.q_scale,
                                          sink=sink)[0]
            checked.append(orig)
    return out, ref, np.array(checked)


def _with(w, **kw):
    import copy
    c = copy.copy(w)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


FULL = [("tiny_fp32", 3, 8), ("decode_bf16", 24, 1), ("mixed_bf16", 12, 24),
        ("prefill_bf16", 2, 24), ("fp8_full", 12, 24), ("long_decode_bf16", 1, 1),
        ("prefill_fp8q", 2, 24), ("mixed_fp8q", 12, 24)]


@pytest.mark.parametrize("name,n_seqs,rows_per_seq", FULL)
def test_full_size_sampled(name, n_seqs, rows_per_seq):
    print(f"\n[case] full {name}", flush=True)
    w = W.make(name, device="cuda")
    poison_unused(w)
    out, ref, rows = _full_check(w, n_seqs, rows_per_seq, seed=7)
    check_output(name, w, out, ref, rows)
    n_valid = int(w.query_start_loc[w.num_seqs])
    assert not torch.isnan(out[:n_valid].float()).any()


@pytest.mark.parametrize("name", ["decode_bf16", "mixed_bf16", "fp8_full", "mixed_fp8q"])
def test_page_permutation_bitwise_invariance(name):
    """Same logical cache on two different page permutations: identical
    output bits (the plan depends only on lengths, not on page ids)."""
    print(f"\n[case] page permutation {name}", flush=True)
    w = W.make(name, device="cuda", small=True)
    out1 = gpu_forward(w, update=False)
    perm = torch.randperm(w.num_pages, generator=torch.Generator().manual_seed(3))
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(w.num_pages)
    cache2 = torch.empty_like(w.kv_cache)
    cache2[perm.cuda()] = w.kv_cache          # page p moves to perm[p]
    w2 = _with(w, kv_cache=cache2,
               block_tables=perm.numpy()[w.block_tables].astype(np.int32))
    out2 = gpu_forward(w2, update=False)
    torch.cuda.synchronize()
    n_valid = int(w.query_start_loc[w.num_seqs])
    assert torch.equal(out1[:n_valid].view(torch.int16 if out1.dtype == torch.bfloat16
                                           else torch.int32),
                       out2[:n_valid].view(torch.int16 if out2.dtype == torch.bfloat16
                                           else torch.int32))


@pytest.mark.parametrize("name", ["mixed_bf16", "fp8_full", "mixed_fp8q"])
def test_value_sensitivity_one_hot_positions(name):
    """V rows set to one-hot codes of their absolute position: a misread page
    moves weight to the wrong position and shows as an O(1) error."""
    print(f"\n[case] one-hot V {name}", flush=True)
    w = W.make(name, device="cuda", small=True)
    D = w.head_dim
    view = w.kv_cache.view(w.num_pages, w.page_size, 2 * w.num_kv_heads, -1)
    for s in range(w.num_seqs):
        kvl = int(w.kv_lens[s])
        for j in range(kvl):
            p = int(w.block_tables[s * w.pages_per_seq + j // w.page_size])
            val = torch.zeros(view.shape[-1], dtype=torch.float32)
            val[j % D] = 1.0
            if w.cache_dtype == "fp8":
                sc = w.v_scale if w.v_scale else 1.0
                code = torch.clamp(val / sc, -448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
                view[p, j % w.page_size, 1::2, :] = code.cuda()
            else:
                view[p, j % w.page_size, 1::2, :] = val.to(view.dtype).cuda()
    before = bits(w.kv_cache, w.cache_dtype)
    out = gpu_forward(w, update=False, softmax_scale=1.0)
    ref, _ = oracle_forward(_with(w, softmax_scale=1.0), cache_bits=before, update=False)
    torch.cuda.synchronize()
    n_valid = int(w.query_start_loc[w.num_seqs])
    check_output(name + "-onehot", w, out, ref, np.arange(n_valid))


def test_update_only_entry_point_bit_exact():
    import ragged_paged_kv_scatter_amd as rpa
    print("\n[case] update only fp8", flush=True)
    w = W.make("fp8_full", device="cuda", small=True)
    before = bits(w.kv_cache, "fp8")
    exp = O.update_kv_cache(before, bits(w.keys, "bf16"), bits(w.values, "bf16"), w.kv_lens,
                            w.block_tables, w.query_start_loc, w.distribution,
                            page_size=w.page_size, pages_per_seq=w.pages_per_seq,
                            kv_in_dtype="bf16", cache_dtype="fp8", k_scale=w.k_scale,
                            v_scale=w.v_scale)
    meta = [torch.from_numpy(getattr(w, k)).cuda() for k in
            ("kv_lens", "block_tables", "query_start_loc", "distribution")]
    rpa.rpa_update_kv_cache(w.keys, w.values, w.kv_cache, *meta, k_scale=w.k_scale,
                            v_scale=w.v_scale)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(w.kv_cache, "fp8"), exp)


def test_fp8_encoder_extremes_bit_exact():
    """Keys chosen on the e4m3 rounding boundaries (ties, subnormals, the
    448 clamp, signed zero) go through the fused quantising update."""
    import ragged_paged_kv_scatter_amd as rpa
    print("\n[case] fp8 encoder extremes", flush=True)
    w = W.build("fp8edge", q_lens=[64], kv_lens=[64], distribution=(0, 1, 0), num_q_heads=8,
                num_kv_heads=8, head_dim=64, page_size=16, q_dtype="bf16", kv_in_dtype="bf16",
                cache_dtype="fp8", softmax_scale=0.125, k_scale=1.0, v_scale=0.5, seed=5,
                device="cuda")
    pats = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    vals = pats.view(torch.bfloat16).float()
    finite = torch.isfinite(vals)
    vals = vals[finite].to(torch.bfloat16)
    n = w.keys.numel()
    reps = (n + vals.numel() - 1) // vals.numel()
    w.keys = vals.repeat(reps)[:n].view(w.keys.shape).cuda().contiguous()
    w.values = vals.flip(0).repeat(reps)[:n].view(w.values.shape).cuda().contiguous()
    before = bits(w.kv_cache, "fp8")
    exp = O.update_kv_cache(before, bits(w.keys, "bf16"), bits(w.values, "bf16"), w.kv_lens,
                            w.block_tables, w.query_start_loc, w.distribution,
                            page_size=w.page_size, pages_per_seq=w.pages_per_seq,
                            kv_in_dtype="bf16", cache_dtype="fp8", k_scale=1.0, v_scale=0.5)
    meta = [torch.from_numpy(getattr(w, k)).cuda() for k in
            ("kv_lens", "block_tables", "query_start_loc", "distribution")]
    rpa.rpa_update_kv_cache(w.keys, w.values, w.kv_cache, *meta, k_scale=1.0, v_scale=0.5)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(w.kv_cache, "fp8"), exp)


@pytest.mark.parametrize("kvs", [[1], [1, 1, 1], [2, 17, 1], [300]])
def test_degenerate_decode_lengths(kvs):
    """kv_len 1 (a single key: out = v exactly up to rounding), and a few
    mixed tiny decode lengths, with empty sequences (q_len 0) interleaved."""
    print(f"\n[case] degenerate {kvs}", flush=True)
    q = [1] * len(kvs) + [0, 0]
    kv = list(kvs) + [5, 0]
    w = W.build("deg", q_lens=q, kv_lens=kv, distribution=(len(kvs), 0, 2), num_q_heads=8,
                num_kv_heads=2, head_dim=128, page_size=16, q_dtype="bf16", kv_in_dtype="bf16",
                cache_dtype="bf16", softmax_scale=0.1, seed=9, device="cuda")
    poison_unused(w)
    before = bits(w.kv_cache, "bf16")
    ref, ref_cache = oracle_forward(w, cache_bits=before)
    out = gpu_forward(w)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(w.kv_cache, "bf16"), ref_cache)
    n_valid = int(w.query_start_loc[w.num_seqs])
    check_output("deg", w, out, ref, np.arange(n_valid))


def test_head_dim_padded_cache():
    print("\n[case] padded head dim", flush=True)
    w = W.make("mixed_bf16", device="cuda", small=True, head_dim=64, head_dim_padded=128)
    poison_unused(w)
    before = bits(w.kv_cache, "bf16")
    ref, ref_cache = oracle_forward(w, cache_bits=before)
    out = gpu_forward(w)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(w.kv_cache, "bf16"), ref_cache)
    n_valid = int(w.query_start_loc[w.num_seqs])
    check_output("dpad", w, out, ref, np.arange(n_valid))


def test_no_split_and_many_splits():
    """One long decode row (many KV splits, merged by log-sum-exp) next to
    short ones (single split, direct output), with a sink."""
    print("\n[case] split mix", flush=True)
    w = W.build("split", q_lens=[1, 1, 1], kv_lens=[100000, 3, 700], distribution=(3, 0, 0),
                num_q_heads=16, num_kv_heads=4, head_dim=128, page_size=32, q_dtype="bf16",
                kv_in_dtype="bf16", cache_dtype="bf16", softmax_scale=0.3, seed=2,
                with_sink=True, device="cuda")
    poison_unused(w)
    before = bits(w.kv_cache, "bf16")
    ref, ref_cache = oracle_forward(w, cache_bits=before)
    out = gpu_forward(w)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(w.kv_cache, "bf16"), ref_cache)
    check_output("split", w, out, ref, np.arange(3))


@pytest.mark.parametrize("G,D", [(4, 64), (4, 128), (8, 64), (8, 128)])
def test_fp8_widening_exact_for_every_code(G, D):
    """The e4m3 -> bf16 widening of every kernel is exact.  With a window of
    one key each query sees only its own position, so its output is that key's
    V row times 1 / 1: the decoded e4m3 value, which bf16 holds exactly.  The
    visible V rows of the decode rows (row kernel: VALU for G = 4, MFMA for
    G = 8) and of the prefill chunk (prefill kernel) each cycle through all
    254 finite codes (no scale, no sink, attention over the cache as it is)."""
    print(f"\n[case] fp8 widening G={G} D={D}", flush=True)
    Hkv = 2
    q_lens, kv_lens = [1, 1, 1, 1, 16], [3, 40, 17, 2, 16]
    w = W.build("fp8widen", q_lens=q_lens, kv_lens=kv_lens, distribution=(4, 1, 0),
                num_q_heads=G * Hkv, num_kv_heads=Hkv, head_dim=D, page_size=16,
                q_dtype="bf16", kv_in_dtype="bf16", cache_dtype="fp8", softmax_scale=0.125,
                sliding_window=1, seed=8000 + G + D, device="cuda")
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert len(finite) == 254
    cache = bits(w.kv_cache, "fp8").copy()
    kcode = np.uint8(0x30)                       # K rows: 0.5 everywhere (finite)
    for group in ([0, 1, 2, 3], [4]):            # decode rows, then the prefill chunk
        i = 0
        for s in group:
            _, ql, ctx, kvl = O.seq_bounds(w.query_start_loc, w.kv_lens, s)
            for pos in range(kvl):
                page, off = O.slot_of(w.block_tables, w.pages_per_seq, w.page_size, s, pos)
                cache[page, off, 0::2, :] = kcode
                if pos < ctx:                    # not visible with a window of one
                    cache[page, off, 1::2, :] = 0x38
                    continue
                for g in range(Hkv):
                    cache[page, off, 2 * g + 1, :D] = finite[(i + np.arange(D)) % 254]
                    i += D
        assert i >= 254
    w.kv_cache.copy_(torch.from_numpy(cache.view(np.uint8)).to(w.kv_cache.device))
    ref, _ = oracle_forward(w, cache_bits=cache, update=False)
    out = gpu_forward(w, update=False)
    torch.cuda.synchronize()
    n_valid = int(w.query_start_loc[w.num_seqs])
    got = out[:n_valid].double().cpu().numpy()
    np.testing.assert_array_equal(got, ref[:n_valid])

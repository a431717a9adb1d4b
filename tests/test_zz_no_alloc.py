"""rpa_forward_noalloc (no workspace, no allocation; the library's own device
scratch) through the C ABI against rpa_forward on the same inputs: the cache
bit for bit, the output to the dtype's tolerance (bit for bit where both run
the same one-stream plan), on two calls in a row with the second smaller, so
the second runs on scratch holding the first call's larger plan."""
import numpy as np
import pytest
import torch

import ragged_paged_kv_scatter_amd as rpa
from ragged_paged_kv_scatter_amd import workloads as W
from tests.helpers import check_output

pytestmark = pytest.mark.gpu

def _f32_batch(seed):
    return W.build("f32_rows", q_lens=[1, 1, 1, 40, 7], kv_lens=[300, 900, 5, 100, 7],
                   distribution=(3, 2, 0), num_q_heads=8, num_kv_heads=2, head_dim=64,
                   page_size=16, q_dtype="f32", kv_in_dtype="f32", cache_dtype="f32",
                   softmax_scale=0.125, seed=seed, with_sink=True, device="cuda")


PAIRS = {
    # first call, then a smaller second call of the same kind
    "decode": (lambda s: W.make("decode_bf16", device="cuda", small=True, seed=s, num_seqs=40,
                                kv_min=20, kv_max=3000),
               lambda s: W.make("decode_bf16", device="cuda", small=True, seed=s, num_seqs=7,
                                kv_min=5, kv_max=400)),
    "mixed": (lambda s: W.make("mixed_bf16", device="cuda", small=True, seed=s, n_decode=12,
                               decode_kv=(40, 900), n_prefill=3, chunk=140, ctx_max=300),
              lambda s: W.make("mixed_bf16", device="cuda", small=True, seed=s, n_decode=3,
                               decode_kv=(10, 100), n_prefill=1, chunk=20, ctx_max=30)),
    "fp8_full": (lambda s: W.make("fp8_full", device="cuda", small=True, seed=s, n_decode=10,
                                  decode_kv=(40, 900), n_prefill=2, chunk=100, ctx=150,
                                  sliding_window=128),
                 lambda s: W.make("fp8_full", device="cuda", small=True, seed=s, n_decode=2,
                                  decode_kv=(40, 60), n_prefill=1, chunk=9, ctx=3,
                                  sliding_window=128)),
    "f32": (_f32_batch, lambda s: W.make("tiny_fp32", device="cuda", seed=s)),
}


def _meta(w):
    return {k: torch.from_numpy(np.ascontiguousarray(getattr(w, k))).cuda()
            for k in ("kv_lens", "block_tables", "query_start_loc", "distribution")}


def _run(w, fn, cache0):
    w.kv_cache.copy_(cache0)
    m = _meta(w)
    out = torch.full(w.queries.shape, float("nan"), dtype=w.queries.dtype, device="cuda")
    fn(w.queries, w.keys, w.values, w.kv_cache, m["kv_lens"], m["block_tables"],
       m["query_start_loc"], m["distribution"], w.attention_sink, out=out, **w.options())
    torch.cuda.synchronize()
    return out, w.kv_cache.clone()


@pytest.mark.parametrize("label", list(PAIRS))
def test_noalloc_matches_forward_twice(label):
    for i, make in enumerate(PAIRS[label]):
        w = make(1500 + i)
        print(f"\n[case] noalloc {label} call {i}: {w.name} tokens={w.total_tokens} "
              f"seqs={w.num_seqs}", flush=True)
        cache0 = w.kv_cache.clone()
        ref_out, ref_cache = _run(w, rpa.rpa_forward, cache0)
        out, cache = _run(w, rpa.rpa_forward_noalloc, cache0)
        assert torch.equal(cache.view(torch.uint8), ref_cache.view(torch.uint8))
        n = int(w.query_start_loc[w.num_seqs])
        if w.total_tokens <= w.max_num_seqs or w.q_dtype == "f32":
            # both run the same plan on one stream: the same bits
            assert torch.equal(out[:n].view(torch.uint8), ref_out[:n].view(torch.uint8))
        check_output(f"noalloc {label} {i}", w, out, ref_out[:n].double().cpu().numpy(),
                     np.arange(n))
        assert torch.isnan(out[n:].float()).all()


def test_noalloc_rejects_sizes_beyond_its_scratch():
    """A batch whose workspace would exceed the scratch array is refused with
    RPA_ERR_WORKSPACE before anything runs; the output stays untouched."""
    print("\n[case] noalloc beyond scratch", flush=True)
    w = W.make("decode_bf16", device="cuda", small=True, num_seqs=1024, kv_min=2, kv_max=20,
               num_q_heads=128, num_kv_heads=8)
    m = _meta(w)
    d = rpa._desc(w.queries, rpa._dtype(w.keys), w.kv_cache, m["kv_lens"], m["block_tables"])
    o = rpa._options(**w.options(), chunk_prefill_size=None, num_kv_pages_per_block=None,
                     num_queries_per_block=None, vmem_limit_bytes=None)
    assert rpa.rpa_workspace_bytes(d, o) > rpa.NOALLOC_SCRATCH_BYTES
    out = torch.full(w.queries.shape, float("nan"), dtype=w.queries.dtype, device="cuda")
    with pytest.raises(rpa.RpaError) as e:
        rpa.rpa_forward_noalloc(w.queries, w.keys, w.values, w.kv_cache, m["kv_lens"],
                                m["block_tables"], m["query_start_loc"], m["distribution"],
                                out=out, **w.options())
    assert e.value.code == 5
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all()

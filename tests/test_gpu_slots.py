"""GPU parity of the update's slot-mapping form (split K / V caches):
rpa_slot_mapping and rpa_reshape_and_cache through the C ABI against the CPU
oracle, bit-exact: every stored row equals the oracle's encoding, every other
byte is unchanged, padding (-1) and out-of-pool slots are skipped."""
import numpy as np
import pytest
import torch

import ragged_paged_kv_scatter_amd as rpa
from oracle import rpa_oracle as O
from ragged_paged_kv_scatter_amd import workloads as W
from tests.helpers import bits

pytestmark = pytest.mark.gpu
NAMES = ["tiny_fp32", "decode_bf16", "mixed_bf16", "prefill_bf16", "fp8_full"]
TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}


def _meta(w):
    return {k: torch.from_numpy(np.ascontiguousarray(getattr(w, k))).cuda()
            for k in ("kv_lens", "block_tables", "query_start_loc", "distribution")}


def _oracle_slots(w, total):
    return O.slot_mapping(w.kv_lens, w.block_tables, w.query_start_loc, w.distribution,
                          page_size=w.page_size, pages_per_seq=w.pages_per_seq,
                          total_tokens=total)


def _split(w):
    """Split caches holding the workload's context (K plane, V plane), on the GPU."""
    c = w.kv_cache
    return c[:, :, 0::2, :].contiguous(), c[:, :, 1::2, :].contiguous()


@pytest.mark.parametrize("name", NAMES)
def test_slot_mapping_matches_oracle(name):
    print(f"\n[case] slot mapping {name}", flush=True)
    w = W.make(name, device="cuda", small=True, extra_seqs=2, extra_tokens=3)
    m = _meta(w)
    got = rpa.rpa_slot_mapping(m["kv_lens"], m["block_tables"], m["query_start_loc"],
                               m["distribution"], page_size=w.page_size,
                               total_tokens=w.total_tokens)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got.cpu().numpy(), _oracle_slots(w, w.total_tokens))


@pytest.mark.parametrize("name", NAMES)
def test_reshape_and_cache_matches_oracle(name):
    print(f"\n[case] reshape_and_cache {name}", flush=True)
    w = W.make(name, device="cuda", small=True, extra_tokens=3)
    kc, vc = _split(w)
    nb, bs = kc.shape[:2]
    slots = _oracle_slots(w, w.total_tokens)
    slots[1] = O.PAD_SLOT                          # a padded row inside the batch
    if w.total_tokens > 4:
        slots[4] = nb * bs + 7                     # a slot past the pool
    kb_before, vb_before = bits(kc, w.cache_dtype), bits(vc, w.cache_dtype)
    ref_k, ref_v = O.reshape_and_cache(kb_before, vb_before, bits(w.keys, w.kv_in_dtype),
                                       bits(w.values, w.kv_in_dtype), slots,
                                       kv_in_dtype=w.kv_in_dtype, cache_dtype=w.cache_dtype,
                                       k_scale=w.k_scale, v_scale=w.v_scale)
    rpa.rpa_reshape_and_cache(w.keys, w.values, kc, vc, torch.from_numpy(slots).cuda(),
                              k_scale=w.k_scale, v_scale=w.v_scale)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(kc, w.cache_dtype), ref_k)
    np.testing.assert_array_equal(bits(vc, w.cache_dtype), ref_v)


def test_slot_mapping_then_store_equals_combined_update_at_full_size():
    """Long-prefill sizes (16384 token rows, 8 kv heads, D 128): the GPU slot
    mapping followed by the GPU split store leaves, plane by plane, the bytes
    of the GPU combined-layout update, whose parity with the oracle the other
    suite checks; and every stored row equals the step's keys / values."""
    print("\n[case] slots full prefill_bf16", flush=True)
    w = W.make("prefill_bf16", device="cuda")
    m = _meta(w)
    kc, vc = _split(w)
    slots = rpa.rpa_slot_mapping(m["kv_lens"], m["block_tables"], m["query_start_loc"],
                                 m["distribution"], page_size=w.page_size,
                                 total_tokens=w.total_tokens)
    rpa.rpa_reshape_and_cache(w.keys, w.values, kc, vc, slots)
    rpa.rpa_update_kv_cache(w.keys, w.values, w.kv_cache, m["kv_lens"], m["block_tables"],
                            m["query_start_loc"], m["distribution"])
    torch.cuda.synchronize()
    assert torch.equal(kc.view(torch.int16), w.kv_cache[:, :, 0::2, :].contiguous().view(torch.int16))
    assert torch.equal(vc.view(torch.int16), w.kv_cache[:, :, 1::2, :].contiguous().view(torch.int16))
    np.testing.assert_array_equal(slots.cpu().numpy(), _oracle_slots(w, w.total_tokens))
    s = slots.long()
    flat_k = kc.view(-1, w.num_kv_heads, w.head_dim_padded)
    rng = np.random.default_rng(3)
    rows = torch.from_numpy(rng.choice(w.total_tokens, 512, replace=False)).cuda()
    assert torch.equal(flat_k[s[rows], :, :w.head_dim].view(torch.int16),
                       w.keys[rows].view(torch.int16))

"""The C-ABI library: it loads, exports every function include/rpa.h declares,
and its host-side validation returns the documented status codes before any
launch (no GPU needed: a failing call never touches the device)."""
import ctypes
import os
import re

import pytest

from ragged_paged_kv_scatter_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "rpa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(rpa_\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) >= {"rpa_update_kv_cache", "rpa_forward", "rpa_workspace_bytes",
                          "rpa_error_string", "rpa_slot_mapping", "rpa_reshape_and_cache",
                          "rpa_copy_blocks", "rpa_swap_blocks"}
    for n in names:
        assert hasattr(lib, n), n


def good_desc(**kw):
    d = _lib.RpaDesc()
    vals = dict(total_tokens=7, max_num_seqs=3, pages_per_seq=2, num_pages=8, page_size=16,
                num_q_heads=4, num_kv_heads=2, head_dim=64, head_dim_padded=64,
                q_dtype=_lib.RPA_F32, kv_in_dtype=_lib.RPA_F32, cache_dtype=_lib.RPA_F32)
    vals.update(kw)
    for k, v in vals.items():
        setattr(d, k, v)
    return d


def good_opts(**kw):
    o = _lib.RpaOptions()
    o.softmax_scale = 0.125
    for k, v in kw.items():
        setattr(o, k, v)
    return o


def ws_status(lib, d, o):
    n = ctypes.c_size_t(0)
    return lib.rpa_workspace_bytes(ctypes.byref(d), ctypes.byref(o), ctypes.byref(n)), n.value


def test_workspace_query_ok(lib):
    st, n = ws_status(lib, good_desc(), good_opts())
    assert st == 0 and n > 0


@pytest.mark.parametrize("kw,code", [
    (dict(num_q_heads=3), 2),                 # Hq % Hkv != 0
    (dict(head_dim_padded=32), 2),            # Dpad < D
    (dict(num_kv_heads=0), 2),
    (dict(page_size=0), 2),
    (dict(head_dim=96, head_dim_padded=96), 3),
    (dict(page_size=24), 3),
    (dict(num_q_heads=6, num_kv_heads=2), 3),  # G = 3
    (dict(q_dtype=_lib.RPA_BF16), 3),         # bf16 q with f32 cache
    (dict(q_dtype=7), 3),
    (dict(cache_dtype=_lib.RPA_FP8_E4M3, kv_in_dtype=_lib.RPA_F32), 3),
    (dict(max_num_seqs=20000), 3),
])
def test_invalid_desc_codes(lib, kw, code):
    st, _ = ws_status(lib, good_desc(**kw), good_opts())
    assert st == code


@pytest.mark.parametrize("kw", [dict(sliding_window=-1), dict(logits_soft_cap=-1.0),
                                dict(logits_soft_cap=float("inf")), dict(k_scale=float("nan")),
                                dict(softmax_scale=float("inf")), dict(v_scale=-0.5),
                                dict(num_queries_per_block=-2)])
def test_invalid_option_codes(lib, kw):
    st, _ = ws_status(lib, good_desc(), good_opts(**kw))
    assert st == 4


def test_null_and_workspace_errors_do_not_launch(lib):
    d, o = good_desc(), good_opts()
    fake = ctypes.c_void_p(4096)   # never dereferenced: every call below fails host checks
    args = [fake] * 10
    # queries NULL
    assert lib.rpa_forward(ctypes.byref(d), ctypes.byref(o), None, None, None, *args[:8],
                           ctypes.c_size_t(1 << 30), None) == 1
    # keys without values
    assert lib.rpa_forward(ctypes.byref(d), ctypes.byref(o), fake, fake, None, fake, fake, fake,
                           fake, fake, None, fake, fake, ctypes.c_size_t(1 << 30), None) == 1
    # workspace too small
    assert lib.rpa_forward(ctypes.byref(d), ctypes.byref(o), fake, None, None, fake, fake, fake,
                           fake, fake, None, fake, fake, ctypes.c_size_t(16), None) == 5
    # misaligned cache pointer
    bad = ctypes.c_void_p(4096 + 8)
    assert lib.rpa_forward(ctypes.byref(d), ctypes.byref(o), fake, None, None, bad, fake, fake,
                           fake, fake, None, fake, fake, ctypes.c_size_t(1 << 30), None) == 2
    # update: NULL metadata, bad scale
    assert lib.rpa_update_kv_cache(ctypes.byref(d), fake, fake, fake, None, fake, fake, fake,
                                   1.0, 1.0, None) == 1
    assert lib.rpa_update_kv_cache(ctypes.byref(d), fake, fake, fake, fake, fake, fake, fake,
                                   float("nan"), 1.0, None) == 4
    assert lib.rpa_update_kv_cache(None, fake, fake, fake, fake, fake, fake, fake, 1.0, 1.0,
                                   None) == 1


def test_split_cache_calls_check_before_launch(lib):
    d = good_desc()
    fake = ctypes.c_void_p(4096)   # never dereferenced: every call below fails host checks
    # slot mapping: NULL output, NULL metadata, bad page size
    assert lib.rpa_slot_mapping(ctypes.byref(d), fake, fake, fake, fake, None, None) == 1
    assert lib.rpa_slot_mapping(ctypes.byref(d), None, fake, fake, fake, fake, None) == 1
    assert lib.rpa_slot_mapping(ctypes.byref(good_desc(page_size=24)), fake, fake, fake, fake,
                                fake, None) == 3
    # reshape_and_cache: NULL cache, bad scale, misaligned keys, unsupported dtype pair
    assert lib.rpa_reshape_and_cache(ctypes.byref(d), fake, fake, None, fake, fake, 1.0, 1.0,
                                     None) == 1
    assert lib.rpa_reshape_and_cache(ctypes.byref(d), fake, fake, fake, fake, fake, -1.0, 1.0,
                                     None) == 4
    assert lib.rpa_reshape_and_cache(ctypes.byref(d), ctypes.c_void_p(4096 + 4), fake, fake, fake,
                                     fake, 1.0, 1.0, None) == 2
    bad = good_desc(kv_in_dtype=_lib.RPA_F32, cache_dtype=_lib.RPA_FP8_E4M3)
    assert lib.rpa_reshape_and_cache(ctypes.byref(bad), fake, fake, fake, fake, fake, 1.0, 1.0,
                                     None) == 3


def test_metadata_check_checks_before_launch(lib):
    d = good_desc()
    fake = ctypes.c_void_p(4096)   # never dereferenced: every call below fails host checks
    # NULL status word, NULL slot bitmap, NULL metadata, NULL or unsupported desc
    assert lib.rpa_validate_metadata(ctypes.byref(d), fake, fake, fake, fake, fake, None,
                                     None) == 1
    assert lib.rpa_validate_metadata(ctypes.byref(d), fake, fake, fake, fake, None, fake,
                                     None) == 1
    assert lib.rpa_validate_metadata(ctypes.byref(d), fake, None, fake, fake, fake, fake,
                                     None) == 1
    assert lib.rpa_validate_metadata(None, fake, fake, fake, fake, fake, fake, None) == 1
    assert lib.rpa_validate_metadata(ctypes.byref(good_desc(page_size=24)), fake, fake, fake,
                                     fake, fake, fake, None) == 3


def test_block_copy_calls_check_before_launch(lib):
    fake = ctypes.c_void_p(4096)
    arr = (ctypes.c_void_p * 2)(4096, 8192)
    bad = (ctypes.c_void_p * 2)(4096, 4096 + 8)
    PP = ctypes.POINTER(ctypes.c_void_p)
    cast = lambda a: ctypes.cast(a, PP)
    assert lib.rpa_copy_blocks(None, cast(arr), 2, 4, 64, fake, 1, None) == 1
    assert lib.rpa_copy_blocks(cast(arr), cast(arr), 65, 4, 64, fake, 1, None) == 2
    assert lib.rpa_copy_blocks(cast(arr), cast(arr), 2, 4, 60, fake, 1, None) == 2
    assert lib.rpa_copy_blocks(cast(bad), cast(arr), 2, 4, 64, fake, 1, None) == 2
    assert lib.rpa_copy_blocks(cast(arr), cast(arr), 2, 4, 64, fake, 0, None) == 0
    pairs = (ctypes.c_int64 * 4)(0, 1, 3, 5)      # second pair: destination 5 >= 4 blocks
    assert lib.rpa_swap_blocks(fake, fake, 4, 4, 64, pairs, 2, None) == 2
    assert lib.rpa_swap_blocks(None, fake, 4, 4, 64, pairs, 1, None) == 1


def test_error_strings(lib):
    for code in range(7):
        assert lib.rpa_error_string(code)
    assert b"unknown" in lib.rpa_error_string(99)


def test_binding_rejects_cpu_tensors():
    import torch
    import ragged_paged_kv_scatter_amd as rpa
    q = torch.zeros(2, 4, 64)
    with pytest.raises(ValueError):
        rpa.rpa_forward(q, None, None, torch.zeros(2, 16, 4, 64), torch.zeros(1, dtype=torch.int32),
                        torch.zeros(1, dtype=torch.int32), torch.zeros(2, dtype=torch.int32),
                        torch.zeros(3, dtype=torch.int32))

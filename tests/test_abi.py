"""The C-ABI library: it loads, exports every function include/rpa.h declares,
and its host-side validation returns the documented status codes before any
launch (no GPU needed: a failing call never touches the device)."""
import ctypes
import os
import re

import pytest

from ragged_paged_kv_scatter_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions(header="rpa.h"):
    src = open(os.path.join(ROOT, "include", header)).read()
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


def test_probe_library_exports_every_declared_symbol():
    from ragged_paged_kv_scatter_amd import _probes
    lib = _probes.load()
    names = declared_functions("rpa_probes.h")
    assert set(names) == set(_probes.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_every_header_is_covered():
    """Each header under include/ belongs to one of the two libraries."""
    assert sorted(os.listdir(os.path.join(ROOT, "include"))) == ["rpa.h", "rpa_probes.h"]


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
    for kv_in in (_lib.RPA_BF16, _lib.RPA_FP8_E4M3):   # e4m3 queries over an e4m3 cache
        d = good_desc(q_dtype=_lib.RPA_FP8_E4M3, kv_in_dtype=kv_in, cache_dtype=_lib.RPA_FP8_E4M3)
        assert ws_status(lib, d, good_opts(q_scale=0.05))[0] == 0


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
    (dict(q_dtype=_lib.RPA_FP8_E4M3, kv_in_dtype=_lib.RPA_BF16, cache_dtype=_lib.RPA_BF16), 3),
    (dict(q_dtype=_lib.RPA_FP8_E4M3), 3),     # e4m3 queries need an e4m3 cache
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


def _cpu_batch(T=7, Hq=4, Hkv=2, D=64, seqs=3, pps=2, pages=8, ps=16):
    import torch
    i32 = torch.int32
    return dict(queries=torch.zeros(T, Hq, D, dtype=torch.bfloat16),
                keys=torch.zeros(T, Hkv, D, dtype=torch.bfloat16),
                values=torch.zeros(T, Hkv, D, dtype=torch.bfloat16),
                kv_cache=torch.zeros(pages, ps, 2 * Hkv, D, dtype=torch.bfloat16),
                kv_lens=torch.zeros(seqs, dtype=i32), block_tables=torch.zeros(seqs * pps, dtype=i32),
                query_start_loc=torch.zeros(seqs + 1, dtype=i32),
                distribution=torch.zeros(3, dtype=i32))


def _forward_err(**over):
    """The binding's error for a CPU batch with one argument replaced: every
    size and dtype check runs before the device check, so the message names
    the mismatch rather than the device."""
    import torch
    import ragged_paged_kv_scatter_amd as rpa
    b = _cpu_batch()
    b.update(over)
    extra = {k: b.pop(k) for k in ("attention_sink", "out") if k in b}
    with pytest.raises((ValueError, TypeError)) as e:
        rpa.rpa_forward(b["queries"], b["keys"], b["values"], b["kv_cache"], b["kv_lens"],
                        b["block_tables"], b["query_start_loc"], b["distribution"],
                        softmax_scale=0.125, **extra)
    assert "GPU" not in str(e.value), str(e.value)
    return str(e.value)


def test_binding_checks_sizes_before_any_launch():
    import torch
    bf = torch.bfloat16
    i32 = torch.int32
    assert "out" in _forward_err(out=torch.zeros(7, 4, 32, dtype=bf))
    assert "out" in _forward_err(out=torch.zeros(7, 4, 64, dtype=torch.float32))
    assert "out" in _forward_err(out=torch.zeros(7, 4, 128, dtype=bf)[..., :64])
    assert "keys" in _forward_err(keys=torch.zeros(6, 2, 64, dtype=bf))
    assert "keys" in _forward_err(keys=torch.zeros(7, 1, 64, dtype=bf))
    assert "values" in _forward_err(values=torch.zeros(7, 2, 32, dtype=bf))
    assert "dtype" in _forward_err(values=torch.zeros(7, 2, 64, dtype=torch.float32))
    assert "attention_sink" in _forward_err(attention_sink=torch.zeros(3))
    assert "attention_sink" in _forward_err(attention_sink=torch.zeros(4, dtype=torch.float64))
    assert "query_start_loc" in _forward_err(query_start_loc=torch.zeros(3, dtype=i32))
    assert "distribution" in _forward_err(distribution=torch.zeros(2, dtype=i32))
    assert "block_tables" in _forward_err(block_tables=torch.zeros(5, dtype=i32))
    assert "int32" in _forward_err(kv_lens=torch.zeros(3, dtype=torch.int64))


def test_update_binding_checks_sizes_before_any_launch():
    import torch
    import ragged_paged_kv_scatter_amd as rpa
    bf = torch.bfloat16

    def err(**over):
        b = _cpu_batch()
        b.update(over)
        with pytest.raises((ValueError, TypeError)) as e:
            rpa.rpa_update_kv_cache(b["keys"], b["values"], b["kv_cache"], b["kv_lens"],
                                    b["block_tables"], b["query_start_loc"], b["distribution"])
        assert "GPU" not in str(e.value), str(e.value)
        return str(e.value)
    assert "values" in err(values=torch.zeros(7, 2, 32, dtype=bf))
    assert "kv_cache" in err(kv_cache=torch.zeros(8, 16, 2, 64, dtype=bf))
    assert "query_start_loc" in err(query_start_loc=torch.zeros(2, dtype=torch.int32))
    assert "distribution" in err(distribution=torch.zeros(4, dtype=torch.int32))


def _kv(line):
    """key=value fields of one trace line."""
    return dict(f.split("=", 1) for f in line.split()[2:] if "=" in f)


@pytest.mark.parametrize("kind", ["decode", "mixed", "f32"])
def test_trace_format_lines(lib, kind):
    """rpa_trace_format runs rpa_forward's host path dry: the forward,
    workspace and stream lines, then one launch line per kernel in launch
    order (decode-only: plan, rows, prefill kernel merging the splits; with
    prefill tiles: plan, rows, the prefill kernels on the side stream, merge; f32: plan,
    rows, merge), and the workspace size rpa_workspace_bytes reports."""
    import ragged_paged_kv_scatter_amd as rpa
    if kind == "f32":
        d = good_desc()
        order = ["prep_kernel", "row_kernel", "merge_kernel"]
    else:
        d = good_desc(q_dtype=_lib.RPA_BF16, kv_in_dtype=_lib.RPA_BF16,
                      cache_dtype=_lib.RPA_BF16, num_q_heads=32, num_kv_heads=8, head_dim=128,
                      head_dim_padded=128, pages_per_seq=128, num_pages=20000, page_size=64)
        if kind == "decode":
            d.total_tokens, d.max_num_seqs = 256, 256
            order = ["prep_kernel", "row_kernel", "prefill_kernel"]
        else:
            d.total_tokens, d.max_num_seqs = 2176, 132
            # bf16 over a bf16 cache, G = 4: the two-group prefill kernel is
            # launched after prefill_kernel, and the planner's co_run flag
            # decides on the device which of the two takes the tiles
            order = ["prep_kernel", "row_kernel", "prefill_kernel", "prefill_pair_kernel",
                     "merge_kernel"]
    o = good_opts()
    text = rpa.rpa_trace_format(d, o, with_update=True)
    lines = text.strip().split("\n")
    assert all(l.startswith("[rpa] ") for l in lines), text
    assert [l.split()[1] for l in lines[:3]] == ["forward", "workspace", "streams"]
    fw = _kv(lines[0])
    assert int(fw["total_tokens"]) == d.total_tokens and int(fw["update"]) == 1
    assert int(fw["num_q_heads"]) == d.num_q_heads and int(fw["head_dim"]) == d.head_dim
    ws = _kv(lines[1])
    assert int(ws["bytes"]) == ws_status(lib, d, o)[1]
    offs = [int(ws[k]) for k in ("header", "zeros", "rows", "items", "chunks", "merge_rows",
                                 "prefill_items", "part_ml", "part_acc")]
    assert offs == sorted(offs) and all(x % 256 == 0 for x in offs)
    assert int(ws["max_parts"]) <= 2 * int(ws["max_chunks"])
    assert lines[2].split()[2] == ("caller+side" if kind == "mixed" else "caller")
    # the update: fused into the prefill kernel for bit-copy updates of batches
    # with a prefill kernel, else in the planner's launch
    assert lines[3].split()[1] == "update"
    assert lines[3].split()[2] == ("prep_kernel" if kind == "f32" else "fused")
    launches = [l for l in lines[4:] if l.split()[1] == "launch"]
    assert len(launches) == len(lines) - 4
    assert [l.split()[2].split("<")[0] for l in launches] == order
    for l in launches:
        f = _kv(l)
        assert int(f["grid"]) >= 1 and int(f["block"]) in (256, 512, 1024)
    # without the update the planner's launch carries no scatter
    text2 = rpa.rpa_trace_format(d, o, with_update=False)
    assert "plan+scatter" not in text2 and "update=0" in text2 and "[rpa] update none" in text2
    if kind != "f32":
        assert "+update)" in text and "+update)" not in text2   # the prefill kernel's share


def test_trace_format_reports_host_errors(lib):
    import ragged_paged_kv_scatter_amd as rpa
    with pytest.raises(rpa.RpaError) as e:
        rpa.rpa_trace_format(good_desc(page_size=24), good_opts())
    assert e.value.code == 3


def test_noalloc_checks_before_touching_the_device(lib):
    """rpa_forward_noalloc makes rpa_forward's host checks, and refuses sizes
    whose workspace exceeds its scratch array, before any device call."""
    fake = ctypes.c_void_p(4096)   # never dereferenced: every call below fails host checks
    o = good_opts()
    args = [fake] * 4 + [fake] * 4 + [None, fake, None]
    assert lib.rpa_forward_noalloc(None, ctypes.byref(o), *args) == 1
    assert lib.rpa_forward_noalloc(ctypes.byref(good_desc(page_size=24)), ctypes.byref(o),
                                   *args) == 3
    assert lib.rpa_forward_noalloc(ctypes.byref(good_desc()),
                                   ctypes.byref(good_opts(sliding_window=-1)), *args) == 4
    big = good_desc(q_dtype=_lib.RPA_BF16, kv_in_dtype=_lib.RPA_BF16, cache_dtype=_lib.RPA_BF16,
                    num_q_heads=128, num_kv_heads=8, head_dim=128, head_dim_padded=128,
                    total_tokens=4096, max_num_seqs=4096)
    st, need = ws_status(lib, big, o)
    assert st == 0 and need > _lib.NOALLOC_SCRATCH_BYTES
    assert lib.rpa_forward_noalloc(ctypes.byref(big), ctypes.byref(o), *args) == 5


@pytest.mark.parametrize("case", ["bf16_even_group", "bf16_odd_group", "fp8_cache", "padded",
                                  "long_table"])
def test_two_group_prefill_kernel_selection(lib, case):
    """Batches with prefill tiles launch the two-group prefill kernel beside
    prefill_kernel only for bf16 queries over a bf16 cache with an even GQA
    group, no lane padding and a block table of at most 8192 pages."""
    import ragged_paged_kv_scatter_amd as rpa
    kw = dict(q_dtype=_lib.RPA_BF16, kv_in_dtype=_lib.RPA_BF16, cache_dtype=_lib.RPA_BF16,
              num_q_heads=8, num_kv_heads=2, head_dim=128, head_dim_padded=128,
              pages_per_seq=64, num_pages=512, page_size=16, total_tokens=600, max_num_seqs=4)
    expect = True
    if case == "bf16_odd_group":
        kw.update(num_q_heads=2)
        expect = False
    elif case == "fp8_cache":
        kw.update(cache_dtype=_lib.RPA_FP8_E4M3)
        expect = False
    elif case == "padded":
        kw.update(head_dim_padded=144)
        expect = False
    elif case == "long_table":
        kw.update(pages_per_seq=8193, num_pages=40000)
        expect = False
    text = rpa.rpa_trace_format(good_desc(**kw), good_opts(), with_update=True)
    names = [l.split()[2].split("<")[0] for l in text.strip().split("\n") if l.split()[1] == "launch"]
    assert "prefill_kernel" in names
    assert ("prefill_pair_kernel" in names) == expect, names

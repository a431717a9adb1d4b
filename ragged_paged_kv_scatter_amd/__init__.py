"""MI355X-native ragged paged attention with paged KV-cache scatter.

Thin Python binding over librpa.so (include/rpa.h).  PyTorch supplies device
memory and the current HIP stream; every step of the computation runs in the
library's HIP kernels.  The two operations follow the ragged paged attention
v3 interface (ejkernel ``ragged_page_attention_v3`` signature):

* :func:`rpa_update_kv_cache` -- scatter new K/V tokens into their pages;
* :func:`rpa_forward` -- optional update, then attention of the ragged query
  batch over the paged cache; returns ``(out, kv_cache)``.
"""
import ctypes
from typing import Optional

import torch

from . import _lib
from ._lib import RpaDesc, RpaError, RpaKernelStat, RpaOptions

__all__ = ["rpa_update_kv_cache", "rpa_forward", "rpa_forward_noalloc", "rpa_workspace_bytes",
           "out_dtype_for",
           "rpa_slot_mapping",
           "rpa_reshape_and_cache", "rpa_copy_blocks", "rpa_swap_blocks",
           "rpa_validate_metadata", "rpa_trace_format", "profile_enable", "profile_read",
           "RpaError",
           "META_QSL", "META_LENS", "META_BLOCK_TABLE", "META_SLOTS", "META_DISTRIBUTION",
           "META_WRITE_IN_CONTEXT"]

# bits of rpa_validate_metadata's status word (include/rpa.h RPA_META_*)
META_QSL, META_LENS, META_BLOCK_TABLE, META_SLOTS, META_DISTRIBUTION = 1, 2, 4, 8, 16
META_WRITE_IN_CONTEXT = 32

_DT = {torch.float32: _lib.RPA_F32, torch.bfloat16: _lib.RPA_BF16, torch.uint8: _lib.RPA_FP8_E4M3,
       torch.float8_e4m3fn: _lib.RPA_FP8_E4M3}


def out_dtype_for(q_dtype: torch.dtype) -> torch.dtype:
    """dtype of the attention output: the queries' own, or bf16 for e4m3
    queries (uint8 codes or float8_e4m3fn)."""
    return torch.bfloat16 if q_dtype in (torch.uint8, torch.float8_e4m3fn) else q_dtype


def _dtype(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return _DT[t.dtype]


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_dev(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("all tensors must be on the same device")
    return dev


def _meta(t: torch.Tensor, name: str):
    if t.dtype != torch.int32:
        raise TypeError(f"{name} must be int32")
    return t


def _check_meta(kv_lens, block_tables, query_start_loc, distribution):
    """dtype and sizes of the metadata: the C ABI reads kv_lens[max_num_seqs],
    block_tables[max_num_seqs * pages_per_seq], query_start_loc[max_num_seqs + 1]
    and distribution[3] and cannot see their lengths."""
    for t, n in ((kv_lens, "kv_lens"), (block_tables, "block_tables"),
                 (query_start_loc, "query_start_loc"), (distribution, "distribution")):
        _meta(t, n)
    if kv_lens.dim() != 1:
        raise ValueError("kv_lens must be 1-D [max_num_seqs]")
    max_num_seqs = kv_lens.shape[0]
    if query_start_loc.numel() < max_num_seqs + 1:
        raise ValueError(f"query_start_loc needs max_num_seqs + 1 = {max_num_seqs + 1} "
                         f"entries, got {query_start_loc.numel()}")
    if distribution.numel() != 3:
        raise ValueError("distribution must hold 3 counts (decode, prefill, mixed)")
    if max_num_seqs > 0 and (block_tables.numel() == 0 or block_tables.numel() % max_num_seqs):
        raise ValueError("block_tables must hold max_num_seqs * pages_per_seq entries")


def _check_new_kv(keys, values, T, Hkv, D):
    """keys / values: [T, Hkv, D], one dtype."""
    if keys.dim() != 3 or tuple(keys.shape) != (T, Hkv, D):
        raise ValueError(f"keys must be [{T}, {Hkv}, {D}] (total_tokens, num_kv_heads, "
                         f"head_dim), got {tuple(keys.shape)}")
    if tuple(values.shape) != tuple(keys.shape):
        raise ValueError(f"values must have the shape of keys {tuple(keys.shape)}, got "
                         f"{tuple(values.shape)}")
    if values.dtype != keys.dtype:
        raise TypeError(f"values dtype {values.dtype} differs from keys dtype {keys.dtype}")


def _cache_dims(kv_cache: torch.Tensor):
    if kv_cache.dim() == 5:       # [P, ps, 2Hkv/packing, packing, Dpad]
        P, ps, a, b, dp = kv_cache.shape
        return P, ps, a * b, dp
    if kv_cache.dim() == 4:       # [P, ps, 2Hkv, Dpad]
        return tuple(kv_cache.shape)
    raise ValueError("kv_cache must be [num_pages, page_size, 2*num_kv_heads(/packing, packing), "
                     "head_dim_padded]")


def _desc(queries, kv_in_dtype, kv_cache, kv_lens, block_tables, num_kv_heads=None):
    T, Hq, D = queries.shape
    P, ps, two_h, dp = _cache_dims(kv_cache)
    if two_h % 2:
        raise ValueError("kv_cache head axis must hold 2 * num_kv_heads rows")
    Hkv = two_h // 2 if num_kv_heads is None else num_kv_heads
    max_num_seqs = kv_lens.shape[0]
    if block_tables.numel() % max(max_num_seqs, 1):
        raise ValueError("block_tables must hold max_num_seqs * pages_per_seq entries")
    pps = block_tables.numel() // max(max_num_seqs, 1)
    d = RpaDesc()
    d.total_tokens, d.max_num_seqs, d.pages_per_seq, d.num_pages, d.page_size = \
        T, max_num_seqs, pps, P, ps
    d.num_q_heads, d.num_kv_heads, d.head_dim, d.head_dim_padded = Hq, Hkv, D, dp
    d.q_dtype, d.kv_in_dtype, d.cache_dtype = _dtype(queries), kv_in_dtype, _dtype(kv_cache)
    return d


def _options(softmax_scale, sliding_window, logits_soft_cap, q_scale, k_scale, v_scale,
             chunk_prefill_size, num_kv_pages_per_block, num_queries_per_block, vmem_limit_bytes):
    o = RpaOptions()
    o.softmax_scale = float(softmax_scale)
    o.sliding_window = int(sliding_window or 0)
    o.logits_soft_cap = float(logits_soft_cap or 0.0)
    o.q_scale = float(q_scale or 0.0)
    o.k_scale = float(k_scale or 0.0)
    o.v_scale = float(v_scale or 0.0)
    o.chunk_prefill_size = int(chunk_prefill_size or 0)
    o.num_kv_pages_per_block = int(num_kv_pages_per_block or 0)
    o.num_queries_per_block = int(num_queries_per_block or 0)
    o.lds_limit_bytes = int(vmem_limit_bytes or 0)
    return o


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def rpa_update_kv_cache(keys, values, kv_cache, kv_lens, block_tables, query_start_loc,
                        distribution, *, k_scale=None, v_scale=None, queries_dtype=None):
    """Write new tokens' K/V ([T, Hkv, D]) into their pages of `kv_cache` in place."""
    _check_meta(kv_lens, block_tables, query_start_loc, distribution)
    if keys.dim() != 3:
        raise ValueError("keys must be [total_tokens, num_kv_heads, head_dim]")
    T, Hkv, D = keys.shape
    _check_new_kv(keys, values, T, Hkv, D)
    _, _, two_h, _ = _cache_dims(kv_cache)
    if two_h != 2 * Hkv:
        raise ValueError(f"kv_cache holds {two_h} head rows per token, keys need 2 * {Hkv}")
    dev = _check_dev(keys, values, kv_cache, kv_lens, block_tables, query_start_loc, distribution)
    qdt = queries_dtype if queries_dtype is not None else (
        torch.float32 if keys.dtype == torch.float32 else torch.bfloat16)
    fake_q = torch.empty((T, Hkv, D), dtype=qdt, device="meta")
    d = _desc(fake_q, _dtype(keys), kv_cache, kv_lens, block_tables, num_kv_heads=Hkv)
    lib = _lib.load()
    _lib.check(lib.rpa_update_kv_cache(
        ctypes.byref(d), _ptr(keys), _ptr(values), _ptr(kv_cache), _ptr(kv_lens),
        _ptr(block_tables), _ptr(query_start_loc), _ptr(distribution),
        float(k_scale or 0.0), float(v_scale or 0.0), _stream(dev)))
    return kv_cache


def rpa_validate_metadata(queries, kv_cache, kv_lens, block_tables, query_start_loc,
                          distribution, *, kv_in_dtype=None, status=None, slot_bits=None):
    """Check on the device the metadata preconditions of rpa_update_kv_cache and
    rpa_forward for these tensors' sizes.  Returns the device int32[1] status
    tensor (the OR of META_* bits, 0 when all hold); the C call does not
    synchronise, so read it with ``int(status.item())``."""
    _check_meta(kv_lens, block_tables, query_start_loc, distribution)
    dev = _check_dev(queries, kv_cache, kv_lens, block_tables, query_start_loc, distribution)
    kin = kv_in_dtype if kv_in_dtype is not None else _dtype(kv_cache)
    d = _desc(queries, kin, kv_cache, kv_lens, block_tables)
    words = (d.num_pages * d.page_size + 31) // 32
    if slot_bits is None:
        slot_bits = torch.empty(words, dtype=torch.int32, device=dev)
    elif slot_bits.numel() < words or slot_bits.dtype != torch.int32:
        raise ValueError(f"slot_bits must be int32 with at least {words} elements")
    if status is None:
        status = torch.empty(1, dtype=torch.int32, device=dev)
    _lib.check(_lib.load().rpa_validate_metadata(
        ctypes.byref(d), _ptr(kv_lens), _ptr(block_tables), _ptr(query_start_loc),
        _ptr(distribution), _ptr(slot_bits), _ptr(status), _stream(dev)))
    return status


def _flat_desc(total_tokens, max_num_seqs, pages_per_seq, num_pages, page_size, num_kv_heads,
               head_dim, head_dim_padded, kv_in_dtype, cache_dtype):
    d = RpaDesc()
    d.total_tokens, d.max_num_seqs, d.pages_per_seq, d.num_pages, d.page_size = \
        total_tokens, max_num_seqs, pages_per_seq, num_pages, page_size
    d.num_q_heads, d.num_kv_heads, d.head_dim, d.head_dim_padded = \
        num_kv_heads, num_kv_heads, head_dim, head_dim_padded
    d.q_dtype = _lib.RPA_F32 if kv_in_dtype == _lib.RPA_F32 else _lib.RPA_BF16
    d.kv_in_dtype, d.cache_dtype = kv_in_dtype, cache_dtype
    return d


def rpa_slot_mapping(kv_lens, block_tables, query_start_loc, distribution, *, page_size,
                     total_tokens, out=None):
    """Flat cache slot (int64 [total_tokens]) of every new token row; -1 for rows
    past the last sequence."""
    _check_meta(kv_lens, block_tables, query_start_loc, distribution)
    dev = _check_dev(kv_lens, block_tables, query_start_loc, distribution, out)
    max_num_seqs = kv_lens.shape[0]
    pps = block_tables.numel() // max(max_num_seqs, 1)
    if out is None:
        out = torch.empty(total_tokens, dtype=torch.int64, device=dev)
    if out.dtype != torch.int64 or out.numel() != total_tokens or not out.is_contiguous():
        raise ValueError("out must be a contiguous int64 tensor of total_tokens entries")
    # only the sequence geometry is used; the head geometry is a valid placeholder
    d = _flat_desc(total_tokens, max_num_seqs, pps, 1, page_size, 1, 64, 64,
                   _lib.RPA_F32, _lib.RPA_F32)
    _lib.check(_lib.load().rpa_slot_mapping(
        ctypes.byref(d), _ptr(kv_lens), _ptr(block_tables), _ptr(query_start_loc),
        _ptr(distribution), _ptr(out), _stream(dev)))
    return out


def rpa_reshape_and_cache(keys, values, key_cache, value_cache, slot_mapping, *, k_scale=None,
                          v_scale=None):
    """Store new K / V rows ([T, Hkv, D]) into split caches ([num_blocks, block_size,
    Hkv, Dpad]) at their flat slots, in place; slots outside the pool (-1
    padding) are skipped.  Returns ``(key_cache, value_cache)``."""
    dev = _check_dev(keys, values, key_cache, value_cache, slot_mapping)
    T, Hkv, D = keys.shape
    if tuple(values.shape) != (T, Hkv, D):
        raise ValueError("values must have the shape of keys")
    if key_cache.dim() != 4 or tuple(value_cache.shape) != tuple(key_cache.shape):
        raise ValueError("key_cache / value_cache must both be [num_blocks, block_size, Hkv, Dpad]")
    nb, bs, hc, dp = key_cache.shape
    if hc != Hkv or key_cache.dtype != value_cache.dtype:
        raise ValueError("cache head count or dtype does not match")
    if slot_mapping.dtype != torch.int64 or slot_mapping.numel() != T:
        raise ValueError("slot_mapping must be int64 with one entry per token row")
    for t in (keys, values, key_cache, value_cache, slot_mapping):
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    d = _flat_desc(T, 1, 1, nb, bs, Hkv, D, dp, _dtype(keys), _dtype(key_cache))
    _lib.check(_lib.load().rpa_reshape_and_cache(
        ctypes.byref(d), _ptr(keys), _ptr(values), _ptr(key_cache), _ptr(value_cache),
        _ptr(slot_mapping), float(k_scale or 0.0), float(v_scale or 0.0), _stream(dev)))
    return key_cache, value_cache


def _block_bytes(cache):
    if cache.dim() < 2 or not cache.is_contiguous():
        raise ValueError("a cache must be a contiguous [num_blocks, ...] tensor")
    return cache[0].numel() * cache.element_size()


def rpa_copy_blocks(key_caches, value_caches, src_to_dst):
    """For every layer's K and V cache ([num_blocks, ...] device tensors), copy
    block d = block s for every (s, d) row of the device int64 table
    ``src_to_dst`` ([n, 2]), in place."""
    if len(key_caches) != len(value_caches) or not key_caches:
        raise ValueError("one key cache and one value cache per layer")
    dev = _check_dev(src_to_dst, *key_caches, *value_caches)
    shape, bb = tuple(key_caches[0].shape), _block_bytes(key_caches[0])
    for c in list(key_caches) + list(value_caches):
        if tuple(c.shape) != shape or _block_bytes(c) != bb:
            raise ValueError("all caches must share one shape and block size")
    if src_to_dst.dtype != torch.int64 or src_to_dst.dim() != 2 or src_to_dst.shape[1] != 2:
        raise ValueError("src_to_dst must be int64 [n, 2]")
    pairs = src_to_dst.contiguous()
    n = len(key_caches)
    ks = (ctypes.c_void_p * n)(*[c.data_ptr() for c in key_caches])
    vs = (ctypes.c_void_p * n)(*[c.data_ptr() for c in value_caches])
    _lib.check(_lib.load().rpa_copy_blocks(ks, vs, n, shape[0], bb, _ptr(pairs), pairs.shape[0],
                                           _stream(dev)))
    return key_caches, value_caches


def rpa_swap_blocks(src_cache, dst_cache, src_to_dst):
    """dst block d = src block s for every (s, d) row of the host int64 table
    ``src_to_dst`` ([n, 2]); either cache may live in pinned host memory.  One
    plane per call (the K and the V plane are swapped by two calls)."""
    if src_to_dst.is_cuda or src_to_dst.dtype != torch.int64 or src_to_dst.dim() != 2 \
            or src_to_dst.shape[1] != 2:
        raise ValueError("src_to_dst must be a host int64 [n, 2] tensor")
    bb = _block_bytes(src_cache)
    if _block_bytes(dst_cache) != bb:
        raise ValueError("caches must share one block size")
    dev = src_cache.device if src_cache.is_cuda else dst_cache.device
    if not dev.type == "cuda":
        raise ValueError("one of the caches must be on the GPU")
    pairs = src_to_dst.contiguous()
    _lib.check(_lib.load().rpa_swap_blocks(
        _ptr(src_cache), _ptr(dst_cache), src_cache.shape[0], dst_cache.shape[0], bb,
        ctypes.c_void_p(pairs.data_ptr()), pairs.shape[0], _stream(dev)))
    return dst_cache


def rpa_workspace_bytes(desc: RpaDesc, opts: RpaOptions) -> int:
    n = ctypes.c_size_t(0)
    _lib.check(_lib.load().rpa_workspace_bytes(ctypes.byref(desc), ctypes.byref(opts),
                                               ctypes.byref(n)))
    return n.value


def _forward_args(queries, keys, values, kv_cache, kv_lens, block_tables, query_start_loc,
                  distribution, attention_sink, out, workspace, softmax_scale, sliding_window,
                  logits_soft_cap, q_scale, k_scale, v_scale, chunk_prefill_size,
                  num_kv_pages_per_block, num_queries_per_block, vmem_limit_bytes):
    """Checks and marshalling shared by rpa_forward and rpa_forward_noalloc:
    every size and dtype check runs before the device check (no launch on a
    mismatch).  Returns (device, desc, options, out)."""
    if (keys is None) != (values is None):
        raise ValueError("keys and values must both be given or both be None")
    _check_meta(kv_lens, block_tables, query_start_loc, distribution)
    if queries.dim() != 3:
        raise ValueError("queries must be [total_tokens, num_q_heads, head_dim]")
    T, Hq, D = queries.shape
    _, _, two_h, _ = _cache_dims(kv_cache)
    if keys is not None:
        _check_new_kv(keys, values, T, two_h // 2, D)
    if attention_sink is not None:
        if attention_sink.dtype != torch.float32:
            raise TypeError("attention_sink must be float32")
        if attention_sink.numel() != Hq:
            raise ValueError(f"attention_sink must hold num_q_heads = {Hq} values, got "
                             f"{attention_sink.numel()}")
    out_dtype = out_dtype_for(queries.dtype)
    if out is not None:
        if tuple(out.shape) != tuple(queries.shape) or out.dtype != out_dtype:
            raise ValueError(f"out must be {tuple(queries.shape)} {out_dtype}, got "
                             f"{tuple(out.shape)} {out.dtype}")
        if not out.is_contiguous():
            raise ValueError("out must be contiguous")
    dev = _check_dev(queries, keys, values, kv_cache, kv_lens, block_tables, query_start_loc,
                     distribution, attention_sink, out, workspace)
    kv_in = _dtype(keys) if keys is not None else _dtype(kv_cache)
    d = _desc(queries, kv_in, kv_cache, kv_lens, block_tables)
    o = _options(softmax_scale, sliding_window, logits_soft_cap, q_scale, k_scale, v_scale,
                 chunk_prefill_size, num_kv_pages_per_block, num_queries_per_block,
                 vmem_limit_bytes)
    if out is None:
        out = torch.empty(queries.shape, dtype=out_dtype, device=dev)
    return dev, d, o, out


def rpa_forward(queries, keys, values, kv_cache, kv_lens, block_tables, query_start_loc,
                distribution, attention_sink=None, *, softmax_scale=1.0, sliding_window=None,
                logits_soft_cap=None, q_scale=None, k_scale=None, v_scale=None,
                chunk_prefill_size=None, num_kv_pages_per_block=None,
                num_queries_per_block=None, vmem_limit_bytes=None, out=None, workspace=None):
    """Ragged paged attention (v3 semantics).  `keys`/`values` may be None to
    attend over the cache as it is.  Returns ``(out, kv_cache)``; the cache is
    updated in place."""
    dev, d, o, out = _forward_args(
        queries, keys, values, kv_cache, kv_lens, block_tables, query_start_loc, distribution,
        attention_sink, out, workspace, softmax_scale, sliding_window, logits_soft_cap, q_scale,
        k_scale, v_scale, chunk_prefill_size, num_kv_pages_per_block, num_queries_per_block,
        vmem_limit_bytes)
    nbytes = rpa_workspace_bytes(d, o)
    if workspace is None or workspace.numel() * workspace.element_size() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    lib = _lib.load()
    with torch.cuda.device(dev):    # the library sizes launches for the current device
        _lib.check(lib.rpa_forward(
            ctypes.byref(d), ctypes.byref(o), _ptr(queries), _ptr(keys), _ptr(values),
            _ptr(kv_cache), _ptr(kv_lens), _ptr(block_tables), _ptr(query_start_loc),
            _ptr(distribution), _ptr(attention_sink), _ptr(out), _ptr(workspace),
            ctypes.c_size_t(workspace.numel() * workspace.element_size()), _stream(dev)))
    return out, kv_cache


def rpa_forward_noalloc(queries, keys, values, kv_cache, kv_lens, block_tables, query_start_loc,
                        distribution, attention_sink=None, *, out, softmax_scale=1.0,
                        sliding_window=None, logits_soft_cap=None, q_scale=None, k_scale=None,
                        v_scale=None, chunk_prefill_size=None, num_kv_pages_per_block=None,
                        num_queries_per_block=None, vmem_limit_bytes=None):
    """rpa_forward with no workspace and no allocation: the library's own
    device scratch (NOALLOC_SCRATCH_BYTES per GPU) holds the plan and split
    partials, and every kernel runs on the current stream.  `out` must be
    given (this call allocates nothing, here or in the library).  Calls that
    overlap on one GPU share that scratch and race."""
    if out is None:
        raise ValueError("rpa_forward_noalloc needs a caller-allocated out")
    dev, d, o, out = _forward_args(
        queries, keys, values, kv_cache, kv_lens, block_tables, query_start_loc, distribution,
        attention_sink, out, None, softmax_scale, sliding_window, logits_soft_cap, q_scale,
        k_scale, v_scale, chunk_prefill_size, num_kv_pages_per_block, num_queries_per_block,
        vmem_limit_bytes)
    lib = _lib.load()
    with torch.cuda.device(dev):
        _lib.check(lib.rpa_forward_noalloc(
            ctypes.byref(d), ctypes.byref(o), _ptr(queries), _ptr(keys), _ptr(values),
            _ptr(kv_cache), _ptr(kv_lens), _ptr(block_tables), _ptr(query_start_loc),
            _ptr(distribution), _ptr(attention_sink), _ptr(out), _stream(dev)))
    return out, kv_cache


NOALLOC_SCRATCH_BYTES = _lib.NOALLOC_SCRATCH_BYTES


def rpa_trace_format(desc: RpaDesc, opts: RpaOptions, with_update: bool = True) -> str:
    """The trace an rpa_forward with these sizes and options prints under
    RPA_TRACE=1 (before its plan line), computed on the host without touching
    the device."""
    need = ctypes.c_size_t(0)
    lib = _lib.load()
    _lib.check(lib.rpa_trace_format(ctypes.byref(desc), ctypes.byref(opts), int(with_update),
                                    None, 0, ctypes.byref(need)))
    buf = ctypes.create_string_buffer(need.value + 1)
    _lib.check(lib.rpa_trace_format(ctypes.byref(desc), ctypes.byref(opts), int(with_update),
                                    buf, need.value + 1, ctypes.byref(need)))
    return buf.value.decode()


def profile_enable(on: bool = True):
    _lib.check(_lib.load().rpa_profile_enable(1 if on else 0))


def profile_read() -> dict:
    """{kernel name: (launches, total_ms)} since the last read."""
    buf = (RpaKernelStat * 32)()
    n = _lib.load().rpa_profile_read(buf, 32)
    if n < 0:
        _lib.check(-n)
    return {buf[i].name.decode(): (buf[i].launches, buf[i].total_ms) for i in range(n)}

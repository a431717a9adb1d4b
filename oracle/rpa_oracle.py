"""CPU oracle for ragged paged attention with paged KV-cache scatter.

TEST INFRASTRUCTURE ONLY.  Nothing in the library may import or call this
module; only the tests, the smoke check and the CPU-baseline leg of the
benchmark do.  It shares no code with the HIP path.

It is the plain definition of what the method computes, written in float64
numpy (the fp8 quantisation decision alone is taken in float32, the precision
the kernels take it in):

* update: every new K/V token of every sequence is written into its page slot
  (``update_kv_cache``);
* attention: for every query row, softmax-weighted sum over the visible keys of
  its own sequence, read from the updated paged cache (``attend_sequence``).

Sources (page titles and sections):

* ejkernel docs, ``ragged_page_attention_v3`` interface: argument names,
  shapes (queries ``[T, Hq, D]``, keys/values ``[T, Hkv, D]``, kv_cache
  ``[num_pages, page_size, 2*Hkv/kv_packing, kv_packing, head_dim_padded]``,
  kv_lens, flat block_tables, query_start_loc, distribution, attention_sink
  ``[Hq]``), and the options softmax_scale (default 1.0), sliding_window,
  logits_soft_cap, q/k/v scales.
* tpu-inference 0.11.1.dev -> 0.12.0.dev diff, v3 ``kernel.py``:
  ``flash_attention_step1_qk_softmax`` / ``flash_attention_step2_pv`` (running
  max, row sum, accumulator; ``pv *= v_scale``), ``_fetch_bkv`` and
  ``_update_kv_cache`` (a token lives at row ``page * page_size + offset`` of
  the page given by the block table), and the note that K and V are packed
  together per head.
* vLLM differential_flash_attn.py: context_len / query_len / seq_len diagram
  (queries are the last query_len tokens of the sequence), query_start_loc
  example ``[4, 6] -> [0, 4, 10]``, causal flag, ``window_size =
  (sliding_window - 1, 0)``, soft cap 0 meaning off, and GQA
  ``num_queries_per_kv = num_heads // num_kv_heads``.
* tpu-inference 0.11.1rc3 ``layers/vllm/attention.py``: new K/V are quantised
  to the cache dtype with k/v scales before the kernel (``quantize_kv``).

Readings taken where the pages are silent:
distribution = (n_decode, n_prefill, n_mixed) counts with num_seqs = their sum;
combined head index 2h holds K and 2h+1 holds V, pad lanes zero-filled;
soft cap is cap*tanh(s/cap) after all scales; the sink is a per-q-head logit
that joins the softmax denominator without a value row; quantisation is
clamp(x/scale, +-448) rounded to nearest-even OCP e4m3fn.
"""
from __future__ import annotations

import math

import numpy as np

# ---------------------------------------------------------------------------
# Element codecs.  Cache images are carried as raw bit patterns:
#   f32 -> uint32, bf16 -> uint16, fp8 (OCP e4m3fn) -> uint8.
# ---------------------------------------------------------------------------

BITS_DTYPE = {"f32": np.uint32, "bf16": np.uint16, "fp8": np.uint8}


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 is the top half of an IEEE binary32 word."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f32_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(bits, dtype=np.uint32).view(np.float32).astype(np.float64)


def e4m3_value(code: int) -> float:
    """Value of one OCP e4m3fn code: 1 sign bit, 4 exponent bits (bias 7),
    3 mantissa bits; exponent 0 is subnormal (m/8 * 2^-6); exponent 15 with
    mantissa 7 is NaN; there is no infinity."""
    s = -1.0 if (code >> 7) & 1 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return s * (m / 8.0) * 2.0 ** -6
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
# Non-negative finite codes 0..126 in increasing value order (0x7F is NaN).
_POS_VALUES = E4M3_TABLE[:127]


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(y: np.ndarray) -> np.ndarray:
    """Round float32 values (already clamped to +-448) to the nearest e4m3fn
    code; an exact tie goes to the code with an even last mantissa bit.
    NaN keeps its sign and becomes the NaN code (0x7F / 0xFF)."""
    y = np.asarray(y, dtype=np.float32).astype(np.float64)
    a = np.abs(y)
    if np.any(a[~np.isnan(a)] > 448.0):
        raise ValueError("e4m3_encode expects values clamped to +-448")
    sign = np.signbit(y).astype(np.uint8) << 7
    hi = np.searchsorted(_POS_VALUES, np.where(np.isnan(a), 0.0, a), side="left")
    hi = np.clip(hi, 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    d_hi = _POS_VALUES[hi] - a
    d_lo = a - _POS_VALUES[lo]
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (lo % 2 == 0))
    code = np.where(pick_lo, lo, hi).astype(np.uint8)
    code = np.where(np.isnan(a), np.uint8(0x7F), code).astype(np.uint8)
    return code | sign


def quantize_e4m3(x_f32: np.ndarray, scale: float) -> np.ndarray:
    """quantize_kv for an e4m3 cache: divide by the scale in float32 (IEEE,
    round to nearest even), clamp to the finite range +-448, round to e4m3fn.
    A scale of 0 means "no scale" (1.0)."""
    s = np.float32(scale if scale else 1.0)
    y = np.asarray(x_f32, dtype=np.float32) / s
    y = np.clip(y, np.float32(-448.0), np.float32(448.0))
    return e4m3_encode(y)


def to_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return f32_bits_to_f64(bits)
    if dtype == "bf16":
        return bf16_bits_to_f64(bits)
    if dtype == "fp8":
        return e4m3_decode(bits)
    raise ValueError(dtype)


def encode_for_cache(bits_in: np.ndarray, in_dtype: str, cache_dtype: str, scale: float):
    """Bit pattern of a new K or V element as stored in the cache."""
    if in_dtype == cache_dtype:
        return bits_in.astype(BITS_DTYPE[cache_dtype])
    if cache_dtype == "fp8" and in_dtype in ("bf16", "f32"):
        x32 = to_f64(bits_in, in_dtype).astype(np.float32)  # exact: both fit fp32
        return quantize_e4m3(x32, scale)
    raise ValueError(f"unsupported conversion {in_dtype} -> {cache_dtype}")


# ---------------------------------------------------------------------------
# Ragged metadata
# ---------------------------------------------------------------------------

def num_seqs_of(distribution) -> int:
    """distribution = (decode, prefill, mixed) sequence counts; their sum is
    the number of valid sequences (the rest of the metadata is padding)."""
    d = np.asarray(distribution, dtype=np.int64)
    return int(d[0] + d[1] + d[2])


def seq_bounds(query_start_loc, kv_lens, s):
    """(q0, q_len, ctx, kv_len) of sequence s.  query_start_loc is the
    cumulative sum of query lengths; kv_len counts the context plus the new
    tokens, so the queries are the last q_len positions of the sequence."""
    q0 = int(query_start_loc[s])
    q_len = int(query_start_loc[s + 1]) - q0
    kv_len = int(kv_lens[s])
    return q0, q_len, kv_len - q_len, kv_len


def slot_of(block_tables, pages_per_seq, page_size, s, pos):
    """Physical (page, offset) of logical token `pos` of sequence `s`: the
    block table row of s lists the pages in token order, page_size tokens per
    page."""
    pos = np.asarray(pos, dtype=np.int64)
    page = np.asarray(block_tables, dtype=np.int64)[s * pages_per_seq + pos // page_size]
    return page, pos % page_size


# ---------------------------------------------------------------------------
# KV-cache update (the scatter)
# ---------------------------------------------------------------------------

def update_kv_cache(cache_bits, keys_bits, values_bits, kv_lens, block_tables,
                    query_start_loc, distribution, *, page_size, pages_per_seq,
                    kv_in_dtype, cache_dtype, k_scale=0.0, v_scale=0.0):
    """Return a copy of `cache_bits` ([P, ps, 2*Hkv, Dpad]) with every new token
    written: K of head h to combined head 2h, V to 2h+1, lanes [D, Dpad) zero.
    No other element changes."""
    out = np.array(cache_bits, copy=True)
    T, Hkv, D = keys_bits.shape
    for s in range(num_seqs_of(distribution)):
        q0, q_len, ctx, _ = seq_bounds(query_start_loc, kv_lens, s)
        if q_len == 0:
            continue
        pos = ctx + np.arange(q_len)
        page, off = slot_of(block_tables, pages_per_seq, page_size, s, pos)
        k = encode_for_cache(keys_bits[q0:q0 + q_len], kv_in_dtype, cache_dtype, k_scale)
        v = encode_for_cache(values_bits[q0:q0 + q_len], kv_in_dtype, cache_dtype, v_scale)
        for h in range(Hkv):
            out[page, off, 2 * h, :] = 0
            out[page, off, 2 * h, :D] = k[:, h, :]
            out[page, off, 2 * h + 1, :] = 0
            out[page, off, 2 * h + 1, :D] = v[:, h, :]
    return out


def gather_kv(cache_bits, s, kv_len, block_tables, *, page_size, pages_per_seq, head_dim,
              cache_dtype, k_scale=0.0, v_scale=0.0):
    """Logical K and V ([kv_len, Hkv, D], float64) of sequence s, read from the
    pages its block-table row names and dequantised: element * scale (a scale
    of 0 means 1)."""
    pos = np.arange(kv_len)
    page, off = slot_of(block_tables, pages_per_seq, page_size, s, pos)
    rows = cache_bits[page, off]                      # [kv_len, 2Hkv, Dpad]
    k = to_f64(rows[:, 0::2, :head_dim], cache_dtype)
    v = to_f64(rows[:, 1::2, :head_dim], cache_dtype)
    return k * (k_scale if k_scale else 1.0), v * (v_scale if v_scale else 1.0)


# ---------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------

def visible(q_pos: np.ndarray, kv_len: int, sliding_window: int) -> np.ndarray:
    """[q, kv] mask: key j is visible from a query at absolute position p iff
    j <= p (causal over the query tail) and, with a window W > 0, p - j < W
    (W keys including the query's own)."""
    j = np.arange(kv_len)[None, :]
    p = np.asarray(q_pos)[:, None]
    m = j <= p
    if sliding_window:
        m &= (p - j) < sliding_window
    return m


def _weighted_sum(w, v, mask):
    """sum over visible j of w[q, j] * v[j]: keys a row cannot see contribute
    nothing whatever their stored bits (a masked slot may hold NaN)."""
    finite = np.isfinite(v).all(axis=1)
    out = w @ np.where(finite[:, None], v, 0.0)
    for j in np.nonzero(~finite)[0]:
        rows = mask[:, j]
        out[rows] += w[rows, j, None] * v[j][None, :]
    return out


def attend_sequence(q, k, v, ctx, *, softmax_scale=1.0, sliding_window=0, logits_soft_cap=0.0,
                    q_scale=0.0, sink=None, return_weights=False):
    """Attention of one sequence's query rows over its own keys.

    q: [q_len, Hq, D]; k, v: [kv_len, Hkv, D] (float64, already dequantised);
    query t sits at position ctx + t.  q head h reads KV head h // (Hq/Hkv).
    Logits s = softmax_scale * q_scale * (q . k); with a soft cap c > 0,
    s = c * tanh(s / c).  With a sink sigma_h, the softmax denominator gains
    exp(sigma_h) and no value row.  Returns [q_len, Hq, D] float64.
    """
    q_len, Hq, D = q.shape
    kv_len, Hkv, _ = k.shape
    G = Hq // Hkv
    out = np.zeros((q_len, Hq, D))
    weights = np.zeros((q_len, Hq, kv_len)) if return_weights else None
    mask = visible(ctx + np.arange(q_len), kv_len, sliding_window)
    scale = softmax_scale * (q_scale if q_scale else 1.0)
    for h in range(Hq):
        g = h // G
        s = (q[:, h, :] @ k[:, g, :].T) * scale                  # [q_len, kv_len]
        if logits_soft_cap:
            s = logits_soft_cap * np.tanh(s / logits_soft_cap)
        s = np.where(mask, s, -np.inf)
        m = s.max(axis=1) if kv_len else np.full(q_len, -np.inf)
        if sink is not None:
            m = np.maximum(m, sink[h])
        w = np.where(mask, np.exp(s - m[:, None]), 0.0)
        z = w.sum(axis=1)
        if sink is not None:
            z = z + np.exp(sink[h] - m)
        out[:, h, :] = _weighted_sum(w, v[:, g, :], mask) / z[:, None]
        if return_weights:
            weights[:, h, :] = w / z[:, None]
    return (out, weights) if return_weights else out


def forward(queries_bits, keys_bits, values_bits, cache_bits, kv_lens, block_tables,
            query_start_loc, distribution, *, page_size, pages_per_seq, q_dtype, kv_in_dtype,
            cache_dtype, softmax_scale=1.0, sliding_window=0, logits_soft_cap=0.0, q_scale=0.0,
            k_scale=0.0, v_scale=0.0, attention_sink=None, seqs=None):
    """The whole step: update the cache with the new tokens (when keys are
    given), then attend over the updated cache.

    Returns (out, new_cache): out is [T, Hq, D] float64 with NaN in rows that
    no valid sequence owns (or that `seqs`, when given, leaves out).
    """
    T, Hq, D = queries_bits.shape
    if keys_bits is not None:
        cache_bits = update_kv_cache(
            cache_bits, keys_bits, values_bits, kv_lens, block_tables, query_start_loc,
            distribution, page_size=page_size, pages_per_seq=pages_per_seq,
            kv_in_dtype=kv_in_dtype, cache_dtype=cache_dtype, k_scale=k_scale, v_scale=v_scale)
    out = np.full((T, Hq, D), np.nan)
    sink = None if attention_sink is None else np.asarray(attention_sink, dtype=np.float64)
    n = num_seqs_of(distribution)
    for s in (range(n) if seqs is None else seqs):
        q0, q_len, ctx, kv_len = seq_bounds(query_start_loc, kv_lens, s)
        if q_len == 0:
            continue
        k, v = gather_kv(cache_bits, s, kv_len, block_tables, page_size=page_size,
                         pages_per_seq=pages_per_seq, head_dim=D, cache_dtype=cache_dtype,
                         k_scale=k_scale, v_scale=v_scale)
        q = to_f64(queries_bits[q0:q0 + q_len], q_dtype)
        out[q0:q0 + q_len] = attend_sequence(
            q, k, v, ctx, softmax_scale=softmax_scale, sliding_window=sliding_window,
            logits_soft_cap=logits_soft_cap, q_scale=q_scale, sink=sink)
    return out, cache_bits


def visible_slots(kv_lens, block_tables, query_start_loc, distribution, *, page_size,
                  pages_per_seq, num_pages, sliding_window=0):
    """Boolean [num_pages, page_size]: slots holding a key that some query of
    some valid sequence can see (after the update).  Every other slot may hold
    anything, NaN included, without changing any output."""
    used = np.zeros((num_pages, page_size), dtype=bool)
    for s in range(num_seqs_of(distribution)):
        _, q_len, ctx, kv_len = seq_bounds(query_start_loc, kv_lens, s)
        if q_len == 0:
            continue
        lo = max(0, ctx - sliding_window + 1) if sliding_window else 0
        page, off = slot_of(block_tables, pages_per_seq, page_size, s, np.arange(lo, kv_len))
        used[page, off] = True
    return used


def written_slots(kv_lens, block_tables, query_start_loc, distribution, *, page_size,
                  pages_per_seq, num_pages):
    """Boolean [num_pages, page_size]: slots the update writes."""
    w = np.zeros((num_pages, page_size), dtype=bool)
    for s in range(num_seqs_of(distribution)):
        _, q_len, ctx, kv_len = seq_bounds(query_start_loc, kv_lens, s)
        page, off = slot_of(block_tables, pages_per_seq, page_size, s, np.arange(ctx, kv_len))
        w[page, off] = True
    return w


# ---------------------------------------------------------------------------
# Slot-mapping form of the update, into split K / V caches
# (vLLM differential_flash_attn.py: the metadata builder's "Compute slot
# mapping" step, cuda-graph padding with PAD_SLOT_ID, and populate_kv_cache's
# reshape_and_cache_flash call on kv_cache[0], kv_cache[1] with the flattened
# slot mapping, the cache dtype and the k/v scales).  The pages show the calls
# only; the readings taken: a slot is
# block * block_size + offset of the token's position, rows past the last
# sequence carry PAD_SLOT, and a store skips PAD_SLOT (and, as a guard, any
# slot outside the pool).
# ---------------------------------------------------------------------------

PAD_SLOT = -1


def slot_mapping(kv_lens, block_tables, query_start_loc, distribution, *, page_size,
                 pages_per_seq, total_tokens):
    """int64 [total_tokens]: flat cache slot of every new token row, the same
    (page, offset) the combined-layout update writes; PAD_SLOT for rows past
    the last valid sequence."""
    out = np.full(total_tokens, PAD_SLOT, dtype=np.int64)
    for s in range(num_seqs_of(distribution)):
        q0, q_len, ctx, _ = seq_bounds(query_start_loc, kv_lens, s)
        if q_len == 0:
            continue
        page, off = slot_of(block_tables, pages_per_seq, page_size, s, ctx + np.arange(q_len))
        out[q0:q0 + q_len] = page.astype(np.int64) * page_size + off
    return out


def reshape_and_cache(key_cache_bits, value_cache_bits, keys_bits, values_bits, slots, *,
                      kv_in_dtype, cache_dtype, k_scale=0.0, v_scale=0.0):
    """Copies of the split caches ([num_blocks, block_size, Hkv, Dpad] each)
    with token i's K row (all heads) stored at flat slot slots[i] of the key
    cache and its V row in the value cache, lanes [D, Dpad) zero.  Tokens whose
    slot is negative or past the pool are skipped; nothing else changes."""
    kc = np.array(key_cache_bits, copy=True)
    vc = np.array(value_cache_bits, copy=True)
    nb, bs, _, _ = kc.shape
    D = keys_bits.shape[2]
    k = encode_for_cache(keys_bits, kv_in_dtype, cache_dtype, k_scale)
    v = encode_for_cache(values_bits, kv_in_dtype, cache_dtype, v_scale)
    for i, sl in enumerate(np.asarray(slots, dtype=np.int64)):
        if sl < 0 or sl >= nb * bs:
            continue
        b, o = divmod(int(sl), bs)
        kc[b, o] = 0
        kc[b, o, :, :D] = k[i]
        vc[b, o] = 0
        vc[b, o, :, :D] = v[i]
    return kc, vc


# ---------------------------------------------------------------------------
# Block copies of the split caches (vLLM differential_flash_attn.py:
# swap_blocks applies ops.swap_blocks to the K plane kv_cache[0] and the V
# plane kv_cache[1] with one src_to_dst table; copy_blocks applies
# ops.copy_blocks to the K and V planes of every layer's cache with one
# src_to_dists table).  The pages show the calls only; the reading taken
# here: a table is int64 [n, 2] of (source block,
# destination block) pairs and each pair copies one whole block, all of its
# bytes; destinations are distinct and no destination is also a source.
# ---------------------------------------------------------------------------

def swap_blocks(src_cache, dst_cache, src_to_dst):
    """Copy of dst_cache ([num_blocks, ...]) with block d replaced by block s of
    src_cache for every (s, d) pair."""
    out = np.array(dst_cache, copy=True)
    for s, d in np.asarray(src_to_dst, dtype=np.int64).reshape(-1, 2):
        out[d] = src_cache[s]
    return out


def copy_blocks(caches, src_to_dists):
    """Copies of every cache in `caches` (each [num_blocks, ...]) with block d
    replaced by block s of the same cache, for every (s, d) pair."""
    out = [np.array(c, copy=True) for c in caches]
    pairs = np.asarray(src_to_dists, dtype=np.int64).reshape(-1, 2)
    for c, o in zip(caches, out):
        for s, d in pairs:
            o[d] = c[s]
    return out

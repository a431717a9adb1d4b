"""Seeded synthetic workloads for ragged paged attention.

This module only draws random inputs: sequence lengths, a page pool handed out
through a random permutation, and tensor contents.  It holds none of the
method's arithmetic (no addressing of tokens into pages, no quantisation rule of
its own, no attention), so that the CPU oracle and the GPU path can both consume
its output without sharing any code with each other.

Layouts follow the ragged-paged-attention v3 interface (ejkernel
``ragged_page_attention_v3`` signature): queries ``[T, Hq, D]``, keys / values
``[T, Hkv, D]``, kv_cache ``[num_pages, page_size, 2*Hkv/kv_packing, kv_packing,
head_dim_padded]`` which, row-major, is the same memory as
``[num_pages, page_size, 2*Hkv, head_dim_padded]``; int32 ``kv_lens``,
flat ``block_tables``, ``query_start_loc`` and a 3-entry ``distribution``.

The recipes are the five named workloads (tiny fp32 mixed batch, bf16 decode,
bf16 mixed prefill+decode, bf16 long prefill, fp8-KV feature-complete batch)
plus scaled-down variants small enough for a CPU oracle.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

DTYPES = ("f32", "bf16", "fp8")
TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}


@dataclass
class Workload:
    name: str
    # shapes
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    head_dim_padded: int
    page_size: int
    num_pages: int
    pages_per_seq: int
    max_num_seqs: int
    total_tokens: int
    q_dtype: str
    kv_in_dtype: str
    cache_dtype: str
    # metadata (host copies, int32)
    kv_lens: np.ndarray
    block_tables: np.ndarray          # flat [max_num_seqs * pages_per_seq]
    query_start_loc: np.ndarray       # [max_num_seqs + 1]
    distribution: np.ndarray          # [3] = (n_decode, n_prefill, n_mixed)
    # options
    softmax_scale: float = 1.0
    sliding_window: int = 0
    logits_soft_cap: float = 0.0
    q_scale: float = 0.0
    k_scale: float = 0.0
    v_scale: float = 0.0
    # tensors (torch, on `device`); fp8 tensors are uint8 code arrays
    queries: Optional[torch.Tensor] = None
    keys: Optional[torch.Tensor] = None
    values: Optional[torch.Tensor] = None
    kv_cache: Optional[torch.Tensor] = None
    attention_sink: Optional[torch.Tensor] = None
    seed: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.distribution.sum())

    def q_lens(self) -> np.ndarray:
        n = self.num_seqs
        return (self.query_start_loc[1:n + 1] - self.query_start_loc[:n]).astype(np.int64)

    def options(self) -> dict:
        return dict(softmax_scale=self.softmax_scale, sliding_window=self.sliding_window,
                    logits_soft_cap=self.logits_soft_cap, q_scale=self.q_scale,
                    k_scale=self.k_scale, v_scale=self.v_scale)


def _rand_tensor(shape, dtype: str, gen: torch.Generator, device, scale: float = 1.0,
                 chunk_elems: int = 1 << 28) -> torch.Tensor:
    """N(0,1) values drawn in fp32 and cast to `dtype`.

    fp8 tensors hold OCP e4m3fn codes of N(0,1)/scale, produced by torch's own
    float8_e4m3fn conversion after a clamp to the format's +-448 range.
    Drawn in chunks so that huge page pools do not need a full fp32 copy.
    """
    out = torch.empty(shape, dtype=TORCH_DTYPE[dtype], device=device)
    flat = out.view(-1)
    n = flat.numel()
    for start in range(0, n, chunk_elems):
        m = min(chunk_elems, n - start)
        x = torch.randn(m, generator=gen, device=device, dtype=torch.float32)
        if dtype == "f32":
            flat[start:start + m] = x
        elif dtype == "bf16":
            flat[start:start + m] = x.to(torch.bfloat16)
        else:
            y = torch.clamp(x / scale, -448.0, 448.0)
            flat[start:start + m] = y.to(torch.float8_e4m3fn).view(torch.uint8)
    return out


def build(name: str, *, q_lens, kv_lens, distribution, num_q_heads, num_kv_heads, head_dim,
          page_size, q_dtype, kv_in_dtype, cache_dtype, softmax_scale, seed,
          head_dim_padded=None, pool_factor=1.5, num_pages=None, sliding_window=0,
          logits_soft_cap=0.0, q_scale=0.0, k_scale=0.0, v_scale=0.0, with_sink=False,
          extra_seqs=0, extra_tokens=0, device="cpu", rng: Optional[np.random.Generator] = None,
          pages_per_seq=None) -> Workload:
    """Assemble a workload from per-sequence lengths.

    `rng` continues the caller's draw stream (lengths were drawn first); the
    page permutation is drawn from it next, then tensors from a torch generator
    seeded with `seed` in the order Q, cache image, new K, new V, sink.
    `extra_seqs` pads the metadata arrays past num_seqs; `extra_tokens` pads
    the token arrays past the last valid row.
    """
    if rng is None:
        rng = np.random.default_rng(seed)
    q_lens = np.asarray(q_lens, dtype=np.int64)
    kv_lens = np.asarray(kv_lens, dtype=np.int64)
    n = len(q_lens)
    assert len(kv_lens) == n and np.all(kv_lens >= q_lens) and np.all(q_lens >= 0)
    dist = np.asarray(distribution, dtype=np.int32)
    assert dist.sum() == n
    hdp = head_dim if head_dim_padded is None else head_dim_padded
    needed = [int(math.ceil(k / page_size)) for k in kv_lens]
    total_needed = sum(needed)
    if num_pages is None:
        num_pages = max(1, int(math.ceil(pool_factor * total_needed)))
    assert num_pages >= total_needed
    if pages_per_seq is None:
        pages_per_seq = max(1, max(needed) if n else 1)
    max_num_seqs = n + extra_seqs
    perm = rng.permutation(num_pages)
    bt = np.zeros((max_num_seqs, pages_per_seq), dtype=np.int32)
    cur = 0
    for s in range(n):
        bt[s, :needed[s]] = perm[cur:cur + needed[s]]
        cur += needed[s]
    qsl = np.zeros(max_num_seqs + 1, dtype=np.int32)
    qsl[1:n + 1] = np.cumsum(q_lens)
    qsl[n + 1:] = qsl[n]
    kvl = np.zeros(max_num_seqs, dtype=np.int32)
    kvl[:n] = kv_lens
    T = int(q_lens.sum()) + extra_tokens

    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    two_h = 2 * num_kv_heads
    queries = _rand_tensor((T, num_q_heads, head_dim), q_dtype, gen, device,
                           scale=q_scale if q_scale else 1.0)
    cache_scale = k_scale if k_scale else 1.0
    kv_cache = _rand_tensor((num_pages, page_size, two_h, hdp), cache_dtype, gen, device,
                            scale=cache_scale)
    keys = _rand_tensor((T, num_kv_heads, head_dim), kv_in_dtype, gen, device,
                        scale=k_scale if k_scale else 1.0)
    values = _rand_tensor((T, num_kv_heads, head_dim), kv_in_dtype, gen, device,
                          scale=v_scale if v_scale else 1.0)
    sink = None
    if with_sink:
        sink = torch.randn(num_q_heads, generator=gen, device=device, dtype=torch.float32)
    return Workload(
        name=name, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
        head_dim_padded=hdp, page_size=page_size, num_pages=num_pages,
        pages_per_seq=pages_per_seq, max_num_seqs=max_num_seqs, total_tokens=T,
        q_dtype=q_dtype, kv_in_dtype=kv_in_dtype, cache_dtype=cache_dtype,
        kv_lens=kvl, block_tables=bt.reshape(-1).copy(), query_start_loc=qsl,
        distribution=dist, softmax_scale=float(softmax_scale),
        sliding_window=int(sliding_window), logits_soft_cap=float(logits_soft_cap),
        q_scale=float(q_scale), k_scale=float(k_scale), v_scale=float(v_scale),
        queries=queries, keys=keys, values=values, kv_cache=kv_cache, attention_sink=sink,
        seed=int(seed), meta=dict(needed_pages=total_needed))


# ---------------------------------------------------------------------------
# Named recipes.  `scale` < 1 shrinks sequence counts and lengths for CPU runs.
# ---------------------------------------------------------------------------

def tiny_fp32(device="cpu", seed=1000, **kw) -> Workload:
    """3 seqs, q_lens {1,1,5}, kv_lens {9,17,5}; page_size 16, pool of 8 pages;
    Hq 4, Hkv 2, D 64, fp32 everywhere, softmax_scale 1/8."""
    rng = np.random.default_rng(seed)
    return build("tiny_fp32", q_lens=[1, 1, 5], kv_lens=[9, 17, 5], distribution=(2, 1, 0),
                 num_q_heads=4, num_kv_heads=2, head_dim=64, page_size=16, num_pages=8,
                 q_dtype="f32", kv_in_dtype="f32", cache_dtype="f32", softmax_scale=1 / 8,
                 seed=seed, device=device, rng=rng, **kw)


def decode_bf16(device="cpu", seed=1001, num_seqs=256, kv_min=512, kv_max=4096, **kw) -> Workload:
    """Decode only: q_len 1, kv_len ~ U{kv_min..kv_max}; page_size 16;
    Hq 32, Hkv 8, D 128, bf16, softmax_scale 1/sqrt(128)."""
    rng = np.random.default_rng(seed)
    kv = rng.integers(kv_min, kv_max, size=num_seqs, endpoint=True)
    args = dict(num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16)
    args.update(kw)
    return build("decode_bf16", q_lens=np.ones(num_seqs, np.int64), kv_lens=kv,
                 distribution=(num_seqs, 0, 0), q_dtype="bf16", kv_in_dtype="bf16",
                 cache_dtype="bf16", softmax_scale=1 / math.sqrt(args["head_dim"]), seed=seed,
                 device=device, rng=rng, **args)


def mixed_bf16(device="cpu", seed=1002, n_decode=128, decode_kv=(1024, 8192), n_prefill=4,
               chunk=512, ctx_max=4096, **kw) -> Workload:
    """128 decode seqs (kv ~ U{1024..8192}) + 4 prefill chunks of 512 tokens with
    prior context ~ U{0..4096}; page_size 64; Hq 32, Hkv 8, D 128, bf16."""
    rng = np.random.default_rng(seed)
    dkv = rng.integers(decode_kv[0], decode_kv[1], size=n_decode, endpoint=True)
    ctx = rng.integers(0, ctx_max, size=n_prefill, endpoint=True)
    q = np.concatenate([np.ones(n_decode, np.int64), np.full(n_prefill, chunk, np.int64)])
    kv = np.concatenate([dkv, ctx + chunk])
    args = dict(num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=64)
    args.update(kw)
    return build("mixed_bf16", q_lens=q, kv_lens=kv, distribution=(n_decode, n_prefill, 0),
                 q_dtype="bf16", kv_in_dtype="bf16", cache_dtype="bf16",
                 softmax_scale=1 / math.sqrt(args["head_dim"]), seed=seed, device=device,
                 rng=rng, **args)


def prefill_bf16(device="cpu", seed=1003, n_seqs=2, seq_len=8192, **kw) -> Workload:
    """2 seqs with q_len = kv_len = 8192 (no prior context), causal;
    Hq 64, Hkv 8, D 128, page_size 128, bf16."""
    rng = np.random.default_rng(seed)
    args = dict(num_q_heads=64, num_kv_heads=8, head_dim=128, page_size=128)
    args.update(kw)
    return build("prefill_bf16", q_lens=[seq_len] * n_seqs, kv_lens=[seq_len] * n_seqs,
                 distribution=(0, n_seqs, 0), q_dtype="bf16", kv_in_dtype="bf16",
                 cache_dtype="bf16", softmax_scale=1 / math.sqrt(args["head_dim"]), seed=seed,
                 device=device, rng=rng, **args)


def fp8_full(device="cpu", seed=1004, n_decode=64, decode_kv=(2048, 16384), n_prefill=2,
             chunk=1024, ctx=2048, sliding_window=4096, **kw) -> Workload:
    """64 decode seqs (kv ~ U{2048..16384}) + 2 prefill chunks of 1024 with
    context 2048; Hq 64, Hkv 8, D 64; e4m3 cache with k_scale = v_scale = 0.05,
    page_size 32; sliding window 4096, soft cap 30, per-head sink ~ N(0,1);
    bf16 queries and new K/V (quantised by the update)."""
    rng = np.random.default_rng(seed)
    dkv = rng.integers(decode_kv[0], decode_kv[1], size=n_decode, endpoint=True)
    q = np.concatenate([np.ones(n_decode, np.int64), np.full(n_prefill, chunk, np.int64)])
    kv = np.concatenate([dkv, np.full(n_prefill, ctx + chunk, np.int64)])
    args = dict(num_q_heads=64, num_kv_heads=8, head_dim=64, page_size=32)
    args.update(kw)
    return build("fp8_full", q_lens=q, kv_lens=kv, distribution=(n_decode, n_prefill, 0),
                 q_dtype="bf16", kv_in_dtype="bf16", cache_dtype="fp8",
                 softmax_scale=1 / math.sqrt(args["head_dim"]), k_scale=0.05, v_scale=0.05,
                 sliding_window=sliding_window, logits_soft_cap=30.0, with_sink=True,
                 seed=seed, device=device, rng=rng, **args)


def long_decode_bf16(device="cpu", seed=1005, kv_len=131072, **kw) -> Workload:
    """One decode sequence over a long context: q_len 1, kv_len 131072;
    page_size 16; Hq 32, Hkv 8, D 128, bf16 (the decode workload's heads).
    Its single row is cut across the GPU and merged by log-sum-exp."""
    rng = np.random.default_rng(seed)
    args = dict(num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16)
    args.update(kw)
    return build("long_decode_bf16", q_lens=[1], kv_lens=[kv_len], distribution=(1, 0, 0),
                 q_dtype="bf16", kv_in_dtype="bf16", cache_dtype="bf16",
                 softmax_scale=1 / math.sqrt(args["head_dim"]), seed=seed, device=device,
                 rng=rng, **args)


def prefill_fp8q(device="cpu", seed=1006, n_seqs=2, seq_len=8192, q_scale=0.05, **kw) -> Workload:
    """The long-prefill shape with 8-bit queries and cache ("w8a8"): 2 seqs
    with q_len = kv_len = 8192, causal; Hq 64, Hkv 8, D 128, page_size 128;
    queries are e4m3 codes of N(0,1) / q_scale, the cache e4m3 with k_scale =
    v_scale = 0.05 (new K/V bf16 N(0,1), quantised by the update)."""
    rng = np.random.default_rng(seed)
    args = dict(num_q_heads=64, num_kv_heads=8, head_dim=128, page_size=128)
    args.update(kw)
    return build("prefill_fp8q", q_lens=[seq_len] * n_seqs, kv_lens=[seq_len] * n_seqs,
                 distribution=(0, n_seqs, 0), q_dtype="fp8", kv_in_dtype="bf16",
                 cache_dtype="fp8", softmax_scale=1 / math.sqrt(args["head_dim"]),
                 q_scale=q_scale, k_scale=0.05, v_scale=0.05, seed=seed, device=device,
                 rng=rng, **args)


def mixed_fp8q(device="cpu", seed=1007, n_decode=64, decode_kv=(512, 4096), n_prefill=4,
               chunk=384, ctx_max=2048, q_scale=0.05, **kw) -> Workload:
    """8-bit queries and cache over a mixed batch: 64 decode rows (kv ~
    U{512..4096}) + 4 prefill chunks of 384 tokens with context ~ U{0..2048};
    Hq 64, Hkv 8, D 128, page_size 32; window 1024, soft cap 30, sinks."""
    rng = np.random.default_rng(seed)
    dkv = rng.integers(decode_kv[0], decode_kv[1], size=n_decode, endpoint=True)
    ctx = rng.integers(0, ctx_max, size=n_prefill, endpoint=True)
    q = np.concatenate([np.ones(n_decode, np.int64), np.full(n_prefill, chunk, np.int64)])
    kv = np.concatenate([dkv, ctx + chunk])
    args = dict(num_q_heads=64, num_kv_heads=8, head_dim=128, page_size=32)
    args.update(kw)
    return build("mixed_fp8q", q_lens=q, kv_lens=kv, distribution=(n_decode, n_prefill, 0),
                 q_dtype="fp8", kv_in_dtype="bf16", cache_dtype="fp8",
                 softmax_scale=1 / math.sqrt(args["head_dim"]), q_scale=q_scale, k_scale=0.05,
                 v_scale=0.05, sliding_window=1024, logits_soft_cap=30.0, with_sink=True,
                 seed=seed, device=device, rng=rng, **args)


RECIPES = {
    "tiny_fp32": tiny_fp32,
    "decode_bf16": decode_bf16,
    "mixed_bf16": mixed_bf16,
    "prefill_bf16": prefill_bf16,
    "fp8_full": fp8_full,
    "long_decode_bf16": long_decode_bf16,
    "prefill_fp8q": prefill_fp8q,
    "mixed_fp8q": mixed_fp8q,
}

# Scaled-down variants with the same structure, for CPU oracle runs and fast
# GPU parity sweeps (several tiles and a ragged tail, but seconds of oracle).
SMALL = {
    "tiny_fp32": dict(),
    "decode_bf16": dict(num_seqs=16, kv_min=20, kv_max=300),
    "mixed_bf16": dict(n_decode=8, decode_kv=(40, 400), n_prefill=3, chunk=77, ctx_max=200),
    "prefill_bf16": dict(n_seqs=2, seq_len=300),
    "fp8_full": dict(n_decode=8, decode_kv=(40, 600), n_prefill=2, chunk=100, ctx=150,
                     sliding_window=128),
    "long_decode_bf16": dict(kv_len=5000),
    "prefill_fp8q": dict(n_seqs=2, seq_len=300),
    "mixed_fp8q": dict(n_decode=8, decode_kv=(40, 600), n_prefill=3, chunk=77, ctx_max=200),
}


def make(name: str, device="cpu", small: bool = False, **kw) -> Workload:
    args = dict(SMALL[name]) if small else {}
    args.update(kw)
    return RECIPES[name](device=device, **args)

"""Test helpers: bit views of torch tensors and a one-call oracle run on a
workload.  Shared by the CPU pin tests and the GPU parity tests."""
import numpy as np
import torch

from oracle import rpa_oracle as O

_VIEW = {"f32": (torch.int32, np.uint32), "bf16": (torch.int16, np.uint16),
         "fp8": (torch.uint8, np.uint8)}


def bits(t: torch.Tensor, dtype: str) -> np.ndarray:
    tv, nv = _VIEW[dtype]
    return t.detach().contiguous().view(tv).cpu().numpy().view(nv)


def oracle_forward(w, cache_bits=None, seqs=None, update=True):
    """Run the oracle on workload `w` (tensors may live on any device)."""
    if cache_bits is None:
        cache_bits = bits(w.kv_cache, w.cache_dtype)
    sink = None if w.attention_sink is None else w.attention_sink.cpu().numpy()
    return O.forward(
        bits(w.queries, w.q_dtype),
        bits(w.keys, w.kv_in_dtype) if update else None,
        bits(w.values, w.kv_in_dtype) if update else None,
        cache_bits, w.kv_lens, w.block_tables, w.query_start_loc, w.distribution,
        page_size=w.page_size, pages_per_seq=w.pages_per_seq, q_dtype=w.q_dtype,
        kv_in_dtype=w.kv_in_dtype, cache_dtype=w.cache_dtype, softmax_scale=w.softmax_scale,
        sliding_window=w.sliding_window, logits_soft_cap=w.logits_soft_cap, q_scale=w.q_scale,
        k_scale=w.k_scale, v_scale=w.v_scale, attention_sink=sink, seqs=seqs)


def oracle_update(w, cache_bits=None):
    if cache_bits is None:
        cache_bits = bits(w.kv_cache, w.cache_dtype)
    return O.update_kv_cache(
        cache_bits, bits(w.keys, w.kv_in_dtype), bits(w.values, w.kv_in_dtype), w.kv_lens,
        w.block_tables, w.query_start_loc, w.distribution, page_size=w.page_size,
        pages_per_seq=w.pages_per_seq, kv_in_dtype=w.kv_in_dtype, cache_dtype=w.cache_dtype,
        k_scale=w.k_scale, v_scale=w.v_scale)


def poison_unused(w, include_written=True):
    """Fill every cache slot that no query can see (after the update) with NaN
    (in place), so that any read outside the visible ranges shows in the
    output.  With `include_written`, slots the update overwrites are poisoned
    too (only valid when the call under test performs the update)."""
    used = O.visible_slots(w.kv_lens, w.block_tables, w.query_start_loc, w.distribution,
                           page_size=w.page_size, pages_per_seq=w.pages_per_seq,
                           num_pages=w.num_pages, sliding_window=w.sliding_window)
    written = O.written_slots(w.kv_lens, w.block_tables, w.query_start_loc, w.distribution,
                              page_size=w.page_size, pages_per_seq=w.pages_per_seq,
                              num_pages=w.num_pages)
    bad = torch.from_numpy((~used) | (written if include_written else False)).reshape(-1).to(w.kv_cache.device)
    flat = w.kv_cache.view(w.num_pages * w.page_size, -1)
    nan = {"f32": float("nan"), "bf16": float("nan")}
    if w.cache_dtype == "fp8":
        flat[bad] = 0x7F
    else:
        flat[bad] = nan[w.cache_dtype]
    return w


TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8": 6e-2}
# Relative L2 error bound ||out - ref|| / ||ref|| over the checked rows.  The
# absolute bounds above are loose for outputs whose rows average thousands of
# N(0,1) values (sigma ~ 0.03): a dropped or misplaced page can pass them.
# bf16 p and output rounding give about 2e-3 here.
REL_TOL = {"f32": 1e-5, "bf16": 1e-2, "fp8": 1e-2}


def tolerance(w):
    """Max-abs-error bound on the attention output: fp32 workloads 1e-5,
    bf16 2e-2, fp8-KV 6e-2."""
    return TOL["fp8"] if w.cache_dtype == "fp8" else TOL[w.q_dtype]


def rel_tolerance(w):
    return REL_TOL["fp8"] if w.cache_dtype == "fp8" else REL_TOL[w.q_dtype]


def check_output(name, w, out, ref, rows):
    """Assert the output rows `rows` against the oracle: max abs error within
    the dtype's bound, relative L2 error within REL_TOL, no NaN."""
    o = out[rows].double().cpu().numpy()
    r = ref[rows]
    err = float(np.abs(o - r).max()) if len(rows) else 0.0
    nr = float(np.linalg.norm(r))
    rel = float(np.linalg.norm(o - r)) / nr if nr > 0 else float(np.linalg.norm(o - r))
    print(f"[{name}] rows={len(rows)} max_abs={err:.3e} rel_l2={rel:.3e} "
          f"tol={tolerance(w):.0e}/{rel_tolerance(w):.0e}", flush=True)
    assert not np.isnan(o).any(), f"{name}: NaN in the output"
    assert err <= tolerance(w), f"{name}: max abs error {err:.3e}"
    assert rel <= rel_tolerance(w), f"{name}: relative L2 error {rel:.3e}"
    return err, rel


def gpu_forward(w, update=True, out=None, **kw):
    """Run rpa_forward on workload `w` (tensors on the GPU).  `out` is
    pre-filled with NaN so unwritten rows stay visible."""
    import ragged_paged_kv_scatter_amd as rpa
    dev = w.queries.device
    meta = {k: torch.from_numpy(np.ascontiguousarray(getattr(w, k))).to(dev)
            for k in ("kv_lens", "block_tables", "query_start_loc", "distribution")}
    if out is None:
        out = torch.full(w.queries.shape, float("nan"), dtype=rpa.out_dtype_for(w.queries.dtype),
                         device=dev)
    opts = w.options()
    opts.update(kw)
    rpa.rpa_forward(w.queries, w.keys if update else None, w.values if update else None,
                    w.kv_cache, meta["kv_lens"], meta["block_tables"], meta["query_start_loc"],
                    meta["distribution"], w.attention_sink, out=out, **opts)
    return out


def compact_pages(w, seqs, cache_dev=None):
    """Copy to the host only the pages the given sequences use, and a block
    table renumbered onto that compact pool (entries of other sequences 0).
    Returns (cache_bits, block_tables)."""
    cache_dev = w.kv_cache if cache_dev is None else cache_dev
    pps, ps = w.pages_per_seq, w.page_size
    bt = np.zeros_like(w.block_tables)
    pages = []
    index = {}
    for s in seqs:
        n = -(-int(w.kv_lens[s]) // ps)
        for i in range(n):
            p = int(w.block_tables[s * pps + i])
            if p not in index:
                index[p] = len(pages)
                pages.append(p)
            bt[s * pps + i] = index[p]
    sel = torch.tensor(pages if pages else [0], dtype=torch.long, device=cache_dev.device)
    sub = cache_dev.index_select(0, sel)
    return bits(sub, w.cache_dtype), bt

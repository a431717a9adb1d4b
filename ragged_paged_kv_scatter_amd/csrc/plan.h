// Device-side planner: reads the ragged metadata (query_start_loc, kv_lens,
// distribution) on the GPU, so no host synchronisation is needed, and writes
// the work lists of the attention kernels into the workspace:
//   * row items: pieces (query row, key range) for rows served by the row
//     kernel, grouped in equal chunks of keys, one chunk per wave and kv head;
//   * prefill items: (sequence, query tile) for the MFMA prefill kernel.
// One workgroup of 1024 threads; per-sequence tables live in LDS.
#pragma once

#include "device_common.h"
#include "rpa_internal.h"

namespace rpa {
namespace plan_detail {

constexpr int kT = kPlanThreads;
constexpr int kWaves = kT / 64;
// Rows cut into more pieces than this have them written by all lanes of
// their wave (one such row after another) rather than by their own thread.
// With at most kTargetItems chunks, at most kTargetItems / 64 rows of a step
// pass it, so the wave's walk over them stays short; a lower bound would
// serialise the many rows of a batch with a handful of pieces each.
constexpr int kWavePieces = 64;
// A row is cut into at most about kRowPieces pieces: chunks hold at least
// (longest row's visible keys) / kRowPieces keys.  One 200K-key row at Hkv 1
// in 128-, 256- and 512-key pieces ran 80, 51 and 41 us in all (the merge of
// its partials shrinks faster than the row kernel slows); batches of short
// rows keep the finer chunks their row kernel needs.
constexpr int kRowPieces = 256;

__device__ __forceinline__ int lane_value(int v, int lane) {
  return __builtin_amdgcn_readlane(v, lane);
}
__device__ __forceinline__ long long lane_value(long long v, int lane) {
  const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)v, lane);
  const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)((unsigned long long)v >> 32), lane);
  return (long long)(((unsigned long long)hi << 32) | lo);
}

// A DPP move of v from another lane; lanes that the row mask leaves out, or
// whose source lies outside their row of 16, get 0.  64-bit values move as
// two 32-bit halves.
template <int CTRL, int ROW_MASK, typename V>
__device__ __forceinline__ V dpp_or_zero(V v) {
  if constexpr (sizeof(V) == 4) {
    return (V)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, false);
  } else {
    const unsigned long long u = (unsigned long long)v;
    const unsigned lo = (unsigned)__builtin_amdgcn_update_dpp(0, (int)(unsigned)u, CTRL, ROW_MASK, 0xF, false);
    const unsigned hi = (unsigned)__builtin_amdgcn_update_dpp(0, (int)(unsigned)(u >> 32), CTRL, ROW_MASK, 0xF, false);
    return (V)(((unsigned long long)hi << 32) | lo);
  }
}

// Inclusive prefix sum over the 64 lanes of a wave (all lanes active), on
// VALU moves only: shifts by 1, 2, 4 and 8 within each row of 16 lanes give
// every row its own prefix; then lane 15's total goes into rows 1 and 3
// (row_bcast:15) and lane 31's, by now the total of rows 0-1, into rows 2
// and 3 (row_bcast:31).
template <typename V>
__device__ __forceinline__ V wave_inclusive_scan(V x) {
  x += dpp_or_zero<0x111, 0xF>(x);                  // row_shr:1
  x += dpp_or_zero<0x112, 0xF>(x);                  // row_shr:2
  x += dpp_or_zero<0x114, 0xF>(x);                  // row_shr:4
  x += dpp_or_zero<0x118, 0xF>(x);                  // row_shr:8
  x += dpp_or_zero<0x142, 0xA>(x);                  // row_bcast:15, rows 1 and 3
  x += dpp_or_zero<0x143, 0xC>(x);                  // row_bcast:31, rows 2 and 3
  return x;
}

// Inclusive running max over the 64 lanes of a wave for values >= 0 (lanes
// outside a shift's reach read 0, the identity), on the same DPP moves.
__device__ __forceinline__ int wave_inclusive_max(int x) {
  x = max(x, dpp_or_zero<0x111, 0xF>(x));
  x = max(x, dpp_or_zero<0x112, 0xF>(x));
  x = max(x, dpp_or_zero<0x114, 0xF>(x));
  x = max(x, dpp_or_zero<0x118, 0xF>(x));
  x = max(x, dpp_or_zero<0x142, 0xA>(x));
  x = max(x, dpp_or_zero<0x143, 0xC>(x));
  return x;
}

// Exclusive prefix sums over the workgroup in three steps, so that several
// sums share one pair of barriers:
//   scan_up    (all threads)  the wave's inclusive sum; lane 63 publishes
//                             the wave total in s_waves[wave];
//   barrier;
//   scan_waves (wave 0 only)  the wave totals -> their exclusive prefixes,
//                             the grand total in s_waves[kWaves];
//   barrier;
//   scan_down  (all threads)  this thread's exclusive prefix and the total.
// Entry w < kWaves of s_waves is read after the scan only by wave w, and the
// grand total is rewritten only behind the next scan's first barrier, so an
// array may serve the next scan with no barrier in between.
template <typename V>
__device__ __forceinline__ V scan_up(V v, V* s_waves) {
  const V x = wave_inclusive_scan(v);
  if ((threadIdx.x & 63) == 63) s_waves[threadIdx.x >> 6] = x;
  return x;
}
template <typename V>
__device__ __forceinline__ void scan_waves(V* s_waves) {
  const int lane = threadIdx.x & 63;
  const V t = lane < kWaves ? s_waves[lane] : V(0);
  const V inc = wave_inclusive_scan(t);
  if (lane < kWaves) s_waves[lane] = inc - t;
  if (lane == kWaves - 1) s_waves[kWaves] = inc;
}
template <typename V>
__device__ __forceinline__ V scan_down(V v, V x, const V* s_waves, V* total) {
  *total = s_waves[kWaves];
  return x - v + s_waves[threadIdx.x >> 6];
}

// One exclusive prefix sum over the workgroup; all threads must call it.
template <typename V>
__device__ V block_exclusive_scan(V v, V* total, V* s_waves) {
  const V x = scan_up(v, s_waves);
  __syncthreads();
  if (threadIdx.x < 64) scan_waves(s_waves);
  __syncthreads();
  return scan_down(v, x, s_waves, total);
}

// a / b for a >= 0, b > 0: a 32-bit division when both fit, as they do but
// for huge batches (the 64-bit one is a long instruction sequence, run here
// by every wave of the workgroup).
__device__ __forceinline__ long long div_nonneg(long long a, long long b) {
  if ((((unsigned long long)a | (unsigned long long)b) >> 32) == 0)
    return (long long)((unsigned)a / (unsigned)b);
  return a / b;
}

__device__ __forceinline__ long long visible_sum(int ctx, int q_len, int window) {
  // sum over t < q_len of the visible length of query t (position ctx + t):
  // min(ctx + t + 1, W) with a window, ctx + t + 1 without.
  long long q = q_len, c = ctx;
  if (window <= 0) return q * (c + 1) + q * (q - 1) / 2;
  long long n1 = min(max((long long)window - c, 0LL), q);
  return n1 * (c + 1) + n1 * (n1 - 1) / 2 + (q - n1) * (long long)window;
}

// The planner, run by one workgroup of kPlanThreads threads; s_seq_rows is
// dynamic LDS of plan_lds_words(max_num_seqs) words: the first row of each
// sequence and, when max_num_seqs <= kPlanCacheSeqs, the sequences' first
// query token and context length, so later passes need no global reads.
__device__ __forceinline__ void plan_body(const PlanParams& p, int32_t* s_seq_rows) {
  const bool cached = p.max_num_seqs <= kPlanCacheSeqs;
  int32_t* s_q0 = s_seq_rows + (p.max_num_seqs + 1);   // qsl[s], s <= num_seqs (cached)
  int32_t* s_ctx = s_q0 + (p.max_num_seqs + 1);        // kv_len - q_len (cached)
  __shared__ long long s_w64[kWaves + 1];
  __shared__ long long s_w64b[kWaves + 1];
  __shared__ int32_t s_w32[kWaves + 1];
  __shared__ int32_t s_w32b[kWaves + 1];
  __shared__ int32_t s_w32c[kWaves + 1];
  __shared__ int32_t s_wmax[kWaves + 1];             // longest row: wave maxima, then the block's
  __shared__ int32_t s_pf_first[kT + 1];            // a block's first prefill item per thread
  __shared__ int32_t s_pf_qlen[kT];

  char* ws = p.ws;
  PlanHeader* hdr = reinterpret_cast<PlanHeader*>(ws + p.lay.header);
  RowDesc* rows = reinterpret_cast<RowDesc*>(ws + p.lay.rows);
  ItemDesc* items = reinterpret_cast<ItemDesc*>(ws + p.lay.items);
  MergeDesc* merge_rows = reinterpret_cast<MergeDesc*>(ws + p.lay.merge_rows);
  PrefillItem* pf = reinterpret_cast<PrefillItem*>(ws + p.lay.pf_items);

  const int num_seqs = min(max(p.dist[0] + p.dist[1] + p.dist[2], 0), p.max_num_seqs);
  const int W = p.window;
  // zero row the prefill kernel reads for keys outside a tile's visible range
  for (int i = threadIdx.x; i < kZeroBytes / 4; i += kT)
    reinterpret_cast<int32_t*>(ws + p.lay.zeros)[i] = 0;

  // ---- pass 1: per-sequence row counts, prefill tiles, visible-key totals ----
  int row_base = 0, pf_base = 0;
  long long vis_total = 0, pf_vis_total = 0;
  int vmax_total = 0;                               // visible keys of the longest row
  for (int base = 0; base < num_seqs; base += kT) {
    const int s = base + threadIdx.x;
    int n_rows = 0, n_pf = 0, vmax = 0;
    long long vis = 0, pf_vis = 0;
    int q0 = 0, q_len = 0, ctx = 0;
    if (s < num_seqs) {
      q0 = p.qsl[s];
      q_len = p.qsl[s + 1] - q0;
      ctx = p.kv_lens[s] - q_len;
      if (cached) {
        s_q0[s] = q0;
        s_ctx[s] = ctx;
        if (s == num_seqs - 1) s_q0[num_seqs] = q0 + q_len;
      }
      if (q_len > 0) {
        if (q_len >= p.prefill_min_q) {
          n_pf = (q_len + kPrefillBQ - 1) / kPrefillBQ;
          pf_vis = visible_sum(ctx, q_len, W);
        } else {
          n_rows = q_len;
          vis = visible_sum(ctx, q_len, W);
          vmax = (W > 0) ? min(ctx + q_len, W) : ctx + q_len;   // its last row
        }
      }
    }
    int tot_rows, tot_pf;
    long long tot_vis, tot_pf_vis;
    const int x_rows = scan_up(n_rows, s_w32);
    const int x_pf = scan_up(n_pf, s_w32b);
    scan_up(vis, s_w64);
    scan_up(pf_vis, s_w64b);
    const int x_max = wave_inclusive_max(vmax);
    if ((threadIdx.x & 63) == 63) s_wmax[threadIdx.x >> 6] = x_max;
    __syncthreads();
    if (threadIdx.x < 64) {
      scan_waves(s_w32);
      scan_waves(s_w32b);
      scan_waves(s_w64);
      scan_waves(s_w64b);
      const int m = wave_inclusive_max(threadIdx.x < kWaves ? s_wmax[threadIdx.x] : 0);
      if (threadIdx.x == kWaves - 1) s_wmax[kWaves] = m;
    }
    __syncthreads();
    vmax_total = max(vmax_total, s_wmax[kWaves]);
    const int my_row = scan_down(n_rows, x_rows, s_w32, &tot_rows) + row_base;
    const int my_pf = scan_down(n_pf, x_pf, s_w32b, &tot_pf) + pf_base;
    tot_vis = s_w64[kWaves];
    tot_pf_vis = s_w64b[kWaves];
    if (s < num_seqs) s_seq_rows[s] = my_row;
    if (tot_pf > 0) {
      // the block's prefill items, written by all threads: item j belongs to
      // the last thread t whose first item is <= j (threads without tiles
      // share the next one's first item, threads past num_seqs have tot_pf)
      s_pf_first[threadIdx.x] = my_pf - pf_base;
      s_pf_qlen[threadIdx.x] = q_len;
      if (threadIdx.x == 0) s_pf_first[kT] = tot_pf;
      __syncthreads();
      for (int j = threadIdx.x; j < tot_pf; j += kT) {
        int a = 0, b = min(kT, num_seqs - base) - 1;
        while (a < b) {
          const int mid = (a + b + 1) >> 1;
          if (s_pf_first[mid] <= j) a = mid; else b = mid - 1;
        }
        // heaviest tiles first within a sequence (causal: later tiles see more keys)
        const int tile = s_pf_first[a + 1] - 1 - j;
        PrefillItem it;
        it.seq = base + a;
        it.q_begin = tile * kPrefillBQ;
        it.q_end = min(s_pf_qlen[a], (tile + 1) * kPrefillBQ);
        it.pad = 0;
        if (pf_base + j < p.lay.max_pf_items) pf[pf_base + j] = it;
      }
    }
    row_base += tot_rows;
    pf_base += tot_pf;
    vis_total += tot_vis;
    pf_vis_total += tot_pf_vis;
  }
  if (threadIdx.x == 0) s_seq_rows[num_seqs] = row_base;
  __syncthreads();
  const int n_rows = min(row_base, p.lay.max_rows);

  // ---- chunks: the visible key ranges of all rows, in row order, form one
  // stream of vis_total keys, cut into n_chunks chunks of C keys (the last one
  // shorter); a chunk is the work of one wave per kv head, so the waves of the
  // row kernel get equal work, and only rows cut by a chunk boundary leave
  // split partials to merge. ----
  // Side by side: when the batch has both decode rows and prefill tiles and
  // the rows' HBM time (KV bytes at ~6 TB/s) is at least the tiles' MFMA time
  // (4 D FLOPs per visible (query, key, q head) at ~1 PFLOP/s), the row kernel
  // keeps kCoRowEighths / 8 of its resident waves and the prefill kernel,
  // running at the same time on another stream, takes the rest of the CUs.
  const long long dec_bytes = vis_total * 2 * p.Hkv * p.D * p.kv_elem;
  const long long pf_flops = pf_vis_total * 4 * p.D * p.Hq;
  const bool co_run = p.co_allowed && row_base > 0 && pf_base > 0 &&
                      dec_bytes * 500 >= pf_flops * 3;
  const long long want = row_chunks_max(co_run ? p.row_waves / 8 * kCoRowEighths : p.row_waves, p.Hkv);
  long long C = div_nonneg(vis_total + want - 1, want);
  if (C < kMinSplit) C = kMinSplit;
  if (C < div_nonneg(vmax_total + kRowPieces - 1, kRowPieces))
    C = div_nonneg(vmax_total + kRowPieces - 1, kRowPieces);
  // (C >= vis_total / want keeps this within `want`, which is at most the
  // layout's max_chunks: the bound only guards the chunk table)
  const int n_chunks = (int)min(div_nonneg(vis_total + C - 1, C), (long long)p.lay.max_chunks);
  int32_t* chunk_first = reinterpret_cast<int32_t*>(ws + p.lay.chunks);

  // row r -> (seq, token, visible range [lo, hi))
  auto row_info = [&](int r, int& seq, int& token, int& lo, int& hi) {
    int a = 0, b = num_seqs - 1;                    // largest s with s_seq_rows[s] <= r
    while (a < b) {
      const int mid = (a + b + 1) >> 1;
      if (s_seq_rows[mid] <= r) a = mid; else b = mid - 1;
    }
    seq = a;
    const int t = r - s_seq_rows[seq];
    int q0, pos;
    if (cached) {
      q0 = s_q0[seq];
      pos = s_ctx[seq] + t;
    } else {
      q0 = p.qsl[seq];
      const int q_len = p.qsl[seq + 1] - q0;
      pos = p.kv_lens[seq] - q_len + t;
    }
    token = q0 + t;
    hi = pos + 1;
    lo = (W > 0) ? max(0, pos - W + 1) : 0;
  };

  // ---- pass 2: rows and their pieces (the parts of a row in different chunks) ----
  long long stream_base = 0;
  int item_base = 0, part_base = 0, merge_base = 0;
  for (int base = 0; base < n_rows; base += kT) {
    const int r = base + threadIdx.x;
    int seq = 0, token = 0, lo = 0, hi = 0;
    long long len = 0;
    if (r < n_rows) {
      row_info(r, seq, token, lo, hi);
      len = hi - lo;                                  // >= 1: a row sees its own key
    }
    long long tot_len;
    const long long off = block_exclusive_scan(len, &tot_len, s_w64) + stream_base;
    const long long c0 = div_nonneg(off, C);
    const int n_split = (r < n_rows) ? (int)(div_nonneg(off + len - 1, C) - c0 + 1) : 0;
    const int v_part = n_split > 1 ? n_split : 0, v_merge = n_split > 1 ? 1 : 0;
    int tot_items, tot_parts, tot_merge;
    const int x_item = scan_up(n_split, s_w32);
    const int x_part = scan_up(v_part, s_w32b);
    const int x_merge = scan_up(v_merge, s_w32c);
    __syncthreads();
    if (threadIdx.x < 64) {
      scan_waves(s_w32);
      scan_waves(s_w32b);
      scan_waves(s_w32c);
    }
    __syncthreads();
    const int my_item = scan_down(n_split, x_item, s_w32, &tot_items) + item_base;
    const int my_part = scan_down(v_part, x_part, s_w32b, &tot_parts) + part_base;
    const int my_merge = scan_down(v_merge, x_merge, s_w32c, &tot_merge) + merge_base;
    // piece j of a row: its part of chunk c0 + j; the piece that starts a
    // chunk is that chunk's first item
    auto write_piece = [&](int j, long long off_r, long long len_r, long long c0_r, int lo_r,
                           int token_r, int seq_r, int item_r, int part_r, int n_split_r,
                           int r_r) {
      const int slot = item_r + j;
      if (slot >= p.lay.max_items) return;
      const long long s0 = max(off_r, (c0_r + j) * C);
      const long long s1 = min(off_r + len_r, (c0_r + j + 1) * C);
      ItemDesc it;
      it.token = token_r;
      it.seq = seq_r;
      it.lo = lo_r + (int)(s0 - off_r);
      it.hi = lo_r + (int)(s1 - off_r);
      it.part = n_split_r > 1 ? part_r + j : -1;
      it.row = r_r;
      it.pad[0] = it.pad[1] = 0;
      items[slot] = it;
      if (s0 == (c0_r + j) * C && c0_r + j < n_chunks) chunk_first[c0_r + j] = slot;
    };
    const bool heavy = n_split > kWavePieces;
    if (r < n_rows) {
      RowDesc rd;
      rd.token = token;
      rd.seq = seq;
      rd.lo = lo;
      rd.hi = hi;
      rd.n_split = n_split;
      rd.part_base = n_split > 1 ? my_part : -1;
      rd.pad[0] = rd.pad[1] = 0;
      rows[r] = rd;
      if (!heavy)
        for (int j = 0; j < n_split; ++j)
          write_piece(j, off, len, c0, lo, token, seq, my_item, my_part, n_split, r);
      if (n_split > 1 && my_merge < p.lay.max_merge_rows) {
        MergeDesc md;
        md.token = token;
        md.part_base = my_part;
        md.n_split = n_split;
        md.pad = 0;
        merge_rows[my_merge] = md;
      }
    }
    // the heavy rows of this wave, one after another, by all 64 lanes
    for (unsigned long long m = __ballot(heavy); m != 0; m &= m - 1) {
      const int L = __builtin_ctzll(m);
      const int n_L = lane_value(n_split, L);
      const long long off_L = lane_value(off, L), len_L = lane_value(len, L),
                      c0_L = lane_value(c0, L);
      const int lo_L = lane_value(lo, L), token_L = lane_value(token, L),
                seq_L = lane_value(seq, L), item_L = lane_value(my_item, L),
                part_L = lane_value(my_part, L), r_L = lane_value(r, L);
      for (int j = threadIdx.x & 63; j < n_L; j += 64)
        write_piece(j, off_L, len_L, c0_L, lo_L, token_L, seq_L, item_L, part_L, n_L, r_L);
    }
    stream_base += tot_len;
    item_base += tot_items;
    part_base += tot_parts;
    merge_base += tot_merge;
  }
  // chunks that hold keys (all of them unless rows were cut off at max_rows)
  const int n_chunks_laid = (int)min((long long)n_chunks, div_nonneg(stream_base + C - 1, C));
  if (threadIdx.x == 0) {
    chunk_first[n_chunks_laid] = min(item_base, p.lay.max_items);
    PlanHeader h = {};
    h.num_seqs = num_seqs;
    h.n_rows = n_rows;
    h.n_items = min(item_base, p.lay.max_items);
    h.split = (int)min(C, (long long)0x7fffffff);
    h.n_chunks = n_chunks_laid;
    h.n_merge_rows = min(merge_base, p.lay.max_merge_rows);
    h.n_pf_items = min(pf_base, p.lay.max_pf_items);
    h.row_next = 0;
    h.pf_next = 0;
    h.co_run = co_run ? 1 : 0;
    *hdr = h;
  }
}

}  // namespace plan_detail

using plan_detail::plan_body;

}  // namespace rpa

// Split planner, argument checks and the host-only helpers of the C ABI.
//
// The split rule follows PR "perf: scale prefill attention splits with GPU
// cores on Apple7/8" ("What changed"): aim for a number of threadgroups per
// core, cap the threadgroups per KV head at the tile slots a full 2048-row
// chunk already uses (so the workspace bound does not grow), divide by the
// piece's row tiles and clamp.  On MI355X one attention workgroup fills a CU
// (it holds 128 KB of LDS at head_dim 256), so the target is one workgroup
// per CU over 256 CUs.
#include "plan.h"

#include <stdlib.h>

namespace ppa {

int log2_exact(int32_t v) {
  if (v <= 0 || (v & (v - 1)) != 0) return -1;
  int r = 0;
  while ((1 << r) < v) ++r;
  return r;
}

int check_shape(const Shape& s) {
  if (s.dtype != PPA_F16 && s.dtype != PPA_BF16) return PPA_ERR_BAD_DTYPE;
  if (s.rows < 0 || s.history < 0 || s.n_q_heads < 1 || s.n_kv_heads < 1) return PPA_ERR_BAD_SHAPE;
  if (s.n_q_heads % s.n_kv_heads != 0) return PPA_ERR_BAD_SHAPE;
  if (s.head_dim != 64 && s.head_dim != 128 && s.head_dim != 256) return PPA_ERR_UNSUPPORTED;
  const int lps = log2_exact(s.page_size);
  if (lps < 0 || lps > 10) return PPA_ERR_UNSUPPORTED;
  // 32-bit index ranges used on the device: token positions, q/out elements.
  const int64_t ctx = s.history + s.rows;
  if (ctx + 2 * kKvTile >= (int64_t(1) << 31)) return PPA_ERR_TOO_LARGE;
  if (int64_t(s.rows) * s.n_q_heads * s.head_dim >= (int64_t(1) << 31)) return PPA_ERR_TOO_LARGE;
  return PPA_OK;
}

int64_t max_workspace_bytes() {
  const char* env = getenv("PPA_MAX_WORKSPACE_BYTES");
  if (env && *env) {
    char* end = nullptr;
    long long v = strtoll(env, &end, 10);
    if (end != env && v >= 0) return v;
  }
  return int64_t(2) << 30;
}

static int split_rule(int32_t cores, int32_t kv_heads, int32_t tiles, int32_t per_core,
                      int32_t floor_tg, int32_t slot_cap, int32_t max_splits) {
  const int64_t want = int64_t(per_core) * cores / kv_heads;
  int64_t per_head = want > floor_tg ? want : floor_tg;
  if (per_head > slot_cap) per_head = slot_cap;
  int64_t splits = per_head / tiles;
  if (splits < 1) splits = 1;
  if (splits > max_splits) splits = max_splits;
  return int(splits);
}

// Split workspace and merge grid of a plan with n_eff splits over ws_rows rows.
static void plan_workspace(const Shape& s, int64_t n_eff, int64_t ws_rows, int64_t grid_rows, int32_t n_seqs,
                           ppa_plan* out) {
  if (n_eff > 1) {
    const int64_t pairs = ws_rows * s.n_q_heads;
    const int64_t o_bytes = (n_eff * pairs * s.head_dim * 4 + 255) / 256 * 256;
    const int64_t lse_bytes = (n_eff * pairs * 4 + 255) / 256 * 256;
    out->workspace_bytes = o_bytes + lse_bytes;
    const int threads_per_pair = s.head_dim / 4 * merge_groups_for(int(n_eff));
    const int pairs_per_block = merge_block_threads(s.head_dim, int(n_eff)) / threads_per_pair;
    out->merge_grid = int32_t((grid_rows * s.n_q_heads + pairs_per_block - 1) / pairs_per_block * n_seqs);
  } else {
    out->workspace_bytes = 0;
    out->merge_grid = 0;
  }
}

// The plan of a launch: split units from the longest context `ctx`, the
// split rule's m tiles `rule_tiles`, the grid's m tiles from `grid_rows`, the
// workspace from `ws_rows`, times `n_seqs` sequences.
static int plan_launch(const Shape& s, int64_t ctx, int64_t rule_tiles, int64_t grid_rows,
                       int64_t ws_rows, int32_t n_seqs, int32_t n_splits_req, int64_t max_ws_bytes,
                       ppa_plan* out) {
  const int32_t group = s.n_q_heads / s.n_kv_heads;
  const int32_t unit = s.page_size > kKvTile ? s.page_size : kKvTile;
  const int64_t n_units = (ctx + unit - 1) / unit;
  const int32_t mt = m_tile_for(s.head_dim, s.q8 != 0, grid_rows * group);
  const int64_t tiles_m = (grid_rows * group + mt - 1) / mt;
  int64_t splits;
  if (n_splits_req <= 0) {
    const int32_t cap = int32_t((int64_t(kChunkRowsForCap) * group + mt - 1) / mt);
    const int64_t t = rule_tiles < 1 ? 1 : rule_tiles > cap ? cap : rule_tiles;
    splits = split_rule(kNumCUs, s.n_kv_heads, int32_t(t), kWgPerCu, 1, cap, kMaxSplits);
  } else {
    splits = n_splits_req;
  }
  if (splits > n_units) splits = n_units;
  if (splits < 1) splits = 1;
  const int64_t units_per_split = (n_units + splits - 1) / splits;
  const int64_t split_tokens = units_per_split * unit;
  int64_t n_eff = split_tokens > 0 ? (ctx + split_tokens - 1) / split_tokens : 1;
  if (n_eff < 1) n_eff = 1;
  if (split_tokens >= (int64_t(1) << 31)) return PPA_ERR_TOO_LARGE;
  out->n_splits = int32_t(n_eff);
  out->split_tokens = int32_t(split_tokens);
  out->m_tile = mt;
  out->kv_tile = kKvTile;
  out->tiles_m = int32_t(tiles_m);
  const int64_t grid = tiles_m * s.n_kv_heads * n_eff * n_seqs;
  if (grid >= (int64_t(1) << 31)) return PPA_ERR_TOO_LARGE;
  out->grid = int32_t(grid);
  out->reserved = 0;
  if (n_eff > 1 && n_eff * ws_rows * s.n_q_heads * s.head_dim >= (int64_t(1) << 31)) return PPA_ERR_TOO_LARGE;
  // the merge kernel: groups of head_dim / 4 threads per pair (4 groups for
  // 16 splits or more, else 1); with several sequences one row of blocks per
  // sequence
  plan_workspace(s, n_eff, ws_rows, grid_rows, n_seqs, out);
  if (n_eff > 1 && n_splits_req > 0 && out->workspace_bytes > max_ws_bytes) return PPA_ERR_WORKSPACE;
  return PPA_OK;
}

// The narrow kernel's plan: splits of whole 32-key tiles (and whole pages),
// one workgroup per CU over the KV heads unless the splits would get fewer
// than kNarrowMinKeys keys, at most kNarrowPages pages per split.  Returns 1
// (not planned) when the call needs more than kNarrowMaxSplits splits, or
// when a planner-chosen split count needs more workspace than the cap.
static int plan_narrow(const Shape& s, int64_t ctx, int64_t grid_rows, int64_t ws_rows, int32_t n_seqs,
                       int64_t busy_seqs, int32_t n_splits_req, int64_t max_ws_bytes, ppa_plan* out) {
  const int32_t unit = s.page_size > kNarrowTile ? s.page_size : kNarrowTile;
  const int64_t n_units = (ctx + unit - 1) / unit;
  int64_t splits;
  if (n_splits_req <= 0) {
    // one workgroup per CU over the sequences that have rows and the KV heads
    const int64_t wgs = (busy_seqs < 1 ? 1 : busy_seqs) * s.n_kv_heads;
    splits = (kNumCUs + wgs - 1) / wgs;
    const int64_t by_keys = (ctx + kNarrowMinKeys - 1) / kNarrowMinKeys;
    if (splits > by_keys) splits = by_keys;
  } else {
    splits = n_splits_req;
  }
  if (splits > n_units) splits = n_units;
  if (splits < 1) splits = 1;
  int64_t units_per_split = (n_units + splits - 1) / splits;
  const int64_t max_units = int64_t(kNarrowPages) * s.page_size / unit;
  if (units_per_split > max_units) units_per_split = max_units;
  const int64_t split_tokens = units_per_split * unit;
  const int64_t n_eff = (ctx + split_tokens - 1) / split_tokens;
  if (n_eff > kNarrowMaxSplits || n_eff * ws_rows * s.n_q_heads * s.head_dim >= (int64_t(1) << 31) ||
      n_eff * s.n_kv_heads * n_seqs >= (int64_t(1) << 31))
    return 1;
  out->n_splits = int32_t(n_eff < 1 ? 1 : n_eff);
  out->split_tokens = int32_t(split_tokens);
  out->m_tile = kNarrowVectors;
  out->kv_tile = kNarrowTile;
  out->tiles_m = 1;
  out->grid = int32_t(s.n_kv_heads * out->n_splits * int64_t(n_seqs));
  out->reserved = 0;
  plan_workspace(s, out->n_splits, ws_rows, grid_rows, n_seqs, out);
  // past the workspace cap: an error for a requested split count; the prefill
  // kernel's plan (whose splits are capped by the full-chunk bound) otherwise
  if (out->workspace_bytes > max_ws_bytes) return n_splits_req > 0 ? PPA_ERR_WORKSPACE : 1;
  return PPA_OK;
}

// m tiles of `rows` rows with the m tile a launch of `grid_rows` rows uses
static int64_t m_tiles(int64_t rows, int64_t grid_rows, const Shape& s) {
  const int64_t group = s.n_q_heads / s.n_kv_heads;
  const int32_t mt = m_tile_for(s.head_dim, s.q8 != 0, grid_rows * group);
  return (rows * group + mt - 1) / mt;
}

int make_plan(const Shape& s, int32_t n_splits_req, int64_t max_ws_bytes, ppa_plan* out) {
  if (s.allow_narrow && narrow_call(s.rows, s.n_q_heads / s.n_kv_heads, s.page_size, s.q8 != 0)) {
    const int rc = plan_narrow(s, s.history + s.rows, s.rows, s.rows, 1, 1, n_splits_req, max_ws_bytes, out);
    if (rc <= 0) return rc;
  }
  return plan_launch(s, s.history + s.rows, m_tiles(s.rows, s.rows, s), s.rows, s.rows, 1, n_splits_req,
                     max_ws_bytes, out);
}

int make_plan_varlen(const Shape& s, int32_t n_seqs, int32_t max_rows, int64_t max_context,
                     int32_t n_splits_req, int64_t max_ws_bytes, ppa_plan* out) {
  // A batch of decode steps (every sequence with few query vectors per KV
  // head, see narrow_call): the narrow kernel, splits over the longest context
  // for the sequences that can have rows (at most total_rows of them).
  if (s.allow_narrow && narrow_call(max_rows, s.n_q_heads / s.n_kv_heads, s.page_size, s.q8 != 0)) {
    const int64_t busy = n_seqs < s.rows ? n_seqs : s.rows;
    const int rc = plan_narrow(s, max_context, max_rows, s.rows, n_seqs, busy, n_splits_req, max_ws_bytes, out);
    if (rc <= 0) return rc;
  }
  // Every sequence with rows has at least one m tile of its own, and at most
  // total_rows sequences have rows: the split rule counts at least that many.
  int64_t tiles = m_tiles(s.rows, max_rows, s);
  const int64_t nonempty = n_seqs < s.rows ? n_seqs : s.rows;
  if (tiles < nonempty) tiles = nonempty;
  return plan_launch(s, max_context, tiles, max_rows, s.rows, n_seqs, n_splits_req, max_ws_bytes,
                     out);
}

}  // namespace ppa

extern "C" {

int paged_prefill_plan(int64_t history_len, int32_t chunk_rows, int32_t n_q_heads,
                       int32_t n_kv_heads, int32_t head_dim, int32_t page_size,
                       int32_t n_splits_req, ppa_plan* plan_out) {
  if (!plan_out) return PPA_ERR_NULL_PTR;
  ppa::Shape s{history_len, chunk_rows, n_q_heads, n_kv_heads, head_dim, page_size, PPA_F16};
  int rc = ppa::check_shape(s);
  if (rc != PPA_OK) return rc;
  if (n_splits_req < 0) return PPA_ERR_BAD_SHAPE;
  return ppa::make_plan(s, n_splits_req, ppa::max_workspace_bytes(), plan_out);
}

int paged_prefill_plan_varlen(int32_t n_seqs, int32_t total_rows, int32_t max_rows,
                              int64_t max_context, int32_t n_q_heads, int32_t n_kv_heads,
                              int32_t head_dim, int32_t page_size, int32_t n_splits_req,
                              ppa_plan* plan_out) {
  if (!plan_out) return PPA_ERR_NULL_PTR;
  if (n_seqs < 1 || total_rows < 1 || max_rows < 1 || max_rows > total_rows ||
      max_context < max_rows || n_splits_req < 0)
    return PPA_ERR_BAD_SHAPE;
  if (n_seqs > 65535) return PPA_ERR_TOO_LARGE;
  ppa::Shape s{max_context > total_rows ? max_context - total_rows : 0, total_rows, n_q_heads,
               n_kv_heads, head_dim, page_size, PPA_F16};
  int rc = ppa::check_shape(s);
  if (rc != PPA_OK) return rc;
  ppa::Shape ps{0, total_rows, n_q_heads, n_kv_heads, head_dim, page_size, PPA_F16};
  return ppa::make_plan_varlen(ps, n_seqs, max_rows, max_context, n_splits_req,
                               ppa::max_workspace_bytes(), plan_out);
}

int paged_prefill_split_rule(int32_t gpu_cores, int32_t kv_heads, int32_t tiles, int32_t per_core,
                             int32_t floor_tg, int32_t slot_cap, int32_t max_splits) {
  if (gpu_cores < 1 || kv_heads < 1 || tiles < 1 || per_core < 1 || floor_tg < 1 ||
      slot_cap < 1 || max_splits < 1)
    return PPA_ERR_BAD_SHAPE;
  return ppa::split_rule(gpu_cores, kv_heads, tiles, per_core, floor_tg, slot_cap, max_splits);
}

int32_t paged_prefill_piece_rows(int64_t history_len, int32_t chunk_rows, int64_t budget) {
  if (budget <= 0) budget = int64_t(1) << 25;
  if (chunk_rows < 1 || history_len < 0) return chunk_rows < 0 ? 0 : chunk_rows;
  int64_t rows = chunk_rows;
  while (rows > 1 && rows * (history_len + rows) > budget) rows /= 2;
  return int32_t(rows);
}

int paged_prefill_check_block_table(const int32_t* bt, int64_t n_entries, int64_t n_pool_pages) {
  if (n_entries < 0 || n_pool_pages < 0) return PPA_ERR_BAD_SHAPE;
  if (n_entries == 0) return PPA_OK;
  if (!bt) return PPA_ERR_NULL_PTR;
  for (int64_t i = 0; i < n_entries; ++i)
    if (bt[i] < 0 || bt[i] >= n_pool_pages) return PPA_ERR_BLOCK_TABLE;
  return PPA_OK;
}

const char* paged_prefill_strerror(int code) {
  switch (code) {
    case PPA_OK: return "ok";
    case PPA_ERR_NULL_PTR: return "a required pointer is NULL";
    case PPA_ERR_BAD_SHAPE: return "bad shape (negative size, heads < 1 or Hq not a multiple of Hkv)";
    case PPA_ERR_UNSUPPORTED: return "unsupported head_dim (64/128/256) or page_size (power of two, 1..1024)";
    case PPA_ERR_BAD_DTYPE: return "dtype must be PPA_F16 or PPA_BF16";
    case PPA_ERR_WORKSPACE: return "split workspace too large or its allocation failed";
    case PPA_ERR_HIP: return "HIP runtime error";
    case PPA_ERR_BLOCK_TABLE: return "block-table entry outside the page pool";
    case PPA_ERR_ALIGNMENT: return "tensor pointer not 16-byte aligned";
    case PPA_ERR_ALIAS: return "out overlaps q";
    case PPA_ERR_TOO_LARGE: return "size beyond the kernels' 32-bit index range";
    default: return "unknown status";
  }
}

int paged_prefill_version(void) { return 1 * 10000 + 1 * 100 + 0; }

}  // extern "C"

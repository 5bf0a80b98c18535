// Host-side planning and argument checks.  HIP-free: builds with g++ alone so
// the planner is testable without a GPU.
#pragma once
#include <stdint.h>

#include "paged_prefill.h"

namespace ppa {

// Work decomposition of the attention kernel (fixed by the kernel design).
// Query vectors per workgroup: 4 waves x 32 x query blocks per wave.  Two
// blocks for head_dim <= 128 (not for 8-bit pages at 128) when the call has
// more query vectors (rows x heads per KV head) than one 128-vector tile,
// else one; the attention kernel is built for both.
constexpr int m_tile_for(int head_dim, bool q8, int64_t query_vectors) {
  const bool two = head_dim <= 64 || (head_dim <= 128 && !q8);
  return two && query_vectors > 128 ? 256 : 128;
}
constexpr int kKvTile = 64;      // keys per inner-loop tile
constexpr int kThreads = 256;    // threads per workgroup
constexpr int kNumCUs = 256;     // MI355X compute units
constexpr int kWgPerCu = 1;      // resident attention workgroups per CU (LDS/VGPR bound)
constexpr int kMaxSplits = 128;
constexpr int kChunkRowsForCap = 2048;  // the cap: tile slots of a full 2048-row chunk

// Thread groups per (row, head) pair in the merge kernel: 16 for
// kMergeSixteenGroups splits or more (decode steps: a few pairs, many splits),
// 4 for kMergeFourGroups or more, else 1; a merge block has max(256, threads
// per pair) threads (the planner sizes the merge grid by these).
constexpr int kMergeFourGroups = 16;
constexpr int kMergeSixteenGroups = 64;
constexpr int merge_groups_for(int n_splits) {
  return n_splits >= kMergeSixteenGroups ? 16 : n_splits >= kMergeFourGroups ? 4 : 1;
}
constexpr int merge_block_threads(int head_dim, int n_splits) {
  return head_dim / 4 * merge_groups_for(n_splits) > 256 ? head_dim / 4 * merge_groups_for(n_splits) : 256;
}

// The narrow kernel (decode steps, appends of a few rows): calls (or
// sequences of a batch) with few query vectors (rows x Hq/Hkv) per KV head
// and pages of 8 tokens or more: at most kNarrowVectors over 8-bit pages, at
// most kNarrowVectors16 over 16-bit K/V (from 17 to 32 the prefill kernel,
// which shares each K/V tile among its waves, measured 4-8% faster there;
// over 8-bit pages the narrow kernel, which widens in registers, is 1.2-1.6x
// faster).  A workgroup is one (split, KV head); its waves stream 32-key
// tiles and keep the pages of their split (at most kNarrowPages) in
// registers.  The planner aims at one workgroup per CU with at least
// kNarrowMinKeys keys per split.  A narrow plan has m_tile kNarrowVectors.
constexpr int kNarrowVectors = 32;
constexpr int kNarrowVectors16 = 16;
constexpr int kNarrowTile = 32;
constexpr int kNarrowPages = 128;
constexpr int kNarrowMinKeys = 256;
constexpr int kNarrowMaxSplits = 4096;
constexpr bool narrow_call(int64_t rows, int64_t group, int32_t page_size, bool q8) {
  return rows * group <= (q8 ? kNarrowVectors : kNarrowVectors16) && page_size >= 8;
}

struct Shape {
  int64_t history;
  int32_t rows, n_q_heads, n_kv_heads, head_dim, page_size, dtype;
  int32_t q8 = 0;            // 8-bit K/V pages (changes the m tile at head_dim 128)
  int32_t allow_narrow = 1;  // 0: plan for the prefill kernel whatever the size
};

// Shape checks shared by every entry point (no pointers).
int check_shape(const Shape& s);

// The plan for a call; assumes check_shape passed.  max_ws_bytes bounds an
// explicitly requested split count.  A narrow call (see narrow_call) gets
// m_tile = kv_tile = 32 and grid = Hkv * n_splits.
int make_plan(const Shape& s, int32_t n_splits_req, int64_t max_ws_bytes, ppa_plan* out);

// The plan of a launch over n_seqs sequences: s.rows is the total row
// count, max_rows the longest sequence's rows, max_context the longest
// history + rows.  Splits are cut for max_context; shorter sequences use the
// leading ones.
int make_plan_varlen(const Shape& s, int32_t n_seqs, int32_t max_rows, int64_t max_context,
                     int32_t n_splits_req, int64_t max_ws_bytes, ppa_plan* out);

// Split workspace cap: PPA_MAX_WORKSPACE_BYTES or 2 GiB.
int64_t max_workspace_bytes();

int log2_exact(int32_t v);  // log2 of a power of two, -1 otherwise

}  // namespace ppa

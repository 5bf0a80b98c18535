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

// Thread groups per (row, head) pair in the merge kernel: 4 for kMergeFourGroups
// splits or more, else 1 (the planner sizes the merge grid by it).
constexpr int kMergeFourGroups = 16;
constexpr int merge_groups_for(int n_splits) { return n_splits >= kMergeFourGroups ? 4 : 1; }

struct Shape {
  int64_t history;
  int32_t rows, n_q_heads, n_kv_heads, head_dim, page_size, dtype;
  int32_t q8 = 0;  // 8-bit K/V pages (changes the m tile at head_dim 128)
};

// Shape checks shared by every entry point (no pointers).
int check_shape(const Shape& s);

// The plan for a call; assumes check_shape passed.  max_ws_bytes bounds an
// explicitly requested split count.
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

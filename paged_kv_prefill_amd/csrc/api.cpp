// C ABI entry points: argument checks, planning, the split workspace and the
// kernel launches.  Every step of the computation runs in the HIP kernels
// (attention*.hip, kv_append.hip); this file only validates, plans and
// enqueues.
#include <hip/hip_runtime.h>
#include <stdlib.h>
#include <string.h>

#include <cmath>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "kernels.h"
#include "paged_prefill.h"
#include "plan.h"
#include "workspace.h"

namespace ppa {
namespace {

// hipMalloc / hipFree for the workspace registry.
struct HipAlloc {
  void* alloc(int64_t bytes) {
    void* p = nullptr;
    if (hipMalloc(&p, size_t(bytes)) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
    return p;
  }
  bool free(void* p) { return hipFree(p) == hipSuccess; }
};

using Registry = WorkspaceRegistry<std::pair<int, hipStream_t>, HipAlloc>;

Registry& registry() {
  static Registry r;
  return r;
}

// Where a call's split workspace comes from: the (device, stream) registry
// (grow-only, held for the whole call), or the library's fixed device array
// (no allocation; calls that need more than it holds are rejected).
struct WsSource {
  bool fixed_array = false;
  void* ws = nullptr;       // a buffer the caller holds (its capacity below), or null
  int64_t ws_bytes = 0;
};

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool env_validate() {
  const char* e = getenv("PPA_VALIDATE");
  return e && e[0] == '1';
}

// Host check of the device block table (PPA_VALIDATE=1): the pool size is
// not an argument, so only negative entries can be rejected here.
int validate_block_table(const int32_t* bt_dev, int64_t n_entries, hipStream_t stream) {
  std::vector<int32_t> host(size_t(n_entries > 0 ? n_entries : 0));
  if (n_entries > 0) {
    if (hipMemcpyAsync(host.data(), bt_dev, size_t(n_entries) * 4, hipMemcpyDeviceToHost, stream) !=
        hipSuccess)
      return PPA_ERR_HIP;
    if (hipStreamSynchronize(stream) != hipSuccess) return PPA_ERR_HIP;
  }
  for (int32_t v : host)
    if (v < 0) return PPA_ERR_BLOCK_TABLE;
  return PPA_OK;
}

// Scale pools of 8-bit K/V pages (null: 16-bit pages).
struct Q8Scales {
  const void* k;
  const void* v;
};

// kv16: k and v are contiguous fp16 (8-bit pages dequantized beforehand)
// whatever dtype says about q and out.
int run(const void* q, const void* k, const void* v, const int32_t* bt, bool paged,
        int64_t history, int32_t rows, int32_t hq, int32_t hkv, int32_t d, int32_t ps,
        int32_t n_splits, void* out, int32_t dtype, hipStream_t stream, const Q8Scales* q8 = nullptr,
        const WsSource& wsrc = WsSource(), bool kv16 = false) {
  Shape shape{history, rows, hq, hkv, d, ps, dtype};
  shape.q8 = q8 ? 1 : 0;
  shape.allow_narrow = kv16 ? 0 : 1;   // the narrow kernel reads 16-bit K/V of q's type or 8-bit pages
  int rc = check_shape(shape);
  if (rc != PPA_OK) return rc;
  if (n_splits < 0) return PPA_ERR_BAD_SHAPE;
  if (q8 && ps < 16) return PPA_ERR_UNSUPPORTED;
  if (rows == 0) return PPA_OK;
  if (!q || !k || !v || !out || (paged && !bt)) return PPA_ERR_NULL_PTR;
  if (q8 && (!q8->k || !q8->v)) return PPA_ERR_NULL_PTR;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return PPA_ERR_ALIGNMENT;
  if (q8 && (!aligned16(q8->k) || !aligned16(q8->v))) return PPA_ERR_ALIGNMENT;
  const int64_t qbytes = int64_t(rows) * hq * d * 2;
  const char* qb = static_cast<const char*>(q);
  const char* ob = static_cast<const char*>(out);
  if (ob < qb + qbytes && qb < ob + qbytes) return PPA_ERR_ALIAS;

  ppa_plan plan;
  rc = make_plan(shape, n_splits, max_workspace_bytes(), &plan);
  if (rc != PPA_OK) return rc;
  if (plan.workspace_bytes > max_workspace_bytes()) return PPA_ERR_WORKSPACE;

  if (wsrc.fixed_array && plan.workspace_bytes > kStaticScratchBytes) return PPA_ERR_WORKSPACE;
  if (wsrc.ws && plan.workspace_bytes > wsrc.ws_bytes) return PPA_ERR_WORKSPACE;

  if (paged && !wsrc.fixed_array && env_validate()) {
    rc = validate_block_table(bt, (history + rows + ps - 1) / ps, stream);
    if (rc != PPA_OK) return rc;
  }

  // The stream's workspace stays held (lease) until both kernels are enqueued.
  void* ws = nullptr;
  Registry::Lease lease;
  if (plan.n_splits > 1) {
    if (wsrc.ws) {
      ws = wsrc.ws;
    } else if (wsrc.fixed_array) {
      rc = static_scratch(&ws);
      if (rc != PPA_OK) return rc;
    } else {
      int dev = 0;
      if (hipGetDevice(&dev) != hipSuccess) return PPA_ERR_HIP;
      if (!registry().acquire({dev, stream}, plan.workspace_bytes, &lease)) return PPA_ERR_WORKSPACE;
      ws = lease.ptr();
    }
  }
  const int64_t pairs = int64_t(rows) * hq;
  const int64_t o_bytes = (int64_t(plan.n_splits) * pairs * d * 4 + 255) / 256 * 256;

  AttnArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.bt = bt;
  a.out = static_cast<uint16_t*>(out);
  a.ws_o = static_cast<float*>(ws);
  a.ws_lse = ws ? reinterpret_cast<float*>(static_cast<char*>(ws) + o_bytes) : nullptr;
  a.history = history;
  a.rows = rows;
  a.n_q_heads = hq;
  a.n_kv_heads = hkv;
  a.group = hq / hkv;
  a.log2_ps = paged ? log2_exact(ps) : 0;
  a.ctx = int32_t(history + rows);
  a.split_tokens = plan.split_tokens;
  a.n_splits = plan.n_splits;
  a.tiles_m = plan.tiles_m;
  a.xcd_remap = (plan.grid % 8 == 0) ? 1 : 0;
  a.scale_log2 = float(1.4426950408889634 / std::sqrt(double(d)));
  a.cu_rows = nullptr;
  a.seq_history = nullptr;
  a.n_seqs = 0;
  a.bt_stride = 0;
  a.ws_rows = rows;
  a.k_scale = q8 ? static_cast<const uint16_t*>(q8->k) : nullptr;
  a.v_scale = q8 ? static_cast<const uint16_t*>(q8->v) : nullptr;
  a.query_blocks = plan.m_tile / 128;

  const bool narrow = plan.m_tile == kNarrowVectors;
  const hipError_t le = narrow ? launch_attention_decode(a, d, dtype, paged, q8 != nullptr, plan.grid, stream)
                        : q8   ? launch_attention_q8(a, d, dtype, plan.grid, stream)
                        : kv16 ? launch_attention_kv16(a, d, dtype, plan.grid, stream)
                               : launch_attention(a, d, dtype, paged, plan.grid, stream);
  if (le != hipSuccess) return PPA_ERR_HIP;
  if (plan.n_splits > 1) {
    MergeArgs m;
    m.ws_o = a.ws_o;
    m.ws_lse = a.ws_lse;
    m.out = a.out;
    m.history = history;
    m.rows = rows;
    m.n_q_heads = hq;
    m.split_tokens = plan.split_tokens;
    m.n_splits = plan.n_splits;
    m.cu_rows = nullptr;
    m.seq_history = nullptr;
    m.n_seqs = 0;
    m.ws_rows = rows;
    if (launch_merge(m, d, dtype, plan.merge_grid, 1, stream) != hipSuccess) return PPA_ERR_HIP;
  }
  return PPA_OK;
}

// Host check of a varlen launch's device arrays (PPA_VALIDATE=1): row offsets
// start at 0, never decrease and end at total_rows; each sequence fits the
// host-side bounds; its block-table entries are not negative.
int validate_varlen(const int32_t* bt, int32_t bt_stride, const int32_t* cu_rows,
                    const int64_t* hist, int32_t n_seqs, int32_t total_rows, int32_t max_rows,
                    int64_t max_context, int32_t ps, hipStream_t stream) {
  std::vector<int32_t> cu(size_t(n_seqs) + 1), table(size_t(n_seqs) * size_t(bt_stride));
  std::vector<int64_t> h(static_cast<size_t>(n_seqs));
  if (hipMemcpyAsync(cu.data(), cu_rows, cu.size() * 4, hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipMemcpyAsync(h.data(), hist, h.size() * 8, hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipMemcpyAsync(table.data(), bt, table.size() * 4, hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return PPA_ERR_HIP;
  if (cu[0] != 0 || cu[size_t(n_seqs)] != total_rows) return PPA_ERR_BAD_SHAPE;
  for (int32_t i = 0; i < n_seqs; ++i) {
    const int64_t r = int64_t(cu[size_t(i) + 1]) - cu[size_t(i)];
    if (r < 0 || r > max_rows || h[size_t(i)] < 0 || h[size_t(i)] + r > max_context) return PPA_ERR_BAD_SHAPE;
    const int64_t pages = (h[size_t(i)] + r + ps - 1) / ps;
    for (int64_t j = 0; j < pages; ++j)
      if (table[size_t(i) * size_t(bt_stride) + size_t(j)] < 0) return PPA_ERR_BLOCK_TABLE;
  }
  return PPA_OK;
}

// k and v: 16-bit pages, or with q8 the quant pools (scales in q8).
int run_varlen(const void* q, const void* k, const void* v, const int32_t* bt, int32_t bt_stride,
               const int32_t* cu_rows, const int64_t* hist, int32_t n_seqs, int32_t total_rows,
               int32_t max_rows, int64_t max_context, int32_t hq, int32_t hkv, int32_t d,
               int32_t ps, int32_t n_splits, void* out, int32_t dtype, hipStream_t stream,
               const Q8Scales* q8 = nullptr) {
  if (n_seqs < 0 || total_rows < 0 || max_rows < 0 || max_rows > total_rows ||
      max_context < max_rows || n_splits < 0)
    return PPA_ERR_BAD_SHAPE;
  if (n_seqs > 65535) return PPA_ERR_TOO_LARGE;  // the merge grid's y extent
  // Shape checks with the batch's bounds: ctx = max_context, q/out rows = total_rows.
  Shape shape{max_context > total_rows ? max_context - total_rows : 0, total_rows, hq, hkv, d, ps, dtype};
  shape.q8 = q8 ? 1 : 0;
  int rc = check_shape(shape);
  if (rc != PPA_OK) return rc;
  if (q8 && ps < 16) return PPA_ERR_UNSUPPORTED;
  if (n_seqs == 0 || total_rows == 0 || max_rows == 0) return PPA_OK;
  if (!q || !k || !v || !out || !bt || !cu_rows || !hist) return PPA_ERR_NULL_PTR;
  if (q8 && (!q8->k || !q8->v)) return PPA_ERR_NULL_PTR;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return PPA_ERR_ALIGNMENT;
  if (q8 && (!aligned16(q8->k) || !aligned16(q8->v))) return PPA_ERR_ALIGNMENT;
  const int lps = log2_exact(ps);
  if (int64_t(bt_stride) < (max_context + ps - 1) / ps) return PPA_ERR_BAD_SHAPE;
  if (int64_t(n_seqs) * bt_stride >= (int64_t(1) << 31)) return PPA_ERR_TOO_LARGE;
  const int64_t qbytes = int64_t(total_rows) * hq * d * 2;
  const char* qb = static_cast<const char*>(q);
  const char* ob = static_cast<const char*>(out);
  if (ob < qb + qbytes && qb < ob + qbytes) return PPA_ERR_ALIAS;

  Shape ps_shape{0, total_rows, hq, hkv, d, ps, dtype};
  ps_shape.q8 = shape.q8;
  ppa_plan plan;
  rc = make_plan_varlen(ps_shape, n_seqs, max_rows, max_context, n_splits, max_workspace_bytes(), &plan);
  if (rc != PPA_OK) return rc;
  if (plan.workspace_bytes > max_workspace_bytes()) return PPA_ERR_WORKSPACE;
  if (env_validate()) {
    rc = validate_varlen(bt, bt_stride, cu_rows, hist, n_seqs, total_rows, max_rows, max_context, ps,
                         stream);
    if (rc != PPA_OK) return rc;
  }
  void* ws = nullptr;
  Registry::Lease lease;
  if (plan.n_splits > 1) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return PPA_ERR_HIP;
    if (!registry().acquire({dev, stream}, plan.workspace_bytes, &lease)) return PPA_ERR_WORKSPACE;
    ws = lease.ptr();
  }
  const int64_t pairs = int64_t(total_rows) * hq;
  const int64_t o_bytes = (int64_t(plan.n_splits) * pairs * d * 4 + 255) / 256 * 256;

  AttnArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.bt = bt;
  a.out = static_cast<uint16_t*>(out);
  a.ws_o = static_cast<float*>(ws);
  a.ws_lse = ws ? reinterpret_cast<float*>(static_cast<char*>(ws) + o_bytes) : nullptr;
  a.history = 0;  // per sequence
  a.rows = 0;
  a.n_q_heads = hq;
  a.n_kv_heads = hkv;
  a.group = hq / hkv;
  a.log2_ps = lps;
  a.ctx = 0;
  a.split_tokens = plan.split_tokens;
  a.n_splits = plan.n_splits;
  a.tiles_m = plan.tiles_m;
  a.xcd_remap = (plan.grid % 8 == 0) ? 1 : 0;
  a.scale_log2 = float(1.4426950408889634 / std::sqrt(double(d)));
  a.cu_rows = cu_rows;
  a.seq_history = hist;
  a.n_seqs = n_seqs;
  a.bt_stride = bt_stride;
  a.ws_rows = total_rows;
  a.k_scale = q8 ? static_cast<const uint16_t*>(q8->k) : nullptr;
  a.v_scale = q8 ? static_cast<const uint16_t*>(q8->v) : nullptr;
  a.query_blocks = plan.m_tile / 128;

  hipError_t le;
  if (plan.m_tile == kNarrowVectors) {
    // every sequence's rows x group fit one wave's MFMA columns: the narrow
    // kernel (its build is chosen by the batch's largest row count)
    a.rows = max_rows;
    le = launch_attention_decode(a, d, dtype, true, q8 != nullptr, plan.grid, stream);
  } else {
    le = q8 ? launch_attention_q8(a, d, dtype, plan.grid, stream) : launch_attention(a, d, dtype, true, plan.grid, stream);
  }
  if (le != hipSuccess) return PPA_ERR_HIP;
  if (plan.n_splits > 1) {
    MergeArgs m;
    m.ws_o = a.ws_o;
    m.ws_lse = a.ws_lse;
    m.out = a.out;
    m.history = 0;
    m.rows = 0;
    m.n_q_heads = hq;
    m.split_tokens = plan.split_tokens;
    m.n_splits = plan.n_splits;
    m.cu_rows = cu_rows;
    m.seq_history = hist;
    m.n_seqs = n_seqs;
    m.ws_rows = total_rows;
    if (launch_merge(m, d, dtype, plan.merge_grid / n_seqs, n_seqs, stream) != hipSuccess) return PPA_ERR_HIP;
  }
  return PPA_OK;
}

// 8-bit pages read by several m tiles per KV head: dequantize the chunk's
// context once into contiguous fp16 K/V (kv_dequant_q8_kernel) and run the
// 16-bit kernels over it, instead of widening every tile in every workgroup
// that reads it (about 30 VALU instructions per 16 values, serialized with a
// wave's MFMAs).  The fp16 values are the ones the in-tile widening computes.
// Returns PPA_OK, an error, or kNoDequant when the in-tile path should run
// (one m tile per KV head: each tile is then widened once anyway; or a buffer
// beyond the workspace cap).
constexpr int kNoDequant = 1;
constexpr int kDequantMinTiles = 4;   // m tiles per KV head over the whole chunk

int run_q8_dequant(const void* q, const void* kq, const void* vq, const int32_t* bt, int64_t history,
                   int32_t rows, int32_t piece_rows, int32_t hq, int32_t hkv, int32_t d, int32_t ps,
                   int32_t n_splits, void* out, int32_t dtype, hipStream_t stream, const Q8Scales& q8) {
  const int64_t qv = int64_t(rows) * (hq / hkv);
  const int32_t mt = m_tile_for(d, false, qv);
  if ((qv + mt - 1) / mt < kDequantMinTiles) return kNoDequant;
  const int32_t p = (piece_rows <= 0 || piece_rows >= rows) ? rows : piece_rows;
  // the pieces' split workspaces (16-bit plans), one after another on the stream
  int64_t split_ws = 0;
  for (int32_t r0 = 0; r0 < rows; r0 += p) {
    const int32_t n = rows - r0 < p ? rows - r0 : p;
    const Shape ps16{history + r0, n, hq, hkv, d, ps, dtype};
    ppa_plan plan;
    const int rc = make_plan(ps16, n_splits, max_workspace_bytes(), &plan);
    if (rc != PPA_OK) return rc;
    if (plan.workspace_bytes > split_ws) split_ws = plan.workspace_bytes;
  }
  const int64_t ctx = history + rows;
  const int64_t tensor_bytes = (ctx * hkv * d * 2 + 255) / 256 * 256;
  const int64_t total = 2 * tensor_bytes + split_ws;
  if (total > max_workspace_bytes()) return kNoDequant;
  if (!q || !kq || !vq || !out || !bt || !q8.k || !q8.v) return PPA_ERR_NULL_PTR;
  const int64_t qbytes = int64_t(rows) * hq * d * 2;
  const char* qc = static_cast<const char*>(q);
  const char* oc = static_cast<const char*>(out);
  if (oc < qc + qbytes && qc < oc + qbytes) return PPA_ERR_ALIAS;
  if (env_validate()) {
    const int rc = validate_block_table(bt, (ctx + ps - 1) / ps, stream);
    if (rc != PPA_OK) return rc;
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PPA_ERR_HIP;
  Registry::Lease lease;   // held until the last piece's kernels are enqueued
  if (!registry().acquire({dev, stream}, total, &lease)) return PPA_ERR_WORKSPACE;
  char* base = static_cast<char*>(lease.ptr());
  DequantQ8Args da;
  da.k_quant = static_cast<const int8_t*>(kq);
  da.v_quant = static_cast<const int8_t*>(vq);
  da.k_scale = static_cast<const uint16_t*>(q8.k);
  da.v_scale = static_cast<const uint16_t*>(q8.v);
  da.bt = bt;
  da.k_out = reinterpret_cast<uint16_t*>(base);
  da.v_out = reinterpret_cast<uint16_t*>(base + tensor_bytes);
  da.ctx = int32_t(ctx);
  da.n_kv_heads = hkv;
  da.head_dim = d;
  da.log2_ps = log2_exact(ps);
  if (launch_kv_dequant_q8(da, stream) != hipSuccess) return PPA_ERR_HIP;
  WsSource src;
  src.ws = split_ws > 0 ? base + 2 * tensor_bytes : nullptr;
  src.ws_bytes = split_ws;
  const int64_t row_bytes = int64_t(hq) * d * 2;
  for (int32_t r0 = 0; r0 < rows; r0 += p) {
    const int32_t n = rows - r0 < p ? rows - r0 : p;
    const int rc = run(static_cast<const char*>(q) + r0 * row_bytes, da.k_out, da.v_out, nullptr, false,
                       history + r0, n, hq, hkv, d, ps, n_splits, static_cast<char*>(out) + r0 * row_bytes,
                       dtype, stream, nullptr, src, true);
    if (rc != PPA_OK) return rc;
  }
  return PPA_OK;
}

int run_pieces(const void* q, const void* k, const void* v, const int32_t* bt, bool paged,
               int64_t history, int32_t rows, int32_t piece_rows, int32_t hq, int32_t hkv,
               int32_t d, int32_t ps, int32_t n_splits, void* out, int32_t dtype,
               hipStream_t stream, const Q8Scales* q8 = nullptr, const WsSource& wsrc = WsSource()) {
  if (piece_rows < 0) return PPA_ERR_BAD_SHAPE;
  Shape shape{history, rows, hq, hkv, d, ps, dtype};
  shape.q8 = q8 ? 1 : 0;
  int rc = check_shape(shape);
  if (rc != PPA_OK) return rc;
  if (q8 && rows > 0 && ps >= 16 && n_splits >= 0 && !wsrc.fixed_array) {
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(q8->k) ||
        !aligned16(q8->v))
      return PPA_ERR_ALIGNMENT;
    rc = run_q8_dequant(q, k, v, bt, history, rows, piece_rows, hq, hkv, d, ps, n_splits, out, dtype, stream, *q8);
    if (rc != kNoDequant) return rc;
  }
  if (piece_rows == 0 || piece_rows >= rows)
    return run(q, k, v, bt, paged, history, rows, hq, hkv, d, ps, n_splits, out, dtype, stream, q8, wsrc);
  const int64_t row_bytes = int64_t(hq) * d * 2;
  for (int32_t r0 = 0; r0 < rows; r0 += piece_rows) {
    const int32_t n = rows - r0 < piece_rows ? rows - r0 : piece_rows;
    rc = run(static_cast<const char*>(q) + r0 * row_bytes, k, v, bt, paged, history + r0, n, hq,
             hkv, d, ps, n_splits, static_cast<char*>(out) + r0 * row_bytes, dtype, stream, q8, wsrc);
    if (rc != PPA_OK) return rc;
  }
  return PPA_OK;
}

}  // namespace
}  // namespace ppa

extern "C" {

int paged_prefill_attention(const void* q, const void* k_pages, const void* v_pages,
                            const int32_t* block_table, int64_t history_len, int32_t chunk_rows,
                            int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                            int32_t page_size, int32_t n_splits, void* out, int32_t dtype,
                            ppa_stream_t stream) {
  return ppa::run(q, k_pages, v_pages, block_table, true, history_len, chunk_rows, n_q_heads,
                  n_kv_heads, head_dim, page_size, n_splits, out, dtype,
                  reinterpret_cast<hipStream_t>(stream));
}

int contiguous_prefill_attention(const void* q, const void* k, const void* v, int64_t history_len,
                                 int32_t chunk_rows, int32_t n_q_heads, int32_t n_kv_heads,
                                 int32_t head_dim, int32_t n_splits, void* out, int32_t dtype,
                                 ppa_stream_t stream) {
  return ppa::run(q, k, v, nullptr, false, history_len, chunk_rows, n_q_heads, n_kv_heads,
                  head_dim, 16, n_splits, out, dtype, reinterpret_cast<hipStream_t>(stream));
}

int paged_prefill_attention_pieces(const void* q, const void* k_pages, const void* v_pages,
                                   const int32_t* block_table, int64_t history_len,
                                   int32_t chunk_rows, int32_t piece_rows, int32_t n_q_heads,
                                   int32_t n_kv_heads, int32_t head_dim, int32_t page_size,
                                   int32_t n_splits, void* out, int32_t dtype,
                                   ppa_stream_t stream) {
  return ppa::run_pieces(q, k_pages, v_pages, block_table, true, history_len, chunk_rows,
                         piece_rows, n_q_heads, n_kv_heads, head_dim, page_size, n_splits, out,
                         dtype, reinterpret_cast<hipStream_t>(stream));
}

int contiguous_prefill_attention_pieces(const void* q, const void* k, const void* v,
                                        int64_t history_len, int32_t chunk_rows,
                                        int32_t piece_rows, int32_t n_q_heads, int32_t n_kv_heads,
                                        int32_t head_dim, int32_t n_splits, void* out,
                                        int32_t dtype, ppa_stream_t stream) {
  return ppa::run_pieces(q, k, v, nullptr, false, history_len, chunk_rows, piece_rows, n_q_heads,
                         n_kv_heads, head_dim, 16, n_splits, out, dtype,
                         reinterpret_cast<hipStream_t>(stream));
}

int paged_prefill_attention_varlen(const void* q, const void* k_pages, const void* v_pages,
                                   const int32_t* block_tables, int32_t block_table_stride,
                                   const int32_t* cu_rows, const int64_t* history_lens,
                                   int32_t n_seqs, int32_t total_rows, int32_t max_rows,
                                   int64_t max_context, int32_t n_q_heads, int32_t n_kv_heads,
                                   int32_t head_dim, int32_t page_size, int32_t n_splits,
                                   void* out, int32_t dtype, ppa_stream_t stream) {
  return ppa::run_varlen(q, k_pages, v_pages, block_tables, block_table_stride, cu_rows,
                         history_lens, n_seqs, total_rows, max_rows, max_context, n_q_heads,
                         n_kv_heads, head_dim, page_size, n_splits, out, dtype,
                         reinterpret_cast<hipStream_t>(stream));
}

int paged_prefill_attention_varlen_q8(const void* q, const void* k_quant, const void* k_scale,
                                      const void* v_quant, const void* v_scale,
                                      const int32_t* block_tables, int32_t block_table_stride,
                                      const int32_t* cu_rows, const int64_t* history_lens,
                                      int32_t n_seqs, int32_t total_rows, int32_t max_rows,
                                      int64_t max_context, int32_t n_q_heads, int32_t n_kv_heads,
                                      int32_t head_dim, int32_t page_size, int32_t n_splits,
                                      void* out, int32_t dtype, ppa_stream_t stream) {
  const ppa::Q8Scales scales{k_scale, v_scale};
  return ppa::run_varlen(q, k_quant, v_quant, block_tables, block_table_stride, cu_rows, history_lens,
                         n_seqs, total_rows, max_rows, max_context, n_q_heads, n_kv_heads, head_dim,
                         page_size, n_splits, out, dtype, reinterpret_cast<hipStream_t>(stream), &scales);
}

int paged_prefill_attention_q8(const void* q, const void* k_quant, const void* k_scale,
                               const void* v_quant, const void* v_scale, const int32_t* block_table,
                               int64_t history_len, int32_t chunk_rows, int32_t piece_rows,
                               int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                               int32_t page_size, int32_t n_splits, void* out, int32_t dtype,
                               ppa_stream_t stream) {
  const ppa::Q8Scales scales{k_scale, v_scale};
  return ppa::run_pieces(q, k_quant, v_quant, block_table, true, history_len, chunk_rows, piece_rows,
                         n_q_heads, n_kv_heads, head_dim, page_size, n_splits, out, dtype,
                         reinterpret_cast<hipStream_t>(stream), &scales);
}

int paged_kv_append_q8(const void* k_new, const void* v_new, void* k_quant, void* k_scale,
                       void* v_quant, void* v_scale, const int32_t* block_table, int64_t history_len,
                       int32_t rows, int32_t n_kv_heads, int32_t head_dim, int32_t page_size,
                       int32_t dtype, ppa_stream_t stream) {
  const ppa::Shape shape{history_len, rows, n_kv_heads, n_kv_heads, head_dim, page_size, dtype};
  int rc = ppa::check_shape(shape);
  if (rc != PPA_OK) return rc;
  if (rows == 0) return PPA_OK;
  if (!k_new || !v_new || !k_quant || !k_scale || !v_quant || !v_scale || !block_table)
    return PPA_ERR_NULL_PTR;
  const void* all[6] = {k_new, v_new, k_quant, k_scale, v_quant, v_scale};
  for (const void* p : all)
    if (!ppa::aligned16(p)) return PPA_ERR_ALIGNMENT;
  // the four pools must be distinct and none may start where a new-row buffer starts
  for (int i = 0; i < 6; ++i)
    for (int j = i + 1; j < 6; ++j)
      if (all[i] == all[j]) return PPA_ERR_ALIAS;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (ppa::env_validate()) {
    const int64_t first = history_len / page_size;
    const int64_t last = (history_len + rows - 1) / page_size;
    rc = ppa::validate_block_table(block_table + first, last - first + 1, s);
    if (rc != PPA_OK) return rc;
  }
  ppa::AppendQ8Args a;
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  a.k_quant = static_cast<int8_t*>(k_quant);
  a.v_quant = static_cast<int8_t*>(v_quant);
  a.k_scale = static_cast<uint16_t*>(k_scale);
  a.v_scale = static_cast<uint16_t*>(v_scale);
  a.bt = block_table;
  a.history = history_len;
  a.rows = rows;
  a.n_kv_heads = n_kv_heads;
  a.head_dim = head_dim;
  a.log2_ps = ppa::log2_exact(page_size);
  return ppa::launch_kv_append_q8(a, dtype, s) == hipSuccess ? PPA_OK : PPA_ERR_HIP;
}

int paged_kv_append(const void* k_new, const void* v_new, void* k_pages, void* v_pages,
                    const int32_t* block_table, int64_t history_len, int32_t rows, int32_t n_kv_heads,
                    int32_t head_dim, int32_t page_size, int32_t dtype, ppa_stream_t stream) {
  const ppa::Shape shape{history_len, rows, n_kv_heads, n_kv_heads, head_dim, page_size, dtype};
  int rc = ppa::check_shape(shape);
  if (rc != PPA_OK) return rc;
  if (rows == 0) return PPA_OK;
  if (!k_new || !v_new || !k_pages || !v_pages || !block_table) return PPA_ERR_NULL_PTR;
  if (!ppa::aligned16(k_new) || !ppa::aligned16(v_new) || !ppa::aligned16(k_pages) || !ppa::aligned16(v_pages))
    return PPA_ERR_ALIGNMENT;
  // The new rows must not start where a pool starts, and K and V need pools
  // of their own (the pool sizes are not arguments, so partial overlaps cannot
  // be checked).
  const char* pools[2] = {static_cast<const char*>(k_pages), static_cast<const char*>(v_pages)};
  const char* news[2] = {static_cast<const char*>(k_new), static_cast<const char*>(v_new)};
  for (const char* nb : news)
    for (const char* pb : pools)
      if (nb == pb) return PPA_ERR_ALIAS;
  if (k_pages == v_pages) return PPA_ERR_ALIAS;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (ppa::env_validate()) {
    const int64_t first = history_len / page_size;
    const int64_t last = (history_len + rows - 1) / page_size;
    rc = ppa::validate_block_table(block_table + first, last - first + 1, s);
    if (rc != PPA_OK) return rc;
  }
  ppa::AppendArgs a;
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  a.k_pages = static_cast<uint16_t*>(k_pages);
  a.v_pages = static_cast<uint16_t*>(v_pages);
  a.bt = block_table;
  a.history = history_len;
  a.rows = rows;
  a.upr = n_kv_heads * head_dim * 2 / 16;
  a.log2_ps = ppa::log2_exact(page_size);
  return ppa::launch_kv_append(a, s) == hipSuccess ? PPA_OK : PPA_ERR_HIP;
}

int paged_prefill_release_workspaces(void) {
  return ppa::registry().release_all() ? PPA_OK : PPA_ERR_HIP;
}

int64_t paged_prefill_workspace_bytes(ppa_stream_t stream) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PPA_ERR_HIP;
  return ppa::registry().capacity({dev, reinterpret_cast<hipStream_t>(stream)});
}

int paged_prefill_attention_pieces_noalloc(const void* q, const void* k_pages, const void* v_pages,
                                           const int32_t* block_table, int64_t history_len,
                                           int32_t chunk_rows, int32_t piece_rows, int32_t n_q_heads,
                                           int32_t n_kv_heads, int32_t head_dim, int32_t page_size,
                                           int32_t n_splits, void* out, int32_t dtype,
                                           ppa_stream_t stream) {
  ppa::WsSource src;
  src.fixed_array = true;
  return ppa::run_pieces(q, k_pages, v_pages, block_table, true, history_len, chunk_rows, piece_rows,
                         n_q_heads, n_kv_heads, head_dim, page_size, n_splits, out, dtype,
                         reinterpret_cast<hipStream_t>(stream), nullptr, src);
}

}  // extern "C"

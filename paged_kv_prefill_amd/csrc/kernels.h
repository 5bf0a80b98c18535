// Device-side argument blocks and launch wrappers shared by the host API and
// the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ppa {

struct AttnArgs {
  const uint16_t* q;       // [R][Hq][D]
  const uint16_t* k;       // paged: [pool][ps][Hkv][D]; contiguous: [ctx][Hkv][D]
  const uint16_t* v;
  const int32_t* bt;       // block table (paged only)
  uint16_t* out;           // [R][Hq][D] (single split)
  float* ws_o;             // [S][R][Hq][D] normalised split partials
  float* ws_lse;           // [S][R][Hq] log2-domain log-sum-exp of each partial
  int64_t history;         // H
  int32_t rows;            // R
  int32_t n_q_heads;       // Hq
  int32_t n_kv_heads;      // Hkv
  int32_t group;           // Hq / Hkv
  int32_t log2_ps;         // log2(page_size) (paged)
  int32_t ctx;             // H + R
  int32_t split_tokens;    // keys per split
  int32_t n_splits;        // S
  int32_t tiles_m;         // m tiles per KV head
  int32_t xcd_remap;       // 1: spread consecutive logical tiles over one XCD
  float scale_log2;        // log2(e) / sqrt(D)
  // Several sequences in one launch (n_seqs > 0): sequence s owns rows
  // [cu_rows[s], cu_rows[s+1]) of q, out and the workspace, has history
  // seq_history[s] and block-table row bt + s * bt_stride.  The workgroup
  // then takes rows, history and ctx above from these arrays; tiles_m and
  // n_splits are the launch's maxima and workgroups beyond a sequence's
  // tiles or splits exit.  n_seqs == 0: one sequence, as described above.
  const int32_t* cu_rows;
  const int64_t* seq_history;
  int32_t n_seqs;
  int32_t bt_stride;
  int32_t ws_rows;         // rows of the workspace layout (all sequences)
  // 8-bit pages: k and v point to int8 quants [pool][ps][Hkv][D], these to
  // their fp16 scales [pool][ps][Hkv][D / 32] (one per 32 values along D).
  const uint16_t* k_scale;
  const uint16_t* v_scale;
  int32_t query_blocks;    // 32-vector query blocks per wave (m tile / 128): 1 or 2
};

struct MergeArgs {
  const float* ws_o;
  const float* ws_lse;
  uint16_t* out;
  int64_t history;
  int32_t rows;
  int32_t n_q_heads;
  int32_t split_tokens;
  int32_t n_splits;
  // As in AttnArgs; with n_seqs > 0 the grid's y index is the sequence.
  const int32_t* cu_rows;
  const int64_t* seq_history;
  int32_t n_seqs;
  int32_t ws_rows;
};

// KV append: rows [R][Hkv][d] of K and V into their pages.
struct AppendArgs {
  const uint16_t* k_new;
  const uint16_t* v_new;
  uint16_t* k_pages;
  uint16_t* v_pages;
  const int32_t* bt;
  int64_t history;
  int32_t rows;
  int32_t upr;      // 16-byte units per token row: Hkv * d * 2 / 16
  int32_t log2_ps;
};

// Quantizing KV append into 8-bit pages: rows [R][Hkv][D] (fp16 or bf16) to
// int8 quants [pool][ps][Hkv][D] and fp16 scales [pool][ps][Hkv][D / 32].
struct AppendQ8Args {
  const uint16_t* k_new;
  const uint16_t* v_new;
  int8_t* k_quant;
  int8_t* v_quant;
  uint16_t* k_scale;
  uint16_t* v_scale;
  const int32_t* bt;
  int64_t history;
  int32_t rows;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t log2_ps;
};

// Dequantizing gather: tokens [0, ctx) of one sequence from 8-bit pages
// (quants [pool][ps][Hkv][D], fp16 scales [pool][ps][Hkv][D / 32]) to
// contiguous fp16 [ctx][Hkv][D], K and V.
struct DequantQ8Args {
  const int8_t* k_quant;
  const int8_t* v_quant;
  const uint16_t* k_scale;
  const uint16_t* v_scale;
  const int32_t* bt;
  uint16_t* k_out;
  uint16_t* v_out;
  int32_t ctx;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t log2_ps;
};

// dtype: 0 = fp16, 1 = bf16.  Returns hipSuccess or the launch error.
hipError_t launch_attention(const AttnArgs& a, int head_dim, int dtype, bool paged, int grid,
                            hipStream_t stream);
hipError_t launch_merge(const MergeArgs& a, int head_dim, int dtype, int grid, int grid_y, hipStream_t stream);
hipError_t launch_kv_append(const AppendArgs& a, hipStream_t stream);
hipError_t launch_kv_append_q8(const AppendQ8Args& a, int dtype, hipStream_t stream);
// The attention kernel over 8-bit pages (page_size >= 16).
hipError_t launch_attention_q8(const AttnArgs& a, int head_dim, int dtype, int grid, hipStream_t stream);
// The attention kernel over contiguous fp16 K/V with q and out of type dtype
// (dequantized 8-bit pages).
hipError_t launch_attention_kv16(const AttnArgs& a, int head_dim, int dtype, int grid, hipStream_t stream);
hipError_t launch_kv_dequant_q8(const DequantQ8Args& a, hipStream_t stream);
// The narrow kernel (at most 32 query vectors per KV head, one sequence;
// 16-bit pages of >= 8 tokens, 8-bit pages of >= 16, or contiguous K/V):
// grid = n_splits * Hkv workgroups.
hipError_t launch_attention_decode(const AttnArgs& a, int head_dim, int dtype, bool paged, bool q8, int grid,
                                   hipStream_t stream);

// The per-head-dimension halves of launch_attention and launch_attention_q8
// (separate translation units).
hipError_t launch_attention_d64_d128(const AttnArgs& a, int head_dim, int dtype, bool paged, int grid,
                                     hipStream_t stream);
hipError_t launch_attention_d256(const AttnArgs& a, int dtype, bool paged, int grid, hipStream_t stream);
hipError_t launch_attention_d256_small_pages(const AttnArgs& a, int dtype, int grid, hipStream_t stream);
hipError_t launch_attention_d64_d128_qb1(const AttnArgs& a, int head_dim, int dtype, bool paged, int grid,
                                         hipStream_t stream);
hipError_t launch_attention_q8_d64_d128(const AttnArgs& a, int head_dim, int dtype, int grid, hipStream_t stream);
hipError_t launch_attention_q8_d256(const AttnArgs& a, int dtype, int grid, hipStream_t stream);
hipError_t launch_attention_kv16_d256(const AttnArgs& a, int grid, hipStream_t stream);
hipError_t launch_attention_kv16_d64_d128(const AttnArgs& a, int head_dim, int grid, hipStream_t stream);
hipError_t launch_attention_kv16_d64_d128_qb1(const AttnArgs& a, int head_dim, int grid, hipStream_t stream);

// Size of the fixed scratch array (noalloc.hip), one per device.
constexpr int64_t kStaticScratchBytes = int64_t(64) << 20;   // 64 MiB
// The current device's fixed scratch array: its device address (looked up
// once per device).  PPA_OK or PPA_ERR_HIP.
int static_scratch(void** ptr);

}  // namespace ppa

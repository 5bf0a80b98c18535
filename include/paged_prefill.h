/*
 * paged_prefill.h -- C ABI of chunked prefill attention over a paged KV cache
 * on AMD Instinct MI355X (gfx950).
 *
 * The operation (issue "Metal: paged-KV prefill is 4.43x slower than
 * contiguous KV at 32K", TL;DR and "Results"; PR "perf: scale prefill
 * attention splits with GPU cores on Apple7/8", "What changed"):
 *
 *   A chunk of R query rows sits at absolute positions H .. H+R-1 after a
 *   history of H tokens.  Its own K/V are already stored, so the cache holds
 *   ctx = H + R tokens.  Row i attends to keys 0 .. H+i (inclusive): the whole
 *   history plus the chunk causally.  Query head h uses KV head h / (Hq/Hkv)
 *   (grouped-query attention).  For every row i and query head h:
 *
 *       out[i][h] = sum_j softmax_j( q[i][h] . K[j][g] / sqrt(d) ) V[j][g]
 *
 *   with the softmax taken over j = 0 .. H+i and g = h / (Hq/Hkv).  The
 *   history is cut into splits, each split writes a partial output and its
 *   log-sum-exp, and a merge kernel combines them (the PR's split-KV prefill
 *   attention and its reduce).  Inputs are fp16 or bf16; scores, the softmax
 *   reference m, the sum l and the output accumulator are fp32; out is
 *   rounded to the input type, to nearest even.
 *
 * Layouts (row-major, element = 2 bytes):
 *   q           [R][Hq][d]
 *   k_pages     [n_pool_pages][page_size][Hkv][d]    (v_pages likewise)
 *   block_table int32, >= ceil(ctx / page_size) entries; logical page j of
 *               the sequence is pool page block_table[j]; token t is slot
 *               t % page_size of logical page t / page_size
 *   k, v        [>= ctx][Hkv][d]  (contiguous entry point: this is the paged
 *               layout with an identity block table)
 *   out         [R][Hq][d]
 *
 * Ownership: every pointer is caller-owned device memory that must stay
 * valid until `stream` has executed the enqueued work; the library keeps no
 * pointer after a call returns.  The library owns one grow-only split
 * workspace per (device, stream), allocated on first need (that first call
 * blocks in hipMalloc).  When a larger call arrives a larger buffer is
 * allocated and the smaller one is kept, not freed, so that work already
 * enqueued and HIP graphs captured earlier keep valid memory; all of them
 * are freed by paged_prefill_release_workspaces() only.
 *
 * Execution: asynchronous, ordered on `stream` (0 = the null stream).  `out`
 * is valid once the stream has synchronised.  Once the stream's workspace is
 * large enough for a call (after a first call of that size on that stream),
 * the call enqueues kernel launches only and can be captured in a HIP graph
 * (PPA_VALIDATE=1 adds host copies, which capture does not allow).  A
 * captured graph stays valid through later calls of any size on that stream
 * (their growth retires the buffer it uses without freeing it) until
 * paged_prefill_release_workspaces() is called.  Replaying it runs its
 * kernels on the workspace it captured: do not replay it while other work
 * that uses the same workspace runs on another stream.  Results are
 * deterministic for a given plan: no atomics; partials merge in a fixed
 * order; identity, permuted and scattered block tables give bit-identical
 * outputs.
 *
 * Errors: 0 on success, a negative PPA_ERR_* code otherwise.  On any argument
 * error nothing is enqueued.  Slots past ctx in the last page may hold any
 * bits (NaN included): they never reach the output.  Block-table entries are
 * not range-checked on the device (the signature carries no pool size): use
 * paged_prefill_check_block_table() on a host copy, or set PPA_VALIDATE=1 to
 * make every paged call copy the table to the host and check it first (slow).
 *
 * Thread safety: concurrent calls on different streams are safe.  Host
 * threads may also call concurrently on one stream: a call holds that
 * stream's workspace from planning until its last kernel is enqueued, so the
 * calls' kernels reach the stream one whole call after another (which call
 * comes first is not defined).  paged_prefill_release_workspaces() must not
 * run concurrently with any other call.
 */
#ifndef PAGED_PREFILL_H
#define PAGED_PREFILL_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* ppa_stream_t; /* a hipStream_t */

enum ppa_dtype { PPA_F16 = 0, PPA_BF16 = 1 };

enum ppa_status {
  PPA_OK = 0,
  PPA_ERR_NULL_PTR = -1,    /* a required pointer is NULL */
  PPA_ERR_BAD_SHAPE = -2,   /* R < 0, H < 0, heads < 1, Hq % Hkv != 0, piece_rows < 0 */
  PPA_ERR_UNSUPPORTED = -3, /* head_dim not 64/128/256, page_size not a power of two in [1, 1024] */
  PPA_ERR_BAD_DTYPE = -4,   /* dtype not PPA_F16 / PPA_BF16 */
  PPA_ERR_WORKSPACE = -5,   /* split workspace above PPA_MAX_WORKSPACE_BYTES or hipMalloc failed */
  PPA_ERR_HIP = -6,         /* a HIP runtime call or kernel launch failed */
  PPA_ERR_BLOCK_TABLE = -7, /* a block-table entry is outside [0, n_pool_pages) (checks only) */
  PPA_ERR_ALIGNMENT = -8,   /* a tensor pointer is not 16-byte aligned */
  PPA_ERR_ALIAS = -9,       /* out overlaps q */
  PPA_ERR_TOO_LARGE = -10   /* a size exceeds the 32-bit index range the kernels use */
};

/* How one call is cut into work: see paged_prefill_plan(). */
typedef struct {
  int32_t n_splits;        /* key-axis splits actually used (>= 1) */
  int32_t split_tokens;    /* keys per split; a multiple of kv_tile and of page_size */
  int32_t m_tile;          /* query vectors (row, head pairs of one KV head) per workgroup */
  int32_t kv_tile;         /* keys per inner-loop tile */
  int32_t tiles_m;         /* m tiles per KV head: ceil(R * Hq/Hkv / m_tile) */
  int32_t grid;            /* attention workgroups: tiles_m * Hkv * n_splits */
  int32_t merge_grid;      /* merge workgroups (0 when n_splits == 1) */
  int32_t reserved;
  int64_t workspace_bytes; /* split workspace bytes (0 when n_splits == 1) */
} ppa_plan;

/*
 * Paged prefill attention for one chunk (or one piece of a chunk).
 * n_splits: 0 lets the planner choose (fill the 256 CUs, see
 * paged_prefill_plan); >= 1 requests that many splits, clamped to the number
 * of kv-tile units of the key axis (a call on the narrow kernel, see
 * paged_prefill_plan, also takes at least ceil((H + R) / (128 * page_size))
 * splits: a split holds at most 128 pages).  A requested count whose
 * partials pass PPA_MAX_WORKSPACE_BYTES or the kernels' 32-bit index range is
 * refused (PPA_ERR_WORKSPACE, PPA_ERR_TOO_LARGE).  chunk_rows == 0 is a
 * no-op (returns 0, pointers unused).
 */
int paged_prefill_attention(const void* q, const void* k_pages, const void* v_pages,
                            const int32_t* block_table, int64_t history_len, int32_t chunk_rows,
                            int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                            int32_t page_size, int32_t n_splits, void* out, int32_t dtype,
                            ppa_stream_t stream);

/*
 * The same computation over contiguous K/V [>= ctx][Hkv][d] (the A/B partner
 * of the issue: same values, no block table).  It runs the same kernels with
 * identity addressing and the same plan as a paged call with page_size 16,
 * so its output is bit-identical to the paged one.
 */
int contiguous_prefill_attention(const void* q, const void* k, const void* v,
                                 int64_t history_len, int32_t chunk_rows, int32_t n_q_heads,
                                 int32_t n_kv_heads, int32_t head_dim, int32_t n_splits, void* out,
                                 int32_t dtype, ppa_stream_t stream);

/*
 * A whole chunk in pieces of piece_rows rows (the PR's prefill pieces): call
 * p covers rows [p*P, min((p+1)*P, R)) of q and out at history
 * history_len + p*P, against the same block table.  piece_rows == 0 or
 * >= chunk_rows is one call.  Each piece is planned on its own.
 */
int paged_prefill_attention_pieces(const void* q, const void* k_pages, const void* v_pages,
                                   const int32_t* block_table, int64_t history_len,
                                   int32_t chunk_rows, int32_t piece_rows, int32_t n_q_heads,
                                   int32_t n_kv_heads, int32_t head_dim, int32_t page_size,
                                   int32_t n_splits, void* out, int32_t dtype, ppa_stream_t stream);

/*
 * Several sequences in one launch (varlen chunked prefill; the issue's
 * opening places paged KV in serving with continuous batching and prefix
 * caching).  Sequence s owns rows [cu_rows[s], cu_rows[s+1]) of q and out,
 * has history history_lens[s], and row s of block_tables as its block table
 * (block_tables[s * block_table_stride + j] = pool page of its logical page
 * j).  Each sequence's rows get exactly the single-sequence result: its rows
 * attend to its own history and, causally, to themselves, never to another
 * sequence's keys.  Tables may name the same pool pages (a shared prefix).
 *
 *   q, out          [total_rows][Hq][d], the sequences' rows back to back
 *   k_pages/v_pages one pool, [n_pool_pages][page_size][Hkv][d]
 *   block_tables    device int32 [n_seqs][block_table_stride],
 *                   block_table_stride >= ceil(max_context / page_size)
 *   cu_rows         device int32 [n_seqs + 1]: 0 = cu_rows[0] <= ... <=
 *                   cu_rows[n_seqs] = total_rows
 *   history_lens    device int64 [n_seqs], >= 0
 *   max_rows        host: >= every sequence's rows (sizes the grid)
 *   max_context     host: >= every history_lens[s] + rows_s (sizes the splits)
 *
 * The device arrays are not read on the host: if they break the bounds above,
 * rows past max_rows or keys past the splits are silently not computed, and
 * an entry of cu_rows past total_rows makes the kernels read outside q.
 * PPA_VALIDATE=1 copies them to the host and checks them first
 * (PPA_ERR_BAD_SHAPE, or PPA_ERR_BLOCK_TABLE for a negative table entry).
 * Splits are cut for max_context (n_splits as in paged_prefill_attention);
 * a shorter sequence uses the leading splits it reaches.  n_seqs == 0 or
 * total_rows == 0 is a no-op.  Errors: PPA_ERR_BAD_SHAPE for negative
 * counts, max_rows > total_rows, max_context < max_rows or a stride below
 * ceil(max_context / page_size); PPA_ERR_TOO_LARGE for n_seqs > 65535.
 */
int paged_prefill_attention_varlen(const void* q, const void* k_pages, const void* v_pages,
                                   const int32_t* block_tables, int32_t block_table_stride,
                                   const int32_t* cu_rows, const int64_t* history_lens,
                                   int32_t n_seqs, int32_t total_rows, int32_t max_rows,
                                   int64_t max_context, int32_t n_q_heads, int32_t n_kv_heads,
                                   int32_t head_dim, int32_t page_size, int32_t n_splits,
                                   void* out, int32_t dtype, ppa_stream_t stream);

/*
 * Attention over 8-bit K/V pages, dequantized in the gather (the 8-bit KV
 * cache types of the report "Research: KVarN V-store per-call latency grows
 * with n_kv at fixed grid", which measures against q8_0, and of the
 * speculative-decoding page's "--kv int8").  Each (token, KV head) row of d
 * values is stored as d int8 quants plus one fp16 scale per block of 32
 * consecutive values; a value reads back as scale * quant:
 *
 *   k_quant, v_quant  int8 [n_pool_pages][page_size][Hkv][d]
 *   k_scale, v_scale  fp16 [n_pool_pages][page_size][Hkv][d / 32]
 *
 * addressed by the same block table as 16-bit pages.  q and out are fp16 or
 * bf16 (dtype) as in paged_prefill_attention; inside, the dequantized K/V,
 * the scores' operands and the softmax weights are fp16 (a bf16 q is
 * converted to fp16, exact for |q| in fp16's normal range; dequantized values
 * above 65504 overflow), accumulation is fp32.  piece_rows as in
 * paged_prefill_attention_pieces (0 = one call).  page_size must be at least
 * 16 (PPA_ERR_UNSUPPORTED otherwise: a 16-row load group then lies in one
 * page).  Quants and scales 16-byte aligned.
 */
int paged_prefill_attention_q8(const void* q, const void* k_quant, const void* k_scale,
                               const void* v_quant, const void* v_scale, const int32_t* block_table,
                               int64_t history_len, int32_t chunk_rows, int32_t piece_rows,
                               int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                               int32_t page_size, int32_t n_splits, void* out, int32_t dtype,
                               ppa_stream_t stream);

/*
 * Several sequences in one launch over 8-bit pages: the arguments, layouts,
 * bounds, checks (PPA_VALIDATE=1 included) and errors of
 * paged_prefill_attention_varlen, with the pool given as the quants and
 * scales of paged_prefill_attention_q8 (page_size >= 16, everything 16-byte
 * aligned) and the same arithmetic as there.  A batch whose sequences all
 * have at most 32 query vectors per KV head (max_rows * Hq/Hkv <= 32: a batch
 * of decode steps) runs the narrow kernel, widening in registers; other
 * batches widen each tile in the prefill kernel's loop (the chunk path's
 * dequantize-once gather needs one block table).
 */
int paged_prefill_attention_varlen_q8(const void* q, const void* k_quant, const void* k_scale,
                                      const void* v_quant, const void* v_scale,
                                      const int32_t* block_tables, int32_t block_table_stride,
                                      const int32_t* cu_rows, const int64_t* history_lens,
                                      int32_t n_seqs, int32_t total_rows, int32_t max_rows,
                                      int64_t max_context, int32_t n_q_heads, int32_t n_kv_heads,
                                      int32_t head_dim, int32_t page_size, int32_t n_splits,
                                      void* out, int32_t dtype, ppa_stream_t stream);

/*
 * Quantizing KV append into 8-bit pages: rows k_new/v_new [R][Hkv][d] (fp16
 * or bf16, dtype) at positions H .. H+R-1 go to slot (H+i) % page_size of
 * pool page block_table[(H+i) / page_size], as in paged_kv_append.  Per
 * block of 32 values: scale = fp16(max|x| / 127) (fp32 division, rounded to
 * nearest even, saturated at 65504); quant = x / scale (fp32 division)
 * rounded to nearest, ties to even, clamped to [-127, 127]; an all-zero block
 * gets scale 0 and quants 0.  Deterministic bit for bit.  The six buffers
 * must be distinct (PPA_ERR_ALIAS) and 16-byte aligned.
 */
int paged_kv_append_q8(const void* k_new, const void* v_new, void* k_quant, void* k_scale,
                       void* v_quant, void* v_scale, const int32_t* block_table, int64_t history_len,
                       int32_t rows, int32_t n_kv_heads, int32_t head_dim, int32_t page_size,
                       int32_t dtype, ppa_stream_t stream);

/*
 * paged_prefill_attention_pieces for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same computation, plan, kernels and bits, but the
 * split workspace is a fixed 64 MiB device array inside the library (one per
 * GPU, held until the process ends) instead of the per-stream workspace, and
 * the call never allocates or frees device memory.  A call whose plan needs
 * more than 64 MiB of workspace (plan.workspace_bytes, per piece) returns
 * PPA_ERR_WORKSPACE before enqueuing anything; planner-chosen plans need at
 * most 2048 * Hq * (d + 1) * 4 bytes, which fits for Hq * d <= 8128.
 * Every call on one GPU shares that GPU's array and leaves its last
 * partials there: calls that overlap on one GPU (several streams, or several
 * threads) race on it and must be serialized by the caller.  PPA_VALIDATE is
 * not applied here.  The first call on a device looks the array's address up
 * (hipGetSymbolAddress) and must not be under stream capture.
 */
int paged_prefill_attention_pieces_noalloc(const void* q, const void* k_pages, const void* v_pages,
                                           const int32_t* block_table, int64_t history_len,
                                           int32_t chunk_rows, int32_t piece_rows, int32_t n_q_heads,
                                           int32_t n_kv_heads, int32_t head_dim, int32_t page_size,
                                           int32_t n_splits, void* out, int32_t dtype,
                                           ppa_stream_t stream);

/* Contiguous-KV counterpart of paged_prefill_attention_pieces. */
int contiguous_prefill_attention_pieces(const void* q, const void* k, const void* v,
                                        int64_t history_len, int32_t chunk_rows,
                                        int32_t piece_rows, int32_t n_q_heads, int32_t n_kv_heads,
                                        int32_t head_dim, int32_t n_splits, void* out,
                                        int32_t dtype, ppa_stream_t stream);

/*
 * Host-only: the plan a call with these arguments would use on an MI355X
 * (256 CUs).  n_splits_req as in paged_prefill_attention.  The planner
 * follows the PR's split rule ("What changed": threadgroups per core times
 * cores over KV heads, capped at a full chunk's tile slots, divided by the
 * piece's tiles, clamped) with MI355X's numbers: one resident workgroup per
 * CU, 256 CUs, the tile slots of a 2048-row chunk as the cap, 128 splits at
 * most, and no split shorter than one kv-tile unit.
 * A call with at most 16 query vectors per KV head (R * Hq/Hkv <= 16: a
 * decode step or an append of a few rows) over pages of at least 8 tokens
 * gets the narrow kernel's plan instead: m_tile = kv_tile = 32, tiles_m = 1,
 * ceil(256 / Hkv) splits (at most one per 256 keys, at most 4096) in units of
 * max(32, page_size) tokens, at most 128 pages each; grid = Hkv * n_splits.
 * When that needs more than 4096 splits, or (split count chosen by the
 * planner) more workspace than PPA_MAX_WORKSPACE_BYTES, the call takes the
 * prefill plan above.
 * This planner describes 16-bit K/V; over 8-bit pages
 * (paged_prefill_attention_q8) calls of up to 32 query vectors per KV head
 * take the narrow kernel's plan.
 */
int paged_prefill_plan(int64_t history_len, int32_t chunk_rows, int32_t n_q_heads,
                       int32_t n_kv_heads, int32_t head_dim, int32_t page_size,
                       int32_t n_splits_req, ppa_plan* plan_out);

/*
 * Host-only: the plan paged_prefill_attention_varlen would use for a batch
 * with these bounds (grid = n_seqs * tiles_m * Hkv * n_splits workgroups, of
 * which those past a sequence's rows or splits exit at once; the split rule
 * counts the m tiles of total_rows).  Arguments as there; n_seqs, total_rows
 * and max_rows >= 1.
 */
int paged_prefill_plan_varlen(int32_t n_seqs, int32_t total_rows, int32_t max_rows,
                              int64_t max_context, int32_t n_q_heads, int32_t n_kv_heads,
                              int32_t head_dim, int32_t page_size, int32_t n_splits_req,
                              ppa_plan* plan_out);

/*
 * Host-only: the PR's split rule with explicit parameters,
 * clamp(min(slot_cap, max(floor, per_core * gpu_cores / kv_heads)) / tiles,
 * 1, max_splits) in integer arithmetic.  Returns the split count, or a
 * negative PPA_ERR_BAD_SHAPE if an argument is < 1.
 */
int paged_prefill_split_rule(int32_t gpu_cores, int32_t kv_heads, int32_t tiles,
                             int32_t per_core, int32_t floor_tg, int32_t slot_cap,
                             int32_t max_splits);

/*
 * Host-only: the PR's piece size (explanatory note after "Testing"): halve
 * chunk_rows until rows * (history + rows) <= budget.  budget <= 0 means 2^25.
 */
int32_t paged_prefill_piece_rows(int64_t history_len, int32_t chunk_rows, int64_t budget);

/*
 * Host-only: check that the first n_entries of a host copy of a block table
 * lie in [0, n_pool_pages).  Returns 0 or PPA_ERR_BLOCK_TABLE (or
 * PPA_ERR_NULL_PTR / PPA_ERR_BAD_SHAPE for bad arguments).
 */
int paged_prefill_check_block_table(const int32_t* block_table_host, int64_t n_entries,
                                    int64_t n_pool_pages);

/*
 * KV append: write a chunk's K and V rows into their pages (the issue's
 * publishing of completed KV pages, after its "Expected vs actual" table;
 * run it before the chunk's attention, whose keys include the chunk's own).
 * Row i of k_new/v_new [rows][Hkv][d] is the token at position
 * history_len + i and goes to slot (history_len + i) % page_size of pool page
 * block_table[(history_len + i) / page_size] of k_pages/v_pages
 * [n_pool_pages][page_size][Hkv][d].  Nothing else in the pools changes; the
 * bits are copied unchanged (dtype only selects the 2-byte element type and
 * is checked like the attention's).  The block table must cover positions
 * 0 .. history_len + rows - 1.  rows == 0 is a no-op.  Errors as for the
 * attention: PPA_ERR_ALIAS when a new-rows pointer equals a pool pointer or
 * K and V share a pool; partial overlaps cannot be checked (the pool size is
 * not an argument).  Asynchronous on `stream`; no workspace.
 */
int paged_kv_append(const void* k_new, const void* v_new, void* k_pages, void* v_pages,
                    const int32_t* block_table, int64_t history_len, int32_t rows,
                    int32_t n_kv_heads, int32_t head_dim, int32_t page_size, int32_t dtype,
                    ppa_stream_t stream);

/*
 * Frees every split workspace, including the smaller ones kept after growth.
 * Call only when no stream still runs, and no captured graph will replay,
 * work that uses one, and not concurrently with any other call.
 */
int paged_prefill_release_workspaces(void);

/*
 * Host-only: bytes of the split workspace the library currently holds for
 * `stream` on the current device (0 if none), or a negative PPA_ERR_HIP.
 * A call with a split plan needs plan.workspace_bytes; below that it
 * allocates (so it cannot run under stream capture).
 */
int64_t paged_prefill_workspace_bytes(ppa_stream_t stream);

/* Static text for a status code. */
const char* paged_prefill_strerror(int code);

/* ABI version: major * 10000 + minor * 100 + patch. */
int paged_prefill_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_PREFILL_H */

// Device code of the split-partial attention kernel, included by the
// translation units that instantiate it per head dimension, query blocks per
// wave, page class and K/V format (they are compiled with their own
// register-allocation options).  The log-sum-exp merge kernel is in
// attention.hip.  Written for gfx950 (CDNA4, wave64).
//
// What is computed (issue "Metal: paged-KV prefill is 4.43x slower than
// contiguous KV at 32K"; PR "perf: scale prefill attention splits with GPU
// cores on Apple7/8", "What changed" and "Testing"): chunk row i at position
// H+i attends to keys 0..H+i; query head h reads KV head h / G; the key axis
// is cut into splits whose partials (output normalised by its own softmax
// sum, plus its log-sum-exp) are merged by a second kernel.
//
// A launch may also cover a packed batch of sequences, each with its own rows,
// history and block-table row over one page pool: each workgroup then first
// finds its sequence (see AttnArgs) and otherwise runs unchanged.
//
// Workgroup = 4 waves = 128 query vectors of one KV head (256 with two query
// blocks per wave, QB = 2).  A query vector is one (row, head) pair of the
// head group, flattened row-major, so the G heads of a row share a causal
// limit and every K/V byte staged in LDS serves 128 (256) queries.  K/V pages
// hold 16-bit values, or 8-bit quants with per-32-value scales (Q8) that are
// widened to fp16 in LDS.  Per 64-key tile:
//   * K and V rows stream from memory straight into LDS with 16-byte
//     buffer_load ... lds (no VGPR staging), double-buffered: K of the next
//     tile and V of this one load while this tile's QK and the previous
//     tile's PV run.  Paged addressing reads the block-table entries of a
//     tile once (one per lane), turns them into per-lane page addresses with
//     one 64-bit multiply-add, and each load takes its page base from one
//     lane; contiguous addressing is a per-tile base.  Rows are stored
//     row-major in 8x8-chunk blocks with an XOR swizzle so the MFMA operand
//     reads below do not collide in LDS banks.
//   * S^T = K Q^T on v_mfma_f32_32x32x16_{f16,bf16}: K is the A operand
//     (ds_read_b128), Q stays in registers as the B operand for the whole
//     kernel.  Each lane then owns one query vector and 32 of the tile's 64
//     keys, so a row max needs only one cross-lane exchange
//     (v_permlane32_swap) with the lane holding the other 32 keys.
//   * Softmax weights exp2(s c - m_ref) in fp32 (scale * log2 e folded into
//     one FMA before v_exp_f32) against a per-row integer reference that only
//     moves when a weight would overflow (see kSumLimit below), so the output
//     accumulators are rescaled only then, by an exact power of two.
//   * O^T += V^T P^T on the same MFMA: V^T is read with ds_read_b64_tr_b16,
//     which transposes 16-bit elements across lanes, so V stays row-major in
//     LDS; P's registers are already the B operand's layout.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "kernels.h"

namespace ppa {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

struct F16 {
  using vec8 = f16x8;
  static __device__ __forceinline__ f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma16(vec8 a, vec8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ vec8 from_f32(const float* x) {
    vec8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (_Float16)x[e];
    return r;
  }
  static __device__ __forceinline__ uint16_t bits(float x) {
    return __builtin_bit_cast(uint16_t, (_Float16)x);
  }
  // acc + the sum of the 8 elements (v_dot2c_f32_f16 against (1, 1), fp32 accumulation)
  static __device__ __forceinline__ float sum8(vec8 v, float acc) {
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int e = 0; e < 8; e += 2) acc = __builtin_amdgcn_fdot2(f16x2{v[e], v[e + 1]}, f16x2{1, 1}, acc, false);
    return acc;
  }
};

struct BF16 {
  using vec8 = bf16x8;
  static __device__ __forceinline__ f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma16(vec8 a, vec8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ vec8 from_f32(const float* x) {
    vec8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (__bf16)x[e];
    return r;
  }
  static __device__ __forceinline__ uint16_t bits(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
  }
  static __device__ __forceinline__ float sum8(vec8 v, float acc) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int e = 0; e < 8; e += 2)
      acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{v[e], v[e + 1]}, bf16x2{1, 1}, acc, false);
    return acc;
  }
};

constexpr int kTK = 64;        // keys per tile
constexpr int kWaves = 4;
// QB: query blocks of 32 vectors per wave.  With 2 (head dimensions up to
// 128), each K/V operand read and each loaded tile feed twice the MFMAs; the
// planner picks it for calls with more than one 128-vector m tile, and its m
// tile (query vectors per workgroup, 4 waves x 32 x QB) is the kernel's.
constexpr float kNegInf = -__builtin_inff();

template <int D>
struct Geom {
  static constexpr int CH = D / 8;                 // 16-byte chunks per K/V row
  static constexpr int TILE_BYTES = kTK * D * 2;   // one K (or V) tile
  static constexpr int BLOCKS = TILE_BYTES / 1024; // 1 KB blocks per tile
  static constexpr int LPW = BLOCKS / kWaves;      // blocks one wave loads per tile
};

// LDS layout of a 64-key K or V tile: 1 KB blocks of 8 rows x 8 chunks
// (16 bytes each).  Block (row / 8, c / 8) sits at ((c / 8) * 8 + row / 8) KB.
// Inside a block, row r and chunk c occupy 16-byte unit
//   (r % 8) * 8 + ((c % 8) ^ g(r)),   g(r) = ((r & 2) << 1) | ((r >> 2) & 3).
// One direct-to-LDS load fills one block; lane L writes unit L, so each group
// of 8 consecutive lanes reads 128 contiguous bytes of one row (in a permuted
// order), which the address unit coalesces (a lane order that spreads
// consecutive lanes over rows streams three times slower).  With pages of 8
// tokens or more the 8 rows of a block lie in one page.  LDS has 64 four-byte
// banks; a 16-byte read is served 16 lanes at a time and an 8-byte read 32
// lanes at a time.  g() makes every such group of the two MFMA operand reads
// below (K: 16 rows x one chunk; V transposed: 4 rows x 4 chunks) cover all 64
// banks once.
__device__ __forceinline__ constexpr int lds_g(int r) { return ((r & 2) << 1) | ((r >> 2) & 3); }
__device__ __forceinline__ constexpr int lds_off(int row, int c) {
  return (c >> 3) * 8192 + (row >> 3) * 1024 + ((row & 7) * 8 + ((c & 7) ^ lds_g(row & 15))) * 16;
}

// Barrier for the tile loop, which keeps direct-to-LDS loads in flight across
// it.  A workgroup-scope release (as in __syncthreads) must wait for every
// LDS write in flight, those loads included (vmcnt(0)); instead the caller
// waits for exactly the loads and LDS operations the next phase needs
// (s_waitcnt vmcnt(n) lgkmcnt(0)), and the wavefront-scope fences only keep
// the compiler from moving LDS accesses across the barrier.  LDS is one
// memory per CU, so a write that has completed is seen by every wave.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// A wave-uniform pointer pinned to scalar registers (a buffer descriptor
// must be uniform; this keeps the compiler from treating it as per-lane).
__device__ __forceinline__ const char* scalar_ptr(const char* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const char*)(((uint64_t)hi << 32) | lo);
}

// 16-byte direct-to-LDS load of lane bytes [base + voff, +16) into lds + 16 lane
// (lds is wave-uniform), as buffer_load_dwordx4 ... lds.  The buffer
// (MUBUF) form rather than global_load_lds: the compiler counts a global
// (FLAT-encoded) load that writes LDS against both vmcnt and lgkmcnt, and
// then waits for lgkmcnt(0) at the next use of any LDS read result, which
// would drain the operand-read prefetch after every K/V load.  Descriptor:
// base = the scalar base, stride 0, no practical range limit (offsets stay
// below 2^31), 32-bit data format (word 3 = 0x20000).
// soff is a wave-uniform byte offset added to every lane's address.
__device__ __forceinline__ void load_lds16(const char* base, uint32_t voff, int soff, void* lds) {
  __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)scalar_ptr(base), (short)0, 0x7fffffff, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, LDS_PTR(void, lds), 16, (int)voff, __builtin_amdgcn_readfirstlane(soff), 0, 0);
}

__device__ __forceinline__ float max_with_partner(float x) {
  // v_permlane32_swap pairs lane l with lane l^32; both results hold the pair.
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_with_partner(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);  // same order on both lanes
}

// acc *= alpha for an output accumulator tile.  Translation units built with
// MFMA results in AGPRs (PPA_MFMA_AGPR_FORM) keep the accumulators there:
// VALU instructions cannot read AGPRs, and plain C++ would move the whole
// tile through VGPRs and make the allocator spill, so each element is read,
// scaled and written back in place.  The nops before the first read cover
// the wait an MFMA result needs before an accumulator read (at most 18 wait
// states), those after each write the wait before an MFMA reads it.
__device__ __forceinline__ void scale_acc(f32x16& acc, float alpha) {
#if defined(PPA_MFMA_AGPR_FORM) && PPA_MFMA_AGPR_FORM
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float x = acc[r], t;
    if (r == 0)
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\tv_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %2, %1\n\t"
                   "v_accvgpr_write_b32 %0, %1\n\ts_nop 4"
                   : "+a"(x), "=&v"(t) : "v"(alpha));
    else
      asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %2, %1\n\tv_accvgpr_write_b32 %0, %1\n\ts_nop 4"
                   : "+a"(x), "=&v"(t) : "v"(alpha));
    acc[r] = x;
  }
#else
  acc *= alpha;
#endif
}

// How K/V rows are addressed.  Contig: [ctx][Hkv][d].  Paged: pages of
// `page_size` tokens, each [page_size][Hkv][d].  PageBig: pages of 64 tokens or
// more, so a 64-key tile lies in one page.  Page16: pages of 16 or 32 tokens,
// so the 16 rows of two neighbouring 8-row groups share a page.  Page8: pages
// of 8 tokens, one page per 8-row group.  In these classes the 8 rows one
// direct-to-LDS load covers lie in one page, the page is wave-uniform, and an
// address is a scalar base plus a per-lane offset that does not change from
// tile to tile.  PageLane: smaller pages; every row looks up its own page.
enum class Addr { Contig, PageBig, Page16, Page8, PageLane };

// The softmax weights are exp2(s c - m_ref) against a reference m_ref per
// query vector that is an integer (log2 domain) and moves only when it must,
// instead of the running max of every tile, so the output accumulators are
// not rescaled on every tile and most tiles compute no max at all.  The first
// reference is the ceiling of the max of the split's first tile (a query
// vector that sees any key of the split sees its first key).  Later weights
// may exceed 1; fp16 or bf16 P and fp32 O and l hold them as long as none
// overflows.  After each tile the row sums are checked: an fp16 weight past
// the format's range rounds to infinity and makes the sum infinite, and a sum
// past kSumLimit bounds the weights of bf16.  Where a query vector fails, its
// wave takes the tile's max, raises the reference to its ceiling, scales O and
// l by 2^(old - new) (exact: both are integers) and recomputes the tile's
// weights.  Because every reference is an integer, a weight's fp16/bf16
// rounding does not depend on which reference (which split) it was computed
// against: exp2(x - n) is 2^-n exp2(x) in both formats' normal range.
constexpr float kSumLimit = 0x1p64f;

// Q8: K and V pages hold 8-bit quants with an fp16 scale per 32 values along
// d (see the q8 loader below); the tiles are widened to fp16 in LDS and the
// MFMA, softmax and P arithmetic run in fp16 whatever the type of q and out.
// KV16: K and V are fp16 (8-bit pages dequantized beforehand into a
// contiguous buffer) while q and out have type E: the same fp16 arithmetic as
// Q8, over 16-bit tiles.
template <int D, class E, Addr AM, bool Q8 = false, int QB = 1, bool KV16 = false>
__global__ __launch_bounds__(256, 1) __attribute__((amdgpu_waves_per_eu(1, 1))) void attn_partial_kernel(AttnArgs a) {
  static_assert(!Q8 || AM == Addr::Page16 || AM == Addr::PageBig, "8-bit pages need pages of 16 tokens or more");
  static_assert(!KV16 || (!Q8 && AM == Addr::Contig), "fp16 K/V under another q type: contiguous buffers");
  using Gm = Geom<D>;
  using M = std::conditional_t<Q8 || KV16, F16, E>;   // element type of the MFMA operands
  using vec8 = typename M::vec8;
  constexpr int EB = Q8 ? 1 : 2;              // bytes per K/V element in memory
  constexpr int MT = kWaves * 32 * QB;        // query vectors per workgroup
  constexpr int CH = Gm::CH;
  constexpr int LPW = Gm::LPW;
  constexpr int KS = D / 16;   // 16-wide d steps of QK
  constexpr int DB = D / 32;   // 32-wide d blocks of O
  constexpr bool PAGED = AM != Addr::Contig;
  // Four separate arrays, each picked statically: the compiler can then see
  // that a read of one buffer does not alias a direct-to-LDS load into another
  // and does not make it wait for those loads (they complete a tile later).
  __shared__ __attribute__((aligned(1024))) uint8_t kbuf0[Gm::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t kbuf1[Gm::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t vbuf0[Gm::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t vbuf1[Gm::TILE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;

  // Workgroup -> (split, KV head, m tile).  Consecutive workgroup ids go to
  // different XCDs; remap so the workgroups one XCD holds are consecutive
  // logical tiles, which share a KV head and split and so share L2.
  int b = blockIdx.x;
  if (a.xcd_remap) b = (b & 7) * (gridDim.x >> 3) + (b >> 3);
  const int mt = b % a.tiles_m;
  const int rest = b / a.tiles_m;
  const int g = rest % a.n_kv_heads;
  const int rest2 = rest / a.n_kv_heads;
  const int s = rest2 % a.n_splits;
  // Several sequences: this workgroup's sequence, its rows and history.
  // Workgroups past the sequence's m tiles or past its last split exit (the
  // merge reads no split that starts after a row's last key).
  int ws_row0 = 0;
  if (a.n_seqs > 0) {
    const int seq = rest2 / a.n_splits;
    const int r0 = a.cu_rows[seq];
    a.rows = a.cu_rows[seq + 1] - r0;
    a.history = a.seq_history[seq];
    a.ctx = (int)a.history + a.rows;
    if (mt * MT >= a.rows * a.group || s * a.split_tokens >= a.ctx) return;
    a.q += (int64_t)r0 * a.n_q_heads * D;
    a.out += (int64_t)r0 * a.n_q_heads * D;
    a.bt += (int64_t)seq * a.bt_stride;
    ws_row0 = r0;
  }

  // Query vector f = (row, head) pair of the head group, row-major; wave w
  // holds blocks of 32 at mt MT + 32 (QB w + b), lane % 32 within the block.
  const int G = a.group;
  const int nqv = a.rows * G;
  bool qv_valid[QB];
  int row[QB], head[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int f = mt * MT + 32 * (QB * wave + qb) + (lane & 31);
    qv_valid[qb] = f < nqv;
    row[qb] = qv_valid[qb] ? f / G : a.rows - 1;
    head[qb] = g * G + (qv_valid[qb] ? f % G : 0);
  }
  const int f_last = min(mt * MT + MT - 1, nqv - 1);
  const int r_first = (mt * MT) / G;
  const int r_last = f_last / G;

  const int k0 = s * a.split_tokens;
  const int k1 = min(k0 + a.split_tokens, a.ctx);
  const int kend = min(k1, (int)(a.history + r_last + 1));
  const int n_tiles = kend > k0 ? (kend - k0 + kTK - 1) / kTK : 0;
  int lim[QB];                                      // last key each query vector sees
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) lim[qb] = (int)a.history + row[qb];
  // Tiles ending at or before the first row's last key need no mask, and they
  // are whole (split bounds are multiples of the tile).  A body works on tile
  // it and loads tile it+1, so the fast body (no mask, no load clamp) runs
  // while both are such tiles: it < n_fast.
  const int mask_x = (int)a.history + r_first - k0 - (kTK - 1);
  const int n_plain = min(n_tiles, mask_x < 0 ? 0 : mask_x / kTK + 1);
  const int n_fast = n_plain > 0 ? n_plain - 1 : 0;

  // Q fragments (B operand of QK): lane holds Q[f][16 ks + 8 h .. +7].
  vec8 qf[QB][KS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const uint16_t* qp = a.q + ((int64_t)row[qb] * a.n_q_heads + head[qb]) * D + 8 * h;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 raw = qv_valid[qb] ? *(const u32x4*)(qp + 16 * ks) : u32x4{0u, 0u, 0u, 0u};
      if constexpr (std::is_same_v<M, E>) {
        qf[qb][ks] = __builtin_bit_cast(vec8, raw);
      } else {
        // bf16 q for the fp16 MFMA: exact for |q| in fp16's normal range
        const bf16x8 qbf = __builtin_bit_cast(bf16x8, raw);
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[qb][ks][e] = (_Float16)(float)qbf[e];
      }
    }
  }
  // Wait for Q here, on every path: otherwise the compiler's wait before the
  // first use of Q inside the tile loop covers every load in flight, on every
  // iteration.
  __builtin_amdgcn_s_waitcnt(0x0F70);

  f32x16 o[QB][DB];
  float m_ref[QB], l[QB];  // per query block:
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_ref[qb] = kNegInf;   // softmax reference, scaled log2 domain, an integer once set
    l[qb] = 0.f;           // this lane's share of the softmax sum
  }
  const float c = a.scale_log2;

  // ---- loader -------------------------------------------------------------
  // Block b = wave * LPW + i of a tile holds rows 8 (b % 8) .. +7 and chunks
  // 8 (b / 8) .. +7 (lds_off).
  const int hkvd = a.n_kv_heads * D * EB;  // bytes per token (all KV heads)
  const int ps_mask = (1 << a.log2_ps) - 1;
  const int cg = (wave * LPW) >> 3;        // the wave's chunk group (same for all its blocks)
  // Lane L fills unit L of a block: row 8 rg + L / 8, chunk 8 cg + ((L % 8) ^ g(row)),
  // rg = the block's row group; g depends on rg only through its parity.
  const int lrow = lane >> 3;
  const int cpart_even = (cg * 8 + ((lane & 7) ^ lds_g(lrow))) << 4;
  const int cpart_odd = (cg * 8 + ((lane & 7) ^ lds_g(8 + lrow))) << 4;
  // Lane byte offsets within an 8-row group for whole tiles (tile to tile only
  // the group's scalar base changes).
  const uint32_t voff_even = lrow * hkvd + cpart_even;
  const uint32_t voff_odd = lrow * hkvd + cpart_odd;
  // Row group rg_i = (wave LPW + i) % 8 of load i starts soff[i] bytes past
  // its base: into the tile (contiguous, PageBig) or into its page.
  int soff[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int rg = (wave * LPW + i) & 7;
    soff[i] = (AM == Addr::Page16 || AM == Addr::Page8 ? ((8 * rg) & ps_mask) : 8 * rg) * hkvd;
  }
  const char* kg = (const char*)a.k + g * D * EB;
  const char* vg = (const char*)a.v + g * D * EB;
  const uint32_t page_bytes = (uint32_t)hkvd << a.log2_ps;
  // Scalar bases of one whole tile's loads for this wave: the tile start
  // (contiguous; with PageBig the tile's place in its page) or the page of
  // each 8-row group the wave loads (Page16: two neighbouring groups share a
  // page, so load i uses base i / 2; Page8: base i).  They are read once per
  // tile, right after the tile loop's barrier, from the per-lane page
  // addresses: the lane holding key t0 + 8 rg holds the page of row group rg,
  // and the wave's first group is (wave LPW) % 8 (even, so group pairs line up
  // with base pairs).  Load i then adds soff[i]; with pages of at most 32
  // tokens a tile starts on a page boundary, so soff[i] is the whole offset.
  constexpr int NBASE = AM == Addr::Page16 ? (LPW + 1) / 2 : AM == Addr::Page8 ? LPW : 1;
  struct TileBases {
    const char* base[NBASE];
  };
  const int lane_base = 8 * ((wave * LPW) & 7);
  auto tile_bases = [&](int j, int page, bool is_v) __attribute__((always_inline)) -> TileBases {
    TileBases tb;
    const int t0 = k0 + j * kTK;
    const char* src = is_v ? vg : kg;
    if constexpr (AM == Addr::Contig) {
      tb.base[0] = src + (int64_t)t0 * hkvd;
    } else if constexpr (AM == Addr::PageBig) {
      // lane 0 holds key t0's page, which holds the whole tile
      const uint64_t paddr = (uint64_t)src + (uint64_t)(uint32_t)page * page_bytes;
      const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)paddr, 0);
      const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(paddr >> 32), 0);
      tb.base[0] = (const char*)(((uint64_t)hi << 32) | lo) + (t0 & ps_mask) * hkvd;
    } else {
      // per lane: address of pool page `page`
      const uint64_t paddr = (uint64_t)src + (uint64_t)(uint32_t)page * page_bytes;
#pragma unroll
      for (int q = 0; q < NBASE; ++q) {
        const int ln = lane_base + (AM == Addr::Page16 ? 16 : 8) * q;
        const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)paddr, ln);
        const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(paddr >> 32), ln);
        tb.base[q] = (const char*)(((uint64_t)hi << 32) | lo);
      }
    }
    return tb;
  };

  // Pool page of key (tile j start + lane).  The key is clamped to kend-1, so
  // the block-table read is always in range (lanes and tiles past the end read
  // an entry nobody uses) and the load needs no branch.
  auto pages = [&](int j) __attribute__((always_inline)) -> int {
    if constexpr (!PAGED) return 0;
    const int key = min(k0 + j * kTK + lane, kend - 1);
    return a.bt[key >> a.log2_ps];
  };

  // Direct-to-LDS load i (of LPW) of tile j of K or V.  Keys at or past `kend`
  // are read from key kend-1 instead: they are masked for every query of the
  // workgroup (weight exactly 0) and a finite row keeps 0 * V finite, so there
  // is no zero fill.  With r0c = min(8 rg, (kend-1-t0) & ~7) and
  // lrow_c = min(lrow, kend-1-t0-r0c), whole tiles read their own rows and the
  // last tile's rows past kend-1 read row kend-1 (same 8-row group, so the
  // same page).  `page` holds the pool page of key (tile start + lane).
  // WHOLE: the caller knows tile j lies below kend, so the clamp is skipped:
  // the address is a scalar base (one lane read for the page) plus a
  // loop-invariant lane offset.
  // `tb` = tile_bases(j, page, is_v), used by the WHOLE form.
  auto issue_one = [&](int j, int page, const TileBases& tb, bool is_v, uint8_t* dst, int i, auto whole)
                       __attribute__((always_inline)) {
    constexpr bool WHOLE = decltype(whole)::value;
    const int t0 = k0 + j * kTK;
    const int last = kend - 1 - t0;
    const char* src = is_v ? vg : kg;
    const int b = wave * LPW + i;
    const int cpart = (b & 1) ? cpart_odd : cpart_even;
    if constexpr (WHOLE && AM != Addr::PageLane) {
      const uint32_t voff = (b & 1) ? voff_odd : voff_even;
      const int q = AM == Addr::Page16 ? i / 2 : AM == Addr::Page8 ? i : 0;
      load_lds16(tb.base[q], voff, soff[i], dst + b * 1024);
    } else if constexpr (AM == Addr::PageLane) {
      const int rr = min(8 * (b & 7) + lrow, last);
      const int pg = __shfl(page, rr, 64);
      const int64_t tok = ((int64_t)pg << a.log2_ps) + ((t0 + rr) & ps_mask);
      __builtin_amdgcn_global_load_lds((const void*)(src + tok * hkvd + cpart), LDS_PTR(void, dst + b * 1024), 16, 0, 0);
    } else {
      const int r0c = __builtin_amdgcn_readfirstlane(min(8 * (b & 7), last & ~7));
      const int lrow_c = min(lrow, last - r0c);
      const char* base;
      if constexpr (AM == Addr::Contig) {
        base = src + (int64_t)(t0 + r0c) * hkvd;
      } else {
        const int pg = __builtin_amdgcn_readlane(page, r0c);
        base = src + (((int64_t)pg << a.log2_ps) + ((t0 + r0c) & ps_mask)) * hkvd;
      }
      load_lds16(base, (uint32_t)(lrow_c * hkvd + cpart), 0, dst + b * 1024);
    }
  };
  auto issue = [&](int j, int page, bool is_v, uint8_t* dst) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < LPW; ++i) issue_one(j, page, TileBases{}, is_v, dst, i, std::false_type{});
  };

  // ---- 8-bit pages (Q8) ---------------------------------------------------
  // A tile arrives as quants, half the bytes of a 16-bit tile, and is widened
  // to fp16 in LDS.  Load i (of NQ = LPW / 2) of a wave covers the rows and
  // values of its 16-bit blocks 2i and 2i+1: rows 8 rg .. 8 rg + 15 (rg even,
  // so one page when pages hold 16 tokens or more) and values 64 cg .. +63.
  // Lane L reads the 16 quants of row 8 rg + L / 4 at value 64 cg + 16 (L % 4)
  // into a staging kilobyte in the upper half of the wave's own part of the
  // destination tile, which no other wave writes.  After reading all of its
  // staging data, the wave writes each lane's 16 values, quant * scale rounded
  // once to fp16, into the two 16-byte chunks they occupy in the tile layout.
  // The scales come with one 4-byte load per lane: lane l holds the scales of
  // blocks 2 cg and 2 cg + 1 of row rbase + l.
  constexpr int NQ = Q8 ? LPW / 2 : 1;
  constexpr int ROWS_W = 8 * LPW < 64 ? 8 * LPW : 64;   // rows one wave's loads cover
  const int rbase = 8 * ((wave * LPW) & 7);
  const uint32_t voff_q = (lane >> 2) * hkvd + 64 * cg + 16 * (lane & 3);
  const int sc_row_bytes = a.n_kv_heads * (D / 32) * 2;   // scale bytes per token
  auto issue_q8 = [&](int j, int page, const TileBases& tb, bool is_v, uint8_t* buf, int i, auto whole)
                      __attribute__((always_inline)) {
    constexpr bool WHOLE = decltype(whole)::value;
    uint8_t* dst = buf + (wave * LPW + NQ + i) * 1024;
    if constexpr (WHOLE) {
      load_lds16(tb.base[AM == Addr::Page16 ? i : 0], voff_q, soff[2 * i], dst);
    } else {
      // rows past kend - 1 read row kend - 1 (same 16-row group, same page)
      const int t0 = k0 + j * kTK;
      const int last = kend - 1 - t0;
      const int rg = (wave * LPW + 2 * i) & 7;
      const int r0c = __builtin_amdgcn_readfirstlane(min(8 * rg, last & ~15));
      const int lrow_c = min(lane >> 2, last - r0c);
      const int pg = __builtin_amdgcn_readlane(page, r0c);
      const char* base = (is_v ? vg : kg) + (((int64_t)pg << a.log2_ps) + ((t0 + r0c) & ps_mask)) * hkvd;
      load_lds16(base, (uint32_t)(lrow_c * hkvd + 64 * cg + 16 * (lane & 3)), 0, dst);
    }
  };
  auto load_scales = [&](int j, int page, bool is_v) __attribute__((always_inline)) -> uint32_t {
    const int t0 = k0 + j * kTK;
    const int r = min(rbase + (lane % ROWS_W), kend - 1 - t0);
    const int pg = __shfl(page, r, 64);
    const char* sp = (const char*)(is_v ? a.v_scale : a.k_scale);
    const int64_t tok = ((int64_t)pg << a.log2_ps) + ((t0 + r) & ps_mask);
    return *(const uint32_t*)(sp + tok * sc_row_bytes + g * (D / 32) * 2 + 4 * cg);
  };
  // Load i's staging kilobyte (wave block NQ + i) is read before load i
  // writes its blocks 2i and 2i+1, and 2i + 1 < NQ + j for every later j: the
  // writes never reach staging data still to be read.
  auto convert_q8 = [&](uint8_t* buf, uint32_t scales) __attribute__((always_inline)) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const u32x4 raw = *LDS_PTR(const u32x4, buf + (wave * LPW + NQ + i) * 1024 + 16 * lane);
      const int r = 8 * ((wave * LPW + 2 * i) & 7) + (lane >> 2);
      const uint32_t s2 = __shfl(scales, r - rbase, 64);
      const uint32_t sb = (lane & 2) ? (s2 >> 16) : (s2 & 0xffffu);
      const h2 ss = __builtin_bit_cast(h2, sb | (sb << 16));
      const h2 bias = {(_Float16)1152.0f, (_Float16)1152.0f};
      uint32_t w[8];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        // byte u = quant ^ 0x80 under exponent byte 0x64 is the fp16 1024 + u:
        // minus 1152 gives the quant exactly, times the scale rounds once
        const uint32_t x = raw[k] ^ 0x80808080u;
        const h2 lo = __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, x, 0x04010400u));
        const h2 hi = __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, x, 0x04030402u));
        w[2 * k] = __builtin_bit_cast(uint32_t, (lo - bias) * ss);
        w[2 * k + 1] = __builtin_bit_cast(uint32_t, (hi - bias) * ss);
      }
      const int c0 = 8 * cg + 2 * (lane & 3);
      *LDS_PTR(u32x4, buf + lds_off(r, c0)) = u32x4{w[0], w[1], w[2], w[3]};
      *LDS_PTR(u32x4, buf + lds_off(r, c0 + 1)) = u32x4{w[4], w[5], w[6], w[7]};
    }
  };

  // ---- MFMA phases --------------------------------------------------------
  // S^T[key][qv] = K Q^T for the 64 keys of a tile: lane holds qv = lane & 31
  // of each query block and keys 32 kb + 8 (r / 4) + 4 h + r % 4.  Each K
  // operand read feeds the MFMAs of all QB query blocks.
  f32x16 sc[QB][2];
  // lds_off(lane % 32 + 32 kb, 2 ks + h) = (kofs ^ (ks % 4) 32) + (ks / 4) 8192 + kb 4096
  const int kofs = ((lane >> 3) & 3) * 1024 + (lane & 7) * 128 + ((h ^ lds_g(lane & 15)) << 4);
  // The operand reads run QPF steps ahead of their MFMAs; sched_barrier pins
  // that order (the compiler otherwise waits on each read right before its
  // MFMA).
  auto qk = [&](const uint8_t* kt, auto&& step_hook) __attribute__((always_inline)) {
    constexpr int QPF = 3;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      sc[qb][0] = f32x16{};
      sc[qb][1] = f32x16{};
    }
    i16x8 k0r[KS], k1r[KS];
    auto load = [&](int ks) __attribute__((always_inline)) {
      const uint8_t* kl = kt + (kofs ^ ((ks & 3) << 5));
      const int imm = (ks >> 2) * 8192;
      k0r[ks] = *LDS_PTR(const i16x8, kl + imm);
      k1r[ks] = *LDS_PTR(const i16x8, kl + imm + 4096);
    };
#pragma unroll
    for (int ks = 0; ks < QPF && ks < KS; ++ks) load(ks);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + QPF < KS) load(ks + QPF);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        sc[qb][0] = M::mfma(__builtin_bit_cast(vec8, k0r[ks]), qf[qb][ks], sc[qb][0]);
        sc[qb][1] = M::mfma(__builtin_bit_cast(vec8, k1r[ks]), qf[qb][ks], sc[qb][1]);
      }
      step_hook(ks);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // PV of the previous tile fused with the row max and softmax of this one:
  // O^T[d][qv] += V^T[d][key] P^T[key][qv] (16 keys per MFMA, V^T read from
  // row-major V by two transposing reads per operand: the 16 lanes of a group
  // read rows 16 kstep + 4 h + (lane % 16) / 4 (and + 8) at columns
  // 32 db + 16 ((lane / 16) % 2) + 4 (lane % 4), each lane receiving one column
  // over 4 rows), while the VALU computes the max, the weights exp2(s c - m)
  // of this tile into pb_new and their sum.  Step i issues the V reads of
  // step i + VPF, one MFMA and a slice of the VALU work; sched_barrier pins
  // the interleave.  The two halves are independent: PV reads pb, softmax
  // writes pb_new.
  vec8 pb[QB][4], pb_new[QB][4];
  float rs[QB];   // this lane's sum of the tile's rounded weights (pb_new)
  // lds_off(16 kstep + vr (+ 8), 4 db + cc) + within = (vofs1 (vofs2) ^ (db % 2) 64)
  // + (db / 2) 8192 + kstep 2048, vr = 4 h + (lane % 16) / 4, cc = 2 ((lane / 16) % 2) + (lane % 4) / 2
  const int v_r = 4 * h + ((lane & 15) >> 2);
  const int v_cc = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int vofs1 = v_r * 128 + ((v_cc ^ lds_g(v_r)) << 4) + (lane & 1) * 8;
  const int vofs2 = 1024 + v_r * 128 + ((v_cc ^ lds_g(v_r + 8)) << 4) + (lane & 1) * 8;
  auto pv_softmax = [&](const uint8_t* vt, auto track, auto&& step_hook) __attribute__((always_inline)) {
    constexpr bool TRACK = decltype(track)::value;
    constexpr int NPV = 4 * DB;
    constexpr int VPF = D >= 256 ? 2 : 3;
    // steps that carry the max reduction (none when the tile's max is not needed)
    constexpr int MAX_STEPS = TRACK ? (NPV >= 16 ? 4 : 2) : 0;
    i16x4 vlo[NPV], vhi[NPV];
    auto load = [&](int i) __attribute__((always_inline)) {
      const int kstep = i / DB, db = i % DB;
      const int imm = (db >> 1) * 8192 + kstep * 2048;
      vlo[i] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, vt + (vofs1 ^ ((db & 1) << 6)) + imm));
      vhi[i] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, vt + (vofs2 ^ ((db & 1) << 6)) + imm));
    };
    // VALU work: max over the lane's 32 QB scores (MAX_STEPS steps, each within
    // one query block) if tracked, then their weights.  Element e is score
    // e % 32 of block e / 32 (kstep-major, 8 per pb entry).
    constexpr int ET = 32 * QB;
    constexpr int PER = TRACK ? ET / MAX_STEPS : 32;
    static_assert(32 % PER == 0, "a max step stays within one query block");
    auto elem = [&](int e) __attribute__((always_inline)) -> float { return sc[e >> 5][(e >> 4) & 1][e & 15]; };
    float part[MAX_STEPS > 0 ? MAX_STEPS : 1];
    float base[QB], p32[ET];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      base[qb] = (TRACK || m_ref[qb] == kNegInf) ? 0.f : m_ref[qb];
      rs[qb] = 0.f;
    }
    auto valu = [&](int i) __attribute__((always_inline)) {
      if (TRACK && i < MAX_STEPS) {
        float mx = elem(i * PER);
#pragma unroll
        for (int e = 1; e < PER; ++e) mx = fmaxf(mx, elem(i * PER + e));
        part[i] = mx;
        if (i == MAX_STEPS - 1) {
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            constexpr int SPB = MAX_STEPS / QB;   // max steps per block
            float m = part[qb * SPB];
#pragma unroll
            for (int j = 1; j < SPB; ++j) m = fmaxf(m, part[qb * SPB + j]);
            // the split's first tile (O and l are still 0): the first reference
            m_ref[qb] = ceilf(max_with_partner(m) * c);
            base[qb] = m_ref[qb] == kNegInf ? 0.f : m_ref[qb];
          }
        }
        return;
      }
      // weights of elements [e0, e1)
      const int n = NPV - MAX_STEPS;
      const int e0 = ((i - MAX_STEPS) * ET) / n, e1 = ((i - MAX_STEPS + 1) * ET) / n;
#pragma unroll
      for (int e = e0; e < e1; ++e) {
        p32[e] = __builtin_amdgcn_exp2f(fmaf(elem(e), c, -base[e >> 5]));
        if ((e & 7) == 7) {
          // The sum takes the rounded weights, the ones the PV product uses.
          pb_new[e >> 5][(e >> 3) & 3] = M::from_f32(p32 + (e & ~7));
          rs[e >> 5] = M::sum8(pb_new[e >> 5][(e >> 3) & 3], rs[e >> 5]);
        }
      }
    };
#pragma unroll
    for (int i = 0; i < VPF && i < NPV; ++i) load(i);
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
      if (i + VPF < NPV) load(i + VPF);
      const int kstep = i / DB, db = i % DB;
      i16x8 av = __builtin_shufflevector(vlo[i], vhi[i], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) o[qb][db] = M::mfma(__builtin_bit_cast(vec8, av), pb[qb][kstep], o[qb][db]);
      valu(i);
      step_hook(i);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // After a tile's weights: where a query vector's sum overflowed (see
  // kSumLimit), its wave raises the reference to the ceiling of the tile's
  // max, scales O and l (tiles up to the previous one) by the exact power of
  // two 2^(old - new) and recomputes this tile's weights.  Then this tile's
  // weights become the next PV's operand.
  auto commit_tile = [&]() __attribute__((always_inline)) {
    bool over = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) over |= !(l[qb] + rs[qb] <= kSumLimit);
    if (__builtin_expect(__ballot(over) != 0, 0)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float mx = sc[qb][0][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[qb][kb][r]);
        const float m_new = fmaxf(m_ref[qb], ceilf(max_with_partner(mx) * c));
        if (m_new != kNegInf && m_new != m_ref[qb]) {
          const float alpha = __builtin_amdgcn_exp2f(m_ref[qb] - m_new);   // 2^-k, 0 if m_ref was -inf
          l[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db) scale_acc(o[qb][db], alpha);
          m_ref[qb] = m_new;
        }
        const float base = m_ref[qb] == kNegInf ? 0.f : m_ref[qb];
        float p32[32];
        rs[qb] = 0.f;
#pragma unroll
        for (int e = 0; e < 32; ++e) {
          p32[e] = __builtin_amdgcn_exp2f(fmaf(sc[qb][e >> 4][e & 15], c, -base));
          if ((e & 7) == 7) {
            pb_new[qb][e >> 3] = M::from_f32(p32 + (e & ~7));
            rs[qb] = M::sum8(pb_new[qb][e >> 3], rs[qb]);
          }
        }
      }
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      l[qb] += rs[qb];
#pragma unroll
      for (int k = 0; k < 4; ++k) pb[qb][k] = pb_new[qb][k];
    }
  };

  // PV of the last tile (no softmax left to overlap).
  auto pv_last = [&](const uint8_t* vt) __attribute__((always_inline)) {
#pragma unroll
    for (int kstep = 0; kstep < 4; ++kstep)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int imm = (db >> 1) * 8192 + kstep * 2048;
        i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, vt + (vofs1 ^ ((db & 1) << 6)) + imm));
        i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, vt + (vofs2 ^ ((db & 1) << 6)) + imm));
        i16x8 av = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) o[qb][db] = M::mfma(__builtin_bit_cast(vec8, av), pb[qb][kstep], o[qb][db]);
      }
  };

  // ---- pipeline -----------------------------------------------------------
  // Iteration it: QK of tile it, then the softmax of tile it interleaved with
  // the PV of tile it-1 (independent of each other).  Loads run one tile
  // ahead: K(it+1) and V(it) are issued at the start of iteration it.  The
  // V buffer of "tile -1" is zeroed and pb starts at 0, so iteration 0 runs
  // the same code (its PV adds exact zeros).
  int pg0 = 0, pg1 = 0;  // pages of tiles it and it+1
  // vmcnt(n) with the other counters left alone (gfx9 s_waitcnt encoding:
  // vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
  constexpr int kWaitVmcnt0 = 0x0F70;
  // vmcnt(LPW) lgkmcnt(0): before the tile loop's barriers.
  constexpr int kWaitVmcntLPW = 0x0070 | (LPW & 15) | ((LPW >> 4) << 14);
  static_assert(LPW < 64, "vmcnt holds 6 bits");
  // At head dimensions up to 128 (16-bit pages) both loads of a body, K(it+1)
  // and V(it), go out during its QK phase, one per MFMA step, and the top
  // barrier of the next body covers both: one barrier per tile.  At d 256
  // V(it) loads during the PV phase instead, with a second barrier before PV
  // (the QK phase there is held by its operand reads; moving the V loads into
  // it gained 1% on a 2048-row chunk and lost 2% on 128-row pieces, and the
  // VGPR-form build of that code crashes the compiler).
  constexpr bool ONE_BARRIER = !Q8 && D <= 128;
  auto body = [&](int it, auto masked, auto track, auto parity) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked)::value;
    constexpr bool ODD = decltype(parity)::value;  // it is odd
    const int t0 = k0 + it * kTK;
    // This wave's loads in flight, oldest first: K(it) (issued during the QK
    // of it-1), V(it-1) (during the PV phase of it-1), LPW each.  Wait for
    // K(it) only; after the barrier K(it) is in LDS and the buffers of K(it-1)
    // and V(it-2) are free (every wave is done with body it-1).  With one
    // barrier per tile both were issued during the QK of it-1: wait for both.
    // Q8: nothing is in flight; the previous body widened K(it) and V(it-1)
    // in LDS.
    __builtin_amdgcn_s_waitcnt((Q8 || ONE_BARRIER) ? kWaitVmcnt0 & ~0x0F00 : kWaitVmcntLPW);
    lds_barrier();
    // The loads of K(it+1) and V(it) are spread over the MFMA steps (one per
    // few MFMAs) rather than issued in a burst, which would stall the waves on
    // a full address queue before any math starts.
    // On the last tile the K load of "tile n_tiles" reads row kend-1 (the
    // clamp above) into a buffer nothing reads again; keeping it unconditional
    // keeps this a straight-line block.
    const int pk = pg1, pv = pg0;
    pg0 = pg1;
    pg1 = pages(it + 2);
    TileBases kb{}, vb{};
    if constexpr (!MASKED) {
      kb = tile_bases(it + 1, pk, false);
      vb = tile_bases(it, pv, true);
    }
    uint32_t ksc = 0, vsc = 0;   // Q8: scales of K(it+1) and V(it)
    qk(ODD ? kbuf1 : kbuf0, [&](int ks) {
      if constexpr (Q8) {
        constexpr int EVERY = KS / NQ;
        if (ks % EVERY == 0)
          issue_q8(it + 1, pk, kb, false, ODD ? kbuf0 : kbuf1, ks / EVERY, std::bool_constant<!MASKED>{});
        if (ks == 1) ksc = load_scales(it + 1, pk, false);
      } else if constexpr (ONE_BARRIER) {
        static_assert(KS == 2 * LPW, "one load per QK step");
        if (ks % 2 == 0)
          issue_one(it + 1, pk, kb, false, ODD ? kbuf0 : kbuf1, ks / 2, std::bool_constant<!MASKED>{});
        else
          issue_one(it, pv, vb, true, ODD ? vbuf1 : vbuf0, ks / 2, std::bool_constant<!MASKED>{});
      } else {
        constexpr int EVERY = KS / LPW;
        if (ks % EVERY == 0)
          issue_one(it + 1, pk, kb, false, ODD ? kbuf0 : kbuf1, ks / EVERY, std::bool_constant<!MASKED>{});
      }
    });
    if constexpr (MASKED) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int rel = lim[qb] - t0;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
            sc[qb][kb][r] = key > rel ? kNegInf : sc[qb][kb][r];
          }
      }
    }
    // Now in flight: V(it-1), then K(it+1).  Wait for V(it-1), which the PV
    // below reads, so that its load latency hides behind the QK phase.  (With
    // one barrier per tile V(it-1) was waited for at the top.)
    if constexpr (!Q8 && !ONE_BARRIER) {
      __builtin_amdgcn_s_waitcnt(kWaitVmcntLPW);
      lds_barrier();
    } else {
      __builtin_amdgcn_sched_barrier(0);   // keep the two phases apart
    }
    // PV(it-1) with the previous weights, fused with this tile's softmax.
    pv_softmax(ODD ? vbuf0 : vbuf1, track, [&](int i) {
      if constexpr (Q8) {
        constexpr int EVERY = 4 * DB / NQ;
        if (i % EVERY == 0)
          issue_q8(it, pv, vb, true, ODD ? vbuf1 : vbuf0, i / EVERY, std::bool_constant<!MASKED>{});
        if (i == 1) vsc = load_scales(it, pv, true);
      } else if constexpr (!ONE_BARRIER) {
        constexpr int EVERY = 4 * DB / LPW;
        if (i % EVERY == 0)
          issue_one(it, pv, vb, true, ODD ? vbuf1 : vbuf0, i / EVERY, std::bool_constant<!MASKED>{});
      }
    });
    commit_tile();
    if constexpr (Q8) {
      // Widen K(it+1) and V(it): their buffers' last readers (QK(it-1) and
      // PV(it-2)) finished before this body's barrier.
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      convert_q8(ODD ? kbuf0 : kbuf1, ksc);
      convert_q8(ODD ? vbuf1 : vbuf0, vsc);
    }
  };
  // Tiles in even/odd pairs so that each body has its buffers fixed at compile
  // time and the output accumulators flow through one chain of code.
  auto run = [&](int& it, int end, auto masked) __attribute__((always_inline)) {
    const std::false_type no_track{};
    if (it < end && (it & 1)) {
      body(it, masked, no_track, std::true_type{});
      ++it;
    }
    for (; it + 1 < end; it += 2) {
      body(it, masked, no_track, std::false_type{});
      body(it + 1, masked, no_track, std::true_type{});
    }
    if (it < end) {
      body(it, masked, no_track, std::false_type{});
      ++it;
    }
  };
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
    for (int db = 0; db < DB; ++db) o[qb][db] = f32x16{};
#pragma unroll
    for (int kstep = 0; kstep < 4; ++kstep) pb[qb][kstep] = vec8{};
  }
  for (int i = tid; i < Gm::TILE_BYTES / 16; i += 256) *LDS_PTR(u32x4, vbuf1 + i * 16) = u32x4{0u, 0u, 0u, 0u};
  if (n_tiles > 0) {
    pg0 = pages(0);
    if constexpr (Q8) {
#pragma unroll
      for (int i = 0; i < NQ; ++i) issue_q8(0, pg0, TileBases{}, false, kbuf0, i, std::false_type{});
      const uint32_t s0 = load_scales(0, pg0, false);
      pg1 = pages(1);
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      convert_q8(kbuf0, s0);
    } else {
      issue(0, pg0, false, kbuf0);
      pg1 = pages(1);
      // K(0) is the only load in flight: the first body's vmcnt(LPW) would not wait for it.
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    }
    // Tile 0 runs in the masked body and takes its max (the first reference);
    // then the fast body (no mask, no clamp) while both its tile and the one
    // it loads lie below the first row's last key; then the masked body.
    body(0, std::true_type{}, std::true_type{}, std::false_type{});
    int it = 1;
    run(it, n_fast, std::false_type{});
    run(it, n_tiles, std::true_type{});
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if ((n_tiles - 1) & 1) pv_last(vbuf1);
    else pv_last(vbuf0);
  }

  // Epilogue: combine the two lanes' sums; lane holds d = 32 db + 8 q + 4 h + 0..3.
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l_tot = sum_with_partner(l[qb]);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (!qv_valid[qb]) continue;
    const int64_t pair = (int64_t)row[qb] * a.n_q_heads + head[qb];
    if (a.n_splits == 1) {
      uint16_t* op = a.out + pair * D + 4 * h;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x16& ov = o[qb][db];
          const uint32_t lo = E::bits(ov[4 * q4 + 0] * inv) | ((uint32_t)E::bits(ov[4 * q4 + 1] * inv) << 16);
          const uint32_t hi = E::bits(ov[4 * q4 + 2] * inv) | ((uint32_t)E::bits(ov[4 * q4 + 3] * inv) << 16);
          *(u32x2*)(op + 32 * db + 8 * q4) = u32x2{lo, hi};
        }
    } else {
      const int64_t pairs = (int64_t)a.ws_rows * a.n_q_heads;
      const int64_t wpair = pair + (int64_t)ws_row0 * a.n_q_heads;
      float* wp = a.ws_o + ((int64_t)s * pairs + wpair) * D + 4 * h;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x16& ov = o[qb][db];
          f32x4 v4 = {ov[4 * q4 + 0] * inv, ov[4 * q4 + 1] * inv, ov[4 * q4 + 2] * inv, ov[4 * q4 + 3] * inv};
          *(f32x4*)(wp + 32 * db + 8 * q4) = v4;
        }
      if (h == 0) a.ws_lse[(int64_t)s * pairs + wpair] = l_tot > 0.f ? m_ref[qb] + log2f(l_tot) : kNegInf;
    }
  }
}

template <int D, class E, Addr AM, bool Q8 = false, int QB = 1, bool KV16 = false>
hipError_t launch_attn_t(const AttnArgs& a, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((attn_partial_kernel<D, E, AM, Q8, QB, KV16>), dim3(grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

// 8-bit pages: 16 tokens per page or more (the host checks).
template <int D, class E, int QB = 1>
hipError_t launch_attn_q8(const AttnArgs& a, int grid, hipStream_t stream) {
  if (a.log2_ps >= 6) return launch_attn_t<D, E, Addr::PageBig, true, QB>(a, grid, stream);
  if (a.log2_ps >= 4) return launch_attn_t<D, E, Addr::Page16, true, QB>(a, grid, stream);
  return hipErrorInvalidValue;
}

// Every addressing class: contiguous K/V, then pages by size.
template <int D, class E, int QB = 1>
hipError_t launch_attn_p(const AttnArgs& a, bool paged, int grid, hipStream_t stream) {
  if (!paged) return launch_attn_t<D, E, Addr::Contig, false, QB>(a, grid, stream);
  if (a.log2_ps >= 6) return launch_attn_t<D, E, Addr::PageBig, false, QB>(a, grid, stream);
  if (a.log2_ps >= 4) return launch_attn_t<D, E, Addr::Page16, false, QB>(a, grid, stream);
  if (a.log2_ps == 3) return launch_attn_t<D, E, Addr::Page8, false, QB>(a, grid, stream);
  return launch_attn_t<D, E, Addr::PageLane, false, QB>(a, grid, stream);
}

// Contiguous K/V or pages of 16 tokens or more.
template <int D, class E>
hipError_t launch_attn_p_large(const AttnArgs& a, bool paged, int grid, hipStream_t stream) {
  if (!paged) return launch_attn_t<D, E, Addr::Contig>(a, grid, stream);
  if (a.log2_ps >= 6) return launch_attn_t<D, E, Addr::PageBig>(a, grid, stream);
  return launch_attn_t<D, E, Addr::Page16>(a, grid, stream);
}

// Pages of fewer than 16 tokens.
template <int D, class E>
hipError_t launch_attn_p_small(const AttnArgs& a, int grid, hipStream_t stream) {
  if (a.log2_ps == 3) return launch_attn_t<D, E, Addr::Page8>(a, grid, stream);
  return launch_attn_t<D, E, Addr::PageLane>(a, grid, stream);
}

}  // namespace
}  // namespace ppa

// Chunked prefill attention over a paged KV cache: the split-partial kernel
// and the log-sum-exp merge kernel, written for gfx950 (CDNA4, wave64).
//
// What is computed (issue "Metal: paged-KV prefill is 4.43x slower than
// contiguous KV at 32K"; PR "perf: scale prefill attention splits with GPU
// cores on Apple7/8", "What changed" and "Testing"): chunk row i at position
// H+i attends to keys 0..H+i; query head h reads KV head h / G; the key axis
// is cut into splits whose partials (output normalised by its own softmax
// sum, plus its log-sum-exp) are merged by a second kernel.
//
// Workgroup = 4 waves = 128 query vectors of one KV head.  A query vector is
// one (row, head) pair of the head group, flattened row-major, so the G heads
// of a row share a causal limit and every K/V byte staged in LDS serves
// 128 queries.  Per 64-key tile:
//   * K and V rows stream from HBM straight into LDS with 16-byte
//     global_load_lds (no VGPR staging), double-buffered so the next tile's
//     loads overlap this tile's math.  Paged addressing reads one block-table
//     entry per key, prefetched one tile ahead and shared across the wave by
//     a lane shuffle; contiguous addressing is the identity.  Chunks are
//     XOR-swizzled per row so the MFMA operand reads below do not collide in
//     LDS banks.
//   * S^T = K Q^T on v_mfma_f32_32x32x16_{f16,bf16}: K is the A operand
//     (ds_read_b128), Q stays in VGPRs as the B operand for the whole kernel.
//     Each lane then owns one query vector and 32 of the tile's 64 keys, so
//     row max and row sum need only one cross-lane exchange
//     (v_permlane32_swap) with the lane holding the other 32 keys.
//   * fp32 online softmax in the log2 domain (scale * log2 e folded into one
//     FMA before v_exp_f32); the O rescale is skipped when no lane's max
//     moved, which is exact (the factor would be 1.0).
//   * O^T += V^T P^T on the same MFMA: V^T is read with ds_read_b64_tr_b16,
//     which transposes 16-bit elements across lanes, so V stays row-major in
//     LDS; P's registers are already the B operand's layout.
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
  static __device__ __forceinline__ vec8 from_f32(const float* x) {
    vec8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (_Float16)x[e];
    return r;
  }
  static __device__ __forceinline__ uint16_t bits(float x) {
    return __builtin_bit_cast(uint16_t, (_Float16)x);
  }
};

struct BF16 {
  using vec8 = bf16x8;
  static __device__ __forceinline__ f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
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
};

constexpr int kTK = 64;        // keys per tile
constexpr int kWaves = 4;
constexpr float kNegInf = -__builtin_inff();

template <int D>
struct Geom {
  static constexpr int CH = D / 8;                 // 16-byte chunks per K/V row
  static constexpr int TILE_BYTES = kTK * D * 2;   // one K (or V) tile
  static constexpr int BLOCKS = TILE_BYTES / 1024; // 1 KB blocks per tile
  static constexpr int LPW = BLOCKS / kWaves;      // blocks one wave loads per tile
};

// LDS layout of a 64-key K or V tile: 1 KB blocks of 8 rows x 8 chunks
// (16 bytes each), chunk-major inside the block.  Block (row / 8, c / 8)
// sits at ((c / 8) * 8 + row / 8) KB.  One direct-to-LDS load fills one
// block: its 64 lanes read 8 rows x 128 contiguous bytes (8 whole cache
// lines), and with pages of 8 tokens or more the 8 rows lie in one page.
// Both MFMA operand reads below (K: 32 rows x one chunk; V transposed:
// 8 rows x 4 chunks) touch every 16-byte bank group the minimum number of
// times, and their addresses are a per-lane base plus compile-time offsets.
__device__ __forceinline__ constexpr int lds_off(int row, int c) {
  return (c >> 3) * 8192 + (row >> 3) * 1024 + (c & 7) * 128 + (row & 7) * 16;
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

// How K/V rows are addressed.  Contig: [ctx][Hkv][d].  PageWave: pages of
// 16 tokens or more; the 16 rows one wave loads per tile then lie in one page,
// so the page is wave-uniform and an address is a scalar base plus a per-lane
// offset that does not change from tile to tile.  PageLane: smaller pages;
// every row looks up its own page.
enum class Addr { Contig, PageWave, PageLane };

// Softmax reference max is only raised when a tile's max exceeds it by more
// than 2^8 (log2 domain): the weights exp2(s c - m) then stay below 256, well
// inside fp16 and bf16 range, and the O/l rescale (128 multiplies per lane at
// head_dim 256) runs a handful of times per row instead of on every tile.
// The result is the same softmax; only rounding differs.
constexpr float kRescaleLog2 = 8.0f;

template <int D, class E, Addr AM>
__global__ __launch_bounds__(256, 1) void attn_partial_kernel(AttnArgs a) {
  using Gm = Geom<D>;
  using vec8 = typename E::vec8;
  constexpr int CH = Gm::CH;
  constexpr int LPW = Gm::LPW;
  constexpr int KS = D / 16;   // 16-wide d steps of QK
  constexpr int DB = D / 32;   // 32-wide d blocks of O
  constexpr bool PAGED = AM != Addr::Contig;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[4 * Gm::TILE_BYTES];
  uint8_t* const kbuf0 = smem;
  uint8_t* const kbuf1 = smem + Gm::TILE_BYTES;
  uint8_t* const vbuf0 = smem + 2 * Gm::TILE_BYTES;
  uint8_t* const vbuf1 = smem + 3 * Gm::TILE_BYTES;

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
  const int s = rest / a.n_kv_heads;

  const int G = a.group;
  const int nqv = a.rows * G;
  const int f = mt * 128 + wave * 32 + (lane & 31);
  const bool qv_valid = f < nqv;
  const int row = qv_valid ? f / G : a.rows - 1;
  const int head = g * G + (qv_valid ? f % G : 0);
  const int f_last = min(mt * 128 + 127, nqv - 1);
  const int r_first = (mt * 128) / G;
  const int r_last = f_last / G;

  const int k0 = s * a.split_tokens;
  const int k1 = min(k0 + a.split_tokens, a.ctx);
  const int kend = min(k1, (int)(a.history + r_last + 1));
  const int n_tiles = kend > k0 ? (kend - k0 + kTK - 1) / kTK : 0;
  const int lim = (int)a.history + row;             // last key this query vector sees
  // Tiles ending at or before the first row's last key need no mask.
  const int mask_x = (int)a.history + r_first - k0 - (kTK - 1);
  const int n_plain = min(n_tiles, mask_x < 0 ? 0 : mask_x / kTK + 1);

  // Q fragments (B operand of QK): lane holds Q[f][16 ks + 8 h .. +7].
  vec8 qf[KS];
  {
    const uint16_t* qp = a.q + ((int64_t)row * a.n_q_heads + head) * D + 8 * h;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 raw = qv_valid ? *(const u32x4*)(qp + 16 * ks) : u32x4{0u, 0u, 0u, 0u};
      qf[ks] = __builtin_bit_cast(vec8, raw);
    }
  }

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  float m_ref = kNegInf;  // reference max, scaled log2 domain
  float l = 0.f;          // this lane's share of the softmax sum
  const float c = a.scale_log2;

  // ---- loader -------------------------------------------------------------
  // Block b = wave * LPW + i of a tile holds rows 8 (b % 8) .. +7 and chunks
  // 8 (b / 8) .. +7; lane L loads row 8 (b % 8) + L % 8, chunk 8 (b / 8) + L / 8.
  const int hkvd2 = a.n_kv_heads * D * 2;  // bytes per token (all KV heads)
  const int ps_mask = (1 << a.log2_ps) - 1;
  const int cg = (wave * LPW) >> 3;        // the wave's chunk group (same for all its blocks)
  const uint32_t lane_off = (lane & 7) * hkvd2 + ((cg * 8 + (lane >> 3)) << 4);
  const char* kg = (const char*)a.k + g * D * 2;
  const char* vg = (const char*)a.v + g * D * 2;

  auto pages = [&](int j) -> int {
    if constexpr (!PAGED) return 0;
    const int key = k0 + j * kTK + lane;
    return (j < n_tiles && key < kend) ? a.bt[key >> a.log2_ps] : 0;
  };

  // Direct-to-LDS loads of tile j of K or V.  Keys at or past `kend` are read
  // from key kend-1 instead: they are masked for every query of the workgroup
  // (weight exactly 0) and a finite row keeps 0 * V finite, so there is no
  // zero fill.  `page` holds the pool page of key (tile start + lane).
  auto issue = [&](int j, int page, bool is_v, uint8_t* dst) {
    const int t0 = k0 + j * kTK;
    const int last = kend - 1 - t0;
    const char* src = is_v ? vg : kg;
    if (AM != Addr::PageLane && last >= kTK - 1) {
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        const int b = wave * LPW + i;
        const int r0 = 8 * (b & 7);   // first row of the block
        const char* base;
        if constexpr (AM == Addr::Contig) {
          base = src + (int64_t)(t0 + r0) * hkvd2;
        } else {
          const int pg = __builtin_amdgcn_readlane(page, r0);
          base = src + (((int64_t)pg << a.log2_ps) + ((t0 + r0) & ps_mask)) * hkvd2;
        }
        __builtin_amdgcn_global_load_lds((const void*)(base + lane_off), LDS_PTR(void, dst + b * 1024), 16, 0, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        const int b = wave * LPW + i;
        const int rr = min(8 * (b & 7) + (lane & 7), last);
        int64_t tok;
        if constexpr (AM == Addr::Contig) {
          tok = t0 + rr;
        } else {
          const int pg = __shfl(page, rr, 64);
          tok = ((int64_t)pg << a.log2_ps) + ((t0 + rr) & ps_mask);
        }
        __builtin_amdgcn_global_load_lds((const void*)(src + tok * hkvd2 + ((cg * 8 + (lane >> 3)) << 4)),
                                         LDS_PTR(void, dst + b * 1024), 16, 0, 0);
      }
    }
  };

  // ---- MFMA phases --------------------------------------------------------
  // S^T[key][qv] = K Q^T for the 64 keys of a tile: lane holds qv = lane & 31
  // and keys 32 kb + 8 (r / 4) + 4 h + r % 4.
  f32x16 sc[2];
  auto qk = [&](const uint8_t* kt) {
    sc[0] = f32x16{};
    sc[1] = f32x16{};
    const uint8_t* kl = kt + lds_off(lane & 31, h);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      i16x8 r0 = *LDS_PTR(const i16x8, kl + lds_off(0, 2 * ks));
      i16x8 r1 = *LDS_PTR(const i16x8, kl + lds_off(32, 2 * ks));
      sc[0] = E::mfma(__builtin_bit_cast(vec8, r0), qf[ks], sc[0]);
      sc[1] = E::mfma(__builtin_bit_cast(vec8, r1), qf[ks], sc[1]);
    }
  };

  // O^T[d][qv] += V^T[d][key] P^T[key][qv], 16 keys per MFMA.  V^T comes from
  // row-major V by two transposing reads per operand: the 16 lanes of a
  // group read rows 16 kstep + 4 h + (lane % 16) / 4 (and + 8) at columns
  // 32 db + 16 ((lane / 16) % 2) + 4 (lane % 4), and each lane receives one
  // column over 4 rows.
  vec8 pb[4];
  auto pv = [&](const uint8_t* vt) {
    const int col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);  // column within a 32-wide block
    const uint8_t* vl = vt + lds_off(4 * h + ((lane & 15) >> 2), col >> 3) + (col & 7) * 2;
#pragma unroll
    for (int kstep = 0; kstep < 4; ++kstep) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, vl + lds_off(16 * kstep, 4 * db)));
        i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, vl + lds_off(16 * kstep + 8, 4 * db)));
        i16x8 av = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        o[db] = E::mfma(__builtin_bit_cast(vec8, av), pb[kstep], o[db]);
      }
    }
  };

  // Weights of the current S into pb (the B operand of PV), and their sum.
  auto softmax = [&](float alpha) {
    const float base = m_ref == kNegInf ? 0.f : m_ref;
    float rs = 0.f;
#pragma unroll
    for (int kstep = 0; kstep < 4; ++kstep) {
      float p8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sc[kstep >> 1][8 * (kstep & 1) + e], c, -base));
        p8[e] = p;
        rs += p;
      }
      pb[kstep] = E::from_f32(p8);
    }
    l = l * alpha + rs;
  };

  // ---- pipeline -----------------------------------------------------------
  // Iteration it: QK of tile it, then the softmax of tile it interleaved with
  // the PV of tile it-1 (independent of each other).  Loads run one tile
  // ahead: K(it+1) and V(it) are issued at the start of iteration it.  The
  // V buffer of "tile -1" is zeroed and pb starts at 0, so iteration 0 runs
  // the same code (its PV adds exact zeros).
#pragma unroll
  for (int kstep = 0; kstep < 4; ++kstep) pb[kstep] = vec8{};
  for (int i = tid; i < Gm::TILE_BYTES / 16; i += 256) *LDS_PTR(u32x4, vbuf1 + i * 16) = u32x4{0u, 0u, 0u, 0u};
  int pg0 = 0, pg1 = 0;  // pages of tiles it and it+1
  if (n_tiles > 0) {
    pg0 = pages(0);
    issue(0, pg0, false, kbuf0);
    pg1 = pages(1);
  }

  bool pend = false;       // O waits for a rescale by pend_alpha
  float pend_alpha = 1.f;
  auto body = [&](int it, auto masked) {
    constexpr bool MASKED = decltype(masked)::value;
    const int t0 = k0 + it * kTK;
    // K(it) and V(it-1) have landed in every wave; K(it-1), V(it-2) are free.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (it + 1 < n_tiles) issue(it + 1, pg1, false, (it & 1) ? kbuf0 : kbuf1);
    issue(it, pg0, true, (it & 1) ? vbuf1 : vbuf0);
    pg0 = pg1;
    pg1 = pages(it + 2);
    qk((it & 1) ? kbuf1 : kbuf0);
    if constexpr (MASKED) {
      const int rel = lim - t0;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
          sc[kb][r] = key > rel ? kNegInf : sc[kb][r];
        }
    }
    float mx = sc[0][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sc[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[1][r]);
    const float mxs = max_with_partner(mx) * c;
    // A raise of the reference max decided on the previous tile moves O to
    // the new reference now, after PV(it-2) and before PV(it-1) (rare).
    if (__ballot(pend)) {
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= pend_alpha;
    }
    // Raise the reference max where this tile exceeds it by more than 2^8.
    pend = mxs > m_ref + kRescaleLog2;
    const float m_new = pend ? mxs : m_ref;
    pend_alpha = __builtin_amdgcn_exp2f(m_ref - m_new);  // 1 where unchanged
    m_ref = m_new;
    // PV(it-1) reads the previous pb before softmax(it) rewrites it; the two
    // are independent and form one block, so MFMA and VALU work interleave.
    pv((it & 1) ? vbuf0 : vbuf1);
    softmax(pend_alpha);
  };

  int it = 0;
  for (; it < n_plain; ++it) body(it, std::false_type{});
  for (; it < n_tiles; ++it) body(it, std::true_type{});
  if (n_tiles > 0) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (__ballot(pend)) {
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= pend_alpha;
    }
    pv(((n_tiles - 1) & 1) ? vbuf1 : vbuf0);
  }

  // Epilogue: combine the two lanes' sums; lane holds d = 32 db + 8 q + 4 h + 0..3.
  const float l_tot = sum_with_partner(l);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (!qv_valid) return;
  const int64_t pair = (int64_t)row * a.n_q_heads + head;
  if (a.n_splits == 1) {
    uint16_t* op = a.out + pair * D + 4 * h;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const uint32_t lo = E::bits(o[db][4 * q4 + 0] * inv) | ((uint32_t)E::bits(o[db][4 * q4 + 1] * inv) << 16);
        const uint32_t hi = E::bits(o[db][4 * q4 + 2] * inv) | ((uint32_t)E::bits(o[db][4 * q4 + 3] * inv) << 16);
        *(u32x2*)(op + 32 * db + 8 * q4) = u32x2{lo, hi};
      }
  } else {
    const int64_t pairs = (int64_t)a.rows * a.n_q_heads;
    float* wp = a.ws_o + ((int64_t)s * pairs + pair) * D + 4 * h;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        f32x4 v4 = {o[db][4 * q4 + 0] * inv, o[db][4 * q4 + 1] * inv, o[db][4 * q4 + 2] * inv,
                    o[db][4 * q4 + 3] * inv};
        *(f32x4*)(wp + 32 * db + 8 * q4) = v4;
      }
    if (h == 0) a.ws_lse[(int64_t)s * pairs + pair] = l_tot > 0.f ? m_ref + log2f(l_tot) : kNegInf;
  }
}

// Log-sum-exp merge of split partials, one (row, head) pair per D/4 threads,
// 4 output elements per thread, splits summed in index order.  Splits that
// start past a row's last key hold nothing for it and are not read.
template <int D, class E>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  constexpr int TPP = D / 4;
  constexpr int PPB = 256 / TPP;
  const int pairs = a.rows * a.n_q_heads;
  const int pair = blockIdx.x * PPB + threadIdx.x / TPP;
  if (pair >= pairs) return;
  const int dl = (threadIdx.x % TPP) * 4;
  const int row = pair / a.n_q_heads;
  int nv = (int)((a.history + row) / a.split_tokens) + 1;
  if (nv > a.n_splits) nv = a.n_splits;
  float mx = kNegInf;
  for (int s = 0; s < nv; ++s) mx = fmaxf(mx, a.ws_lse[(int64_t)s * pairs + pair]);
  float wsum = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < nv; ++s) {
    const float w = exp2f(a.ws_lse[(int64_t)s * pairs + pair] - mx);
    const f32x4 ov = *(const f32x4*)(a.ws_o + ((int64_t)s * pairs + pair) * D + dl);
    acc += w * ov;
    wsum += w;
  }
  const float inv = 1.f / wsum;
  const uint32_t lo = E::bits(acc[0] * inv) | ((uint32_t)E::bits(acc[1] * inv) << 16);
  const uint32_t hi = E::bits(acc[2] * inv) | ((uint32_t)E::bits(acc[3] * inv) << 16);
  *(u32x2*)(a.out + (int64_t)pair * D + dl) = u32x2{lo, hi};
}

template <int D, class E, Addr AM>
hipError_t launch_attn_t(const AttnArgs& a, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((attn_partial_kernel<D, E, AM>), dim3(grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int D, class E>
hipError_t launch_attn_p(const AttnArgs& a, bool paged, int grid, hipStream_t stream) {
  if (!paged) return launch_attn_t<D, E, Addr::Contig>(a, grid, stream);
  if (a.log2_ps >= 3) return launch_attn_t<D, E, Addr::PageWave>(a, grid, stream);
  return launch_attn_t<D, E, Addr::PageLane>(a, grid, stream);
}

template <class E>
hipError_t launch_attn_d(const AttnArgs& a, int head_dim, bool paged, int grid, hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_attn_p<64, E>(a, paged, grid, stream);
    case 128: return launch_attn_p<128, E>(a, paged, grid, stream);
    case 256: return launch_attn_p<256, E>(a, paged, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

template <class E>
hipError_t launch_merge_d(const MergeArgs& a, int head_dim, int grid, hipStream_t stream) {
  switch (head_dim) {
    case 64: hipLaunchKernelGGL((merge_kernel<64, E>), dim3(grid), dim3(256), 0, stream, a); break;
    case 128: hipLaunchKernelGGL((merge_kernel<128, E>), dim3(grid), dim3(256), 0, stream, a); break;
    case 256: hipLaunchKernelGGL((merge_kernel<256, E>), dim3(grid), dim3(256), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, int head_dim, int dtype, bool paged, int grid,
                            hipStream_t stream) {
  return dtype == 1 ? launch_attn_d<BF16>(a, head_dim, paged, grid, stream)
                    : launch_attn_d<F16>(a, head_dim, paged, grid, stream);
}

hipError_t launch_merge(const MergeArgs& a, int head_dim, int dtype, int grid, hipStream_t stream) {
  return dtype == 1 ? launch_merge_d<BF16>(a, head_dim, grid, stream)
                    : launch_merge_d<F16>(a, head_dim, grid, stream);
}

}  // namespace ppa

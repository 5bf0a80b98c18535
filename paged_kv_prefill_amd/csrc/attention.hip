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
  static constexpr int LPW = TILE_BYTES / 1024 / kWaves;  // 1 KB direct loads per wave per tile
  static constexpr int RPI = 64 / CH;              // rows covered by one 1 KB load
};

// Chunk swizzles: LDS chunk position of (row, chunk c) is c ^ swz(row).
// K: the 32 rows one QK operand read touches land on distinct 16-byte bank
// groups.  V: the 8 rows x 4 chunks one transposing read touches cover each
// bank group exactly twice.
template <int CH>
__device__ __forceinline__ int swz_k(int row) {
  if constexpr (CH >= 16) return row & 15;
  else return (row >> 1) & 7;
}
template <int CH>
__device__ __forceinline__ int swz_v(int row) {
  if constexpr (CH >= 16) return (row & 3) << 2;
  else return ((row >> 1) & 1) << 2;
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

// Issue the direct-to-LDS loads of one 64-key tile of K and V.  `page` is the
// pool page of key t0 + lane (paged), keys at or past `kend` are not read and
// their V rows are zeroed (K rows there are masked by the softmax).
template <int D, bool PAGED>
__device__ __forceinline__ void issue_tile(const AttnArgs& a, int g, int t0, int kend, int wave,
                                           int lane, int page, uint8_t* kbuf, uint8_t* vbuf) {
  using Gm = Geom<D>;
  const int ps_mask = (1 << a.log2_ps) - 1;
#pragma unroll
  for (int i = 0; i < Gm::LPW; ++i) {
    const int instr = wave * Gm::LPW + i;
    const int slot = instr * 64 + lane;
    const int row = slot / Gm::CH;
    const int pos = slot % Gm::CH;
    const int t = t0 + row;
    int64_t tok;
    if constexpr (PAGED) {
      const int pg = __shfl(page, row, 64);
      tok = ((int64_t)pg << a.log2_ps) + (t & ps_mask);
    } else {
      tok = t;
    }
    const int64_t base = (tok * a.n_kv_heads + g) * D;
    const int ck = pos ^ swz_k<Gm::CH>(row);
    const int cv = pos ^ swz_v<Gm::CH>(row);
    uint8_t* kd = kbuf + instr * 1024;
    uint8_t* vd = vbuf + instr * 1024;
    if (t < kend) {
      __builtin_amdgcn_global_load_lds((const void*)(a.k + base + ck * 8), LDS_PTR(void, kd), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(a.v + base + cv * 8), LDS_PTR(void, vd), 16, 0, 0);
    } else {
      *LDS_PTR(u32x4, vd + lane * 16) = u32x4{0u, 0u, 0u, 0u};
    }
  }
}

template <int D, class E, bool PAGED>
__global__ __launch_bounds__(256, 1) void attn_partial_kernel(AttnArgs a) {
  using Gm = Geom<D>;
  using vec8 = typename E::vec8;
  constexpr int CH = Gm::CH;
  constexpr int KS = D / 16;   // 16-wide d steps of QK
  constexpr int DB = D / 32;   // 32-wide d blocks of O
  __shared__ __attribute__((aligned(1024))) uint8_t smem[4 * Gm::TILE_BYTES];

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
  const int mask_from = (int)a.history + r_first;   // tiles ending past this need the mask

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
  float m = kNegInf;  // running max of raw scores
  float l = 0.f;      // this lane's share of the running sum
  const float c = a.scale_log2;

  // Block-table prefetch: lane k holds the page of key (tile start + k).
  int page_next = 0;
  if constexpr (PAGED) {
    if (n_tiles > 0 && k0 + lane < kend) page_next = a.bt[(k0 + lane) >> a.log2_ps];
  }
  if (n_tiles > 0) {
    issue_tile<D, PAGED>(a, g, k0, kend, wave, lane, page_next, smem, smem + Gm::TILE_BYTES);
    if constexpr (PAGED) {
      const int tn = k0 + kTK + lane;
      page_next = (n_tiles > 1 && tn < kend) ? a.bt[tn >> a.log2_ps] : 0;
    }
  }

  for (int it = 0; it < n_tiles; ++it) {
    const int t0 = k0 + it * kTK;
    uint8_t* kt = smem + (it & 1) * 2 * Gm::TILE_BYTES;
    uint8_t* vt = kt + Gm::TILE_BYTES;
    // This tile's loads (and the page prefetch) have landed in every wave,
    // and every wave is done reading the other buffer.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (it + 1 < n_tiles) {
      uint8_t* kn = smem + ((it + 1) & 1) * 2 * Gm::TILE_BYTES;
      issue_tile<D, PAGED>(a, g, t0 + kTK, kend, wave, lane, page_next, kn, kn + Gm::TILE_BYTES);
      if constexpr (PAGED) {
        const int tn = t0 + 2 * kTK + lane;
        page_next = (it + 2 < n_tiles && tn < kend) ? a.bt[tn >> a.log2_ps] : 0;
      }
    }

    // S^T[key][qv] for keys 32 kb + (lane's C rows), qv = lane & 31.
    f32x16 sc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sc[kb] = f32x16{};
      const int krow = 32 * kb + (lane & 31);
      const uint8_t* kr = kt + krow * CH * 16;
      const int sw = swz_k<CH>(krow);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int pos = (2 * ks + h) ^ sw;
        i16x8 raw = *LDS_PTR(const i16x8, kr + pos * 16);
        sc[kb] = E::mfma(__builtin_bit_cast(vec8, raw), qf[ks], sc[kb]);
      }
    }

    if (t0 + kTK - 1 > mask_from) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = t0 + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
          sc[kb][r] = key > lim ? kNegInf : sc[kb][r];
        }
    }

    float mx = sc[0][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sc[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[1][r]);
    mx = max_with_partner(mx);
    const float m_new = fmaxf(m, mx);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f((m - m_use) * c);
    const float mc = m_use * c;
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sc[kb][r], c, -mc));
        sc[kb][r] = p;
        rs += p;
      }
    l = l * alpha + rs;
    m = m_new;
    if (__ballot(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
    }

    // O^T[d][qv] += V^T[d][key] P^T[key][qv], 16 keys per MFMA.
    const int grp = (lane >> 4) & 1;
    const int sub = (lane & 15) >> 2;
#pragma unroll
    for (int kstep = 0; kstep < 4; ++kstep) {
      const int kb = kstep >> 1;
      const int tt = kstep & 1;
      float pv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) pv[e] = sc[kb][8 * tt + e];
      const vec8 pb = E::from_f32(pv);
      const int row1 = 16 * kstep + 4 * h + sub;
      const int row2 = row1 + 8;
      const int sw1 = swz_v<CH>(row1), sw2 = swz_v<CH>(row2);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int col = 32 * db + 16 * grp + 4 * (lane & 3);
        const int cc = col >> 3;
        const int within = (col & 7) * 2;
        const uint8_t* p1 = vt + (row1 * CH + (cc ^ sw1)) * 16 + within;
        const uint8_t* p2 = vt + (row2 * CH + (cc ^ sw2)) * 16 + within;
        i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, p1));
        i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, p2));
        i16x8 av = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        o[db] = E::mfma(__builtin_bit_cast(vec8, av), pb, o[db]);
      }
    }
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
    if (h == 0) a.ws_lse[(int64_t)s * pairs + pair] = l_tot > 0.f ? m * c + __log2f(l_tot) : kNegInf;
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

template <int D, class E, bool PAGED>
hipError_t launch_attn_t(const AttnArgs& a, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((attn_partial_kernel<D, E, PAGED>), dim3(grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int D, class E>
hipError_t launch_attn_p(const AttnArgs& a, bool paged, int grid, hipStream_t stream) {
  return paged ? launch_attn_t<D, E, true>(a, grid, stream) : launch_attn_t<D, E, false>(a, grid, stream);
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

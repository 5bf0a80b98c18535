// The log-sum-exp merge kernel and the dispatch of both kernels by head
// dimension and element type.
#include "attn_kernel.h"
#include "plan.h"

namespace ppa {
namespace {

// Log-sum-exp merge of split partials.  A (row, head) pair is served by GR
// groups of D/4 threads, 4 output elements per thread; group g sums its own
// contiguous share of the pair's splits.  GR = 16 for 64 splits or more (a
// decode step: a few pairs, up to thousands of splits; one 8-split batch per
// group for up to 128 splits), 4 for 16 or more (a short append on a long
// history), GR = 1 below (many pairs, few splits: no cross-group exchange).
// A block has max(256, GR D / 4) threads.
// One pass: each thread keeps 8 splits' loads in flight and a running
// reference M (the largest lse it has read); a batch's weights are
// exp2(lse_s - M) after the sums so far are scaled to the batch's M.  Groups
// then scale their sums to the pair's largest lse and add in index order.
// Within a group the splits are summed in index order: the order is fixed,
// so results are reproducible.  Splits that start past the row's last key
// hold nothing for it and are not read.
template <int D, class E, int GR>
__global__ __launch_bounds__(D / 4 * GR > 256 ? D / 4 * GR : 256) void merge_kernel(MergeArgs a) {
  constexpr int TPP = D / 4;                      // threads per (pair, group)
  constexpr int TPAIR = TPP * GR;                 // threads per pair
  constexpr int BLOCK = TPAIR > 256 ? TPAIR : 256;
  constexpr int PPB = BLOCK / TPAIR;              // pairs per block
  __shared__ f32x4 acc_part[GR > 1 ? PPB : 1][GR][TPP];
  __shared__ float w_part[GR > 1 ? PPB : 1][GR], m_part[GR > 1 ? PPB : 1][GR];

  // The sequence (grid y with several sequences): its first row in the
  // workspace and output, its rows and history.
  int r0 = 0, rows = a.rows;
  int64_t history = a.history;
  if (a.n_seqs > 0) {
    r0 = a.cu_rows[blockIdx.y];
    rows = a.cu_rows[blockIdx.y + 1] - r0;
    history = a.seq_history[blockIdx.y];
  }
  const int pairs_seq = rows * a.n_q_heads;
  if ((int)blockIdx.x * PPB >= pairs_seq) return;   // the whole block
  const int64_t pairs = (int64_t)a.ws_rows * a.n_q_heads;  // workspace stride per split
  const int pl = threadIdx.x / TPAIR;             // pair within the block
  const int tp = threadIdx.x % TPAIR;             // thread within the pair
  const int grp = tp / TPP;
  const int t = tp % TPP;
  const int pair_raw = blockIdx.x * PPB + pl;
  const bool valid = pair_raw < pairs_seq;
  const int pair_l = valid ? pair_raw : pairs_seq - 1;  // keep every thread's reads in range
  const int row = pair_l / a.n_q_heads;
  const int64_t pair = (int64_t)r0 * a.n_q_heads + pair_l;
  int nv = (int)((history + row) / a.split_tokens) + 1;
  if (nv > a.n_splits) nv = a.n_splits;
  const float* lse = a.ws_lse + pair;

  // This group's splits [sb, se).
  const int per = (nv + GR - 1) / GR;
  const int sb = min(grp * per, nv);
  const int se = min(sb + per, nv);
  const float* op = a.ws_o + pair * D + 4 * t;
  const int64_t ostride = (int64_t)pairs * D;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f, m = kNegInf;
  for (int s0 = sb; s0 < se; s0 += 8) {
    float l8[8];
    f32x4 v8[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      l8[j] = kNegInf;
      v8[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (s0 + j < se) {
        l8[j] = lse[(int64_t)(s0 + j) * pairs];
        v8[j] = *(const f32x4*)(op + (int64_t)(s0 + j) * ostride);
      }
    }
    float mb = m;
#pragma unroll
    for (int j = 0; j < 8; ++j) mb = fmaxf(mb, l8[j]);
    if (mb == kNegInf) continue;                  // nothing with weight yet
    const float scale = exp2f(m - mb);            // 0 while nothing has been added
    acc *= scale;
    wsum *= scale;
    m = mb;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float w = exp2f(l8[j] - m);          // 0 for the padding entries
      acc += w * v8[j];
      wsum += w;
    }
  }
  if constexpr (GR > 1) {
    acc_part[pl][grp][t] = acc;
    if (t == 0) {
      w_part[pl][grp] = wsum;
      m_part[pl][grp] = m;
    }
    __syncthreads();
    if (grp != 0 || !valid) return;
    float mx = m_part[pl][0];
#pragma unroll
    for (int g = 1; g < GR; ++g) mx = fmaxf(mx, m_part[pl][g]);
    acc = f32x4{0.f, 0.f, 0.f, 0.f};
    wsum = 0.f;
#pragma unroll
    for (int g = 0; g < GR; ++g) {
      const float mg = m_part[pl][g];
      const float sg = mg == kNegInf ? 0.f : exp2f(mg - mx);  // an empty group adds nothing
      acc += sg * acc_part[pl][g][t];
      wsum += sg * w_part[pl][g];
    }
  } else {
    if (!valid) return;
  }
  const float inv = 1.f / wsum;
  const uint32_t lo = E::bits(acc[0] * inv) | ((uint32_t)E::bits(acc[1] * inv) << 16);
  const uint32_t hi = E::bits(acc[2] * inv) | ((uint32_t)E::bits(acc[3] * inv) << 16);
  *(u32x2*)(a.out + pair * D + 4 * t) = u32x2{lo, hi};
}

template <int D, class E>
void launch_merge_gr(const MergeArgs& a, dim3 g, hipStream_t stream) {
  switch (merge_groups_for(a.n_splits)) {
    case 16: hipLaunchKernelGGL((merge_kernel<D, E, 16>), g, dim3(merge_block_threads(D, a.n_splits)), 0, stream, a); break;
    case 4: hipLaunchKernelGGL((merge_kernel<D, E, 4>), g, dim3(256), 0, stream, a); break;
    default: hipLaunchKernelGGL((merge_kernel<D, E, 1>), g, dim3(256), 0, stream, a); break;
  }
}

template <class E>
hipError_t launch_merge_d(const MergeArgs& a, int head_dim, int grid, int grid_y, hipStream_t stream) {
  const dim3 g(grid, grid_y);
  switch (head_dim) {
    case 64: launch_merge_gr<64, E>(a, g, stream); break;
    case 128: launch_merge_gr<128, E>(a, g, stream); break;
    case 256: launch_merge_gr<256, E>(a, g, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, int head_dim, int dtype, bool paged, int grid,
                            hipStream_t stream) {
  if (head_dim == 256) return launch_attention_d256(a, dtype, paged, grid, stream);
  return launch_attention_d64_d128(a, head_dim, dtype, paged, grid, stream);
}

hipError_t launch_attention_q8(const AttnArgs& a, int head_dim, int dtype, int grid, hipStream_t stream) {
  if (head_dim == 256) return launch_attention_q8_d256(a, dtype, grid, stream);
  return launch_attention_q8_d64_d128(a, head_dim, dtype, grid, stream);
}

hipError_t launch_attention_kv16(const AttnArgs& a, int head_dim, int dtype, int grid, hipStream_t stream) {
  // fp16 q: the ordinary fp16 kernel over contiguous K/V
  if (dtype == 0) return launch_attention(a, head_dim, dtype, false, grid, stream);
  if (head_dim == 256) return launch_attention_kv16_d256(a, grid, stream);
  return launch_attention_kv16_d64_d128(a, head_dim, grid, stream);
}

hipError_t launch_merge(const MergeArgs& a, int head_dim, int dtype, int grid, int grid_y, hipStream_t stream) {
  return dtype == 1 ? launch_merge_d<BF16>(a, head_dim, grid, grid_y, stream)
                    : launch_merge_d<F16>(a, head_dim, grid, grid_y, stream);
}

}  // namespace ppa

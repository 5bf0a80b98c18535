// The log-sum-exp merge kernel and the dispatch of both kernels by head
// dimension and element type.
#include "attn_kernel.h"

namespace ppa {
namespace {

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
  if (head_dim == 256) return launch_attention_d256(a, dtype, paged, grid, stream);
  return launch_attention_d64_d128(a, head_dim, dtype, paged, grid, stream);
}

hipError_t launch_merge(const MergeArgs& a, int head_dim, int dtype, int grid, hipStream_t stream) {
  return dtype == 1 ? launch_merge_d<BF16>(a, head_dim, grid, stream)
                    : launch_merge_d<F16>(a, head_dim, grid, stream);
}

}  // namespace ppa

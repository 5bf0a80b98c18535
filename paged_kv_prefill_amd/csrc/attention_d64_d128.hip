// Split-partial attention kernels for head dimensions 64 and 128 with two
// query blocks per wave (calls of more than one 128-vector m tile); one query
// block per wave is in attention_d64_d128_qb1.hip (own register options).
#include "attn_kernel.h"

namespace ppa {

hipError_t launch_attention_d64_d128(const AttnArgs& a, int head_dim, int dtype, bool paged, int grid,
                                     hipStream_t stream) {
  if (a.query_blocks != 2) return launch_attention_d64_d128_qb1(a, head_dim, dtype, paged, grid, stream);
  const bool bf = dtype == 1;
  switch (head_dim) {
    case 64: return bf ? launch_attn_p<64, BF16, 2>(a, paged, grid, stream) : launch_attn_p<64, F16, 2>(a, paged, grid, stream);
    case 128: return bf ? launch_attn_p<128, BF16, 2>(a, paged, grid, stream) : launch_attn_p<128, F16, 2>(a, paged, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ppa

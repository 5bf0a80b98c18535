// Split-partial attention kernels over 8-bit K/V pages, head dimensions 64 and 128
// (two query blocks per wave at 64 for calls of more than one m tile; one at 128,
// where the widening step needs the registers).
#include "attn_kernel.h"

namespace ppa {

hipError_t launch_attention_q8_d64_d128(const AttnArgs& a, int head_dim, int dtype, int grid, hipStream_t stream) {
  const bool bf = dtype == 1;
  const bool two = a.query_blocks == 2;
  switch (head_dim) {
    case 64:
      if (two) return bf ? launch_attn_q8<64, BF16, 2>(a, grid, stream) : launch_attn_q8<64, F16, 2>(a, grid, stream);
      return bf ? launch_attn_q8<64, BF16>(a, grid, stream) : launch_attn_q8<64, F16>(a, grid, stream);
    case 128: return bf ? launch_attn_q8<128, BF16>(a, grid, stream) : launch_attn_q8<128, F16>(a, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ppa

// Split-partial attention kernels over 8-bit K/V pages, head dimension 256.
#include "attn_kernel.h"

namespace ppa {

hipError_t launch_attention_q8_d256(const AttnArgs& a, int dtype, int grid, hipStream_t stream) {
  return dtype == 1 ? launch_attn_q8<256, BF16>(a, grid, stream) : launch_attn_q8<256, F16>(a, grid, stream);
}

}  // namespace ppa

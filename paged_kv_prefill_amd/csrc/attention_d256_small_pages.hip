// Split-partial attention kernels for head dimension 256 over pages of fewer
// than 16 tokens.
#include "attn_kernel.h"

namespace ppa {

hipError_t launch_attention_d256_small_pages(const AttnArgs& a, int dtype, int grid, hipStream_t stream) {
  return dtype == 1 ? launch_attn_p_small<256, BF16>(a, grid, stream) : launch_attn_p_small<256, F16>(a, grid, stream);
}

}  // namespace ppa

// Split-partial attention kernels for head dimension 256.
#include "attn_kernel.h"

namespace ppa {

hipError_t launch_attention_d256(const AttnArgs& a, int dtype, bool paged, int grid, hipStream_t stream) {
  return dtype == 1 ? launch_attn_p<256, BF16>(a, paged, grid, stream) : launch_attn_p<256, F16>(a, paged, grid, stream);
}

}  // namespace ppa

// Split-partial attention kernels for head dimension 256, contiguous K/V and
// pages of 16 tokens or more (the smaller page classes are in
// attention_d256_small_pages.hip, built with other register options).
#include "attn_kernel.h"

namespace ppa {

hipError_t launch_attention_d256(const AttnArgs& a, int dtype, bool paged, int grid, hipStream_t stream) {
  if (paged && a.log2_ps < 4) return launch_attention_d256_small_pages(a, dtype, grid, stream);
  return dtype == 1 ? launch_attn_p_large<256, BF16>(a, paged, grid, stream)
                    : launch_attn_p_large<256, F16>(a, paged, grid, stream);
}

// bf16 q and out over contiguous fp16 K/V (dequantized 8-bit pages)
hipError_t launch_attention_kv16_d256(const AttnArgs& a, int grid, hipStream_t stream) {
  return launch_attn_t<256, BF16, Addr::Contig, false, 1, true>(a, grid, stream);
}

}  // namespace ppa

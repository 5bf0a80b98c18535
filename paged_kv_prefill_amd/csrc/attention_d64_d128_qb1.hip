// Split-partial attention kernels for head dimensions 64 and 128 with one
// query block per wave (calls whose query vectors fit one 128-vector m tile:
// short appends, decode steps).
#include "attn_kernel.h"

namespace ppa {

hipError_t launch_attention_d64_d128_qb1(const AttnArgs& a, int head_dim, int dtype, bool paged, int grid,
                                         hipStream_t stream) {
  const bool bf = dtype == 1;
  switch (head_dim) {
    case 64: return bf ? launch_attn_p<64, BF16>(a, paged, grid, stream) : launch_attn_p<64, F16>(a, paged, grid, stream);
    case 128: return bf ? launch_attn_p<128, BF16>(a, paged, grid, stream) : launch_attn_p<128, F16>(a, paged, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

// bf16 q and out over contiguous fp16 K/V (dequantized 8-bit pages), one
// query block per wave
hipError_t launch_attention_kv16_d64_d128_qb1(const AttnArgs& a, int head_dim, int grid, hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_attn_t<64, BF16, Addr::Contig, false, 1, true>(a, grid, stream);
    case 128: return launch_attn_t<128, BF16, Addr::Contig, false, 1, true>(a, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ppa

// Instantiations of the narrow (decode) attention kernel: head dimensions
// 64, 128 and 256, fp16 or bf16 q and out, paged or contiguous 16-bit K/V,
// and 8-bit pages.
#include "decode_kernel.h"

namespace ppa {
namespace {

template <class E, bool PAGED, bool Q8>
hipError_t launch_decode_d(const AttnArgs& a, int head_dim, int grid, hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_decode_t<64, E, PAGED, Q8>(a, grid, stream);
    case 128: return launch_decode_t<128, E, PAGED, Q8>(a, grid, stream);
    case 256: return launch_decode_t<256, E, PAGED, Q8>(a, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

template <class E>
hipError_t launch_decode_e(const AttnArgs& a, int head_dim, bool paged, bool q8, int grid, hipStream_t stream) {
  if (q8) return launch_decode_d<E, true, true>(a, head_dim, grid, stream);
  if (paged) return launch_decode_d<E, true, false>(a, head_dim, grid, stream);
  return launch_decode_d<E, false, false>(a, head_dim, grid, stream);
}

}  // namespace

hipError_t launch_attention_decode(const AttnArgs& a, int head_dim, int dtype, bool paged, bool q8, int grid,
                                   hipStream_t stream) {
  return dtype == 1 ? launch_decode_e<BF16>(a, head_dim, paged, q8, grid, stream)
                    : launch_decode_e<F16>(a, head_dim, paged, q8, grid, stream);
}

}  // namespace ppa

// Instantiations of the narrow (decode) attention kernel with 16 query
// vectors per wave (16 x 16 x 32 MFMAs): calls of at most 16 query vectors
// per KV head (rows x group), e.g. a decode step under grouped-query
// attention with up to 16 query heads per KV head.
#include "decode_kernel.h"

namespace ppa {

hipError_t launch_attention_decode16(const AttnArgs& a, int head_dim, int dtype, bool paged, bool q8, int grid,
                                     hipStream_t stream) {
  return launch_decode_nq<16>(a, head_dim, dtype, paged, q8, grid, stream);
}

}  // namespace ppa

// Instantiations of the narrow (decode) attention kernel with 32 query
// vectors per wave (32 x 32 MFMAs) over 8-bit pages: head dimensions 64, 128
// and 256, fp16 or bf16 q and out; and the choice between them and the
// 16-vector build (decode16.hip).
#include "decode_kernel.h"

namespace ppa {

hipError_t launch_attention_decode(const AttnArgs& a, int head_dim, int dtype, bool paged, bool q8, int grid,
                                   hipStream_t stream) {
  // A call's query vectors per KV head, rows x group, sit in one wave's MFMA
  // columns: at most 16 take the 16 x 16 x 32 MFMAs (half the matrix work).
  if (a.rows * a.group <= 16) return launch_attention_decode16(a, head_dim, dtype, paged, q8, grid, stream);
  return launch_decode_nq<32>(a, head_dim, dtype, paged, q8, grid, stream);
}

}  // namespace ppa

// KV append: the chunk's K and V rows written into their pages through the
// block table (issue "Metal: paged-KV prefill is 4.43x slower than contiguous
// KV at 32K": publishing completed KV pages, after its "Expected vs actual"
// table).  Chunk row i is the token at position H + i; it goes to slot
// (H + i) % page_size of pool page block_table[(H + i) / page_size].
//
// A pure copy of 16-bit patterns, bound by HBM: every 16-byte unit is read
// once and written once.  One thread moves one unit; consecutive threads move
// consecutive units of a token row (Hkv * d * 2 bytes, contiguous both in the
// chunk's rows and in the page slot), so reads and writes coalesce.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace ppa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void kv_append_kernel(AppendArgs a) {
  // units of 16 bytes: per token row `upr`, per tensor rows * upr; K first, then V
  const uint32_t per_tensor = uint32_t(a.rows) * uint32_t(a.upr);
  const uint32_t ps_mask = (1u << a.log2_ps) - 1u;
  for (uint32_t u = blockIdx.x * 256u + threadIdx.x; u < 2u * per_tensor; u += gridDim.x * 256u) {
    const bool is_v = u >= per_tensor;
    const uint32_t w = is_v ? u - per_tensor : u;
    const uint32_t i = w / uint32_t(a.upr);
    const uint32_t c = w - i * uint32_t(a.upr);
    const int64_t pos = a.history + i;
    const int64_t page = a.bt[pos >> a.log2_ps];
    const int64_t dst_unit = ((page << a.log2_ps) + (pos & ps_mask)) * a.upr + c;
    const u32x4* src = reinterpret_cast<const u32x4*>(is_v ? a.v_new : a.k_new) + w;
    u32x4* dst = reinterpret_cast<u32x4*>(is_v ? a.v_pages : a.k_pages) + dst_unit;
    *dst = *src;
  }
}

}  // namespace

hipError_t launch_kv_append(const AppendArgs& a, hipStream_t stream) {
  const int64_t units = 2 * int64_t(a.rows) * a.upr;
  int64_t grid = (units + 255) / 256;
  if (grid > 8192) grid = 8192;  // grid-stride beyond 32 workgroups per CU
  hipLaunchKernelGGL(kv_append_kernel, dim3(uint32_t(grid)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace ppa

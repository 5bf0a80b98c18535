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

// Quantizing append into 8-bit pages: one thread per 32-value block of a
// token row (the q8_0 block structure named by the KVarN report's format
// comparison).  The block's max |x| over 127, an fp32 division rounded once to
// fp16 (saturated at 65504), is its scale; each value becomes x / scale (fp32
// division) rounded to the nearest integer, ties to even, clamped to
// [-127, 127]; an all-zero block has scale 0 and quants 0.  Every step is a
// correctly rounded fp32 operation, so the result is reproducible bit for bit.
template <bool BF>
__global__ __launch_bounds__(256) void kv_append_q8_kernel(AppendQ8Args a) {
  const int nb = a.head_dim / 32;
  const int64_t per_tensor = int64_t(a.rows) * a.n_kv_heads * nb;   // blocks per tensor
  const int64_t ps_mask = (int64_t(1) << a.log2_ps) - 1;
  for (int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x; t < 2 * per_tensor; t += int64_t(gridDim.x) * 256) {
    const bool is_v = t >= per_tensor;
    const int64_t u = is_v ? t - per_tensor : t;
    const int blk = int(u % nb);
    const int64_t rh = u / nb;                 // row * Hkv + head
    const int64_t row = rh / a.n_kv_heads;
    const int head = int(rh % a.n_kv_heads);
    const u32x4* src = reinterpret_cast<const u32x4*>((is_v ? a.v_new : a.k_new) + rh * a.head_dim + blk * 32);
    float x[32];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const u32x4 w = src[k];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t bits = (w[e >> 1] >> (16 * (e & 1))) & 0xffffu;
        x[8 * k + e] = BF ? __uint_as_float(bits << 16) : (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
      }
    }
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) amax = fmaxf(amax, fabsf(x[e]));
    _Float16 s16 = (_Float16)(amax / 127.0f);
    if (!(s16 <= (_Float16)65504.0f)) s16 = (_Float16)65504.0f;
    const float sf = (float)s16;
    uint32_t qw[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      uint32_t word = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float q = sf > 0.f ? rintf(x[4 * k + e] / sf) : 0.f;
        q = fminf(fmaxf(q, -127.f), 127.f);
        word |= (uint32_t)((int)q & 0xff) << (8 * e);
      }
      qw[k] = word;
    }
    const int64_t pos = a.history + row;
    const int64_t page = a.bt[pos >> a.log2_ps];
    const int64_t slot_row = ((page << a.log2_ps) + (pos & ps_mask)) * a.n_kv_heads + head;   // token-head row
    u32x4* qdst = reinterpret_cast<u32x4*>((is_v ? a.v_quant : a.k_quant) + slot_row * a.head_dim + blk * 32);
    qdst[0] = u32x4{qw[0], qw[1], qw[2], qw[3]};
    qdst[1] = u32x4{qw[4], qw[5], qw[6], qw[7]};
    (is_v ? a.v_scale : a.k_scale)[slot_row * nb + blk] = __builtin_bit_cast(uint16_t, s16);
  }
}

// Dequantizing gather of 8-bit pages into contiguous fp16 K and V: token j
// of the sequence, KV head h, values 16 c .. 16 c + 15 come from slot j % ps
// of pool page bt[j / ps]; each value is quant * scale of its 32-value block,
// rounded once to fp16 (the product of a 7-bit integer and an fp16 scale is
// exact in fp32), the same value the attention kernel's in-LDS widening
// computes.  One thread per 16 values; consecutive threads take consecutive
// 16-byte quant units of a token's rows, so reads and writes coalesce.
__global__ __launch_bounds__(256) void kv_dequant_q8_kernel(DequantQ8Args a) {
  const int upr = a.head_dim / 16;                                  // units per token-head row
  const int64_t per_tensor = int64_t(a.ctx) * a.n_kv_heads * upr;
  const int64_t ps_mask = (int64_t(1) << a.log2_ps) - 1;
  for (int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x; t < 2 * per_tensor; t += int64_t(gridDim.x) * 256) {
    const bool is_v = t >= per_tensor;
    const int64_t u = is_v ? t - per_tensor : t;
    const int c = int(u % upr);
    const int64_t rh = u / upr;                       // token * Hkv + head
    const int64_t j = rh / a.n_kv_heads;
    const int head = int(rh % a.n_kv_heads);
    const int64_t page = a.bt[j >> a.log2_ps];
    const int64_t src_row = ((page << a.log2_ps) + (j & ps_mask)) * a.n_kv_heads + head;
    const u32x4 qw = *reinterpret_cast<const u32x4*>((is_v ? a.v_quant : a.k_quant) + src_row * a.head_dim + 16 * c);
    const uint16_t sb = (is_v ? a.v_scale : a.k_scale)[src_row * (a.head_dim / 32) + c / 2];
    const float sf = (float)__builtin_bit_cast(_Float16, sb);
    uint32_t ow[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t w = qw[k >> 1];
      const int sh = 16 * (k & 1);
      const float x0 = (float)(int8_t)((w >> sh) & 0xffu) * sf;
      const float x1 = (float)(int8_t)((w >> (sh + 8)) & 0xffu) * sf;
      ow[k] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x0) |
              ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x1) << 16);
    }
    u32x4* dst = reinterpret_cast<u32x4*>((is_v ? a.v_out : a.k_out) + rh * a.head_dim + 16 * c);
    dst[0] = u32x4{ow[0], ow[1], ow[2], ow[3]};
    dst[1] = u32x4{ow[4], ow[5], ow[6], ow[7]};
  }
}

}  // namespace

hipError_t launch_kv_dequant_q8(const DequantQ8Args& a, hipStream_t stream) {
  const int64_t units = 2 * int64_t(a.ctx) * a.n_kv_heads * (a.head_dim / 16);
  int64_t grid = (units + 255) / 256;
  if (grid > 8192) grid = 8192;
  hipLaunchKernelGGL(kv_dequant_q8_kernel, dim3(uint32_t(grid)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_kv_append_q8(const AppendQ8Args& a, int dtype, hipStream_t stream) {
  const int64_t blocks = 2 * int64_t(a.rows) * a.n_kv_heads * (a.head_dim / 32);
  int64_t grid = (blocks + 255) / 256;
  if (grid > 8192) grid = 8192;
  if (dtype == 1)
    hipLaunchKernelGGL(kv_append_q8_kernel<true>, dim3(uint32_t(grid)), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(kv_append_q8_kernel<false>, dim3(uint32_t(grid)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_kv_append(const AppendArgs& a, hipStream_t stream) {
  const int64_t units = 2 * int64_t(a.rows) * a.upr;
  int64_t grid = (units + 255) / 256;
  if (grid > 8192) grid = 8192;  // grid-stride beyond 32 workgroups per CU
  hipLaunchKernelGGL(kv_append_kernel, dim3(uint32_t(grid)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace ppa

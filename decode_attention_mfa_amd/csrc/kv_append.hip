// KV append with a device-owned length counter (duck-llm chapter 7, section
// 7.6: the decode context kernel writes the new token's K/V and owns the
// active length, which then counts the token).  One workgroup per slot: every
// thread reads the slot's length, writes its channels of the new K row and V
// column for each KV head, and after a barrier (every thread has read the old
// length) thread 0 advances the length.
//
// FP8 E4M3FN encoding of q = x / scale (fp32): magnitudes below 2^-6 are
// multiples of 2^-9 (subnormal codes m = 0..8, where m = 8 is the smallest
// normal); above, q = 2^E (1 + f) keeps three fraction bits.  Both are a
// round-to-nearest-even of q scaled by a power of two (exact in fp32), so
// rintf does the rounding; |q| is first saturated to 448, the largest finite
// code, and NaN maps to 0x7F with its sign.
#include "device_common.h"
#include "kernel_params.h"

namespace mfa {
namespace {

__device__ __forceinline__ uint8_t e4m3fn_encode(float q) {
  const uint32_t bits = __builtin_bit_cast(uint32_t, q);
  const uint32_t sign = (bits >> 24) & 0x80u;
  if (q != q) return (uint8_t)(sign | 0x7Fu);
  const float a = fminf(fabsf(q), 448.f);
  uint32_t mag;
  if (a < 0.015625f) {                       // below 2^-6: steps of 2^-9
    mag = (uint32_t)__builtin_rintf(a * 512.f);   // 0 .. 8 (8 = smallest normal)
  } else {
    const int e = (int)((__builtin_bit_cast(uint32_t, a) >> 23) & 0xFF) - 127;   // -6 .. 8
    const float m = __builtin_rintf(a * __builtin_ldexpf(8.f, -e));            // 8 .. 16
    uint32_t mi = (uint32_t)m;
    int eb = e + 7;
    if (mi == 16) {
      mi = 8;
      ++eb;
    }
    mag = ((uint32_t)eb << 3) | (mi - 8);
  }
  return (uint8_t)(sign | mag);
}

template <typename TNew>
__device__ __forceinline__ float widen(TNew v);
template <>
__device__ __forceinline__ float widen<uint16_t>(uint16_t v) {
  return __builtin_bit_cast(float, (uint32_t)v << 16);
}

// kKv: 0 = copy the new value's bits (bf16 -> bf16, f32 -> f32), 1 = E4M3FN.
template <typename TNew, typename TKv, int kKv>
__global__ void __launch_bounds__(256) kv_append_kernel(AppendParams p) {
  const int b = blockIdx.x;
  if (p.active && p.active[b] == 0) return;
  const int pos = p.ctx_lens[b];
  const int64_t cap = (int64_t)p.max_blocks * kPage;
  if (pos < 0 || pos >= cap) return;
  const int row = pos & (kPage - 1);
  int64_t blk = 0;
  if (p.block_table) {
    blk = p.block_table[(int64_t)b * p.max_blocks + (pos >> 6)];
    if (blk < 0 || blk >= p.num_blocks) return;
  }
  const int d = p.head_dim, hkv = p.hkv;
  const TNew* kn = static_cast<const TNew*>(p.k_new) + (int64_t)b * hkv * d;
  const TNew* vn = static_cast<const TNew*>(p.v_new) + (int64_t)b * hkv * d;
  TKv* kc = static_cast<TKv*>(p.k_cache);
  TKv* vc = static_cast<TKv*>(p.v_cache);
  for (int g = 0; g < hkv; ++g) {
    // Paged: K [blocks, Hkv, 64, d], V [blocks, Hkv, d, 64];
    // contiguous: K [B, cap, Hkv, d], V [B, Hkv, d, cap].
    const int64_t k_row = p.block_table ? ((blk * hkv + g) * kPage + row) * d
                                        : (((int64_t)b * cap + pos) * hkv + g) * d;
    const int64_t v_col = p.block_table ? (blk * hkv + g) * (int64_t)d * kPage + row
                                        : ((int64_t)b * hkv + g) * (int64_t)d * cap + pos;
    const int64_t v_stride = p.block_table ? kPage : cap;
    const float ks = kKv == 1 ? p.k_scale[g] : 1.f;
    const float vs = kKv == 1 ? p.v_scale[g] : 1.f;
    for (int ch = threadIdx.x; ch < d; ch += blockDim.x) {
      const TNew kv = kn[g * d + ch];
      const TNew vv = vn[g * d + ch];
      if constexpr (kKv == 1) {
        kc[k_row + ch] = e4m3fn_encode(widen<TNew>(kv) / ks);
        vc[v_col + ch * v_stride] = e4m3fn_encode(widen<TNew>(vv) / vs);
      } else {
        kc[k_row + ch] = kv;
        vc[v_col + ch * v_stride] = vv;
      }
    }
  }
  __syncthreads();   // every thread has used the old length
  if (threadIdx.x == 0) p.ctx_lens[b] = pos + 1;
}

}  // namespace

hipError_t launch_kv_append(const AppendParams& p, int new_dtype, int kv_dtype, hipStream_t stream) {
  const dim3 grid(p.batch), block(256);
  if (new_dtype == 1 && kv_dtype == 1)   // bf16 -> bf16
    hipLaunchKernelGGL((kv_append_kernel<uint16_t, uint16_t, 0>), grid, block, 0, stream, p);
  else if (new_dtype == 1 && kv_dtype == 2)   // bf16 -> E4M3FN
    hipLaunchKernelGGL((kv_append_kernel<uint16_t, uint8_t, 1>), grid, block, 0, stream, p);
  else if (new_dtype == 0 && kv_dtype == 0)   // f32 -> f32
    hipLaunchKernelGGL((kv_append_kernel<uint32_t, uint32_t, 0>), grid, block, 0, stream, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace mfa

// KV append with a device-owned length counter (duck-llm chapter 7, section
// 7.6: the decode context kernel writes the new token's K/V and owns the
// active length, which then counts the token).  One workgroup per slot: every
// thread reads the slot's length, writes its channel of the new K row and V
// column for each KV head, and after a barrier (every thread has read the old
// length) thread 0 advances the length.
//
// FP8 caches store the E4M3FN code of x / scale (fp32 quotient, nearest,
// ties to even, saturating at 448, NaN kept).
#include "device_common.h"
#include "fp8_encode.h"
#include "kernel_params.h"

namespace mfa {
namespace {

template <typename TNew>
__device__ __forceinline__ float widen(TNew v);
template <>
__device__ __forceinline__ float widen<uint16_t>(uint16_t v) {
  return __builtin_bit_cast(float, (uint32_t)v << 16);
}

// kKv: 0 = copy the new value's bits (bf16 -> bf16, f32 -> f32), 1 = E4M3FN.
// Thread t owns channel t (d <= 256): its new K/V values, the slot's length
// and its activity flag are all loaded before the first dependent step, so
// the call costs two memory round trips (length, then block id) before the
// writes.
template <typename TNew, typename TKv, int kKv>
__global__ void __launch_bounds__(256) kv_append_kernel(AppendParams p) {
  constexpr int kPre = 4;   // KV heads whose new values are loaded up front
  const int b = blockIdx.x;
  const int ch = threadIdx.x;
  const int d = p.head_dim, hkv = p.hkv;
  const TNew* kn = static_cast<const TNew*>(p.k_new) + (int64_t)b * hkv * d;
  const TNew* vn = static_cast<const TNew*>(p.v_new) + (int64_t)b * hkv * d;
  const bool mine = ch < d;
  TNew kpre[kPre], vpre[kPre];
#pragma unroll
  for (int g = 0; g < kPre; ++g) {
    const int i = min(g, hkv - 1) * d + min(ch, d - 1);
    kpre[g] = kn[i];
    vpre[g] = vn[i];
  }
  const int pos = p.ctx_lens[b];
  const int act = p.active ? p.active[b] : 1;
  const int64_t cap = (int64_t)p.max_blocks * kPage;
  if (act == 0 || pos < 0 || pos >= cap) return;
  const int row = pos & (kPage - 1);
  int64_t blk = 0;
  if (p.block_table) {
    blk = p.block_table[(int64_t)b * p.max_blocks + (pos >> 6)];
    if (blk < 0 || blk >= p.num_blocks) return;
  }
  TKv* kc = static_cast<TKv*>(p.k_cache);
  TKv* vc = static_cast<TKv*>(p.v_cache);
  for (int g = 0; g < hkv; ++g) {
    // Paged: K [blocks, Hkv, 64, d], V [blocks, Hkv, d, 64] or, cut into
    // 8-token sub-blocks, [blocks, Hkv, 8, d, 8];
    // contiguous: K [B, cap, Hkv, d], V [B, Hkv, d, cap] or [B, Hkv, cap/8, d, 8].
    const int64_t k_row = p.block_table ? ((blk * hkv + g) * kPage + row) * d
                                        : (((int64_t)b * cap + pos) * hkv + g) * d;
    const int tok = p.block_table ? row : pos;   // key index inside the V run
    const int64_t v_base = p.block_table ? (blk * hkv + g) * (int64_t)d * kPage
                                         : ((int64_t)b * hkv + g) * (int64_t)d * cap;
    const int64_t v_col = p.v_sub8 ? v_base + (int64_t)(tok >> 3) * d * 8 + (tok & 7)
                                   : v_base + tok;
    const int64_t v_stride = p.v_sub8 ? 8 : (p.block_table ? kPage : cap);
    TNew kv, vv;
    if (g < kPre) {
      kv = kpre[g];
      vv = vpre[g];
    } else {
      kv = kn[g * d + min(ch, d - 1)];
      vv = vn[g * d + min(ch, d - 1)];
    }
    if (mine) {
      if constexpr (kKv == 1) {
        kc[k_row + ch] = e4m3fn_encode(widen<TNew>(kv) / p.k_scale[g]);
        vc[v_col + ch * v_stride] = e4m3fn_encode(widen<TNew>(vv) / p.v_scale[g]);
      } else {
        kc[k_row + ch] = kv;
        vc[v_col + ch * v_stride] = vv;
      }
    }
  }
  __syncthreads();   // every thread has used the old length
  if (ch == 0) p.ctx_lens[b] = pos + 1;
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

// fp32 decode attention: exact fp32 products and sums on the vector ALUs.
//
// For fp32 caches (small, accuracy-first calls).  One workgroup of 256
// threads per (slot, query head).  Keys are processed in chunks of 256: each
// thread scores one key (dot product over d), the block takes the chunk max
// and sum, and thread t then accumulates channel t of sum_j p_j V_j with an
// online-softmax rescale between chunks.  Any group size, any window,
// d <= 256, paged or contiguous cache in the library's layouts.
#include "device_common.h"
#include "kernel_params.h"

namespace mfa {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float block_reduce_max(float x, float* red) {
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  const float r = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return r;
}

__device__ __forceinline__ float block_reduce_sum(float x, float* red) {
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  const float r = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return r;
}

__global__ void __launch_bounds__(kThreads) f32_decode_kernel(DecodeParams p, int d) {
  __shared__ float probs[kThreads];
  __shared__ float qs[256];
  __shared__ float red[4];
  const int t = threadIdx.x;
  const int b = blockIdx.y;
  const int h = blockIdx.x;
  const int group = p.hq / p.hkv;
  const int g = h / group;
  const int L = slot_len(p.ctx_lens[b], p.max_blocks);
  const int lo = (p.window > 0 && L > p.window) ? L - p.window : 0;
  const float* q = static_cast<const float*>(p.q) + ((int64_t)b * p.hq + h) * d;
  const float* kpool = static_cast<const float*>(p.k);
  const float* vpool = static_cast<const float*>(p.v);
  if (t < d) qs[t] = q[t];
  __syncthreads();

  float m = kNegInf, l = 0.f, o = 0.f;
  for (int j0 = lo; j0 < L; j0 += kThreads) {
    const int j = j0 + t;
    float s = kNegInf;
    if (j < L) {
      const float* krow;
      if (p.block_table) {
        const int64_t blk = pool_block(p.block_table[(int64_t)b * p.max_blocks + j / kPage], p.num_blocks);
        krow = kpool + blk * p.k_block_stride + (int64_t)g * p.k_head_stride + (int64_t)(j % kPage) * p.k_row_stride;
      } else {
        krow = kpool + ((int64_t)b * p.max_blocks + j / kPage) * p.k_block_stride +
               (int64_t)g * p.k_head_stride + (int64_t)(j % kPage) * p.k_row_stride;
      }
      float acc = 0.f;
      for (int c = 0; c < d; ++c) acc = fmaf(qs[c], krow[c], acc);
      s = acc * p.scale;
    }
    const float cmax = block_reduce_max(s, red);
    const float m_new = fmaxf(m, cmax);
    const float alpha = expf(m - m_new);
    const float pj = (j < L) ? expf(s - m_new) : 0.f;
    probs[t] = pj;
    const float csum = block_reduce_sum(pj, red);   // also publishes probs[]
    l = l * alpha + csum;
    o *= alpha;
    m = m_new;
    if (t < d) {
      const int n = min(kThreads, L - j0);
      for (int jj = 0; jj < n; ++jj) {
        const int jk = j0 + jj;
        float v;
        if (p.block_table) {
          const int64_t blk = pool_block(p.block_table[(int64_t)b * p.max_blocks + jk / kPage], p.num_blocks);
          v = vpool[blk * p.v_block_stride + (int64_t)g * p.v_head_stride + (int64_t)t * p.v_row_stride + jk % kPage];
        } else {
          v = vpool[(int64_t)b * p.v_seq_stride + (int64_t)g * p.v_head_stride + (int64_t)t * p.v_row_stride + jk];
        }
        o = fmaf(probs[jj], v, o);
      }
    }
    __syncthreads();
  }
  if (t < d) {
    const float res = L > 0 ? o / l : 0.f;
    const int64_t off = ((int64_t)b * p.hq + h) * d + t;
    if (p.out_f32) static_cast<float*>(p.out)[off] = res;
    else static_cast<uint16_t*>(p.out)[off] = (uint16_t)(pack_bf16x2(res, 0.f) & 0xffffu);
  }
}

}  // namespace

hipError_t launch_f32(const DecodeParams& p, int d, hipStream_t stream) {
  hipLaunchKernelGGL(f32_decode_kernel, dim3(p.hq, p.batch), dim3(kThreads), 0, stream, p, d);
  return hipGetLastError();
}

}  // namespace mfa

// Low-rank MFA query path on gfx950: q = RMSNorm(x W_qdown^T) W_qup^T.
//
// "Step-3 is Large yet Affordable", section 2 (the attention design): the
// query is produced from the hidden state through a low-rank bottleneck that
// is normalised before the up projection.  Both projections are dense
// contractions, so they run on MFMA (16x16x32 bf16, fp32 accumulation):
//
//   1. gemm_nt (split-K over hidden): y_part[s] = x[:, Ks] W_qdown[:, Ks]^T   fp32
//   2. rms_norm: y = sum_s y_part[s]; r = y / sqrt(mean(y^2) + eps) * gain,
//      stored as bf16 hi + bf16 lo (r = hi + lo to ~16 mantissa bits)
//   3. gemm_nt: q = (r_hi + r_lo) W_qup^T                                     bf16|f32
//
// The weights are row-major [out, in], so both operands of each product are
// contiguous along the contracted axis and MFMA fragments load straight from
// global memory (16 bytes per lane).  Fixed summation order: results are
// bit-identical from call to call.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "host_plan.h"

namespace mfa {
namespace {

constexpr int kTileM = 64;   // rows per workgroup (4 waves x 16)
constexpr int kTileN = 64;   // columns per workgroup (4 MFMA tiles of 16)
constexpr int kThreads = 256;

enum GemmOut : int { kPartialF32 = 0, kOutBf16 = 1, kOutF32 = 2 };

// Workgroup b of a 1-D grid of `tiles` blocks; consecutive tile numbers are
// kept on one XCD (dispatch is round-robin over 8 XCDs) so that the M tiles
// of one N column of W share that XCD's L2.
__device__ __forceinline__ int xcd_tile(int b, int tiles) {
  if (tiles % 8) return b;
  return (b % 8) * (tiles / 8) + b / 8;
}

// C[m, n] (+)= sum_k A[m, k] * W[n, k] for one 64x64 tile and one K chunk.
// A (and A_lo when kLo) are [M, lda] bf16, W is [N, ldw] bf16.
template <int kMode, bool kLo>
__global__ __launch_bounds__(kThreads) void gemm_nt_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ A_lo, int lda,
    const uint16_t* __restrict__ W, int ldw, int M, int n_tiles, int m_tiles, int k_len,
    void* __restrict__ C, int ldc, size_t c_split_stride) {
  const int t = xcd_tile((int)blockIdx.x, n_tiles * m_tiles);
  const int m_tile = t % m_tiles;
  const int n_tile = t / m_tiles;
  const int split = (int)blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int row = lane & 15;
  const int kq = (lane >> 4) * 8;   // this lane's 8 K-indices within a 32-slice

  const int m = m_tile * kTileM + wave * 16 + row;
  const bool m_ok = m < M;
  const int k0 = split * k_len;
  const uint16_t* a_ptr = A + (size_t)(m_ok ? m : 0) * lda + k0 + kq;
  const uint16_t* alo_ptr = kLo ? A_lo + (size_t)(m_ok ? m : 0) * lda + k0 + kq : nullptr;
  const uint16_t* w_ptr = W + (size_t)(n_tile * kTileN + row) * ldw + k0 + kq;

  floatx4 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = floatx4{0.f, 0.f, 0.f, 0.f};

  const intx4 zero = {0, 0, 0, 0};
  for (int k = 0; k < k_len; k += 64) {
    intx4 a[2], alo[2], w[2][4];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      a[h] = m_ok ? *reinterpret_cast<const intx4*>(a_ptr + k + 32 * h) : zero;
      if (kLo) alo[h] = m_ok ? *reinterpret_cast<const intx4*>(alo_ptr + k + 32 * h) : zero;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        w[h][j] = *reinterpret_cast<const intx4*>(w_ptr + (size_t)16 * j * ldw + k + 32 * h);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[j] = mfma_bf16_16x16x32(a[h], w[h][j], acc[j]);
        if (kLo) acc[j] = mfma_bf16_16x16x32(alo[h], w[h][j], acc[j]);
      }
    }
  }

  // Lane holds C[4*(lane/16) + i][lane % 16] of each 16x16 tile j.
  const int col0 = n_tile * kTileN + row;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int mr = m_tile * kTileM + wave * 16 + 4 * (lane >> 4) + i;
    if (mr >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const size_t off = (size_t)mr * ldc + col0 + 16 * j;
      if (kMode == kPartialF32) {
        reinterpret_cast<float*>(C)[split * c_split_stride + off] = acc[j][i];
      } else if (kMode == kOutF32) {
        reinterpret_cast<float*>(C)[off] = acc[j][i];
      } else {
        __bf16 v = (__bf16)acc[j][i];
        reinterpret_cast<uint16_t*>(C)[off] = __builtin_bit_cast(uint16_t, v);
      }
    }
  }
}

// One workgroup per row: sum the split-K partials, RMS-normalise, apply the
// gain and write r as bf16 hi/lo.
__global__ __launch_bounds__(kThreads) void rms_norm_kernel(const float* __restrict__ y_part,
                                                            int k_splits, int batch, int rank,
                                                            float eps,
                                                            const float* __restrict__ gain,
                                                            uint16_t* __restrict__ r_hi,
                                                            uint16_t* __restrict__ r_lo) {
  constexpr int kMaxPer = 4096 / kThreads;
  const int b = blockIdx.x;
  float y[kMaxPer];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) {
    const int c = i * kThreads + threadIdx.x;
    float v = 0.f;
    if (c < rank) {
      for (int s = 0; s < k_splits; ++s) v += y_part[((size_t)s * batch + b) * rank + c];
    }
    y[i] = v;
    ss += v * v;
  }
  __shared__ float red[kThreads / 64];
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) tot += red[w];
  const float inv = 1.0f / sqrtf(tot / (float)rank + eps);
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) {
    const int c = i * kThreads + threadIdx.x;
    if (c >= rank) continue;
    const float r = y[i] * inv * (gain ? gain[c] : 1.0f);
    const __bf16 hi = (__bf16)r;
    const __bf16 lo = (__bf16)(r - (float)hi);
    r_hi[(size_t)b * rank + c] = __builtin_bit_cast(uint16_t, hi);
    r_lo[(size_t)b * rank + c] = __builtin_bit_cast(uint16_t, lo);
  }
}

}  // namespace

mfa_status query_proj_enqueue(const mfa_query_proj_desc* d, const QueryProjPlan& pl,
                              const void* x, const void* w_down, const void* w_up,
                              const float* gain, void* q_out, void* workspace,
                              hipStream_t stream) {
  const int B = d->batch, H = d->hidden, R = d->rank, N = d->num_heads * d->head_dim;
  char* ws = static_cast<char*>(workspace);
  float* y_part = reinterpret_cast<float*>(ws + pl.y_partial_offset);
  uint16_t* r_hi = reinterpret_cast<uint16_t*>(ws + pl.r_offset);
  uint16_t* r_lo = r_hi + (size_t)B * R;
  const int m_tiles = (B + kTileM - 1) / kTileM;

  {
    const int n_tiles = R / kTileN;
    dim3 grid(n_tiles * m_tiles, pl.k_splits);
    hipLaunchKernelGGL((gemm_nt_kernel<kPartialF32, false>), grid, dim3(kThreads), 0, stream,
                       static_cast<const uint16_t*>(x), nullptr, H,
                       static_cast<const uint16_t*>(w_down), H, B, n_tiles, m_tiles,
                       H / pl.k_splits, y_part, R, (size_t)B * R);
  }
  hipLaunchKernelGGL(rms_norm_kernel, dim3(B), dim3(kThreads), 0, stream, y_part, pl.k_splits, B,
                     R, d->eps, gain, r_hi, r_lo);
  {
    const int n_tiles = N / kTileN;
    dim3 grid(n_tiles * m_tiles, 1);
    if (d->out_dtype == MFA_F32)
      hipLaunchKernelGGL((gemm_nt_kernel<kOutF32, true>), grid, dim3(kThreads), 0, stream, r_hi,
                         r_lo, R, static_cast<const uint16_t*>(w_up), R, B, n_tiles, m_tiles, R,
                         q_out, N, (size_t)0);
    else
      hipLaunchKernelGGL((gemm_nt_kernel<kOutBf16, true>), grid, dim3(kThreads), 0, stream, r_hi,
                         r_lo, R, static_cast<const uint16_t*>(w_up), R, B, n_tiles, m_tiles, R,
                         q_out, N, (size_t)0);
  }
  return hipGetLastError() == hipSuccess ? MFA_OK : MFA_ERR_LAUNCH;
}

}  // namespace mfa

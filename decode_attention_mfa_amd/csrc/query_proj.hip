// Low-rank MFA query path on gfx950: q = RMSNorm(x W_qdown^T) W_qup^T.
//
// "Step-3 is Large yet Affordable", section 2 (the attention design): the
// query is produced from the hidden state through a low-rank bottleneck that
// is normalised before the up projection.  Both projections are dense
// contractions and run on MFMA (16x16x32 bf16, fp32 accumulation):
//
//   1. gemm (split-K over hidden): y_part[s] = x[:, Ks] W_qdown[:, Ks]^T    fp32
//   2. rms_norm: y = sum_s y_part[s]; r = y / sqrt(mean(y^2) + eps) * gain,
//      rounded once to bf16 (the normalised rank vector is the one
//      intermediate of the path that is rounded)
//   3. gemm: q = r W_qup^T                                                    bf16|f32
//
// GEMM: C[M, N] = A[M, K] B[N, K]^T, both operands K-contiguous (the weights
// are row-major [out, in]).  One workgroup of eight waves computes a 128 x 128
// tile of C.  The contraction runs in steps of kStepK; each step's A and B
// slices go global -> LDS by direct 16-byte DMA (global_load_lds_dwordx4)
// into a ring of kStages stages, kStages - 1 steps ahead of the step being
// computed, so that enough bytes are in flight per CU to cover memory latency
// with one workgroup per CU.  One workgroup barrier per step: after it, the
// stage read in the previous step is refilled.  Each 64 x 64 quarter of the
// tile belongs to two waves (one per SIMD pair slot), each taking half of
// every step's k range, so that one can issue MFMAs while the other waits on
// LDS or the barrier; their sums are added through LDS at the end (first k
// half + second k half, a fixed order).  Fragments for the 16x16x32 MFMAs come
// from LDS.  A slice row is kStepK bf16; its 16-byte chunks are XOR-swizzled
// so that the lanes reading one fragment column spread over every bank of a
// 128-byte LDS line.  A DMA instruction writes its 64 lanes' 16 bytes to
// consecutive LDS chunks, so the swizzle is applied on the global side: the
// lane that lands at LDS chunk p fetches the global chunk meant to sit there.
// The products are formed as C^T = B A^T so that each lane ends up with four
// consecutive columns of one row, stored as one vector.  Rows past M or N
// read a clamped row and are not stored.
//
// Fixed summation order throughout (split partials summed in split order by
// the norm kernel): results are bit-identical from call to call.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "host_plan.h"

namespace mfa {
namespace {

constexpr int kTile = 128;                 // rows and columns of C per workgroup
constexpr int kStepK = 64;                 // contraction per step
constexpr int kStages = 4;                 // ring depth
// Waves per output quarter: each takes its own part of every step's k range,
// so that two waves share each SIMD and one issues MFMAs while the other
// waits on LDS or the barrier.
constexpr int kKGroups = 2;
constexpr int kThreads = 256 * kKGroups;
constexpr int kNormThreads = 512;
constexpr int kRowBytes = kStepK * 2;
constexpr int kChunksPerRow = kRowBytes / 16;
constexpr int kRowsPerLine = 128 / kRowBytes;                // rows sharing a 128-byte line
constexpr int kSliceBytes = kTile * kRowBytes;               // one operand, one step
constexpr int kStageBytes = 2 * kSliceBytes;                 // A and B slices
constexpr int kDmaPerThread = kStageBytes / 16 / kThreads;
static_assert(kChunksPerRow == 4 || kChunksPerRow == 8, "slice rows of 64 or 128 bytes");
static_assert((kStages - 2) * kDmaPerThread < 64, "vmcnt range");
static_assert((kStepK / 32) % kKGroups == 0, "k groups split a step evenly");

// Stored chunk of logical chunk c of slice row r (an involution).
__device__ __forceinline__ int swz(int r, int c) {
  return c ^ ((r / kRowsPerLine) & (kChunksPerRow - 1));
}

// Wait until at most n steps of this thread's copies are still in flight.
template <int N>
__device__ __forceinline__ void wait_steps(int n) {
  if constexpr (N == 0) {
    wait_vmcnt<0>();
  } else {
    if (n >= N) wait_vmcnt<N * kDmaPerThread>();
    else wait_steps<N - 1>(n);
  }
}

enum GemmOut : int { kPartialF32 = 0, kOutBf16 = 1, kOutF32 = 2 };

// Work item of workgroup b in a 1-D grid of n: dispatch deals workgroups to
// the 8 XCDs in turn, so b is renumbered XCD-major and consecutive work items
// share one XCD and its L2.  Work item i is (split i / tiles, tile i % tiles),
// tile t = (m tile t % m_tiles, n tile t / m_tiles): with 8 splits each XCD
// takes one k range (every operand byte is fetched from HBM once), with one
// split the M tiles of one column of B share an XCD.
__device__ __forceinline__ int xcd_item(int b, int n) {
  if (n % 8) return b;
  return (b % 8) * (n / 8) + b / 8;
}

template <int kMode>
__global__ __launch_bounds__(kThreads) void gemm_kernel(
    const uint16_t* __restrict__ A, int lda, const uint16_t* __restrict__ Bm, int ldb, int M, int N,
    int m_tiles, int n_tiles, int k_len, void* __restrict__ C, int ldc, size_t c_split_stride) {
  __shared__ __attribute__((aligned(1024))) uint8_t ring[kStages * kStageBytes];
  const int tiles = m_tiles * n_tiles;
  const int item = xcd_item((int)blockIdx.x, (int)gridDim.x);
  const int split = item / tiles;
  const int t = item - split * tiles;
  const int m_tile = t % m_tiles;
  const int n_tile = t / m_tiles;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int k_begin = split * k_len;
  const int steps = k_len / kStepK;

  // DMA sources: LDS chunk p of a stage (the A slice first, then the B slice)
  // is slice row q / kChunksPerRow, stored chunk q % kChunksPerRow, q = p mod
  // the chunks of one slice.
  constexpr int kSliceChunks = kSliceBytes / 16;
  const uint16_t* src[kDmaPerThread];
#pragma unroll
  for (int i = 0; i < kDmaPerThread; ++i) {
    const int p = wave * (kDmaPerThread * 64) + i * 64 + lane;
    const int q = p % kSliceChunks;
    const int row = q / kChunksPerRow;
    const int chunk = swz(row, q % kChunksPerRow);
    if (p < kSliceChunks) {
      const int m = min(m_tile * kTile + row, M - 1);
      src[i] = A + (size_t)m * lda + k_begin + chunk * 8;
    } else {
      const int n = min(n_tile * kTile + row, N - 1);
      src[i] = Bm + (size_t)n * ldb + k_begin + chunk * 8;
    }
  }
  auto issue = [&](int s) __attribute__((always_inline)) {
    uint8_t* stage = ring + (s % kStages) * kStageBytes + wave * (kDmaPerThread * 1024);
#pragma unroll
    for (int i = 0; i < kDmaPerThread; ++i) dma16(src[i] + s * kStepK, stage + i * 1024);
  };

  // This wave's quarter: rows 64 (quarter / 2) .., columns 64 (quarter % 2) ..;
  // its k group takes 32-wide slices kg * kSlices .. of every step.
  const int quarter = wave & 3;
  const int kg = wave >> 2;
  constexpr int kSlices = kStepK / 32 / kKGroups;
  const int r16 = lane & 15;
  const int kq = lane >> 4;                 // chunk within a 32-wide k slice
  const int row_a0 = 64 * (quarter >> 1);
  const int row_b0 = 64 * (quarter & 1);
  floatx4 acc[4][4];                        // [n block j][m block i], transposed
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[j][i] = floatx4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int s = 0; s < kStages - 1; ++s)
    if (s < steps) issue(s);
  for (int s = 0; s < steps; ++s) {
    wait_steps<kStages - 2>(steps - 1 - s);   // step s landed for this thread
    __syncthreads();                          // ... and for every thread
    if (s + kStages - 1 < steps) issue(s + kStages - 1);   // refills the stage of step s - 1
    const uint8_t* stage = ring + (s % kStages) * kStageBytes;
#pragma unroll
    for (int hh = 0; hh < kSlices; ++hh) {
      const int chunk = (32 / 8) * (kg * kSlices + hh) + kq;
      intx4 a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ra = row_a0 + 16 * i + r16;
        const int rb = row_b0 + 16 * i + r16;
        a[i] = *reinterpret_cast<const intx4*>(stage + ra * kRowBytes + (swz(ra, chunk) << 4));
        b[i] = *reinterpret_cast<const intx4*>(stage + kSliceBytes + rb * kRowBytes +
                                               (swz(rb, chunk) << 4));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[j][i] = mfma_bf16_16x16x32(b[j], a[i], acc[j][i]);
    }
  }

  if constexpr (kKGroups == 2) {
    // Add the second k group's sums into the first's through the (now idle)
    // ring: 16 KB per wave, lane-contiguous, in k-group order.
    floatx4* xfer = reinterpret_cast<floatx4*>(ring) + quarter * (16 * 64) + lane;
    __syncthreads();
    if (kg == 1) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) xfer[(j * 4 + i) * 64] = acc[j][i];
    }
    __syncthreads();
    if (kg == 1) return;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[j][i] += xfer[(j * 4 + i) * 64];
  }

  // Lane holds C^T[4 (lane / 16) + e][lane % 16] of each 16 x 16 block: row
  // m = lane % 16, columns n .. n + 3.
  const bool vec = (ldc % 4) == 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m_tile * kTile + row_a0 + 16 * i + r16;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n_tile * kTile + row_b0 + 16 * j + 4 * kq;
      if (n >= N) continue;
      const size_t off = (size_t)m * ldc + n;
      const floatx4 v = acc[j][i];
      if (vec && n + 3 < N) {
        if (kMode == kPartialF32) {
          *reinterpret_cast<floatx4*>(reinterpret_cast<float*>(C) + split * c_split_stride + off) = v;
        } else if (kMode == kOutF32) {
          *reinterpret_cast<floatx4*>(reinterpret_cast<float*>(C) + off) = v;
        } else {
          typedef __attribute__((ext_vector_type(4))) unsigned short ushortx4;
          ushortx4 h;
#pragma unroll
          for (int e = 0; e < 4; ++e) h[e] = __builtin_bit_cast(uint16_t, (__bf16)v[e]);
          *reinterpret_cast<ushortx4*>(reinterpret_cast<uint16_t*>(C) + off) = h;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (n + e >= N) break;
          if (kMode == kPartialF32)
            reinterpret_cast<float*>(C)[split * c_split_stride + off + e] = v[e];
          else if (kMode == kOutF32)
            reinterpret_cast<float*>(C)[off + e] = v[e];
          else
            reinterpret_cast<uint16_t*>(C)[off + e] = __builtin_bit_cast(uint16_t, (__bf16)v[e]);
        }
      }
    }
  }
}

// One workgroup per row: sum the split-K partials in split order, RMS-normalise,
// apply the gain and write r in bf16.  Each thread owns kGroups groups of four
// consecutive columns (kGroups = 1 up to rank 2048, else 2).  Every load is
// issued before any is used: indices are clamped into range and the extra
// splits and columns masked, since a load inside a branch makes the compiler
// wait for each one in turn (one memory round trip per split).
template <int kGroups>
__global__ __launch_bounds__(kNormThreads) void rms_norm_kernel(const float* __restrict__ y_part,
                                                            int k_splits, int batch, int rank,
                                                            float eps,
                                                            const float* __restrict__ gain,
                                                            uint16_t* __restrict__ r_out) {
  const int b = blockIdx.x;
  floatx4 part[kGroups][kMaxQueryKSplits], gn[kGroups];
#pragma unroll
  for (int g = 0; g < kGroups; ++g) {
    const int cc = min(4 * (g * kNormThreads + (int)threadIdx.x), rank - 4);
#pragma unroll
    for (int s = 0; s < kMaxQueryKSplits; ++s)
      part[g][s] = *reinterpret_cast<const floatx4*>(y_part + ((size_t)min(s, k_splits - 1) * batch + b) * rank + cc);
    gn[g] = gain ? *reinterpret_cast<const floatx4*>(gain + cc) : floatx4{1.f, 1.f, 1.f, 1.f};
  }
  floatx4 y[kGroups];
  float ss = 0.f;
#pragma unroll
  for (int g = 0; g < kGroups; ++g) {
    floatx4 v = part[g][0];
#pragma unroll
    for (int s = 1; s < kMaxQueryKSplits; ++s) v += s < k_splits ? part[g][s] : floatx4{0.f, 0.f, 0.f, 0.f};
    y[g] = 4 * (g * kNormThreads + (int)threadIdx.x) < rank ? v : floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 4; ++e) ss += y[g][e] * y[g][e];
  }
  __shared__ float red[kNormThreads / 64];
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < kNormThreads / 64; ++w) tot += red[w];
  const float inv = 1.0f / sqrtf(tot / (float)rank + eps);
#pragma unroll
  for (int g = 0; g < kGroups; ++g) {
    const int c = 4 * (g * kNormThreads + threadIdx.x);
    if (c >= rank) continue;
    typedef __attribute__((ext_vector_type(4))) unsigned short ushortx4;
    ushortx4 h;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float r = y[g][e] * inv * gn[g][e];
      h[e] = __builtin_bit_cast(uint16_t, (__bf16)r);
    }
    *reinterpret_cast<ushortx4*>(r_out + (size_t)b * rank + c) = h;
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
  uint16_t* r = reinterpret_cast<uint16_t*>(ws + pl.r_offset);
  const int m_tiles = (B + kTile - 1) / kTile;
  {
    const int n_tiles = (R + kTile - 1) / kTile;
    dim3 grid(m_tiles * n_tiles * pl.k_splits);
    hipLaunchKernelGGL((gemm_kernel<kPartialF32>), grid, dim3(kThreads), 0, stream,
                       static_cast<const uint16_t*>(x), H, static_cast<const uint16_t*>(w_down), H,
                       B, R, m_tiles, n_tiles, H / pl.k_splits, y_part, R, (size_t)B * R);
  }
  if (R > 4 * kNormThreads)
    hipLaunchKernelGGL(rms_norm_kernel<2>, dim3(B), dim3(kNormThreads), 0, stream, y_part, pl.k_splits, B,
                       R, d->eps, gain, r);
  else
    hipLaunchKernelGGL(rms_norm_kernel<1>, dim3(B), dim3(kNormThreads), 0, stream, y_part, pl.k_splits, B,
                       R, d->eps, gain, r);
  {
    const int n_tiles = (N + kTile - 1) / kTile;
    dim3 grid(m_tiles * n_tiles);
    if (d->out_dtype == MFA_F32)
      hipLaunchKernelGGL((gemm_kernel<kOutF32>), grid, dim3(kThreads), 0, stream, r, R,
                         static_cast<const uint16_t*>(w_up), R, B, N, m_tiles, n_tiles, R, q_out, N,
                         (size_t)0);
    else
      hipLaunchKernelGGL((gemm_kernel<kOutBf16>), grid, dim3(kThreads), 0, stream, r, R,
                         static_cast<const uint16_t*>(w_up), R, B, N, m_tiles, n_tiles, R, q_out, N,
                         (size_t)0);
  }
  return hipGetLastError() == hipSuccess ? MFA_OK : MFA_ERR_LAUNCH;
}

}  // namespace mfa

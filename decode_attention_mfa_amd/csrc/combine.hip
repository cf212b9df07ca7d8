// Split-K merge (log-sum-exp combine) of decode-attention partials.
//
// Split c of slot b covers a contiguous chunk of the attended keys and leaves
// (m_c, l_c, O_c) per head, where m_c is the chunk's reference max (log2
// domain), l_c = sum 2^(s - m_c) and O_c = sum 2^(s - m_c) V (unnormalised).
// The exact result over the union of the chunks is
//     M = max_c m_c,  out = sum_c 2^(m_c - M) O_c / sum_c 2^(m_c - M) l_c
// (softmax is invariant to the reference max; the chunks partition the keys).
// A split without keys leaves m_c = -inf and contributes nothing (its O_c is
// never read into the sum); a slot without keys gets zeros.
//
// O_c is stored in fp32 in channel order, or, when the call's result is bf16
// (the shared-tile MQA kernel, d = 256), rounded to bf16 with each group of
// 32 channels stored as four 8-element runs: run q of group j holds channels
// 32j + 4q .. +3, then 32j + 16 + 4q .. +3.  Rows go in pairs: group j of
// rows 2i and 2i+1 shares one 128-byte line (row 2i first), so each store of
// the producing wave writes whole lines.  m_c and l_c stay fp32.
//
// fp32 partials: one wave per (slot, head), lane l owns channels 4l .. 4l+3.
// bf16 partials: one wave per two rows, lane l owns run l % 32 of row l / 32.
// Every load of a row (all splits' m, l and O) is issued before the first
// use, so the kernel costs one memory round trip; splits are merged in
// increasing order, so the result depends only on the split count.
#include "device_common.h"
#include "kernel_params.h"

namespace mfa {
namespace {

typedef __attribute__((ext_vector_type(8))) float floatx8;

__device__ __forceinline__ void store_out4(const DecodeParams& p, int64_t off, floatx4 v) {
  if (p.out_f32)
    *reinterpret_cast<floatx4*>(static_cast<float*>(p.out) + off) = v;
  else
    *reinterpret_cast<intx2*>(static_cast<uint16_t*>(p.out) + off) =
        intx2{(int)pack_bf16x2(v.x, v.y), (int)pack_bf16x2(v.z, v.w)};
}

// The channels one lane merges: four of an fp32 partial row, or one 8-element
// run of a bf16 row.
template <bool kBf16>
struct MergeLane;

template <>
struct MergeLane<false> {
  using vec = floatx4;
  static constexpr int kRowsPerWave = 1;
  int ch;      // first channel (lanes past d re-read the last ones and store nothing)
  bool live;
  __device__ MergeLane(int lane, int d) : ch(min(lane * 4, d - 4)), live(lane * 4 < d) {}
  __device__ vec load(const DecodeParams& p, int64_t r, int d) const {
    return *reinterpret_cast<const floatx4*>(p.part_o + r * d + ch);
  }
  __device__ void store(const DecodeParams& p, int64_t out_row, vec v) const {
    store_out4(p, out_row + ch, v);
  }
};

template <>
struct MergeLane<true> {   // d = 256, bf16 partials and a bf16 result
  using vec = floatx8;
  static constexpr int kRowsPerWave = 2;
  int run;
  bool live = true;
  __device__ MergeLane(int lane, int) : run(lane & 31) {}
  // Run 4j + q of row r sits in the lines of the row pair (r & ~1), at
  // 64 j + 32 (r & 1) + 8 q elements: a wave merging rows 2i, 2i+1 reads
  // one contiguous kilobyte per partial.
  __device__ vec load(const DecodeParams& p, int64_t r, int) const {
    const intx4 h = *reinterpret_cast<const intx4*>(reinterpret_cast<const uint16_t*>(p.part_o) +
                                                    (r & ~(int64_t)1) * 256 + (run >> 2) * 64 +
                                                    (r & 1) * 32 + (run & 3) * 8);
    vec v;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_lo_to_f32((uint32_t)h[i]);
      v[2 * i + 1] = bf16_hi_to_f32((uint32_t)h[i]);
    }
    return v;
  }
  // The lane holds channels 32j + 4q .. +3 (v[0..3]) and 32j + 16 + 4q ..
  // +3 (v[4..7]) of run 4j + q.  The four lanes of a run group (one lane
  // quad) trade halves so that lane q stores the 8 consecutive channels
  // 32j + 8q .. +7: lanes 2(q & 1) and 2(q & 1) + 1 of the quad supply their
  // low halves (q < 2) or their high halves (q >= 2).  A row is then 32
  // stores of 16 bytes, four whole lines, streamed out.
  __device__ void store(const DecodeParams& p, int64_t out_row, vec v) const {
    const int lo0 = (int)pack_bf16x2(v[0], v[1]), lo1 = (int)pack_bf16x2(v[2], v[3]);
    const int hi0 = (int)pack_bf16x2(v[4], v[5]), hi1 = (int)pack_bf16x2(v[6], v[7]);
    const int q = run & 3;
    const int src0 = (int)(threadIdx.x & 60) | ((q & 1) << 1);
    const int src1 = src0 + 1;
    const int a0 = __shfl(lo0, src0), a1 = __shfl(lo1, src0), a2 = __shfl(lo0, src1), a3 = __shfl(lo1, src1);
    const int b0 = __shfl(hi0, src0), b1 = __shfl(hi1, src0), b2 = __shfl(hi0, src1), b3 = __shfl(hi1, src1);
    const intx4 w = q < 2 ? intx4{a0, a1, a2, a3} : intx4{b0, b1, b2, b3};
    __builtin_nontemporal_store(
        w, reinterpret_cast<intx4*>(static_cast<uint16_t*>(p.out) + out_row + 32 * (run >> 2) + 8 * q));
  }
};

// An empty asm that uses v: every load feeding v has completed here.
__device__ __forceinline__ void keep(floatx4 v) { asm volatile("" ::"v"(v)); }
__device__ __forceinline__ void keep(floatx8 v) {
  asm volatile("" ::"v"(floatx4{v[0], v[1], v[2], v[3]}), "v"(floatx4{v[4], v[5], v[6], v[7]}));
}

// Merge row of this thread: 4 waves per workgroup, kRowsPerWave rows per wave;
// workgroups numbered XCD-major when kXcd (the balanced merge: a slot's rows
// then run on the XCD whose attention workgroups wrote its pieces).
template <bool kBf16, bool kXcd = false>
__device__ __forceinline__ int64_t merge_row() {
  constexpr int kR = MergeLane<kBf16>::kRowsPerWave;
  const int64_t wg = kXcd ? xcd_major(blockIdx.x, gridDim.x) : blockIdx.x;
  return (wg * 4 + (threadIdx.x >> 6)) * kR + (kR == 2 ? (threadIdx.x & 63) >> 5 : 0);
}

template <int kMaxSplits, bool kBf16>
__global__ void __launch_bounds__(256) combine_kernel(DecodeParams p, int group, int d) {
  using Lane = MergeLane<kBf16>;
  using vec = typename Lane::vec;
  const Lane ln(threadIdx.x & 63, d);
  const int64_t row = merge_row<kBf16>();   // over B*Hkv*G
  const int64_t nrows = (int64_t)p.batch * p.hkv * group;
  if (row >= nrows) return;
  const int64_t bg = row / group;
  const int h = (int)(row - bg * group);
  const int b = (int)(bg / p.hkv);
  const int g = (int)(bg - (int64_t)b * p.hkv);
  const int64_t base = bg * p.splits;

  floatx2 ml[kMaxSplits];
  vec o[kMaxSplits];
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s) {
    const int64_t r = (base + min(s, p.splits - 1)) * group + h;
    ml[s] = *reinterpret_cast<const floatx2*>(p.part_ml + r * 2);
    o[s] = ln.load(p, r, d);
  }
  float M = kNegInf;
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s)
    if (s < p.splits) M = fmaxf(M, ml[s].x);
  vec acc = {};
  float lsum = 0.f;
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s) {
    if (s < p.splits && ml[s].x != kNegInf) {
      const float w = fast_exp2(ml[s].x - M);
      lsum += w * ml[s].y;
      acc += w * o[s];
    }
  }
  const float inv = lsum > 0.f ? (p.v_scale ? p.v_scale[g] : 1.f) / lsum : 0.f;
  if (!ln.live) return;
  ln.store(p, ((int64_t)b * p.hq + (int64_t)g * group + h) * d, acc * inv);
}

// Any split count: a running (online) merge, one split at a time.
template <bool kBf16>
__global__ void __launch_bounds__(256) combine_any_kernel(DecodeParams p, int group, int d) {
  using Lane = MergeLane<kBf16>;
  using vec = typename Lane::vec;
  const Lane ln(threadIdx.x & 63, d);
  const int64_t row = merge_row<kBf16>();
  const int64_t nrows = (int64_t)p.batch * p.hkv * group;
  if (row >= nrows) return;
  const int64_t bg = row / group;
  const int h = (int)(row - bg * group);
  const int b = (int)(bg / p.hkv);
  const int g = (int)(bg - (int64_t)b * p.hkv);
  const int64_t base = bg * p.splits;
  float M = kNegInf, lsum = 0.f;
  vec acc = {};
  for (int s = 0; s < p.splits; ++s) {
    const int64_t r = (base + s) * group + h;
    const floatx2 ml = *reinterpret_cast<const floatx2*>(p.part_ml + r * 2);
    if (ml.x == kNegInf) continue;
    const vec os = ln.load(p, r, d);
    const float m_new = fmaxf(M, ml.x);
    const float a = M == kNegInf ? 0.f : fast_exp2(M - m_new);
    const float w = fast_exp2(ml.x - m_new);
    lsum = a * lsum + w * ml.y;
    acc = a * acc + w * os;
    M = m_new;
  }
  const float inv = lsum > 0.f ? (p.v_scale ? p.v_scale[g] : 1.f) / lsum : 0.f;
  if (!ln.live) return;
  ln.store(p, ((int64_t)b * p.hq + (int64_t)g * group + h) * d, acc * inv);
}

// Balanced partition (one KV head, d = 256): slot b's pieces were computed
// by workgroups w_lo .. w_hi (unit_desc[b]) of the G = S * B attention
// workgroups; workgroup w's partial for the slot is w, except the first
// one's when the slot is that workgroup's last piece (G + w).  A slot held by one workgroup already has its output, and
// a slot without keys gets zeros here.  When every slot has the same page
// count (a multiple of the split count), the cut is the split plan's: slot
// b's pieces are workgroups b*S .. b*S+S-1, each its first piece; those
// partials are loaded together with the descriptor (one memory round trip)
// and merged like the split combine.  Otherwise pieces are merged in
// increasing workgroup order, four loads at a time.
template <int kMaxSplits, bool kBf16>
__global__ void __launch_bounds__(256) combine_balanced_kernel(DecodeParams p) {
  constexpr int kD = 256;
  using Lane = MergeLane<kBf16>;
  using vec = typename Lane::vec;
  const Lane ln(threadIdx.x & 63, kD);
  const int64_t row = merge_row<kBf16, true>();   // over B*Hq
  if (row >= (int64_t)p.batch * p.hq) return;
  const int b = (int)(row / p.hq);
  const int h = (int)(row - (int64_t)b * p.hq);
  const int S = p.splits;
  const int L = query_len_flat(p, b);   // (no branch: its load goes out with the others)
  const intx4 dsc = *reinterpret_cast<const intx4*>(p.unit_desc + 4 * (int64_t)b);
  floatx2 ml[kMaxSplits];
  vec o[kMaxSplits];
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s) {
    const int64_t r = ((int64_t)b * S + min(s, S - 1)) * p.hq + h;
    ml[s] = *reinterpret_cast<const floatx2*>(p.part_ml + r * 2);
    o[s] = ln.load(p, r, kD);
  }
  // Every load above is in flight before the first branch: the compiler
  // would otherwise sink each into the branch that uses it (three round
  // trips instead of one).
  asm volatile("" ::"v"(L), "v"(dsc.x), "v"(dsc.y), "v"(dsc.z));
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s) {
    asm volatile("" ::"v"(ml[s]));
    keep(o[s]);
  }
  const int64_t out_row = ((int64_t)b * p.hq + h) * kD;
  if (L == 0) {
    ln.store(p, out_row, vec{});
    return;
  }
  const int w_lo = dsc.x, w_hi = dsc.z;
  if (w_lo >= w_hi) return;   // one workgroup held the whole slot
  float M = kNegInf, lsum = 0.f;
  vec acc = {};
  if (S <= kMaxSplits && w_lo == b * S && w_hi == w_lo + S - 1 && dsc.y == 1) {
#pragma unroll
    for (int s = 0; s < kMaxSplits; ++s)
      if (s < S) M = fmaxf(M, ml[s].x);
#pragma unroll
    for (int s = 0; s < kMaxSplits; ++s) {
      if (s < S && ml[s].x != kNegInf) {
        const float wgt = fast_exp2(ml[s].x - M);
        lsum += wgt * ml[s].y;
        acc += wgt * o[s];
      }
    }
  } else {
    const int64_t G = (int64_t)S * p.batch;   // workgroups of the attention grid
    auto piece_of = [&](int w) -> int64_t { return (w == w_lo && dsc.y == 0) ? G + w : w; };
    for (int w0 = w_lo; w0 <= w_hi; w0 += 4) {
      floatx2 ml4[4];
      vec o4[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int64_t r = piece_of(min(w0 + s, w_hi)) * p.hq + h;
        ml4[s] = *reinterpret_cast<const floatx2*>(p.part_ml + r * 2);
        o4[s] = ln.load(p, r, kD);
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if (w0 + s > w_hi || ml4[s].x == kNegInf) continue;
        const float m_new = fmaxf(M, ml4[s].x);
        const float a = M == kNegInf ? 0.f : fast_exp2(M - m_new);
        const float wgt = fast_exp2(ml4[s].x - m_new);
        lsum = a * lsum + wgt * ml4[s].y;
        acc = a * acc + wgt * o4[s];
        M = m_new;
      }
    }
  }
  const float inv = lsum > 0.f ? (p.v_scale ? p.v_scale[0] : 1.f) / lsum : 0.f;
  ln.store(p, out_row, acc * inv);
}

template <bool kBf16>
hipError_t launch_combine_t(const DecodeParams& p, int group, int d, hipStream_t stream) {
  if (kBf16 && d != 256) return hipErrorInvalidValue;
  constexpr int kR = MergeLane<kBf16>::kRowsPerWave;
  const int64_t waves = ((int64_t)p.batch * p.hkv * group + kR - 1) / kR;
  const dim3 grid((unsigned)((waves + 3) / 4)), block(256);
  if (p.balanced) {
    if (p.hkv != 1 || d != 256 || group != p.hq) return hipErrorInvalidValue;
    if (p.splits <= 2)
      hipLaunchKernelGGL((combine_balanced_kernel<2, kBf16>), grid, block, 0, stream, p);
    else if (p.splits <= 4)
      hipLaunchKernelGGL((combine_balanced_kernel<4, kBf16>), grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL((combine_balanced_kernel<8, kBf16>), grid, block, 0, stream, p);
    return hipGetLastError();
  }
  if (p.splits <= 2)
    hipLaunchKernelGGL((combine_kernel<2, kBf16>), grid, block, 0, stream, p, group, d);
  else if (p.splits <= 4)
    hipLaunchKernelGGL((combine_kernel<4, kBf16>), grid, block, 0, stream, p, group, d);
  else if (p.splits <= 8)
    hipLaunchKernelGGL((combine_kernel<8, kBf16>), grid, block, 0, stream, p, group, d);
  else
    hipLaunchKernelGGL((combine_any_kernel<kBf16>), grid, block, 0, stream, p, group, d);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const DecodeParams& p, int group, int d, hipStream_t stream) {
  return p.part_bf16 ? launch_combine_t<true>(p, group, d, stream)
                     : launch_combine_t<false>(p, group, d, stream);
}

}  // namespace mfa

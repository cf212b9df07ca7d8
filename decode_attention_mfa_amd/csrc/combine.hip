// Split-K merge (log-sum-exp combine) of decode-attention partials.
//
// Split c of slot b covers a contiguous chunk of the attended keys and leaves
// (m_c, l_c, O_c) per head, where m_c is the chunk's reference max (log2
// domain), l_c = sum 2^(s - m_c) and O_c = sum 2^(s - m_c) V (unnormalised).
// The exact result over the union of the chunks is
//     M = max_c m_c,  out = sum_c 2^(m_c - M) O_c / sum_c 2^(m_c - M) l_c
// (softmax is invariant to the reference max; the chunks partition the keys).
// One wave per (slot, head); lane l owns channels 4l .. 4l+3.  Splits are
// merged in increasing order, so the result depends only on the split count.
#include "device_common.h"
#include "kernel_params.h"

namespace mfa {
namespace {

__global__ void __launch_bounds__(256) combine_kernel(DecodeParams p, int group, int d) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // over B*Hkv*G
  const int64_t nrows = (int64_t)p.batch * p.hkv * group;
  if (row >= nrows) return;
  const int64_t bg = row / group;
  const int h = (int)(row - bg * group);
  const int b = (int)(bg / p.hkv);
  const int g = (int)(bg - (int64_t)b * p.hkv);
  const int L = p.ctx_lens[b];
  const int lo = (p.window > 0 && L > p.window) ? L - p.window : 0;
  const int n_tiles = L > 0 ? (L - 1) / kPage - lo / kPage + 1 : 0;
  const int n_active = min(p.splits, (n_tiles + p.chunk_tiles - 1) / p.chunk_tiles);
  const int ch = lane * 4;
  if (ch >= d) return;

  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  float inv = 0.f;
  if (n_active > 0) {
    const int64_t base = bg * p.splits;
    float M = kNegInf;
    for (int s = 0; s < n_active; ++s) M = fmaxf(M, p.part_ml[((base + s) * group + h) * 2]);
    float lsum = 0.f;
    for (int s = 0; s < n_active; ++s) {
      const int64_t r = (base + s) * group + h;
      const float w = fast_exp2(p.part_ml[r * 2] - M);
      lsum += w * p.part_ml[r * 2 + 1];
      acc += w * *reinterpret_cast<const floatx4*>(p.part_o + r * d + ch);
    }
    inv = (p.v_scale ? p.v_scale[g] : 1.f) / lsum;
  }
  const floatx4 v = acc * inv;
  const int64_t o = ((int64_t)b * p.hq + (int64_t)g * group + h) * d + ch;
  if (p.out_f32)
    *reinterpret_cast<floatx4*>(static_cast<float*>(p.out) + o) = v;
  else
    *reinterpret_cast<intx2*>(static_cast<uint16_t*>(p.out) + o) =
        intx2{(int)pack_bf16x2(v.x, v.y), (int)pack_bf16x2(v.z, v.w)};
}

}  // namespace

hipError_t launch_combine(const DecodeParams& p, int group, int d, hipStream_t stream) {
  const int64_t rows = (int64_t)p.batch * p.hkv * group;
  const unsigned blocks = (unsigned)((rows + 3) / 4);
  hipLaunchKernelGGL(combine_kernel, dim3(blocks), dim3(256), 0, stream, p, group, d);
  return hipGetLastError();
}

}  // namespace mfa

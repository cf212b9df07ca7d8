// GQA / sliding-window decode attention on gfx950: 16 query heads share each
// KV group, d = 192 or 256 ("Step-5-Preview: Sparse GQA, Indexer und
// KV-Speicher": 64 query heads, 4 KV groups, width 192, head h reads group
// floor(h / 16); local layers attend to a 512-token window that includes the
// current token; the dense global layer attends to everything).
//
// V is read channel-major ([d][64] per block) or in 8-token sub-blocks
// ([8][d][8] per block, the layout of the sparse global attention, so that
// one cache serves both calls); either way a 16-byte run holds 8 keys of one
// channel, which is all the V^T tile copy needs.
//
// Workgroup = 4 waves = one (slot, KV group, split).  The split's keys are
// streamed in 64-key tiles through the same LDS phase ring as the MQA kernel
// (phase 2t = K tile [64][d], phase 2t+1 = V^T tile [d][64], 16-byte
// non-temporal global->LDS DMA, kRing - 2 phases in flight).  With 16 heads
// per group a single MFMA row block covers all heads, so the waves split the
// keys instead: wave w takes keys 16w .. 16w+15 of every tile.
//   S^T[key, head] = K . Q^T            16x16x32 bf16 MFMA, d/32 K-steps
//   O^T[ch, head] += V^T . P^T          16x16x16 bf16 MFMA over the wave's
//                                       16 keys (the S^T lane layout is the
//                                       B operand as is)
// Each wave keeps its own online softmax (m, l, O) over its key subset; the
// four are merged through LDS at the end (the same log-sum-exp merge as the
// split combine).
#include <type_traits>

#include "device_common.h"
#include "kernel_params.h"

namespace mfa {
namespace {

constexpr int kG = 16;
constexpr int kMaxChunkTiles = 2048;
constexpr float kLazyRescale = 8.f;

typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;

__device__ __forceinline__ floatx4 mfma_bf16_16x16x16(intx2 a, intx2 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4_t, a),
                                                   __builtin_bit_cast(bf16x4_t, b), c, 0, 0, 0);
}

// Tile geometry: bf16 or E4M3 (one byte per value) K/V.  The ring takes
// 144 KB of LDS for d = 192 and 128 KB for d = 256, so E4M3 tiles keep twice
// as many phases in flight.
template <int D, bool kFp8>
struct GqaCfg {
  static constexpr int kElem = kFp8 ? 1 : 2;                       // bytes per cached value
  static constexpr int kPhaseBytes = 64 * D * kElem;               // one K or V^T tile
  static constexpr int kRing = (D == 192 ? 147456 : 131072) / kPhaseBytes;   // LDS slots
  static constexpr int kAhead = kRing - 2;                         // phases in flight while computing
  static constexpr int kDmaPerWave = kPhaseBytes / 1024 / 4;       // 16-byte copies per lane per phase
  static constexpr int kChunks = D * kElem / 16;                   // 16-byte chunks per K row
  static_assert(kRing % 2 == 0 && kAhead * kDmaPerWave < 64, "ring shape");
};

// Eight E4M3 codes (two dwords) to the eight bf16 of an MFMA operand, and four
// codes to four bf16: exact (every E4M3FN value is a bf16 value, scale 1).
template <bool kUpper>
__device__ __forceinline__ int e4m3x2_bf16x2(int w) {
  return __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, kUpper));
}
__device__ __forceinline__ intx4 e4m3x8_bf16(int w0, int w1) {
  return intx4{e4m3x2_bf16x2<false>(w0), e4m3x2_bf16x2<true>(w0), e4m3x2_bf16x2<false>(w1),
               e4m3x2_bf16x2<true>(w1)};
}

// K rows (D values): XOR the chunk index with a key-dependent value so that
// the lanes of one MFMA operand read conflict-free (checked with the LDS
// bank-conflict counter: folding key bit 3 into the bf16 d = 192 map cost
// every K read a 2-way conflict).  The XOR stays inside aligned groups of 8
// chunks (bf16 d = 192: 24 chunks per row) or 4 (E4M3 d = 192: 12 chunks of
// 16 codes, where key bits 1-2 are the conflict-free choice).
template <int D, bool kFp8>
__device__ __forceinline__ int swz_k(int key) {
  if constexpr (kFp8) return D == 256 ? (key & 15) : ((key >> 1) & 3);
  return D == 256 ? (key & 15) : (key & 7);
}
// V^T rows: bf16 128 bytes (8 chunks of 8 keys), E4M3 64 bytes (4 chunks of
// 16 keys; the 4-byte operand reads keep a 2-way bank conflict under every
// XOR map of four chunks, and this one is among the best measured).
__device__ __forceinline__ int swz_v(int ch) { return (ch & 7) ^ ((ch >> 3) & 1); }
__device__ __forceinline__ int swz_v8(int ch) { return (ch >> 2) & 3; }

template <int N>
__device__ __forceinline__ void phase_barrier() {
  wait_vmcnt<N>();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int D, bool kFp8>
__global__ void __launch_bounds__(256) gqa_decode_kernel(DecodeParams p) {
  using C = GqaCfg<D, kFp8>;
  using T = std::conditional_t<kFp8, uint8_t, uint16_t>;     // cached value
  __shared__ __attribute__((aligned(1024))) uint8_t ring[C::kRing * C::kPhaseBytes];
  __shared__ int blk_ids[kMaxChunkTiles];
  __shared__ float wave_ml[4][kG][2];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15;
  const int q4 = lane >> 4;
  const int bg = blockIdx.y;
  const int b = bg / p.hkv;
  const int g = bg - b * p.hkv;
  const int split = blockIdx.x;
  const int L = slot_len(p.ctx_lens[b], p.max_blocks);
  const int lo = (p.window > 0 && L > p.window) ? L - p.window : 0;
  int n_tiles = 0, t_lo = 0;
  if (L > 0) {
    t_lo = lo / kPage;
    n_tiles = (L - 1) / kPage - t_lo + 1;
  }
  const int t_begin = t_lo + split * p.chunk_tiles;
  const int t_end = min(t_lo + n_tiles, t_begin + p.chunk_tiles);
  const int head = g * kG + r;          // this lane's query head

  if (t_begin >= t_end) {
    if (p.splits == 1) {   // empty slot: zeros (wave w writes channel tiles w, w+4, ...)
      for (int ct = wave; ct < D / 16; ct += 4) {
        const int64_t o = ((int64_t)b * p.hq + head) * D + ct * 16 + q4 * 4;
        if (p.out_f32)
          *reinterpret_cast<floatx4*>(static_cast<float*>(p.out) + o) = floatx4{0.f, 0.f, 0.f, 0.f};
        else
          *reinterpret_cast<intx2*>(static_cast<uint16_t*>(p.out) + o) = intx2{0, 0};
      }
    } else if (wave == 0 && q4 == 0) {   // no keys in this split: an empty partial
      const int64_t row = ((int64_t)bg * p.splits + split) * kG + r;
      *reinterpret_cast<floatx2*>(p.part_ml + row * 2) = floatx2{kNegInf, 0.f};
    }
    return;
  }
  const int nt = t_end - t_begin;
  const int nphase = 2 * nt;
  const float qk_scale = p.scale * kLog2e * (p.k_scale ? p.k_scale[g] : 1.f);
  const float v_scale = p.v_scale ? p.v_scale[g] : 1.f;

  for (int i = threadIdx.x; i < nt; i += 256)
    blk_ids[i] = p.block_table ? pool_block(p.block_table[(int64_t)b * p.max_blocks + t_begin + i], p.num_blocks) : 0;

  // Q fragments: head r of the group.  bf16 K: step s takes channels
  // 32s + 8q4 .. +7.  E4M3 K: step s takes channels 64(s/2) + 16q4 + 8(s%2)
  // .. +7, so that one 16-byte read of codes holds the K operands of steps
  // 2u and 2u + 1.
  intx4 qf[D / 32];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(p.q) + ((int64_t)b * p.hq + head) * D;
#pragma unroll
    for (int s = 0; s < D / 32; ++s)
      qf[s] = *reinterpret_cast<const intx4*>(qp + (kFp8 ? 64 * (s >> 1) + 16 * q4 + 8 * (s & 1)
                                                        : 32 * s + 8 * q4));
  }
  wait_vmcnt<0>();   // the copies below are invisible to the compiler's wait bookkeeping
  __syncthreads();

  const T* kpool = static_cast<const T*>(p.k);
  const T* vpool = static_cast<const T*>(p.v);
  constexpr int kChunkElems = 16 / C::kElem;   // values per 16-byte chunk
  auto issue_phase = [&](int ph_req, uint8_t* dst) {
    const int ph = ph_req < nphase ? ph_req : nphase - 2 + (ph_req & 1);
    const int tile_rel = ph >> 1;
    const int tile = t_begin + tile_rel;
    const T* kt;
    const T* vt;
    if (p.block_table) {
      const int64_t blk = readfirstlane(blk_ids[tile_rel]);
      kt = kpool + blk * p.k_block_stride + (int64_t)g * p.k_head_stride;
      vt = vpool + blk * p.v_block_stride + (int64_t)g * p.v_head_stride;
    } else {
      kt = kpool + ((int64_t)b * p.max_blocks + tile) * p.k_block_stride + (int64_t)g * p.k_head_stride;
      vt = vpool + (int64_t)b * p.v_seq_stride + (int64_t)g * p.v_head_stride + (int64_t)tile * p.v_tile_stride;
    }
    if ((ph & 1) == 0) {
      // K tile: 64 rows of kChunks chunks; copy i covers 1 KB = 64 chunks.
#pragma unroll
      for (int k = 0; k < C::kDmaPerWave; ++k) {
        const int i = wave * C::kDmaPerWave + k;
        const int idx = i * 64 + lane;                 // chunk index in the tile
        const int row = idx / C::kChunks;
        const int ch = (idx - row * C::kChunks) ^ swz_k<D, kFp8>(row);
        dma16_nt(kt + row * p.k_row_stride + ch * kChunkElems, dst + i * 1024);
      }
    } else {
      // V^T tile: D rows of 8 chunks (64 keys); copy i covers 8 rows.  Chunk
      // ch of row (channel) `row` is keys 8ch .. 8ch + 7 of that channel,
      // wherever the layout keeps them (channel-major or 8-token sub-blocks).
      // E4M3: D rows of 4 chunks (16 keys each); copy i covers 16 rows, and
      // V is channel-major (a chunk is 16 consecutive bytes).
      if constexpr (kFp8) {
#pragma unroll
        for (int k = 0; k < C::kDmaPerWave; ++k) {
          const int i = wave * C::kDmaPerWave + k;
          const int row = 16 * i + (lane >> 2);
          const int ch = (lane & 3) ^ swz_v8(row);
          dma16_nt(vt + row * p.v_row_stride + ch * 16, dst + i * 1024);
        }
      } else {
#pragma unroll
        for (int k = 0; k < C::kDmaPerWave; ++k) {
          const int i = wave * C::kDmaPerWave + k;
          const int row = 8 * i + (lane >> 3);
          const int ch = (lane & 7) ^ swz_v(row);
          dma16_nt(vt + row * p.v_row_stride + ch * p.v_chunk_stride, dst + i * 1024);
        }
      }
    }
  };

#pragma unroll
  for (int ph = 0; ph < C::kRing - 1; ++ph) issue_phase(ph, ring + ph * C::kPhaseBytes);

  const int my_key = 16 * wave + r;                    // K operand row of this lane
  const int xk = swz_k<D, kFp8>(my_key);
  const int xv = kFp8 ? swz_v8(r) : swz_v(r);

  float m_run = kNegInf;
  float l_run = 0.f;
  floatx4 acc[D / 16];
#pragma unroll
  for (int ct = 0; ct < D / 16; ++ct) acc[ct] = floatx4{0.f, 0.f, 0.f, 0.f};
  intx2 pb;

  auto k_phase = [&](const uint8_t* buf, int key0) {
    floatx4 st = {0.f, 0.f, 0.f, 0.f};
    if constexpr (kFp8) {
#pragma unroll
      for (int u = 0; u < D / 64; ++u) {
        const int chunk = (4 * u + q4) ^ xk;
        const intx4 c = *reinterpret_cast<const intx4*>(buf + my_key * D + chunk * 16);
        st = mfma_bf16_16x16x32(e4m3x8_bf16(c.x, c.y), qf[2 * u], st);
        st = mfma_bf16_16x16x32(e4m3x8_bf16(c.z, c.w), qf[2 * u + 1], st);
      }
    } else {
#pragma unroll
      for (int s = 0; s < D / 32; ++s) {
        const int chunk = (4 * s + q4) ^ xk;
        const intx4 a = *reinterpret_cast<const intx4*>(buf + my_key * (2 * D) + chunk * 16);
        st = mfma_bf16_16x16x32(a, qf[s], st);
      }
    }
    float sv[4];
    const bool partial = (key0 < lo) || (key0 + kPage > L);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float x = st[i] * qk_scale;
      if (partial) {
        const int key = key0 + 16 * wave + 4 * q4 + i;
        x = (key >= lo && key < L) ? x : kNegInf;
      }
      sv[i] = x;
    }
    float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    mx = wave_max_xor16_32(mx);
    // A wave can see a tile whose 16 keys are all masked: mx = -inf, nothing moves.
    const bool move = mx > m_run + kLazyRescale;
    const float m_new = move ? mx : m_run;
    if (__any(move && m_run != kNegInf)) {
      const float alpha = fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int ct = 0; ct < D / 16; ++ct) acc[ct] *= alpha;
    }
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[i] = (m_new == kNegInf) ? 0.f : fast_exp2(sv[i] - m_new);
      psum += sv[i];
    }
    l_run += psum;
    pb = intx2{(int)pack_bf16x2(sv[0], sv[1]), (int)pack_bf16x2(sv[2], sv[3])};
  };

  auto v_phase = [&](const uint8_t* buf, int key0) {
    const int kfirst = 16 * wave + 4 * q4;             // this lane's 4 keys
    const int vvalid = L - key0;
    uint32_t keep0 = 0xffffffffu, keep1 = 0xffffffffu;
    if (vvalid < kPage) {   // rows past the end may hold NaN
      keep0 = ((kfirst + 0 < vvalid) ? 0x0000ffffu : 0u) | ((kfirst + 1 < vvalid) ? 0xffff0000u : 0u);
      keep1 = ((kfirst + 2 < vvalid) ? 0x0000ffffu : 0u) | ((kfirst + 3 < vvalid) ? 0xffff0000u : 0u);
    }
#pragma unroll
    for (int ct = 0; ct < D / 16; ++ct) {
      intx2 a;
      if constexpr (kFp8) {
        // Codes of keys kfirst .. +3: chunk kfirst / 16 of row 16 ct + r, byte
        // kfirst % 16.
        const uint32_t c = *reinterpret_cast<const uint32_t*>(
            buf + ct * 1024 + r * 64 + (((kfirst >> 4) ^ xv) << 4) + (kfirst & 15));
        a = intx2{e4m3x2_bf16x2<false>((int)c), e4m3x2_bf16x2<true>((int)c)};
      } else {
        a = *reinterpret_cast<const intx2*>(buf + ct * 2048 + r * 128 + (((kfirst >> 3) ^ xv) << 4) +
                                            (q4 & 1) * 8);
      }
      a.x &= keep0;
      a.y &= keep1;
      acc[ct] = mfma_bf16_16x16x16(a, pb, acc[ct]);
    }
  };

  auto step = [&](int ph, int slot) {
    phase_barrier<C::kAhead * C::kDmaPerWave>();
    issue_phase(ph + C::kRing - 1, ring + ((slot + C::kRing - 1) % C::kRing) * C::kPhaseBytes);
    const uint8_t* cur = ring + slot * C::kPhaseBytes;
    const int key0 = (t_begin + (ph >> 1)) * kPage;
    if ((slot & 1) == 0) k_phase(cur, key0);
    else v_phase(cur, key0);
  };

  for (int ph = 0; ph < nphase; ph += C::kRing) {
#pragma unroll
    for (int s = 0; s < C::kRing; s += 2) {
      if (ph + s >= nphase) break;
      step(ph + s, s);
      step(ph + s + 1, s + 1);
    }
  }
  wait_vmcnt<0>();
  __syncthreads();   // every wave is done with the ring: reuse it for the merge

  // ---- merge the four waves' (m, l, O) ----
  const float l_w = wave_sum_xor16_32(l_run);
  if (q4 == 0) {
    wave_ml[wave][r][0] = m_run;
    wave_ml[wave][r][1] = l_w;
  }
  // [4][kG][D + 4]: the 16-byte pad per head row spreads the 16 rows a
  // store instruction touches over every bank (a row of D floats is a whole
  // number of bank rows, which made each store a 16-way conflict).
  constexpr int kOStride = D + 4;
  float* obuf = reinterpret_cast<float*>(ring);
#pragma unroll
  for (int ct = 0; ct < D / 16; ++ct)
    *reinterpret_cast<floatx4*>(obuf + ((wave * kG + r) * kOStride + ct * 16 + q4 * 4)) = acc[ct];
  __syncthreads();

  // Thread t: head t / 16, channels 4*(t % 16) + 64*k.
  const int h = threadIdx.x >> 4;
  float M = kNegInf;
#pragma unroll
  for (int w = 0; w < 4; ++w) M = fmaxf(M, wave_ml[w][h][0]);
  float wgt[4];
  float lsum = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    wgt[w] = (wave_ml[w][h][0] == kNegInf) ? 0.f : fast_exp2(wave_ml[w][h][0] - M);
    lsum += wgt[w] * wave_ml[w][h][1];
  }
  const int64_t ghead = (int64_t)g * kG + h;
  const int64_t prow = ((int64_t)bg * p.splits + split) * kG + h;
  for (int c4 = (threadIdx.x & 15) * 4; c4 < D; c4 += 64) {
    floatx4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < 4; ++w) o += wgt[w] * *reinterpret_cast<const floatx4*>(obuf + (w * kG + h) * kOStride + c4);
    if (p.splits == 1) {
      const floatx4 v = o * (v_scale / lsum);
      const int64_t off = ((int64_t)b * p.hq + ghead) * D + c4;
      if (p.out_f32)
        *reinterpret_cast<floatx4*>(static_cast<float*>(p.out) + off) = v;
      else
        *reinterpret_cast<intx2*>(static_cast<uint16_t*>(p.out) + off) =
            intx2{(int)pack_bf16x2(v.x, v.y), (int)pack_bf16x2(v.z, v.w)};
    } else {
      *reinterpret_cast<floatx4*>(p.part_o + prow * D + c4) = o;
    }
  }
  if (p.splits > 1 && (threadIdx.x & 15) == 0)
    *reinterpret_cast<floatx2*>(p.part_ml + prow * 2) = floatx2{M, lsum};
}

}  // namespace

hipError_t launch_gqa(const DecodeParams& p, int d, bool fp8, hipStream_t stream) {
  dim3 grid(p.splits, p.batch * p.hkv);
  if (d == 192 && !fp8)
    hipLaunchKernelGGL((gqa_decode_kernel<192, false>), grid, dim3(256), 0, stream, p);
  else if (d == 256 && !fp8)
    hipLaunchKernelGGL((gqa_decode_kernel<256, false>), grid, dim3(256), 0, stream, p);
  else if (d == 192)
    hipLaunchKernelGGL((gqa_decode_kernel<192, true>), grid, dim3(256), 0, stream, p);
  else if (d == 256)
    hipLaunchKernelGGL((gqa_decode_kernel<256, true>), grid, dim3(256), 0, stream, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace mfa

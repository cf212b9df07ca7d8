// Step-5 sparse global attention for one decode token per request
// ("Step-5-Preview: Sparse GQA, Indexer und KV-Speicher"):
//   1. sparse_summary_kernel: the summary of every complete 8-token block,
//      c[r, d] = sum_j softmax_j(z[8r + j, d]) kI[8r + j, d], one coordinate
//      per thread, fp32, rounded to bf16 and stored as E4M3 (section "Acht
//      Tokens ergeben einen Such-Key - koordinatenweise").
//   2. sparse_score_kernel: for the token at t = L - 1 and every provider
//      group g, s[g, r] = sum_h w[g, h] ReLU(Q8(qI[g, h]) . c[r]) over the
//      candidate blocks r < floor(t / 8); sparse_select_kernel: the 512
//      highest (equal scores to the lower block id), listed in ascending id
//      order (section "Auswahl per gewichtetem ReLU-Score").
//   3. sparse_attention_kernel: the 16 heads of group g attend the selected
//      blocks' original K/V plus the current block up to t (section "Die
//      eigentliche Attention liest weiterhin originale K/V").
//
// The scores are one matrix product per request: S^T[block, (g, h)] =
// C[block, :] . Q8^T, with the 16 columns exactly the 4 groups x 4 search
// heads, on the 16x16x32 bf16 MFMA (E4M3 codes widen to bf16 exactly; the
// products are exact, the sums fp32).  The top-512 is a radix select on the
// key (order-preserving score bits less those of the smallest score, then
// 4095 - id, so every key is distinct and equal scores rank the lower id
// first), in 11-bit passes over the scores kept in LDS, then an ordered
// compaction.
//
// The attention kernel is the GQA decode kernel's pipeline (4 waves, 64-key
// tiles through an LDS ring filled by 16-byte non-temporal global->LDS
// copies, wave w takes keys 16w .. 16w+15 of every tile, the four waves
// merged through LDS)
// with a gathered tile: tile i holds list entries 8i .. 8i+7, each an 8-token
// block.  Its K is 8 consecutive rows of a 64-token page (3 KB); its V^T is
// one contiguous [192][8] sub-block, because this layer's V cache is stored
// channel-major per 8-token sub-block ([blocks, 4, 8, 192, 8]) rather than
// per page: a selected block then costs two 3 KB reads, where a page-wide
// V^T row would give 16 isolated bytes per channel.
#include "device_common.h"
#include "fp8_encode.h"
#include "sparse_params.h"

namespace mfa {
hipError_t launch_combine(const DecodeParams& p, int group, int d, hipStream_t stream);

namespace {

constexpr int kD = 192;
constexpr int kG = 16;                          // query heads per KV group
constexpr int kPhaseBytes = 64 * kD * 2;        // one K or V^T tile
constexpr int kRing = 6;                        // LDS slots
constexpr int kAhead = kRing - 2;               // phases in flight while computing
constexpr int kDmaPerWave = kPhaseBytes / 1024 / 4;
constexpr int kChunks = kD / 8;                 // 16-byte chunks per K row
constexpr int kMaxEntries = 8 * kSparseMaxTiles;
constexpr float kLazyRescale = 8.f;

typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;

__device__ __forceinline__ floatx4 mfma_bf16_16x16x16(intx2 a, intx2 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4_t, a),
                                                   __builtin_bit_cast(bf16x4_t, b), c, 0, 0, 0);
}

// Eight E4M3 codes to the eight bf16 of an MFMA operand (exact, scale 1).
template <bool kUpper>
__device__ __forceinline__ int e4m3x2_to_bf16x2(int w) {
  return __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, kUpper));
}
__device__ __forceinline__ intx4 e4m3x8_to_bf16(int w0, int w1) {
  return intx4{e4m3x2_to_bf16x2<false>(w0), e4m3x2_to_bf16x2<true>(w0),
               e4m3x2_to_bf16x2<false>(w1), e4m3x2_to_bf16x2<true>(w1)};
}

__device__ __forceinline__ float bf16_bits_to_float(uint16_t v) {
  return __builtin_bit_cast(float, (uint32_t)v << 16);
}
// Nearest bf16 of a finite fp32 value, ties to even.
__device__ __forceinline__ float round_bf16(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return __builtin_bit_cast(float, u & 0xFFFF0000u);
}

// ---------------------------------------------------------------------------
// 1. Block summaries: grid (blocks / 4, B), thread d = coordinate.  Blocks
// r0 .. nb - 1 of each request, r0 = 0 (every complete block) or, with
// new_tokens = n > 0, r0 = floor((L - n) / 8): the blocks that the last n
// tokens completed (a decode step completes a block at its eighth token).
__global__ void __launch_bounds__(256) sparse_summary_kernel(SparseParams p) {
  const int b = blockIdx.y;
  const int d = threadIdx.x;
  const int L = slot_len(p.dp.ctx_lens[b], p.dp.max_blocks);
  const int nb = min(L / kSparseBlock, p.cap8);
  const int r0 = p.new_tokens > 0 ? max(L - p.new_tokens, 0) / kSparseBlock : 0;
  const int64_t cap = (int64_t)p.dp.max_blocks * kPage;
  const uint16_t* kp = static_cast<const uint16_t*>(p.k_idx) + (int64_t)b * cap * kSparseWidth + d;
  const uint16_t* zp = static_cast<const uint16_t*>(p.z) + (int64_t)b * cap * kSparseWidth + d;
  uint8_t* cp = p.summ_out + (int64_t)b * p.cap8 * kSparseWidth + d;
  const int r_end = min(nb, r0 + (int)(blockIdx.x + 1) * 4);
  for (int r = r0 + blockIdx.x * 4; r < r_end; ++r) {
    float zv[kSparseBlock], kv[kSparseBlock];
#pragma unroll
    for (int j = 0; j < kSparseBlock; ++j) {
      const int64_t row = (int64_t)(kSparseBlock * r + j) * kSparseWidth;
      zv[j] = bf16_bits_to_float(zp[row]);
      kv[j] = bf16_bits_to_float(kp[row]);
    }
    float m = zv[0];
#pragma unroll
    for (int j = 1; j < kSparseBlock; ++j) m = fmaxf(m, zv[j]);
    float den = 0.f, num = 0.f;
#pragma unroll
    for (int j = 0; j < kSparseBlock; ++j) {
      const float e = fast_exp2((zv[j] - m) * kLog2e);
      den += e;
      num += e * kv[j];
    }
    cp[(int64_t)r * kSparseWidth] = e4m3fn_encode(round_bf16(num / den));
  }
}

// ---------------------------------------------------------------------------
// 2. Scores, then the top-512.

// Order-preserving 32-bit image of a float (larger float -> larger integer).
__device__ __forceinline__ uint32_t mono_bits(float s) {
  const uint32_t u = __builtin_bit_cast(uint32_t, s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kSelThreads = 512;   // 8 waves per (request, group)
constexpr int kScoreChunk = 256;   // candidates per scoring workgroup

// Inclusive prefix sum of one value per thread over the workgroup.
__device__ __forceinline__ int sel_scan_incl(int v, int* wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int a = __shfl_up(v, off);
    if (lane >= off) v += a;
  }
  if (lane == 63) wsum[wave] = v;
  __syncthreads();
  int pre = 0;
#pragma unroll
  for (int w2 = 0; w2 < kSelThreads / 64; ++w2) pre += (w2 < wave) ? wsum[w2] : 0;
  __syncthreads();
  return v + pre;
}

// 2a. Scores: one workgroup of 4 waves per (request, 256 candidates), each
// wave 4 tiles of 16 candidates with all summary loads issued before the
// first product; scores[b, g, r] (fp32) go to the workspace.
__global__ void __launch_bounds__(256) sparse_score_kernel(SparseParams p) {
  constexpr int kUnroll = kScoreChunk / 16 / 4;
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int L = slot_len(p.dp.ctx_lens[b], p.dp.max_blocks);
  const int t = L - 1;
  const int R = t >= 0 ? min(t / kSparseBlock, p.cap8) : 0;   // candidate blocks
  const int t0 = (blockIdx.x * kScoreChunk) / 16 + wave * kUnroll;   // first tile of this wave
  if (R <= kSparseBudget || 16 * (blockIdx.x * kScoreChunk / 16) >= R) return;   // all selected / no candidate here

  // Q8 of the request's 16 search queries, once per workgroup: thread t
  // rounds values 16t .. 16t+15 to E4M3 and widens them back to bf16 (exact)
  // into LDS.  Fragments: column col = 4g + h of lane l % 16; K-step c takes
  // coordinates 64(c/2) + 16(l/16) + 8(c%2) .. +7, the channel map under
  // which one 16-byte read of codes holds two steps' A operands.
  // Rows of kSparseWidth + 8 values: the 16-byte pad spreads the 16 columns a
  // fragment read touches over every bank (unpadded rows are whole bank rows).
  constexpr int kQ8Stride = kSparseWidth + 8;
  __shared__ __attribute__((aligned(16))) uint16_t q8s[kSparseGroups * kSparseHeads * kQ8Stride];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(p.q_idx) +
                         (int64_t)b * kSparseGroups * kSparseHeads * kSparseWidth + 16 * threadIdx.x;
    uint16_t* qs = q8s + (threadIdx.x >> 4) * kQ8Stride + 16 * (threadIdx.x & 15);
    const intx4 v0 = *reinterpret_cast<const intx4*>(qp), v1 = *reinterpret_cast<const intx4*>(qp + 8);
    const int w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    int codes[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      codes[k] = (int)((uint32_t)e4m3fn_encode(bf16_bits_to_float((uint16_t)(w[2 * k] & 0xFFFF))) |
                       ((uint32_t)e4m3fn_encode(bf16_bits_to_float((uint16_t)((uint32_t)w[2 * k] >> 16))) << 8) |
                       ((uint32_t)e4m3fn_encode(bf16_bits_to_float((uint16_t)(w[2 * k + 1] & 0xFFFF)))) << 16 |
                       ((uint32_t)e4m3fn_encode(bf16_bits_to_float((uint16_t)((uint32_t)w[2 * k + 1] >> 16))) << 24));
    *reinterpret_cast<intx4*>(qs) = e4m3x8_to_bf16(codes[0], codes[1]);
    *reinterpret_cast<intx4*>(qs + 8) = e4m3x8_to_bf16(codes[2], codes[3]);
  }
  __syncthreads();
  const int col = lane & 15, q4 = lane >> 4;
  const int grp = col >> 2, sh = col & 3;
  intx4 qf[kSparseWidth / 32];
#pragma unroll
  for (int c = 0; c < kSparseWidth / 32; ++c)
    qf[c] = *reinterpret_cast<const intx4*>(q8s + col * kQ8Stride + 64 * (c >> 1) + 16 * q4 + 8 * (c & 1));
  const float wgt = p.w[(b * kSparseGroups + grp) * kSparseHeads + sh];
  if (16 * t0 >= R) return;   // this wave's tiles are past the candidates

  const uint8_t* cb = p.summ + (int64_t)b * p.cap8 * kSparseWidth + 16 * q4;
  intx4 raw[kUnroll][kSparseWidth / 64];
#pragma unroll
  for (int k = 0; k < kUnroll; ++k) {
    const int row = min(16 * (t0 + k) + col, R - 1);
#pragma unroll
    for (int u = 0; u < kSparseWidth / 64; ++u)
      raw[k][u] = *reinterpret_cast<const intx4*>(cb + (int64_t)row * kSparseWidth + 64 * u);
  }
  float* scb = p.scores + (int64_t)(b * kSparseGroups + grp) * p.cap8;
#pragma unroll
  for (int k = 0; k < kUnroll; ++k) {
    floatx4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < kSparseWidth / 64; ++u) {
      st = mfma_bf16_16x16x32(e4m3x8_to_bf16(raw[k][u].x, raw[k][u].y), qf[2 * u], st);
      st = mfma_bf16_16x16x32(e4m3x8_to_bf16(raw[k][u].z, raw[k][u].w), qf[2 * u + 1], st);
    }
    // Lane (col, q4) holds candidates 16 tile + 4 q4 + i for column col;
    // the sum over the group's four search heads is over lanes col ^ 1, ^ 2.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = wgt * fmaxf(st[i], 0.f);
      v += __shfl_xor(v, 1);
      v += __shfl_xor(v, 2);
      const int cand = 16 * (t0 + k) + 4 * q4 + i;
      if (sh == 0 && cand < R) scb[cand] = v + 0.f;   // -0 -> +0: equal scores compare equal
    }
  }
}

// 2b. Top-512: one workgroup of 8 waves per (request, group) over the scores.
__global__ void __launch_bounds__(kSelThreads) sparse_select_kernel(SparseParams p) {
  constexpr int kWaves = kSelThreads / 64;
  constexpr int kDigitBits = 11, kBins = 1 << kDigitBits;   // 4 bins per thread
  static_assert(kBins == 4 * kSelThreads, "radix bins");
  __shared__ float sc[kSparseMaxCand];   // 16 KB
  __shared__ int hist[kBins];
  __shared__ int wsum[kWaves];
  __shared__ int pick[2];

  const int bg = blockIdx.x;
  const int b = bg / kSparseGroups;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int L = slot_len(p.dp.ctx_lens[b], p.dp.max_blocks);
  const int t = L - 1;
  const int R = t >= 0 ? min(t / kSparseBlock, p.cap8) : 0;   // candidate blocks

  int32_t* out = p.sel_out + (int64_t)bg * kSparseBudget;
  if (R <= kSparseBudget) {
    for (int r = tid; r < R; r += kSelThreads) out[r] = r;
    if (tid == 0) p.nsel_out[bg] = R;
    return;
  }
  const float* scg = p.scores + (int64_t)bg * p.cap8;
  for (int r = tid; r < R; r += kSelThreads) sc[r] = scg[r];
  __syncthreads();

  // Keys relative to the smallest score: key = mono(s) - mono(min) keeps the
  // order and drops the leading bits all scores share (sign, exponent), so
  // the first radix digit already spreads the keys and only as many radix
  // passes run as the spread needs (none when every score is equal).  Equal
  // keys are told apart by block id at the end, lower ids first.
  uint32_t lo_m = 0xFFFFFFFFu, hi_m = 0;
  for (int r = tid; r < R; r += kSelThreads) {
    const uint32_t m = mono_bits(sc[r]);
    lo_m = min(lo_m, m);
    hi_m = max(hi_m, m);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    lo_m = min(lo_m, (uint32_t)__shfl_xor((int)lo_m, off));
    hi_m = max(hi_m, (uint32_t)__shfl_xor((int)hi_m, off));
  }
  if (lane == 0) {
    wsum[wave] = (int)lo_m;
    hist[wave] = (int)hi_m;
  }
  __syncthreads();
  lo_m = 0xFFFFFFFFu;
  hi_m = 0;
#pragma unroll
  for (int w2 = 0; w2 < kWaves; ++w2) {
    lo_m = min(lo_m, (uint32_t)wsum[w2]);
    hi_m = max(hi_m, (uint32_t)hist[w2]);
  }
  __syncthreads();
  const int bits = hi_m > lo_m ? 32 - __builtin_clz(hi_m - lo_m) : 0;
  auto rel_key = [&](int r) { return mono_bits(sc[r]) - lo_m; };
  // Radix select of the 512th largest key T, most significant 11-bit digit
  // first (thread i owns digits 2047 - 4i .. 2044 - 4i of the histogram);
  // afterwards `need` counts the keys equal to T that are taken.
  uint32_t prefix = 0, mask = 0;
  int need = kSparseBudget;
  const int passes = (bits + kDigitBits - 1) / kDigitBits;
  for (int pass = 0; pass < passes; ++pass) {
    const int shift = kDigitBits * (passes - 1 - pass);
    for (int i = tid; i < kBins; i += kSelThreads) hist[i] = 0;
    __syncthreads();
    for (int r = tid; r < R; r += kSelThreads) {
      const uint32_t key = rel_key(r);
      if ((key & mask) == prefix) atomicAdd(&hist[(int)((key >> shift) & (kBins - 1))], 1);
    }
    __syncthreads();
    int cnt[4], own = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      cnt[k] = hist[kBins - 1 - (4 * tid + k)];
      own += cnt[k];
    }
    int before = sel_scan_incl(own, wsum) - own;   // keys with higher digits than this thread's
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (before < need && before + cnt[k] >= need) {
        pick[0] = kBins - 1 - (4 * tid + k);
        pick[1] = need - before;
      }
      before += cnt[k];
    }
    __syncthreads();
    prefix |= (uint32_t)pick[0] << shift;
    mask |= (uint32_t)(kBins - 1) << shift;
    need = pick[1];
    __syncthreads();
  }
  // Every key above T and the `need` lowest-id keys equal to T: exactly
  // 512, written in ascending id order.  One scan carries both counts
  // (above in the low 16 bits, equal in the high; each at most 4096).
  constexpr int kPer = kSparseMaxCand / kSelThreads;
  int mine = 0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int r = tid * kPer + k;
    if (r < R) {
      const uint32_t key = rel_key(r);
      mine += key > prefix ? 1 : (key == prefix ? 1 << 16 : 0);
    }
  }
  const int before = sel_scan_incl(mine, wsum) - mine;
  int eq_before = before >> 16;
  int pos = (before & 0xFFFF) + min(eq_before, need);
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int r = tid * kPer + k;
    if (r < R) {
      const uint32_t key = rel_key(r);
      if (key > prefix) {
        out[pos++] = r;
      } else if (key == prefix) {
        if (eq_before < need) out[pos++] = r;
        ++eq_before;
      }
    }
  }
  if (tid == 0) p.nsel_out[bg] = kSparseBudget;
}

// ---------------------------------------------------------------------------
// 3. Attention over the selected blocks: one workgroup of 4 waves per
// (request, group, split).

// K rows of 384 bytes: XOR with the key's low three bits (inside aligned
// groups of 8 chunks) keeps the K operand reads free of bank conflicts.
__device__ __forceinline__ int swz_k(int key) { return key & 7; }
__device__ __forceinline__ int swz_v(int ch) { return (ch & 7) ^ ((ch >> 3) & 1); }

template <int N>
__device__ __forceinline__ void phase_barrier() {
  wait_vmcnt<N>();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__global__ void __launch_bounds__(256) sparse_attention_kernel(SparseParams sp) {
  const DecodeParams& p = sp.dp;
  __shared__ __attribute__((aligned(1024))) uint8_t ring[kRing * kPhaseBytes];
  __shared__ int ent_blk[kMaxEntries];     // pool block of list entry e
  __shared__ int ent_row[kMaxEntries];     // its first row in that 64-token page
  __shared__ int ent_cnt[kMaxEntries];     // its attended tokens (8, 1..8 for the current block, 0)
  __shared__ float wave_ml[4][kG][2];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15;
  const int q4 = lane >> 4;
  const int bg = blockIdx.y;
  const int b = bg / kSparseGroups;
  const int g = bg - b * kSparseGroups;
  const int split = blockIdx.x;
  const int L = slot_len(p.ctx_lens[b], p.max_blocks);
  const int t = L - 1;
  // List: the selected blocks (clamped to the candidates, so a bad id stays
  // in bounds), then the current block; 64-key tiles of 8 entries.
  const int R = t >= 0 ? t / kSparseBlock : 0;
  const int nsel = L > 0 ? min(max(sp.nsel[bg], 0), min(R, kSparseBudget)) : 0;
  const int n_ent = L > 0 ? nsel + 1 : 0;
  const int n_tiles = (n_ent + 7) / 8;
  const int t_begin = split * p.chunk_tiles;
  const int t_end = min(n_tiles, t_begin + p.chunk_tiles);
  const int head = g * kG + r;

  if (t_begin >= t_end) {
    if (p.splits == 1) {   // empty request: zeros
      for (int ct = wave; ct < kD / 16; ct += 4) {
        const int64_t o = ((int64_t)b * p.hq + head) * kD + ct * 16 + q4 * 4;
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
  const float qk_scale = p.scale * kLog2e;

  const int cur = (t / kSparseBlock) * kSparseBlock;
  const int32_t* selp = sp.sel + (int64_t)bg * kSparseBudget;
  for (int i = threadIdx.x; i < 8 * nt; i += 256) {
    const int e = 8 * t_begin + i;
    int tb = cur, cnt = 0;
    if (e < nsel) {
      tb = kSparseBlock * min(max(selp[e], 0), R - 1);
      cnt = kSparseBlock;
    } else if (e == nsel) {
      cnt = t - cur + 1;
    }
    ent_blk[i] = p.block_table ? pool_block(p.block_table[(int64_t)b * p.max_blocks + tb / kPage], p.num_blocks) : 0;
    ent_row[i] = tb % kPage;
    ent_cnt[i] = cnt;
  }

  // Q fragments: head r of the group, channels 32s + 8q4 .. +7.
  intx4 qf[kD / 32];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(p.q) + ((int64_t)b * p.hq + head) * kD + q4 * 8;
#pragma unroll
    for (int s = 0; s < kD / 32; ++s) qf[s] = *reinterpret_cast<const intx4*>(qp + s * 32);
  }
  wait_vmcnt<0>();   // the copies below are invisible to the compiler's wait bookkeeping
  __syncthreads();

  const uint16_t* kpool = static_cast<const uint16_t*>(p.k) + (int64_t)g * p.k_head_stride;
  const uint16_t* vpool = static_cast<const uint16_t*>(p.v) + (int64_t)g * p.v_head_stride;
  auto issue_phase = [&](int ph_req, uint8_t* dst) {
    const int ph = ph_req < nphase ? ph_req : nphase - 2 + (ph_req & 1);
    const int e0 = 8 * (ph >> 1);
    if ((ph & 1) == 0) {
      // K tile: row j is token ent_row + j % 8 of entry e0 + j / 8.
#pragma unroll
      for (int k = 0; k < kDmaPerWave; ++k) {
        const int i = wave * kDmaPerWave + k;
        const int idx = i * 64 + lane;
        const int row = idx / kChunks;
        const int ch = (idx - row * kChunks) ^ swz_k(row);
        const int e = e0 + (row >> 3);
        dma16_nt(kpool + (int64_t)ent_blk[e] * p.k_block_stride + (ent_row[e] + (row & 7)) * p.k_row_stride + ch * 8,
              dst + i * 1024);
      }
    } else {
      // V^T tile: chunk c of row (channel) ch holds entry e0 + c's 8 keys,
      // the 16 bytes of channel ch in that block's [192][8] V^T sub-block.
#pragma unroll
      for (int k = 0; k < kDmaPerWave; ++k) {
        const int i = wave * kDmaPerWave + k;
        const int row = 8 * i + (lane >> 3);
        const int c = (lane & 7) ^ swz_v(row);
        const int e = e0 + c;
        dma16_nt(vpool + (int64_t)ent_blk[e] * p.v_block_stride + (ent_row[e] >> 3) * (kD * kSparseBlock) +
                  row * kSparseBlock,
              dst + i * 1024);
      }
    }
  };

#pragma unroll
  for (int ph = 0; ph < kRing - 1; ++ph) issue_phase(ph, ring + ph * kPhaseBytes);

  const int my_key = 16 * wave + r;                    // K operand row of this lane
  const int xk = swz_k(my_key);
  const int xv = swz_v(r);

  float m_run = kNegInf;
  float l_run = 0.f;
  floatx4 acc[kD / 16];
#pragma unroll
  for (int ct = 0; ct < kD / 16; ++ct) acc[ct] = floatx4{0.f, 0.f, 0.f, 0.f};
  intx2 pb;

  auto k_phase = [&](const uint8_t* buf, int tile_rel) {
    floatx4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kD / 32; ++s) {
      const int chunk = (4 * s + q4) ^ xk;
      const intx4 a = *reinterpret_cast<const intx4*>(buf + my_key * (2 * kD) + chunk * 16);
      st = mfma_bf16_16x16x32(a, qf[s], st);
    }
    // Keys 16 wave + 4 q4 + i: entry 2 wave + q4 / 2, token (4 q4 + i) % 8.
    const int e = 8 * tile_rel + 2 * wave + (q4 >> 1);
    const int valid = ent_cnt[e] - 4 * (q4 & 1);
    float sv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sv[i] = i < valid ? st[i] * qk_scale : kNegInf;
    float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    mx = wave_max_xor16_32(mx);
    const bool move = mx > m_run + kLazyRescale;
    const float m_new = move ? mx : m_run;
    if (__any(move && m_run != kNegInf)) {
      const float alpha = fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int ct = 0; ct < kD / 16; ++ct) acc[ct] *= alpha;
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

  auto v_phase = [&](const uint8_t* buf, int tile_rel) {
    const int kfirst = 16 * wave + 4 * q4;             // this lane's 4 keys
    const int vvalid = ent_cnt[8 * tile_rel + (kfirst >> 3)] - (kfirst & 7);
    // Rows of unattended keys may hold anything (NaN included): zero them.
    const uint32_t keep0 = ((0 < vvalid) ? 0x0000ffffu : 0u) | ((1 < vvalid) ? 0xffff0000u : 0u);
    const uint32_t keep1 = ((2 < vvalid) ? 0x0000ffffu : 0u) | ((3 < vvalid) ? 0xffff0000u : 0u);
    const int chunk = (kfirst >> 3) ^ xv;
    const int half = (q4 & 1) * 8;
#pragma unroll
    for (int ct = 0; ct < kD / 16; ++ct) {
      intx2 a = *reinterpret_cast<const intx2*>(buf + ct * 2048 + r * 128 + chunk * 16 + half);
      a.x &= keep0;
      a.y &= keep1;
      acc[ct] = mfma_bf16_16x16x16(a, pb, acc[ct]);
    }
  };

  auto step = [&](int ph, int slot) {
    phase_barrier<kAhead * kDmaPerWave>();
    issue_phase(ph + kRing - 1, ring + ((slot + kRing - 1) % kRing) * kPhaseBytes);
    const uint8_t* cur_buf = ring + slot * kPhaseBytes;
    if ((slot & 1) == 0) k_phase(cur_buf, ph >> 1);
    else v_phase(cur_buf, ph >> 1);
  };

  for (int ph = 0; ph < nphase; ph += kRing) {
#pragma unroll
    for (int s = 0; s < kRing; s += 2) {
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
  // [4][kG][kD + 4]: the 16-byte pad per head row spreads the 16 rows a
  // store instruction touches over every bank (a row of kD floats is a whole
  // number of bank rows, which made each store a 16-way conflict).
  constexpr int kOStride = kD + 4;
  float* obuf = reinterpret_cast<float*>(ring);
#pragma unroll
  for (int ct = 0; ct < kD / 16; ++ct)
    *reinterpret_cast<floatx4*>(obuf + ((wave * kG + r) * kOStride + ct * 16 + q4 * 4)) = acc[ct];
  __syncthreads();

  // Thread t: head t / 16, channels 4 (t % 16) + 64 k.
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
  for (int c4 = (threadIdx.x & 15) * 4; c4 < kD; c4 += 64) {
    floatx4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < 4; ++w) o += wgt[w] * *reinterpret_cast<const floatx4*>(obuf + (w * kG + h) * kOStride + c4);
    if (p.splits == 1) {
      const floatx4 v = o * (1.f / lsum);
      const int64_t off = ((int64_t)b * p.hq + ghead) * kD + c4;
      if (p.out_f32)
        *reinterpret_cast<floatx4*>(static_cast<float*>(p.out) + off) = v;
      else
        *reinterpret_cast<intx2*>(static_cast<uint16_t*>(p.out) + off) =
            intx2{(int)pack_bf16x2(v.x, v.y), (int)pack_bf16x2(v.z, v.w)};
    } else {
      *reinterpret_cast<floatx4*>(p.part_o + prow * kD + c4) = o;
    }
  }
  if (p.splits > 1 && (threadIdx.x & 15) == 0)
    *reinterpret_cast<floatx2*>(p.part_ml + prow * 2) = floatx2{M, lsum};
}

}  // namespace

hipError_t launch_sparse_summary(const SparseParams& p, hipStream_t stream) {
  // The last n tokens complete at most ceil(n / 8) blocks.
  const int new_blocks = (p.new_tokens + kSparseBlock - 1) / kSparseBlock;
  const int blocks = (p.new_tokens > 0 && new_blocks < p.cap8) ? new_blocks : p.cap8;
  const dim3 grid((unsigned)((blocks + 3) / 4), (unsigned)p.dp.batch);
  hipLaunchKernelGGL(sparse_summary_kernel, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_sparse_select(const SparseParams& p, hipStream_t stream) {
  if (p.cap8 > kSparseMaxCand || !p.scores) return hipErrorInvalidValue;
  hipLaunchKernelGGL(sparse_score_kernel, dim3((unsigned)((p.cap8 + kScoreChunk - 1) / kScoreChunk), (unsigned)p.dp.batch),
                     dim3(256), 0, stream, p);
  hipLaunchKernelGGL(sparse_select_kernel, dim3((unsigned)(p.dp.batch * kSparseGroups)), dim3(kSelThreads), 0,
                     stream, p);
  return hipGetLastError();
}

hipError_t launch_sparse_attention(const SparseParams& p, hipStream_t stream) {
  if (p.dp.hkv != kSparseGroups || p.dp.hq != kSparseGroups * kG || p.dp.chunk_tiles <= 0 ||
      p.dp.chunk_tiles * p.dp.splits < kSparseMaxTiles)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(sparse_attention_kernel, dim3((unsigned)p.dp.splits, (unsigned)(p.dp.batch * kSparseGroups)),
                     dim3(256), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.dp.splits == 1) return e;
  return launch_combine(p.dp, kG, kD, stream);
}

}  // namespace mfa

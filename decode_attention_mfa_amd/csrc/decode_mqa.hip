// MQA decode attention on gfx950: 64 query heads share one K head and one V
// head of width 256 ("Step-3 is Large yet Affordable", section 2 and
// Table 1).  Hand-written split-K flash decoding over a bf16 cache.
//
// Workgroup = 8 waves (two per SIMD) = one (slot, KV group, split).  Wave w
// owns heads 16*(w%4) .. +15 and key half w/4 (keys 32*(w/4) .. +31 of every
// 64-key tile).  The split's keys stream through a ring of three 32 KB LDS
// slots, one "phase" per slot:
//   phase 2t   : K tile   [64 keys][256 ch]  bf16, rows 512 B
//   phase 2t+1 : V^T tile [256 ch][64 keys]  bf16, rows 128 B
// Each thread stages its share of a phase (four 16-byte non-temporal loads,
// fully coalesced) in registers two phases ahead and writes it into the
// swizzled slot one phase ahead, so 64 KB per CU is in flight while the
// waves compute.  The K/V bytes of a tile reach HBM->LDS once per workgroup
// and are read from LDS by the four head groups.
//
// Products are transposed so the softmax statistics stay in lanes:
//   S^T[key, head] = K[key, :] . Q^T[:, head]       (MFMA A = K rows from LDS,
//                                                    B = Q fragments in VGPRs)
//   O^T[ch, head] += V^T[ch, key] . P^T[key, head]  (A = V^T from LDS, B = P)
// With MFMA row r of S^T tile j mapped to key 8(r/4) + 4j + r%4 of the wave's
// half, the S^T values a lane holds (4 keys x 2 tiles of one head) are exactly
// the B operand of the PV product: no lane shuffle between the products.  Each
// lane owns one head: the row max is a 4-lane reduction per tile, the row sum
// is reduced once at the end, and the two key halves of a head group are
// merged through LDS (log-sum-exp) before the output or split partial is
// written.
//
// Online softmax in the log2 domain, fp32 state.  The running max only moves
// when a tile's max exceeds it by more than kLazyRescale (2^8 headroom for
// p = 2^(s - m) in fp32/bf16), so O is rescaled a handful of times per split;
// the algebra is unchanged.  P is rounded to bf16 for the PV operand.
#include <type_traits>

#include "device_common.h"
#include "kernel_params.h"

namespace mfa {
namespace {

constexpr int kD = 256;
constexpr int kG = 64;
constexpr int kThreads = 512;
constexpr int kPhaseBytes = 32768;   // one bf16 K or V^T tile in LDS
constexpr int kRing = 3;
constexpr int kMaxChunkTiles = 2048;   // block ids cached per workgroup
constexpr float kLazyRescale = 8.f;    // log2 headroom before the max moves

// LDS swizzles (XOR on the 16-byte chunk index) so that the 16 lanes reading
// one MFMA operand hit 16 distinct bank quads (and any 8 consecutive lanes 8).
__device__ __forceinline__ int swz_k(int key) { return (key & 3) | (((key >> 3) & 3) << 2); }
__device__ __forceinline__ int swz_v(int ch) { return (ch & 7) ^ ((ch >> 3) & 1); }

// Workgroup barrier ordering LDS only: release/acquire fences scoped to the
// workgroup and to the local (LDS) address space, around s_barrier.  The
// global loads still in flight only target registers, so unlike
// __syncthreads (whose fence covers global memory too) this does not wait for
// them.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Converts 16 E4M3 codes (one 16-byte chunk) to two 16-byte bf16 chunks.
// Every E4M3FN value is a bf16 value, and the conversion scale is 1, so this
// is exact (NaN codes stay NaN).
template <bool kUpper>
__device__ __forceinline__ int e4m3x2_to_bf16x2(int w) {   // codes of bytes 0,1 (or 2,3)
  return __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, kUpper));
}
__device__ __forceinline__ void e4m3x16_to_bf16(intx4 raw, intx4& lo, intx4& hi) {
  lo = intx4{e4m3x2_to_bf16x2<false>(raw.x), e4m3x2_to_bf16x2<true>(raw.x),
             e4m3x2_to_bf16x2<false>(raw.y), e4m3x2_to_bf16x2<true>(raw.y)};
  hi = intx4{e4m3x2_to_bf16x2<false>(raw.z), e4m3x2_to_bf16x2<true>(raw.z),
             e4m3x2_to_bf16x2<false>(raw.w), e4m3x2_to_bf16x2<true>(raw.w)};
}

// kDense: no window (the split's first page is known before the length).
// kFp8: the cache holds OCP E4M3 codes with one fp32 scale per KV head; tiles
// are converted to bf16 as they are written to LDS, and the scales are
// applied to the logits (k) and to the normalised output (v).
template <bool kDense, bool kFp8>
__global__ void __launch_bounds__(kThreads) mqa_decode_kernel(DecodeParams p) {
  constexpr int kElem = kFp8 ? 1 : 2;                 // bytes per cached element
  constexpr int kPerThread = kPhaseBytes * kElem / 2 / 16 / kThreads;   // 16-byte loads per phase
  // Register stages: phases in flight while a phase is computed (3 bf16
  // phases = 96 KB of cache data per CU; 4 FP8 phases = 64 KB, as many as
  // the conversion temporaries leave registers for).
  constexpr int kStages = kFp8 ? 4 : 3;
  constexpr int kUnroll = kStages == 3 ? 6 : 4;    // steps per unrolled group: kStages | kUnroll, 2 | kUnroll
  constexpr int kFirstTiles = (kStages + 1) / 2;   // tiles the start-up loads touch
  __shared__ __attribute__((aligned(1024))) uint8_t ring[kRing * kPhaseBytes];
  __shared__ int blk_ids[kMaxChunkTiles];
  __shared__ float half_ml[4][16][2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hg = wave & 3;     // head group
  const int kh = wave >> 2;    // key half
  const int r = lane & 15;     // MFMA row / column index of this lane
  const int q4 = lane >> 4;    // K-group of this lane
  const int bg = blockIdx.y;
  const int b = bg / p.hkv;
  const int g = bg - b * p.hkv;
  const int split = blockIdx.x;
  const int head = g * kG + hg * 16 + r;    // this lane's query head
  const float qk_scale = p.scale * kLog2e * (kFp8 ? p.k_scale[g] : 1.f);
  const int32_t* trow = p.block_table ? p.block_table + (int64_t)b * p.max_blocks : nullptr;

  // Dense attention: the split's first page (split * chunk) does not depend
  // on the slot length, so its block id is fetched together with the length
  // and its K/V loads are in flight before the length is known (a split that
  // turns out to be past the end simply drops them).  With a window the
  // first page moves with the length.
  int t_begin = kDense ? min(split * p.chunk_tiles, p.max_blocks - 1) : 0;
  int blk_first[kFirstTiles];
#pragma unroll
  for (int i = 0; i < kFirstTiles; ++i)
    blk_first[i] = (kDense && trow) ? trow[min(t_begin + i, p.max_blocks - 1)] : 0;
  const int L = slot_len(p.ctx_lens[b], p.max_blocks);
  int nphase = 0;   // two phases (K, V) per tile of this split; set once L is known

  const char* kpool = static_cast<const char*>(p.k);
  const char* vpool = static_cast<const char*>(p.v);
  // This thread's 16-byte chunks of a phase, idx = tid + 512 k.
  //  bf16: rows (tid >> 5) + 16k of a K tile (32 chunks per row), rows
  //        (tid >> 3) + 64k of a V^T tile (8 chunks per row).  The V^T
  //        swizzle repeats every 16 rows, the K swizzle every 32: odd k flip
  //        bit 3 of the K chunk index.
  //  FP8:  rows (tid >> 4) + 32k of a K tile (16 code chunks per row) and
  //        rows (tid >> 2) + 128k of a V^T tile (4 per row); code chunk c
  //        becomes bf16 chunks 2c and 2c + 1 of the same LDS row, and the
  //        row steps keep the swizzle.
  const int krow0 = kFp8 ? tid >> 4 : tid >> 5, kc = kFp8 ? tid & 15 : tid & 31;
  const int vrow0 = kFp8 ? tid >> 2 : tid >> 3, vc = kFp8 ? tid & 3 : tid & 7;
  const int64_t kgoff0 = ((int64_t)krow0 * p.k_row_stride + kc * (16 / kElem)) * kElem;
  const int64_t vgoff0 = ((int64_t)vrow0 * p.v_row_stride + vc * (16 / kElem)) * kElem;
  const int64_t kgstep = (int64_t)(kFp8 ? 32 : 16) * p.k_row_stride * kElem;
  const int64_t vgstep = (int64_t)(kFp8 ? 128 : 64) * p.v_row_stride * kElem;
  const uint32_t klds_even = krow0 * 512 + ((kc ^ swz_k(krow0)) << 4);
  const uint32_t klds_odd = krow0 * 512 + ((kc ^ swz_k(krow0 + 16)) << 4);
  const uint32_t vlds0 = vrow0 * 128 + ((vc ^ swz_v(vrow0)) << 4);
  const uint32_t k8_lo = krow0 * 512 + (((2 * kc) ^ swz_k(krow0)) << 4);
  const uint32_t k8_hi = krow0 * 512 + (((2 * kc + 1) ^ swz_k(krow0)) << 4);
  const uint32_t v8_lo = vrow0 * 128 + (((2 * vc) ^ swz_v(vrow0)) << 4);
  const uint32_t v8_hi = vrow0 * 128 + (((2 * vc + 1) ^ swz_v(vrow0)) << 4);

  // Register-staged loads of one phase (nothing past the end of the split).
  // The first two phases take their block ids straight from the table, so
  // they are in flight before the id cache in LDS is filled.
  auto load_phase = [&](int ph, intx4* st, int blk) {
    const int tile = min(t_begin + (ph >> 1), p.max_blocks - 1);   // start-up loads run ahead
    if ((ph & 1) == 0) {
      const char* base =
          kpool + ((p.block_table ? (int64_t)blk : (int64_t)b * p.max_blocks + tile) * p.k_block_stride +
                   (int64_t)g * p.k_head_stride) * kElem + kgoff0;
#pragma unroll
      for (int k = 0; k < kPerThread; ++k)
        st[k] = __builtin_nontemporal_load(reinterpret_cast<const intx4*>(base + k * kgstep));
    } else {
      const char* base =
          vpool + ((p.block_table ? (int64_t)blk * p.v_block_stride
                                  : (int64_t)b * p.v_seq_stride + (int64_t)tile * kPage) +
                   (int64_t)g * p.v_head_stride) * kElem + vgoff0;
#pragma unroll
      for (int k = 0; k < kPerThread; ++k)
        st[k] = __builtin_nontemporal_load(reinterpret_cast<const intx4*>(base + k * vgstep));
    }
  };
  auto load_phase_cached = [&](int ph, intx4* st) {
    load_phase(ph, st, p.block_table ? readfirstlane(blk_ids[ph >> 1]) : 0);
  };

  // Publishing a V^T phase also zeroes the keys past the slot end (their
  // cache rows may hold anything, NaN included), so the PV product never
  // multiplies garbage by a zero probability.  A bf16 chunk holds 8
  // consecutive keys of one channel (vc*8 .. vc*8+7; FP8: 16 keys vc*16 ..).
  auto keep_mask = [&](int valid, uint32_t* keep) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      keep[e] = ((2 * e < valid) ? 0x0000ffffu : 0u) | ((2 * e + 1 < valid) ? 0xffff0000u : 0u);
  };
  auto apply = [](intx4 v, const uint32_t* keep) {
    v.x &= keep[0];
    v.y &= keep[1];
    v.z &= keep[2];
    v.w &= keep[3];
    return v;
  };
  auto store_phase = [&](int ph, const intx4* st) {
    if (ph >= nphase) return;
    uint8_t* dst = ring + (ph % kRing) * kPhaseBytes;
    const int key_rel = L - (t_begin + (ph >> 1)) * kPage;   // keys of this tile < L
    if (kFp8) {
      if (ph & 1) {
        uint32_t keep_lo[4], keep_hi[4];
        keep_mask(key_rel - vc * 16, keep_lo);
        keep_mask(key_rel - vc * 16 - 8, keep_hi);
#pragma unroll
        for (int k = 0; k < kPerThread; ++k) {
          intx4 lo, hi;
          e4m3x16_to_bf16(st[k], lo, hi);
          *reinterpret_cast<intx4*>(dst + v8_lo + k * 128 * 128) = apply(lo, keep_lo);
          *reinterpret_cast<intx4*>(dst + v8_hi + k * 128 * 128) = apply(hi, keep_hi);
        }
      } else {
#pragma unroll
        for (int k = 0; k < kPerThread; ++k) {
          intx4 lo, hi;
          e4m3x16_to_bf16(st[k], lo, hi);
          *reinterpret_cast<intx4*>(dst + k8_lo + k * 32 * 512) = lo;
          *reinterpret_cast<intx4*>(dst + k8_hi + k * 32 * 512) = hi;
        }
      }
    } else if (ph & 1) {
      uint32_t keep[4];
      keep_mask(key_rel - vc * 8, keep);
#pragma unroll
      for (int k = 0; k < kPerThread; ++k)
        *reinterpret_cast<intx4*>(dst + vlds0 + k * 64 * 128) = apply(st[k], keep);
    } else {
#pragma unroll
      for (int k = 0; k < kPerThread; ++k) {
        const uint32_t base_off = (k & 1) ? klds_odd : klds_even;
        *reinterpret_cast<intx4*>(dst + base_off + k * 16 * 512) = st[k];
      }
    }
  };

  intx4 stage[kStages][kPerThread];
  // The first kStages phases, block ids straight from the table (tiles past
  // the split's end are clamped into the table row and never published).
  auto load_first = [&]() {
#pragma unroll
    for (int ph = 0; ph < kStages; ++ph)
      load_phase(ph, stage[ph], pool_block(readfirstlane(blk_first[ph >> 1]), p.num_blocks));
  };
  if (kDense) load_first();

  const int lo = (!kDense && L > p.window) ? L - p.window : 0;
  int n_tiles = 0, t_lo = 0;
  if (L > 0) {
    t_lo = lo / kPage;
    n_tiles = (L - 1) / kPage - t_lo + 1;
  }
  if (!kDense) t_begin = t_lo + split * p.chunk_tiles;
  const int t_end = min(t_lo + n_tiles, t_begin + p.chunk_tiles);

  if (t_begin >= t_end || (kDense && split * p.chunk_tiles >= p.max_blocks)) {
    if (kh == 0) {
      if (p.splits == 1) {   // empty slot: zeros
        for (int ct = 0; ct < kD / 16; ++ct) {
          const int64_t o = ((int64_t)b * p.hq + head) * kD + ct * 16 + q4 * 4;
          if (p.out_f32)
            *reinterpret_cast<floatx4*>(static_cast<float*>(p.out) + o) = floatx4{0.f, 0.f, 0.f, 0.f};
          else
            *reinterpret_cast<intx2*>(static_cast<uint16_t*>(p.out) + o) = intx2{0, 0};
        }
      } else if (q4 == 0) {  // no keys in this split: an empty partial for the merge
        const int64_t row = ((int64_t)bg * p.splits + split) * kG + hg * 16 + r;
        *reinterpret_cast<floatx2*>(p.part_ml + row * 2) = floatx2{kNegInf, 0.f};
      }
    }
    return;
  }
  const int nt = t_end - t_begin;
  nphase = 2 * nt;

  // Start-up order: the first kStages phases are in flight (dense) or go
  // first, then the block-id cache (rows t_begin .. t_end-1 of the table),
  // then Q; only LDS is fenced before the loop.  (Loads are issued
  // unconditionally, indices clamped: the compiler's wait counts stay exact
  // only when every path issues the same loads.)
  if (!kDense) {
#pragma unroll
    for (int i = 0; i < kFirstTiles; ++i)
      blk_first[i] = trow ? trow[min(t_begin + i, p.max_blocks - 1)] : 0;
    load_first();
  }
  const int32_t* btab = trow ? trow + t_begin : static_cast<const int32_t*>(p.ctx_lens);
  int blk_cache[(kMaxChunkTiles + kThreads - 1) / kThreads];
#pragma unroll
  for (int k = 0; k < (kMaxChunkTiles + kThreads - 1) / kThreads; ++k)
    blk_cache[k] = btab[trow ? min(tid + k * kThreads, nt - 1) : 0];
  // Q fragments (B operand of S^T): this lane's head, channels 32s + 8q4 .. +7.
  intx4 qf[kD / 32];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(p.q) + ((int64_t)b * p.hq + head) * kD + q4 * 8;
#pragma unroll
    for (int s = 0; s < kD / 32; ++s) qf[s] = *reinterpret_cast<const intx4*>(qp + s * 32);
  }
#pragma unroll
  for (int k = 0; k < (kMaxChunkTiles + kThreads - 1) / kThreads; ++k) {
    const int i = tid + k * kThreads;
    if (i < nt) blk_ids[i] = pool_block(blk_cache[k], p.num_blocks);
  }
  store_phase(0, stage[0]);
  lds_barrier();   // block ids and phase 0 visible
  // Phase kStages into the freed stage (clamped to the last tile, same K/V
  // parity, when the split is shorter; such a copy is never published).
  load_phase_cached(min(kStages, nphase - 2 + (kStages & 1)), stage[0]);

  // K operand row of S^T tile j: key = 32kh + 8(r/4) + 4j + r%4; its swizzle
  // does not depend on j (bit 2 of the key is not used).
  const int key_lane = 32 * kh + 8 * (r >> 2) + (r & 3);
  const int xk = swz_k(key_lane);
  const int xv = swz_v(r);

  float m_run = kNegInf;
  float l_run = 0.f;
  floatx4 acc[kD / 16];
#pragma unroll
  for (int ct = 0; ct < kD / 16; ++ct) acc[ct] = floatx4{0.f, 0.f, 0.f, 0.f};
  intx4 pb;

  auto k_phase = [&](const uint8_t* buf, int key0) {
    floatx4 st[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int s = 0; s < kD / 32; ++s) {
      const int chunk = (4 * s + q4) ^ xk;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const intx4 a = *reinterpret_cast<const intx4*>(buf + (key_lane + 4 * j) * 512 + chunk * 16);
        st[j] = mfma_bf16_16x16x32(a, qf[s], st[j]);
      }
    }
    // This lane's keys are key0 + 32kh + 8q4 + e, e = 4j + i; those in
    // [lo, L) are attended.  Interior tiles have e_lo <= 0 and e_hi >= 8.
    const int ebase = key0 + 32 * kh + 8 * q4;
    const int e_lo = lo - ebase, e_hi = L - ebase;
    float sv[2][4];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = 4 * j + i;
        const float x = st[j][i] * qk_scale;
        sv[j][i] = (e >= e_lo && e < e_hi) ? x : kNegInf;
      }
    float mx = fmaxf(fmaxf(fmaxf(sv[0][0], sv[0][1]), fmaxf(sv[0][2], sv[0][3])),
                     fmaxf(fmaxf(sv[1][0], sv[1][1]), fmaxf(sv[1][2], sv[1][3])));
    mx = wave_max_xor16_32(mx);
    // Lazy max: keep the old reference unless this tile exceeds it by > 2^8.
    // (A half-tile can be fully masked: mx = -inf and nothing moves.)
    const bool move = mx > m_run + kLazyRescale;
    const float m_new = move ? mx : m_run;
    if (__any(move && m_run != kNegInf)) {
      const float alpha = fast_exp2(m_run - m_new);   // 1 where the max stays
      l_run *= alpha;
#pragma unroll
      for (int ct = 0; ct < kD / 16; ++ct) acc[ct] *= alpha;
    }
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sv[j][i] = m_new == kNegInf ? 0.f : fast_exp2(sv[j][i] - m_new);
        psum += sv[j][i];
      }
    l_run += psum;
    // P^T B operand (keys 8q4 .. 8q4+7 of the half).
    pb = intx4{(int)pack_bf16x2(sv[0][0], sv[0][1]), (int)pack_bf16x2(sv[0][2], sv[0][3]),
               (int)pack_bf16x2(sv[1][0], sv[1][1]), (int)pack_bf16x2(sv[1][2], sv[1][3])};
  };

  auto v_phase = [&](const uint8_t* buf) {
    const int chunk = (4 * kh + q4) ^ xv;
#pragma unroll
    for (int ct = 0; ct < kD / 16; ++ct) {
      const intx4 a = *reinterpret_cast<const intx4*>(buf + ct * 2048 + r * 128 + chunk * 16);
      acc[ct] = mfma_bf16_16x16x32(a, pb, acc[ct]);
    }
  };

  // Step ph: publish phase ph+1 (loaded kStages steps ago) into its slot,
  // start loading phase ph+1+kStages into the freed registers, barrier,
  // compute phase ph.  Slot ph+1 last held phase ph-2, finished by every wave
  // before the barrier of step ph-1.  Phase q lives in stage q % kStages;
  // steps are unrolled kUnroll at a time (a multiple of kStages and of the
  // K/V period), so every stage index is a constant.
  auto step = [&](auto ic, int ph, bool more) {
    constexpr int I = decltype(ic)::value;        // ph % kUnroll
    constexpr int st = (I + 1) % kStages;
    store_phase(ph + 1, stage[st]);
    if (more) load_phase_cached(ph + 1 + kStages, stage[st]);
    lds_barrier();
    if ((I & 1) == 0)
      k_phase(ring + (ph % kRing) * kPhaseBytes, (t_begin + (ph >> 1)) * kPage);
    else
      v_phase(ring + (ph % kRing) * kPhaseBytes);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using I4 = std::integral_constant<int, 4>;
  using I5 = std::integral_constant<int, 5>;
  // Main loop: every load it issues is in range, so the issue pattern (and
  // the compiler's wait counts) is the same in every iteration.
  int ph = 0;
  for (; ph + kUnroll + kStages < nphase; ph += kUnroll) {
    step(I0{}, ph, true);
    step(I1{}, ph + 1, true);
    step(I2{}, ph + 2, true);
    step(I3{}, ph + 3, true);
    if constexpr (kUnroll == 6) {
      step(I4{}, ph + 4, true);
      step(I5{}, ph + 5, true);
    }
  }
  // Tail: the last tiles (loads only while in range).
  for (; ph < nphase; ph += kUnroll) {
    step(I0{}, ph, ph + 1 + kStages < nphase);
    step(I1{}, ph + 1, ph + 2 + kStages < nphase);
    if (ph + 2 >= nphase) break;
    step(I2{}, ph + 2, ph + 3 + kStages < nphase);
    step(I3{}, ph + 3, ph + 4 + kStages < nphase);
    if constexpr (kUnroll == 6) {
      if (ph + 4 >= nphase) break;
      step(I4{}, ph + 4, ph + 5 + kStages < nphase);
      step(I5{}, ph + 5, ph + 6 + kStages < nphase);
    }
  }

  // ---- merge the two key halves of each head group ----
  lds_barrier();   // every wave is done with the ring
  const float l_half = wave_sum_xor16_32(l_run);
  float* obuf = reinterpret_cast<float*>(ring);   // [4 head groups][16 heads][256]
  if (kh == 1) {
    if (q4 == 0) {
      half_ml[hg][r][0] = m_run;
      half_ml[hg][r][1] = l_half;
    }
#pragma unroll
    for (int ct = 0; ct < kD / 16; ++ct)
      *reinterpret_cast<floatx4*>(obuf + (hg * 16 + r) * kD + ct * 16 + q4 * 4) = acc[ct];
  }
  lds_barrier();
  if (kh == 1) return;
  const float m1 = half_ml[hg][r][0], l1 = half_ml[hg][r][1];
  const float M = fmaxf(m_run, m1);
  const float w0 = m_run == kNegInf ? 0.f : fast_exp2(m_run - M);
  const float w1 = m1 == kNegInf ? 0.f : fast_exp2(m1 - M);
  const float l_tot = w0 * l_half + w1 * l1;
#pragma unroll
  for (int ct = 0; ct < kD / 16; ++ct)
    acc[ct] = w0 * acc[ct] + w1 * *reinterpret_cast<const floatx4*>(obuf + (hg * 16 + r) * kD + ct * 16 + q4 * 4);

  if (p.splits == 1) {
    const float inv = (kFp8 ? p.v_scale[g] : 1.f) / l_tot;
#pragma unroll
    for (int ct = 0; ct < kD / 16; ++ct) {
      const int64_t o = ((int64_t)b * p.hq + head) * kD + ct * 16 + q4 * 4;
      const floatx4 v = acc[ct] * inv;
      if (p.out_f32)
        *reinterpret_cast<floatx4*>(static_cast<float*>(p.out) + o) = v;
      else
        *reinterpret_cast<intx2*>(static_cast<uint16_t*>(p.out) + o) =
            intx2{(int)pack_bf16x2(v.x, v.y), (int)pack_bf16x2(v.z, v.w)};
    }
  } else {
    const int64_t row = ((int64_t)bg * p.splits + split) * kG + hg * 16 + r;
#pragma unroll
    for (int ct = 0; ct < kD / 16; ++ct)
      *reinterpret_cast<floatx4*>(p.part_o + row * kD + ct * 16 + q4 * 4) = acc[ct];
    if (q4 == 0) *reinterpret_cast<floatx2*>(p.part_ml + row * 2) = floatx2{M, l_tot};
  }
}

}  // namespace

hipError_t launch_mqa(const DecodeParams& p, bool fp8, hipStream_t stream) {
  dim3 grid(p.splits, p.batch * p.hkv);
  const bool dense = p.window == 0;
  if (fp8) {
    if (dense)
      hipLaunchKernelGGL((mqa_decode_kernel<true, true>), grid, dim3(kThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((mqa_decode_kernel<false, true>), grid, dim3(kThreads), 0, stream, p);
  } else {
    if (dense)
      hipLaunchKernelGGL((mqa_decode_kernel<true, false>), grid, dim3(kThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((mqa_decode_kernel<false, false>), grid, dim3(kThreads), 0, stream, p);
  }
  return hipGetLastError();
}

int mqa_max_chunk_tiles() { return kMaxChunkTiles; }

}  // namespace mfa

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
#include "device_common.h"
#include "kernel_params.h"

namespace mfa {
namespace {

constexpr int kD = 256;
constexpr int kG = 64;
constexpr int kThreads = 512;
constexpr int kPhaseBytes = 32768;
constexpr int kRing = 3;
constexpr int kPerThread = kPhaseBytes / 16 / kThreads;   // 16-byte chunks per thread per phase
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

template <bool kDense>
__global__ void __launch_bounds__(kThreads) mqa_decode_bf16_kernel(DecodeParams p) {
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
  const float qk_scale = p.scale * kLog2e;   // bf16 cache: no dequantisation scales
  const int32_t* trow = p.block_table ? p.block_table + (int64_t)b * p.max_blocks : nullptr;

  // Dense attention: the split's first page (split * chunk) does not depend
  // on the slot length, so its block id is fetched together with the length
  // and its K/V loads are in flight before the length is known (a split that
  // turns out to be past the end simply drops them).  With a window the
  // first page moves with the length.
  int t_begin = kDense ? min(split * p.chunk_tiles, p.max_blocks - 1) : 0;
  const int blk_spec = (kDense && trow) ? trow[t_begin] : 0;
  const int L = slot_len(p.ctx_lens[b], p.max_blocks);
  int nphase = 0;   // two phases (K, V) per tile of this split; set once L is known

  const uint16_t* kpool = static_cast<const uint16_t*>(p.k);
  const uint16_t* vpool = static_cast<const uint16_t*>(p.v);
  // This thread's chunks of a phase: idx = tid + 512 k, i.e. rows
  // (tid >> 5) + 16k of a K tile (32 chunks per row) and rows (tid >> 3) + 64k
  // of a V^T tile (8 chunks per row).  The V^T swizzle repeats every 16 rows,
  // the K swizzle every 32: odd k flip bit 3 of the K chunk index.
  const int krow0 = tid >> 5, kc = tid & 31;
  const int vrow0 = tid >> 3, vc = tid & 7;
  const int32_t kgoff0 = krow0 * (int32_t)p.k_row_stride + kc * 8;
  const int32_t vgoff0 = vrow0 * (int32_t)p.v_row_stride + vc * 8;
  const uint32_t klds_even = krow0 * 512 + ((kc ^ swz_k(krow0)) << 4);
  const uint32_t klds_odd = krow0 * 512 + ((kc ^ swz_k(krow0 + 16)) << 4);
  const uint32_t vlds0 = vrow0 * 128 + ((vc ^ swz_v(vrow0)) << 4);

  // Register-staged loads of one phase (nothing past the end of the split).
  // The first two phases take their block ids straight from the table, so
  // they are in flight before the id cache in LDS is filled.
  auto load_phase = [&](int ph, intx4* st, int blk) {
    const int tile = t_begin + (ph >> 1);
    if ((ph & 1) == 0) {
      const uint16_t* base =
          (p.block_table ? kpool + (int64_t)blk * p.k_block_stride
                         : kpool + ((int64_t)b * p.max_blocks + tile) * p.k_block_stride) +
          (int64_t)g * p.k_head_stride;
#pragma unroll
      for (int k = 0; k < kPerThread; ++k)
        st[k] = __builtin_nontemporal_load(
            reinterpret_cast<const intx4*>(base + kgoff0 + k * 16 * (int32_t)p.k_row_stride));
    } else {
      const uint16_t* base =
          (p.block_table ? vpool + (int64_t)blk * p.v_block_stride
                         : vpool + (int64_t)b * p.v_seq_stride + (int64_t)tile * kPage) +
          (int64_t)g * p.v_head_stride;
#pragma unroll
      for (int k = 0; k < kPerThread; ++k)
        st[k] = __builtin_nontemporal_load(
            reinterpret_cast<const intx4*>(base + vgoff0 + k * 64 * (int32_t)p.v_row_stride));
    }
  };
  auto load_phase_cached = [&](int ph, intx4* st) {
    load_phase(ph, st, p.block_table ? readfirstlane(blk_ids[ph >> 1]) : 0);
  };

  // Publishing a V^T phase also zeroes the keys past the slot end (their
  // cache rows may hold anything, NaN included), so the PV product never
  // multiplies garbage by a zero probability.  A chunk holds 8 consecutive
  // keys vc*8 .. vc*8+7 of one channel.
  auto store_phase = [&](int ph, const intx4* st) {
    if (ph >= nphase) return;
    uint8_t* dst = ring + (ph % kRing) * kPhaseBytes;
    if (ph & 1) {
      const int valid = L - (t_begin + (ph >> 1)) * kPage - vc * 8;   // keys of this chunk < L
      uint32_t keep[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        keep[e] = ((2 * e < valid) ? 0x0000ffffu : 0u) | ((2 * e + 1 < valid) ? 0xffff0000u : 0u);
#pragma unroll
      for (int k = 0; k < kPerThread; ++k) {
        intx4 v = st[k];
        v.x &= keep[0];
        v.y &= keep[1];
        v.z &= keep[2];
        v.w &= keep[3];
        *reinterpret_cast<intx4*>(dst + vlds0 + k * 64 * 128) = v;
      }
    } else {
#pragma unroll
      for (int k = 0; k < kPerThread; ++k) {
        const uint32_t base_off = (k & 1) ? klds_odd : klds_even;
        *reinterpret_cast<intx4*>(dst + base_off + k * 16 * 512) = st[k];
      }
    }
  };

  intx4 stage0[kPerThread], stage1[kPerThread];
  auto load_first = [&](int blk) {
    const int blk0 = pool_block(readfirstlane(blk), p.num_blocks);
    load_phase(0, stage0, blk0);
    load_phase(1, stage1, blk0);
  };
  if (kDense) load_first(blk_spec);

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

  // Start-up order: phases 0 and 1 are in flight (dense) or go first, then the
  // block-id cache (rows t_begin .. t_end-1 of the table), then Q; only LDS
  // is fenced before the loop.  (Loads are issued unconditionally, indices
  // clamped: the compiler's wait counts stay exact only when every path
  // issues the same loads.)
  if (!kDense) load_first(trow ? trow[t_begin] : 0);
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
  store_phase(0, stage0);
  lds_barrier();   // block ids and phase 0 visible
  load_phase_cached(min(2, nphase - 2), stage0);   // (a one-tile split re-loads phase 0; unused)

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

  // Step ph: publish phase ph+1 (staged two steps ago) into its slot, start
  // loading phase ph+3 into the freed registers, barrier, compute phase ph.
  // Slot ph+1 last held phase ph-2, finished by every wave before the barrier
  // of step ph-1.  Even steps are K phases, odd steps V phases.
  auto k_step = [&](int ph, bool more) {
    store_phase(ph + 1, stage1);              // phase ph+1 was staged in stage1
    if (more) load_phase_cached(ph + 3, stage1);
    lds_barrier();
    k_phase(ring + (ph % kRing) * kPhaseBytes, (t_begin + (ph >> 1)) * kPage);
  };
  auto v_step = [&](int ph, bool more) {
    store_phase(ph + 1, stage0);              // phase ph+1 (next K) was staged in stage0
    if (more) load_phase_cached(ph + 3, stage0);
    lds_barrier();
    v_phase(ring + (ph % kRing) * kPhaseBytes);
  };
  // Main loop: every load it issues is in range, so the issue pattern (and
  // the compiler's wait counts) is the same in every iteration.
  int ph = 0;
  for (; ph + 4 < nphase; ph += 2) {
    k_step(ph, true);
    v_step(ph + 1, true);
  }
  // Tail: the last one or two tiles.
  for (; ph < nphase; ph += 2) {
    k_step(ph, ph + 3 < nphase);
    v_step(ph + 1, ph + 4 < nphase);
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
    const float inv = 1.f / l_tot;
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

hipError_t launch_mqa_bf16(const DecodeParams& p, hipStream_t stream) {
  dim3 grid(p.splits, p.batch * p.hkv);
  if (p.window == 0)
    hipLaunchKernelGGL(mqa_decode_bf16_kernel<true>, grid, dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(mqa_decode_bf16_kernel<false>, grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

int mqa_max_chunk_tiles() { return kMaxChunkTiles; }

}  // namespace mfa

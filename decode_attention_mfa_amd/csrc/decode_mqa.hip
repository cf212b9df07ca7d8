// MQA decode attention on gfx950: 64 query heads share one K head and one V
// head of width 256 ("Step-3 is Large yet Affordable", section 2 and
// Table 1).  Hand-written split-K flash decoding over a bf16 or FP8 cache.
//
// Workgroup = 8 waves (two per SIMD) = one (slot, KV group, split), split by
// role:
//   waves 4..7 (loaders)  stream the split's keys HBM -> registers -> LDS in
//                          32 KB "phases", kStages phases ahead (16-byte
//                          non-temporal loads, fully coalesced; FP8 codes are
//                          widened to bf16 on the way), zeroing V rows past
//                          the slot end;
//   waves 0..3 (compute)  each own 16 query heads over every key of a tile.
// Phase 2t is the K tile [64 keys][256 ch] (rows 512 B) in slot 0, phase
// 2t+1 the V^T tile [256 ch][64 keys] (rows 128 B) in slot 1.  One barrier
// per phase: after barrier q the compute waves read phase q while the
// loaders publish phase q+1 into the other slot (last read before barrier q)
// and issue the loads of phase q+1+kStages.  Loads, LDS stores and the
// matrix work of one phase therefore overlap instead of running one after
// the other in every wave.
//
// Products are transposed so the softmax statistics stay in lanes (16x16x32
// bf16 MFMA, fp32 accumulation):
//   S^T[key, head] = K[key, :] . Q^T[:, head]       (A = K rows from LDS,
//                                                    B = Q fragments in VGPRs)
//   O^T[ch, head] += V^T[ch, key] . P^T[key, head]  (A = V^T rows from LDS, B = P)
// Row r of S^T tile j (4 tiles of 16 rows per 64-key page) is key
// 32(j/2) + 8(r/4) + 4(j%2) + r%4, so the 16 S^T values a lane holds (head
// l%16) are exactly the B operands of its two 32-key PV steps: no lane
// shuffle.  The row max is a 4-lane reduction per tile and the row sum is
// reduced once at the end; a compute wave holds all keys of its heads, so
// its output (or split partial) is final without any merge between waves.
//
// FP8 E4M3 caches stay 8-bit in LDS (K rows of 256 B, V^T rows of 64 B).
// Single-token slots form S^T on the E4M3 matrix unit straight from the
// 8-bit K rows, with the query split exactly into two E4M3 terms (below);
// token pairs and V^T operands are widened to bf16 in registers after the
// read.  The MFMA k-index <-> channel and row <-> key maps are chosen so
// that one 16-byte LDS read of a lane holds the operands of two bf16
// products: QK^T step c takes channels 64(c/2) + 16(l/16) + 8(c%2) + e,
// S^T row r of tile j is key 16(r/4) + 4j + r%4, and PV step s takes keys
// 16(l/16) + 8s + e.
//
// Multi-token queries ("Step-3 is Large yet Affordable", section 5.2, MTP):
// a call with tq new tokens per cached sequence runs B * tq query slots;
// slot s reads sequence s / tq's table row and attends its first
// L - (tq - 1 - s % tq) keys, so the new tokens are causal among themselves.
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
constexpr int kLoaders = 256;          // four loader waves (plus four compute waves)
constexpr int kPhaseBytes = 32768;     // one bf16 K or V^T tile in LDS
constexpr int kMaxChunkTiles = 2048;   // block ids cached per workgroup
constexpr int kMaxBalancedSlots = 512; // balanced partition: slots per batch at most
constexpr int kMaxBalancedTiles = 512; // and pages per workgroup at most
constexpr int kMinBalancedPages = 4;   // pages per workgroup at least
constexpr float kLazyRescale = 8.f;    // log2 headroom before the max moves

// LDS swizzles (XOR on the 16-byte chunk index).  The 16 lanes reading one
// K operand hold keys {0..3, 8..11, 16..19, 24..27} + const: swz_k gives
// them 16 distinct bank quads.  A V^T read has 16 lanes on 16 consecutive
// channels (rows of 128 bytes) and four key chunks across q4.  With the bf16
// key map (chunk 4s + q4) the chunk is XORed with the channel's low three
// bits; an earlier map that also folded in channel bit 3 cost every such read
// a 2-way bank conflict (LDS bank-conflict counter, a quarter of the kernel's
// LDS cycles).  The 8-bit key map (chunks 2q4 + s) keeps that older map,
// which is conflict-free for its reads.
__device__ __forceinline__ int swz_k(int key) { return (key & 3) | (((key >> 3) & 3) << 2); }
template <bool kMap16>
__device__ __forceinline__ int swz_v(int ch) {
  return kMap16 ? (ch & 7) ^ ((ch >> 3) & 1) : (ch & 7);
}
// FP8 tiles (16-byte chunks of 16 codes): the 16 lanes of one K read hold
// keys {0..3, 16..19, 32..35, 48..51} + const (rows of 256 B, one bank row
// each); the 16 lanes of one V^T read hold 16 consecutive channels (rows of
// 64 B, four per bank row).
__device__ __forceinline__ int swz_k8(int key) { return (key & 3) | (((key >> 4) & 3) << 2); }
__device__ __forceinline__ int swz_v8(int ch) { return (ch >> 2) & 3; }

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

// Eight E4M3 codes (two dwords, codes in byte order) to the eight bf16 of
// an MFMA operand.  Every E4M3FN value is a bf16 value and the conversion
// scale is 1, so this is exact (NaN codes stay NaN).
template <bool kUpper>
__device__ __forceinline__ int e4m3x2_to_bf16x2(int w) {   // codes of bytes 0,1 (or 2,3)
  return __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, kUpper));
}
__device__ __forceinline__ intx4 e4m3x8_to_bf16(int w0, int w1) {
  return intx4{e4m3x2_to_bf16x2<false>(w0), e4m3x2_to_bf16x2<true>(w0),
               e4m3x2_to_bf16x2<false>(w1), e4m3x2_to_bf16x2<true>(w1)};
}

// Keep masks for a bf16 chunk of 8 consecutive keys of which `valid` (may be
// <= 0 or >= 8) are below the slot end.
__device__ __forceinline__ void keep_mask(int valid, uint32_t* keep) {
#pragma unroll
  for (int e = 0; e < 4; ++e)
    keep[e] = ((2 * e < valid) ? 0x0000ffffu : 0u) | ((2 * e + 1 < valid) ? 0xffff0000u : 0u);
}
// The same for a chunk of 16 consecutive E4M3 keys (one byte each).
__device__ __forceinline__ void keep_mask8(int valid, uint32_t* keep) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) m |= (4 * e + i < valid) ? (0xffu << (8 * i)) : 0u;
    keep[e] = m;
  }
}
__device__ __forceinline__ intx4 apply_keep(intx4 v, const uint32_t* keep) {
  v.x &= keep[0];
  v.y &= keep[1];
  v.z &= keep[2];
  v.w &= keep[3];
  return v;
}

// Every lambda of the kernels below is forced inline: one that the compiler
// outlines (store_result, called at two sites) makes everything it captures
// by reference live in scratch memory, the O^T accumulators included, which
// then make a round trip through memory on every tile.
template <int N>
using Int = std::integral_constant<int, N>;

// f(Int<I>{}) for I = I0 .. N-1, unrolled at compile time.
template <int I0, int N, class F>
__device__ __forceinline__ void unroll(F&& f) {
  if constexpr (I0 < N) {
    f(Int<I0>{});
    unroll<I0 + 1, N>(f);
  }
}

// kK8 / kV8 (FP8 only): K / V^T tiles stay E4M3 codes in LDS and the
// compute waves widen their operands; otherwise the loaders widen the codes
// to bf16 as they publish a phase.  8-bit K tiles use the key <-> row map
// that lets one 16-byte read feed two products (see above).
//
// kBal (paged, dense, one KV head): instead of cutting every slot into the
// same number of chunks of its capacity, the workgroups of a 1-D grid split
// the batch's actual pages evenly.  Slot b's pages are the global page range
// [P_b, P_b + ceil(L_b/64)) with P_b the prefix sum over earlier slots; with
// T pages in all and Ge active workgroups, workgroup w takes global pages
// [wT/Ge, (w+1)T/Ge).  A workgroup thus walks one or more slot pieces back
// to back: the loaders stream across piece boundaries and the compute waves
// start a fresh softmax state and load the new slot's query at each one.  A
// piece that is a whole slot writes its output; the others write partials
// for the merge (workgroup w's first piece to partial w, its last to G + w).  The compute waves work the partition out (synchronising
// among themselves through an LDS counter) while the loaders already stream
// the pages the split plan would give, which is the partition of a batch of
// full slots.  The partition depends only on the lengths, so results are
// reproducible.
//
// kTps = 2 (multi-token queries, an even number per sequence): a query slot
// is a pair of consecutive new tokens, 128 query rows over one cache row, so
// each K/V tile is read once for both.  Compute wave w holds heads 16w ..
// 16w + 15 of both tokens: softmax state, accumulators and P operands are
// per token, and every K or V^T operand read from LDS (and, FP8, widened)
// feeds one product per token.  The first token of the pair attends one key
// fewer than the second.
template <bool kDense, bool kFp8, bool kK8, bool kV8, bool kBal, int kTps>
__global__ void __launch_bounds__(256 + kLoaders) mqa_decode_kernel(DecodeParams p) {
  static_assert(kFp8 || (!kK8 && !kV8), "8-bit LDS tiles need an FP8 cache");
  static_assert(kK8 || !kV8, "8-bit V^T tiles use the 8-bit K key map");
  static_assert(!kBal || kDense, "the balanced partition covers dense attention");
  static_assert(kTps == 1 || (kTps == 2 && kDense), "token pairs are built for dense attention");
  constexpr int kCw = 4;                              // compute waves (each holds every token of a slot)
  constexpr int kCt = 64 * kCw;                       // compute threads
  constexpr int kNt = kCt + kLoaders;                 // threads
  constexpr int kRows = kG * kTps;                    // query rows per slot and KV group
  constexpr int kSpt = kMaxBalancedSlots / kCt;       // balanced partition: slots
  constexpr int kTpt = kMaxBalancedTiles / kCt;       // and tiles per compute thread
  static_assert(kSpt * kCt == kMaxBalancedSlots && kTpt * kCt == kMaxBalancedTiles &&
                kMaxBalancedTiles <= kMaxChunkTiles, "slots and tiles split evenly over compute threads");
  constexpr bool kMap16 = kK8;                          // key map of 8-bit K tiles
  // 8-bit K tiles of single-token slots multiply on the E4M3 matrix unit;
  // token pairs widen them to bf16 (their two tokens' accumulators leave no
  // registers for the split query's fragments: the E4M3 form spilled in
  // the tile loop and ran 55 % slower).
  constexpr bool kE4m3 = kK8 && kTps == 1;
  constexpr int kElem = kFp8 ? 1 : 2;                 // bytes per cached element
  constexpr int kPerThread = kPhaseBytes * kElem / 2 / 16 / kLoaders;   // 16-byte loads per phase
  constexpr int kKSlot = kK8 ? kPhaseBytes / 2 : kPhaseBytes;   // LDS bytes of a K tile
  constexpr int kVSlot = kV8 ? kPhaseBytes / 2 : kPhaseBytes;   // and of a V^T tile
  // Phases in flight in the loaders' registers: 4 bf16 or 8 FP8 phases,
  // 128 KB of cache data per CU either way.
  constexpr int kStages = kFp8 ? 8 : 4;
  constexpr int kFirstTiles = (kStages + 1) / 2;      // tiles the start-up loads touch
  __shared__ __attribute__((aligned(1024))) uint8_t kslot[kKSlot];
  __shared__ __attribute__((aligned(1024))) uint8_t vslot[kVSlot];
  __shared__ int blk_ids[kMaxChunkTiles];
  __shared__ intx4 qlds[kTps == 2 ? kCw * kTps * (kD / 32) * 64 : 1];   // token pairs: Q fragments
  // Balanced partition: first global page and length of every slot, each
  // tile's (slot << 20 | page) and keys below the slot end, scan partials, a
  // counter the compute waves synchronise on, and {tiles, speculation held}.
  __shared__ int bal_first[kBal ? kMaxBalancedSlots : 1];
  __shared__ int bal_len[kBal ? kMaxBalancedSlots : 1];
  __shared__ int tile_pg[kBal ? kMaxBalancedTiles : 1];
  __shared__ uint8_t tile_keys[kBal ? kMaxBalancedTiles : 1];
  __shared__ int bal_wsum[kBal ? kCw : 1];
  __shared__ int bal_sync[1];
  __shared__ int bal_hdr[2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const bool loader = wave >= kCw;
  const int bg = kBal ? 0 : blockIdx.y;
  int b = bg / p.hkv;          // slot (changes per piece under the balanced partition)
  const int g = bg - b * p.hkv;
  const int split = kBal ? 0 : blockIdx.x;
  // Balanced partition: the workgroup's place in the cut, numbered XCD-major
  // (launch slots go round-robin over the 8 XCDs), so that consecutive
  // ranges -- the pieces of one slot -- run on one XCD, where the merge
  // kernel reads them back.
  const int wl = kBal ? xcd_major(blockIdx.x, gridDim.x) : 0;
  const int32_t* trow = p.block_table ? p.block_table + (int64_t)seq_of(p, b) * p.max_blocks : nullptr;

  // Dense attention: the split's first page (split * chunk) does not depend
  // on the slot length, so its block ids are fetched together with the
  // length and the loaders' first K/V loads are in flight before the length
  // is known (a split that turns out to be past the end simply drops them).
  // With a window the first page moves with the length.
  int t_begin = kDense ? min(split * p.chunk_tiles, p.max_blocks - 1) : 0;
  // Balanced partition: a batch whose slots all have the same number of
  // pages, a multiple of the split count, is cut exactly like the split plan
  // (workgroup w = slot w / splits, pages from (w % splits) * chunk), so
  // those block ids are fetched alongside the lengths and used if the real
  // partition agrees.
  const int spec_b = kBal ? wl / p.splits : 0;
  const int spec_pg = kBal ? (wl - spec_b * p.splits) * p.chunk_tiles : 0;
  const int32_t* spec_row = kBal ? p.block_table + (int64_t)seq_of(p, spec_b) * p.max_blocks : trow;
  int blk_first[kFirstTiles];
#pragma unroll
  for (int i = 0; i < kFirstTiles; ++i)
    blk_first[i] = (kDense && spec_row && (kBal || loader)) ? spec_row[min((kBal ? spec_pg : t_begin) + i, p.max_blocks - 1)] : 0;
  int L = kBal ? 0 : query_len(p, b);
  int nphase = 0;   // two phases (K, V) per tile of this split; set once L is known
  int bal_nt = 0;   // balanced partition: tiles of this workgroup

  // ---- loader state ----
  // Loader thread lt copies 16-byte chunks idx = lt + 256 k of a phase.
  //  bf16: rows (lt >> 5) + 8k of a K tile (32 chunks per row), rows
  //        (lt >> 3) + 32k of a V^T tile (8 chunks per row).
  //  FP8:  rows (lt >> 4) + 16k of a K tile (16 code chunks per row) and
  //        rows (lt >> 2) + 64k of a V^T tile (4 per row), copied as codes.
  const int lt = tid & (kLoaders - 1);
  const char* kpool = static_cast<const char*>(p.k);
  const char* vpool = static_cast<const char*>(p.v);
  const int krow0 = kFp8 ? lt >> 4 : lt >> 5, kc = kFp8 ? lt & 15 : lt & 31;
  const int vrow0 = kFp8 ? lt >> 2 : lt >> 3, vc = kFp8 ? lt & 3 : lt & 7;
  const int64_t kgoff0 = ((int64_t)krow0 * p.k_row_stride + kc * (16 / kElem)) * kElem;
  const int64_t vgoff0 = ((int64_t)vrow0 * p.v_row_stride + vc * (16 / kElem)) * kElem;
  const int64_t kgstep = (int64_t)(kFp8 ? 16 : 8) * p.k_row_stride * kElem;
  const int64_t vgstep = (int64_t)(kFp8 ? 64 : 32) * p.v_row_stride * kElem;
  // LDS position of stored chunk c (16 codes or 8 bf16) of K row
  // krow0 + (8 or 16) k.
  auto klds = [&](int k, int c) __attribute__((always_inline)) {
    const int row = krow0 + (kFp8 ? 16 : 8) * k;
    return kK8 ? (uint32_t)(row * 256 + ((c ^ swz_k8(row)) << 4))
               : (uint32_t)(row * 512 + ((c ^ swz_k(row)) << 4));
  };
  // V^T rows step by 32 or 64: the swizzle of the first row holds for all.
  auto vlds = [&](int k, int c) __attribute__((always_inline)) {
    const int row = vrow0 + (kFp8 ? 64 : 32) * k;
    return kV8 ? (uint32_t)(row * 64 + ((c ^ swz_v8(vrow0)) << 4))
               : (uint32_t)(row * 128 + ((c ^ swz_v<kMap16>(vrow0)) << 4));
  };

  // Register-staged loads of one phase (tiles clamped into the table row:
  // the start-up loads may run past the split).
  auto load_phase = [&](int ph, intx4* st, int blk) __attribute__((always_inline)) {
    const int tile = min(t_begin + (ph >> 1), p.max_blocks - 1);
    if ((ph & 1) == 0) {
      const char* base =
          kpool + ((p.block_table ? (int64_t)blk : (int64_t)seq_of(p, b) * p.max_blocks + tile) * p.k_block_stride +
                   (int64_t)g * p.k_head_stride) * kElem + kgoff0;
#pragma unroll
      for (int k = 0; k < kPerThread; ++k)
        st[k] = __builtin_nontemporal_load(reinterpret_cast<const intx4*>(base + k * kgstep));
    } else {
      const char* base =
          vpool + ((p.block_table ? (int64_t)blk * p.v_block_stride
                                  : (int64_t)seq_of(p, b) * p.v_seq_stride + (int64_t)tile * kPage) +
                   (int64_t)g * p.v_head_stride) * kElem + vgoff0;
#pragma unroll
      for (int k = 0; k < kPerThread; ++k)
        st[k] = __builtin_nontemporal_load(reinterpret_cast<const intx4*>(base + k * vgstep));
    }
  };
  auto load_phase_cached = [&](int ph, intx4* st) __attribute__((always_inline)) {
    load_phase(ph, st, p.block_table ? readfirstlane(blk_ids[ph >> 1]) : 0);
  };

  // Publishing a V^T phase also zeroes the keys past the slot end (their
  // cache rows may hold anything, NaN included), so the PV product never
  // multiplies garbage by a zero probability.  A bf16 chunk holds 8
  // consecutive keys of one channel (vc*8 .. vc*8+7; FP8: 16 keys vc*16 ..).
  auto store_phase = [&](int ph, const intx4* st) __attribute__((always_inline)) {
    if (ph >= nphase) return;
    // Keys of this tile below the slot end (read for V^T phases only).
    auto keys_of = [&]() __attribute__((always_inline)) { return kBal ? (int)tile_keys[ph >> 1] : L - (t_begin + (ph >> 1)) * kPage; };
    if ((ph & 1) == 0) {
#pragma unroll
      for (int k = 0; k < kPerThread; ++k) {
        if (kFp8 && !kK8) {   // 16 codes -> bf16 chunks 2kc, 2kc + 1
          const intx4 c = st[k];
          *reinterpret_cast<intx4*>(kslot + klds(k, 2 * kc)) = e4m3x8_to_bf16(c.x, c.y);
          *reinterpret_cast<intx4*>(kslot + klds(k, 2 * kc + 1)) = e4m3x8_to_bf16(c.z, c.w);
        } else {
          *reinterpret_cast<intx4*>(kslot + klds(k, kc)) = st[k];
        }
      }
    } else if (kFp8 && !kV8) {   // 16 keys -> bf16 chunks 2vc (keys 16vc ..) and 2vc + 1
      // Single-token slots: the key count is the same in every lane, so a
      // scalar branch lets a tile wholly below the slot end -- every tile
      // but a slot's last -- skip the masks (64 of the 96 VALU instructions
      // of this step).  Token pairs keep one path: the branch cost their
      // register allocation a spill.
      const int key_rel = kTps == 1 ? readfirstlane(keys_of()) : keys_of();
      if (kTps == 1 && key_rel >= kPage) {
#pragma unroll
        for (int k = 0; k < kPerThread; ++k) {
          const intx4 c = st[k];
          *reinterpret_cast<intx4*>(vslot + vlds(k, 2 * vc)) = e4m3x8_to_bf16(c.x, c.y);
          *reinterpret_cast<intx4*>(vslot + vlds(k, 2 * vc + 1)) = e4m3x8_to_bf16(c.z, c.w);
        }
      } else {
        uint32_t keep_lo[4], keep_hi[4];
        keep_mask(key_rel - vc * 16, keep_lo);
        keep_mask(key_rel - vc * 16 - 8, keep_hi);
#pragma unroll
        for (int k = 0; k < kPerThread; ++k) {
          const intx4 c = st[k];
          *reinterpret_cast<intx4*>(vslot + vlds(k, 2 * vc)) = apply_keep(e4m3x8_to_bf16(c.x, c.y), keep_lo);
          *reinterpret_cast<intx4*>(vslot + vlds(k, 2 * vc + 1)) = apply_keep(e4m3x8_to_bf16(c.z, c.w), keep_hi);
        }
      }
    } else {
      const int key_rel = keys_of();
      uint32_t keep[4];
      if (kFp8)
        keep_mask8(key_rel - vc * 16, keep);
      else
        keep_mask(key_rel - vc * 8, keep);
#pragma unroll
      for (int k = 0; k < kPerThread; ++k) *reinterpret_cast<intx4*>(vslot + vlds(k, vc)) = apply_keep(st[k], keep);
    }
  };

  intx4 stage[kStages][kPerThread];
  // The first kStages phases, block ids straight from the table, or (balanced
  // partition, other cut) from the tile list, clamped to its last tile.
  auto load_first = [&](bool from_list) __attribute__((always_inline)) {
#pragma unroll
    for (int ph = 0; ph < kStages; ++ph)
      load_phase(ph, stage[ph],
                 from_list ? readfirstlane(blk_ids[min(ph >> 1, bal_nt - 1)])
                           : pool_block(readfirstlane(blk_first[ph >> 1]), p.num_blocks));
  };
  if (kDense && !kBal && loader) load_first(false);

  // ---- compute-wave identity ----
  const int hg = wave & 3;     // head group: heads 16hg .. 16hg+15 of the KV group
  const int r = lane & 15;     // MFMA row / column of this lane
  const int q4 = lane >> 4;    // K-group of this lane
  // This lane's query row for token tk of the slot (one token, or a pair).
  const int head = g * kRows + hg * 16 + r;
  auto head_of = [&](int tk) __attribute__((always_inline)) { return head + tk * kG; };
  // Token pairs: the per-piece code (query loads, result stores) inside the
  // balanced partition's tile loop forms its lane addresses afresh from a
  // copy of the lane index that the compiler cannot see through, rather
  // than hoisting them out of the loop into registers the accumulators of
  // two tokens need.
  struct LaneIds {
    int ln, q4, head;   // lane, K-group, token-0 query row
  };
  auto lane_ids = [&]() __attribute__((always_inline)) {
    int ln = lane;
    if constexpr (kTps == 2) asm volatile("" : "+v"(ln));
    return LaneIds{ln, ln >> 4, g * kRows + hg * 16 + (ln & 15)};
  };
  // Q fragments (B operand of S^T): this lane's head, channels 32c + 8q4 ..
  // +7 (FP8: 64(c/2) + 16q4 + 8(c%2) .. +7).  With token pairs each compute
  // wave parks both tokens' fragments in its own LDS rows and reads them
  // back per K tile, so that they are not held across the V phase.
  //
  // Single-token slots over 8-bit K tiles (kE4m3) multiply on the E4M3
  // matrix unit instead: the 16x16x128 product pairs byte i of lane group
  // l/16 in both operands, so
  // lane (r, q4) takes channels 128m + 32q4 .. +31 of K row and query for
  // product m = 0, 1.  The query of a head is scaled by a power of two
  // 2^e (its largest magnitude below 256) and split into two E4M3 terms,
  // hi = E4M3(2^e q) and lo = E4M3(2^e q - hi): a bf16 value has 8
  // significant bits and each term holds 4, so hi + lo is 2^e q exactly
  // for elements down to ~2^-10 of the head's largest; below that lo is
  // rounded to the E4M3 subnormal step 2^-9, an error under 2^-17 of the
  // largest element.  S^T = K.hi + K.lo, descaled by 2^-e with the logit
  // scale.  Fragment c = 4m + 2t + h holds term t (hi, lo), bytes
  // 16h .. 16h + 15 of product m's 32 channels.
  intx4 qf[kD / 32];
  float q_descale[kTps] = {};
  auto load_q = [&](int slot) __attribute__((always_inline)) {
    const LaneIds id = lane_ids();
#pragma unroll
    for (int tk = 0; tk < kTps; ++tk) {
      const uint16_t* qp = static_cast<const uint16_t*>(p.q) + ((int64_t)slot * p.hq + id.head + tk * kG) * kD;
#pragma unroll
      for (int c = 0; c < kD / 32; ++c) {
        const int ch = kE4m3 ? 128 * (c >> 2) + 32 * id.q4 + 8 * (c & 3)
                             : kMap16 ? 64 * (c >> 1) + 16 * id.q4 + 8 * (c & 1) : 32 * c + 8 * id.q4;
        qf[c] = *reinterpret_cast<const intx4*>(qp + ch);
      }
      if constexpr (kE4m3) {
        float amax = 0.f;
#pragma unroll
        for (int c = 0; c < kD / 32; ++c)
#pragma unroll
          for (int w = 0; w < 4; ++w)
            amax = fmaxf(amax, fmaxf(fabsf(bf16_lo_to_f32((uint32_t)qf[c][w])), fabsf(bf16_hi_to_f32((uint32_t)qf[c][w]))));
        amax = wave_max_xor16_32(amax);   // the four lanes of this head
        int ex = 0;
        frexpf(amax, &ex);                // amax < 2^ex
        const int sh = amax > 0.f ? min(max(8 - ex, -100), 100) : 0;
        const float up = ldexpf(1.f, sh);
        q_descale[tk] = ldexpf(1.f, -sh);
        intx4 t8[kD / 32];
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int c = 0; c < 4; ++c) {   // 8 channels 128m + 32q4 + 8c .. +7
            int hi[2], lo[2];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              const float x0 = bf16_lo_to_f32((uint32_t)qf[4 * m + c][w]) * up;
              const float x1 = bf16_hi_to_f32((uint32_t)qf[4 * m + c][w]) * up;
              const int h2 = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
              const floatx2 hv = __builtin_amdgcn_cvt_pk_f32_fp8(h2, false);
              const int l2 = __builtin_amdgcn_cvt_pk_fp8_f32(x0 - hv.x, x1 - hv.y, 0, false);
              const int sh16 = 16 * (w & 1);
              if ((w & 1) == 0) { hi[w >> 1] = h2 & 0xffff; lo[w >> 1] = l2 & 0xffff; }
              else { hi[w >> 1] |= (h2 & 0xffff) << sh16; lo[w >> 1] |= (l2 & 0xffff) << sh16; }
            }
            // term t, half h = c / 2 of product m: dwords 2 (c % 2) .. +1
            t8[4 * m + 0 + (c >> 1)][2 * (c & 1)] = hi[0];
            t8[4 * m + 0 + (c >> 1)][2 * (c & 1) + 1] = hi[1];
            t8[4 * m + 2 + (c >> 1)][2 * (c & 1)] = lo[0];
            t8[4 * m + 2 + (c >> 1)][2 * (c & 1) + 1] = lo[1];
          }
#pragma unroll
        for (int c = 0; c < kD / 32; ++c) qf[c] = t8[c];
      }
      if constexpr (kTps == 2) {
#pragma unroll
        for (int c = 0; c < kD / 32; ++c) qlds[((wave * kTps + tk) * (kD / 32) + c) * 64 + id.ln] = qf[c];
      }
    }
  };
  auto qfrag = [&](int tk, int c) __attribute__((always_inline)) {
    if constexpr (kTps == 1)
      return qf[c];
    else
      return qlds[((wave * kTps + tk) * (kD / 32) + c) * 64 + lane];
  };

  // ---- balanced partition: this workgroup's slot pieces and tile list ----
  if constexpr (kBal) {
    if (tid == 0) bal_sync[0] = 0;
    lds_barrier();   // counter ready
    // Speculation: if the first, the last and this workgroup's split-plan
    // slot have the same length, take the batch to be uniform and predict
    // the cut from that length alone (for full slots it is the split plan's
    // own); the loaders publish the predicted first pages as phase 0 while
    // the compute waves work out the real partition.
    const int l_spec = query_len(p, spec_b);
    const int l_first = query_len(p, 0);
    const int l_last = query_len(p, p.batch - 1);
    const int p_spec = (l_spec + kPage - 1) / kPage;
    const int tot_spec = p.batch * p_spec;
    const int ge_spec = max(1, min((int)gridDim.x, tot_spec / kMinBalancedPages));
    int pred_b = 0, pred_pg = 0;
    bool spec_issued = false;
    if (l_first == l_spec && l_last == l_spec && p_spec > 0 && wl < ge_spec) {
      const int s_pred = (int)((int64_t)wl * tot_spec / ge_spec);
      const int e_pred = (int)((int64_t)(wl + 1) * tot_spec / ge_spec);
      pred_b = s_pred / p_spec;
      pred_pg = s_pred - pred_b * p_spec;
      spec_issued = e_pred - s_pred >= kFirstTiles && pred_pg + kFirstTiles <= p_spec;
    }
    if (loader) {
      if (spec_issued) {
        if (pred_b != spec_b || pred_pg != spec_pg) {   // not the split plan's cut
          const int32_t* row = p.block_table + (int64_t)seq_of(p, pred_b) * p.max_blocks;
#pragma unroll
          for (int i = 0; i < kFirstTiles; ++i) blk_first[i] = row[pred_pg + i];
        }
        load_first(false);
        nphase = 2;
        store_phase(0, stage[0]);
      }
    } else {
      b = spec_b;
      // Block ids of the split plan's pages for this workgroup, fetched
      // with the lengths (tile i = tid + kCt k); used where the partition
      // agrees.
      int spec_ids[kTpt];
#pragma unroll
      for (int k = 0; k < kTpt; ++k)
        spec_ids[k] = spec_row[min(spec_pg + tid + k * kCt, p.max_blocks - 1)];
      // The compute waves only: wait until all have passed sync point n.
      auto cw_sync = [&](int n) __attribute__((always_inline)) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        if (lane == 0) __hip_atomic_fetch_add(bal_sync, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        while (__hip_atomic_load(bal_sync, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < kCw * n)
          __builtin_amdgcn_s_sleep(1);
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
      };
      // Thread t owns slots kSpt t .. kSpt t + kSpt - 1: their lengths and
      // pages, scanned.
      int len[kSpt], pg[kSpt];
      int incl = 0;
      int raw[kSpt];
#pragma unroll
      for (int k = 0; k < kSpt; ++k) raw[k] = query_len_flat(p, min(kSpt * tid + k, p.batch - 1));
      // The query after the lengths: the wave's loads complete in order, and
      // the scan needs only the lengths (kept out of a branch, where the
      // compiler would wait for the query too).
      asm volatile("" ::: "memory");
      load_q(b);
#pragma unroll
      for (int k = 0; k < kSpt; ++k) asm volatile("" : "+v"(raw[k]));
#pragma unroll
      for (int k = 0; k < kSpt; ++k) {
        const int sk = kSpt * tid + k;
        len[k] = sk < p.batch ? raw[k] : 0;
        pg[k] = (len[k] + kPage - 1) / kPage;
        incl += pg[k];
      }
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int a = __shfl_up(incl, off);
        if (lane >= off) incl += a;
      }
      if (lane == 63) bal_wsum[wave] = incl;
      cw_sync(1);
      int pre = 0, total = 0;
#pragma unroll
      for (int w2 = 0; w2 < kCw; ++w2) {
        const int a = bal_wsum[w2];
        if (w2 < wave) pre += a;
        total += a;
      }
      int first[kSpt];
      first[0] = pre + incl;
#pragma unroll
      for (int k = 0; k < kSpt; ++k) first[0] -= pg[k];
#pragma unroll
      for (int k = 1; k < kSpt; ++k) first[k] = first[k - 1] + pg[k - 1];
#pragma unroll
      for (int k = 0; k < kSpt; ++k) {
        bal_first[kSpt * tid + k] = first[k];
        bal_len[kSpt * tid + k] = len[k];
      }
      const int ge = max(1, min((int)gridDim.x, total / kMinBalancedPages));
      const int w = wl;
      const bool active = total > 0 && w < ge;
      const int s_w = active ? (int)((int64_t)w * total / ge) : 0;
      const int e_w = active ? (int)((int64_t)(w + 1) * total / ge) : 0;
      // A slot whose first page falls in this range: tell the merge which
      // workgroups hold its pieces (the last one holds its last page) and
      // whether it is this workgroup's first piece.
#pragma unroll
      for (int k = 0; k < kSpt; ++k) {
        if (pg[k] > 0 && first[k] >= s_w && first[k] < e_w) {
          const int w_hi = (int)(((int64_t)(first[k] + pg[k]) * ge + total - 1) / total) - 1;
          *reinterpret_cast<intx4*>(p.unit_desc + 4 * (int64_t)(kSpt * tid + k)) =
              intx4{w, first[k] == s_w ? 1 : 0, w_hi, 0};
        }
      }
      cw_sync(2);
      const int nt_here = min(e_w - s_w, kMaxBalancedTiles);
      // Slot of global page x: the last slot starting at or before it.
      auto slot_of = [&](int x) __attribute__((always_inline)) {
        int lo_s = 0, hi_s = p.batch - 1;
        while (lo_s < hi_s) {
          const int mid = (lo_s + hi_s + 1) >> 1;
          if (bal_first[mid] <= x) lo_s = mid; else hi_s = mid - 1;
        }
        return lo_s;
      };
#pragma unroll
      for (int k = 0; k < kTpt; ++k) {
        const int i = tid + k * kCt;
        if (i < nt_here) {
          const int x = s_w + i;
          const int slot = slot_of(x);
          const int page = x - bal_first[slot];
          tile_pg[i] = (slot << 20) | page;
          const bool spec_tile = slot == spec_b && page == spec_pg + i;
          blk_ids[i] = pool_block(spec_tile ? spec_ids[k] : p.block_table[(int64_t)seq_of(p, slot) * p.max_blocks + page],
                                  p.num_blocks);
          tile_keys[i] = (uint8_t)min(kPage, bal_len[slot] - page * kPage);
        }
      }
      const int b0 = nt_here > 0 ? readfirstlane(slot_of(s_w)) : spec_b;
      const int pred_left = bal_first[pred_b] + (bal_len[pred_b] + kPage - 1) / kPage - s_w;
      const bool spec_ok = spec_issued && nt_here >= kFirstTiles && b0 == pred_b &&
                           s_w - bal_first[pred_b] == pred_pg && pred_left >= kFirstTiles;
      if (tid == 0) {
        bal_hdr[0] = nt_here;
        bal_hdr[1] = spec_ok ? 1 : 0;
      }
      if (b0 != b) {
        b = b0;
        load_q(b);
      }
    }
    lds_barrier();   // tile list, block ids, key counts and phase 0 visible
    bal_nt = readfirstlane(bal_hdr[0]);
    if (bal_nt == 0) return;
    nphase = 2 * bal_nt;
    if (!readfirstlane(bal_hdr[1])) {   // the speculation missed: phase 0 from the tile list
      if (loader) {
        load_first(true);
        store_phase(0, stage[0]);
      }
      lds_barrier();
    }
  }

  const int lo = (!kDense && L > p.window) ? L - p.window : 0;
  // Keys token tk of the slot attends: the slot's (its last token's) length,
  // one fewer for the first token of a pair.
  int Lq[kTps];
  auto set_query_keys = [&](int len) __attribute__((always_inline)) {
#pragma unroll
    for (int tk = 0; tk < kTps; ++tk) Lq[tk] = max(len - (kTps - 1 - tk), 0);
  };
  set_query_keys(L);
  int n_tiles = 0, t_lo = 0;
  if (L > 0) {
    t_lo = lo / kPage;
    n_tiles = (L - 1) / kPage - t_lo + 1;
  }
  if (!kDense) t_begin = t_lo + split * p.chunk_tiles;
  const int t_end = min(t_lo + n_tiles, t_begin + p.chunk_tiles);

  // A split without keys: zeros for a single-split slot; otherwise an empty
  // partial (m = -inf) that still takes part in the merge.
  const bool empty = !kBal && (t_begin >= t_end || (kDense && split * p.chunk_tiles >= p.max_blocks));
  if (empty && p.splits == 1) {
    if (loader) return;
    for (int tk = 0; tk < kTps; ++tk)
      for (int ct = 0; ct < kD / 16; ++ct) {
        const int64_t o = ((int64_t)b * p.hq + head_of(tk)) * kD + ct * 16 + q4 * 4;
        if (p.out_f32)
          *reinterpret_cast<floatx4*>(static_cast<float*>(p.out) + o) = floatx4{0.f, 0.f, 0.f, 0.f};
        else
          *reinterpret_cast<intx2*>(static_cast<uint16_t*>(p.out) + o) = intx2{0, 0};
      }
    return;
  }
  const int nt = kBal ? bal_nt : (empty ? 0 : t_end - t_begin);
  nphase = 2 * nt;

  // Online-softmax state of a compute lane, per token tk (row head_of(tk),
  // channels 16ct + 4q4 .. +3 of O^T tile ct).
  float m_run[kTps], l_run[kTps];
  floatx4 acc[kTps][kD / 16];
  auto reset_state = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int tk = 0; tk < kTps; ++tk) {
      m_run[tk] = kNegInf;
      l_run[tk] = 0.f;
#pragma unroll
      for (int ct = 0; ct < kD / 16; ++ct) acc[tk][ct] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
  };
  reset_state();

  // A compute wave holds every key of its 16 heads for the piece it has
  // walked: the final output of slot b, or partial `piece` for the merge.
  auto store_result = [&](bool final_out, int64_t piece) __attribute__((always_inline)) {
    const LaneIds id = lane_ids();
#pragma unroll
    for (int tk = 0; tk < kTps; ++tk) {
      const float l_tot = wave_sum_xor16_32(l_run[tk]);
      if (final_out) {
        // (The first token of a pair may have no key at all: zeros.)
        const float inv = (kTps == 1 || l_tot > 0.f) ? (kFp8 ? p.v_scale[g] : 1.f) / l_tot : 0.f;
#pragma unroll
        for (int ct = 0; ct < kD / 16; ++ct) {
          const int64_t o = ((int64_t)b * p.hq + (id.head + tk * kG)) * kD + ct * 16 + id.q4 * 4;
          const floatx4 v = acc[tk][ct] * inv;
          if (p.out_f32)
            *reinterpret_cast<floatx4*>(static_cast<float*>(p.out) + o) = v;
          else
            *reinterpret_cast<intx2*>(static_cast<uint16_t*>(p.out) + o) =
                intx2{(int)pack_bf16x2(v.x, v.y), (int)pack_bf16x2(v.z, v.w)};
        }
        continue;
      }
      // Split partials are read once, by the merge kernel.
      const int64_t row = piece * kRows + ((id.head + tk * kG) - g * kRows);
      if (p.part_bf16) {
        // bf16 rows, stored by row pairs: tiles 2j and 2j+1 of this lane
        // form run 4j + q4 (8 elements), and the runs 4j .. 4j+3 of rows 2i
        // and 2i+1 (the lanes of heads r and r ^ 1) fill one 128-byte line,
        // so every store of the wave writes whole lines: cached for single
        // tokens, streamed out for token pairs (each measured the faster).
        uint16_t* po = reinterpret_cast<uint16_t*>(p.part_o) + (row & ~(int64_t)1) * kD + (row & 1) * 32 + id.q4 * 8;
#pragma unroll
        for (int j = 0; j < kD / 32; ++j) {
          const intx4 v = intx4{(int)pack_bf16x2(acc[tk][2 * j].x, acc[tk][2 * j].y),
                                (int)pack_bf16x2(acc[tk][2 * j].z, acc[tk][2 * j].w),
                                (int)pack_bf16x2(acc[tk][2 * j + 1].x, acc[tk][2 * j + 1].y),
                                (int)pack_bf16x2(acc[tk][2 * j + 1].z, acc[tk][2 * j + 1].w)};
          if constexpr (kTps == 1)
            *reinterpret_cast<intx4*>(po + j * 64) = v;
          else
            __builtin_nontemporal_store(v, reinterpret_cast<intx4*>(po + j * 64));
        }
      } else {
        // fp32 rows (whole 64-byte quarters of a line per store): streamed
        // out rather than kept dirty in L2 for the write-back at the
        // kernel's end.
#pragma unroll
        for (int ct = 0; ct < kD / 16; ++ct)
          __builtin_nontemporal_store(acc[tk][ct], reinterpret_cast<floatx4*>(p.part_o + row * kD + ct * 16 + id.q4 * 4));
      }
      if (id.q4 == 0) {   // (m, l): cached for single tokens, streamed for pairs, as the rows
        if constexpr (kTps == 1)
          *reinterpret_cast<floatx2*>(p.part_ml + row * 2) = floatx2{m_run[tk], l_tot};
        else
          __builtin_nontemporal_store(floatx2{m_run[tk], l_tot}, reinterpret_cast<floatx2*>(p.part_ml + row * 2));
      }
    }
  };


  if (!empty) {

  // Start-up: the loaders' first kStages phases are in flight (dense) or go
  // first; every thread fills part of the block-id cache (rows t_begin ..
  // t_end-1 of the table); the compute waves load Q; the loaders publish
  // phase 0.  (Loads are issued unconditionally, indices clamped: the
  // compiler's wait counts stay exact only when every path issues the same
  // loads.)
  if (!kDense && loader) {
#pragma unroll
    for (int i = 0; i < kFirstTiles; ++i)
      blk_first[i] = trow ? trow[min(t_begin + i, p.max_blocks - 1)] : 0;
    load_first(false);
  }
  if constexpr (!kBal) {
    constexpr int kIdsPerThread = (kMaxChunkTiles + kNt - 1) / kNt;
    const int32_t* btab = trow ? trow + t_begin : static_cast<const int32_t*>(p.ctx_lens);
    int blk_cache[kIdsPerThread];
#pragma unroll
    for (int k = 0; k < kIdsPerThread; ++k)
      blk_cache[k] = btab[trow ? min(tid + k * kNt, nt - 1) : 0];
#pragma unroll
    for (int k = 0; k < kIdsPerThread; ++k) {
      const int i = tid + k * kNt;
      if (i < nt) blk_ids[i] = pool_block(blk_cache[k], p.num_blocks);
    }
  }

  if (loader) {
    if constexpr (!kBal) {
      store_phase(0, stage[0]);
      lds_barrier();   // block ids and phase 0 visible
    }
    // Phase kStages into the freed stage (clamped to the last phase of the
    // same K/V parity when the split is shorter; such a copy is never
    // published).
    load_phase_cached(min(kStages, nphase - 2 + (kStages & 1)), stage[0]);
    // Step q: barrier q, publish phase q+1 (loaded kStages steps ago) into
    // its slot, load phase q+1+kStages into the registers it freed.  Phase
    // i lives in stage i % kStages; steps are unrolled kStages at a time.
    auto step = [&](auto ic, int q, bool more) __attribute__((always_inline)) {
      constexpr int I = decltype(ic)::value;     // q % kStages
      constexpr int st = (I + 1) % kStages;
      lds_barrier();
      store_phase(q + 1, stage[st]);
      if (more) load_phase_cached(q + 1 + kStages, stage[st]);
    };
    auto group = [&](int q, auto all_in_range) __attribute__((always_inline)) {
      auto one = [&](auto ic) __attribute__((always_inline)) {
        constexpr int I = decltype(ic)::value;
        if constexpr (decltype(all_in_range)::value) {
          step(ic, q + I, true);
        } else {
          if (q + I < nphase) step(ic, q + I, q + I + 1 + kStages < nphase);
        }
      };
      unroll<0, kStages>(one);
    };
    // Main loop: every load it issues is in range, so the issue pattern (and
    // the compiler's wait counts) is the same in every iteration.
    int q = 0;
    for (; q + 2 * kStages < nphase; q += kStages) group(q, std::true_type{});
    for (; q < nphase; q += kStages) group(q, std::false_type{});
  } else {

  // ---------------- compute waves ----------------
  // bf16 single-token slots: the compute waves win issue arbitration against
  // the loader on their SIMD (measured ~0.1 us faster per call; even or
  // slower for FP8 caches, which keep equal priority).
  if constexpr (!kFp8 && kTps == 1) __builtin_amdgcn_s_setprio(2);
  const float qk_scale = p.scale * kLog2e * (kFp8 ? p.k_scale[g] : 1.f);
  if constexpr (!kBal) {
    load_q(b);
    lds_barrier();   // block ids and phase 0 visible
  }

  // K operand of S^T tile j: row r is key 32(j/2) + 8(r/4) + 4(j%2) + r%4,
  // whose swizzle is r itself; fragment c (channels 32c + 8q4 .. +7) is
  // chunk (4c + q4) ^ r = 4c ^ (q4 ^ r), at byte (kfrag ^ (c << 6)) +
  // 512 (32(j/2) + 4(j%2)).
  // FP8: row r of tile j is key 16(r/4) + 4j + r%4 (swizzle r again); the
  // 32 codes of product m are chunks (8m + 2q4 + h) ^ r, h = 0, 1, at byte
  // (kfrag ^ ((8m + h) << 4)) + 1024 j (the chunk bits of 8m, 2q4 and h do
  // not overlap, so the sum is an XOR).
  const uint32_t kfrag = kK8 ? (16 * (r >> 2) + (r & 3)) * 256 + (((kE4m3 ? 2 * q4 : q4) ^ r) << 4)
                             : (8 * (r >> 2) + (r & 3)) * 512 + ((q4 ^ r) << 4);
  // V^T operand of channel tile t, key step s: row 16t + r, chunk
  // (4s + q4) ^ swz_v(r) (8-bit K map: 2q4 + s), at byte vfrag_s + 2048 t.
  // 8-bit V^T: code chunk q4 ^ swz_v8(r) holds keys 16q4 .. +15, both
  // steps, at vfrag0 + 1024 t.
  const uint32_t vfrag0 = kV8 ? r * 64 + ((q4 ^ swz_v8(r)) << 4)
                              : r * 128 + (((kMap16 ? 2 * q4 : q4) ^ swz_v<kMap16>(r)) << 4);
  const uint32_t vfrag1 = r * 128 + (((kMap16 ? 2 * q4 + 1 : 4 + q4) ^ swz_v<kMap16>(r)) << 4);

  intx4 pb[kTps][2];
  // LDS operand reads issued ahead of the products (16-byte reads; FP8 K
  // reads feed two products each, per token).
  constexpr int kAhead = 8;
  constexpr int kAhead8 = 6;

  auto k_phase = [&](int key0) __attribute__((always_inline)) {
    uint32_t kb = kfrag;
    asm volatile("" : "+v"(kb));   // addresses formed here, not hoisted and kept live
    floatx4 st[kTps][4];
#pragma unroll
    for (int tk = 0; tk < kTps; ++tk)
#pragma unroll
      for (int j = 0; j < 4; ++j) st[tk][j] = floatx4{0.f, 0.f, 0.f, 0.f};
    if constexpr (kE4m3) {
      // Product m of S^T tile j: A = K row (32 codes: chunks 8m + 2q4 and
      // 8m + 2q4 + 1 of the row), B = the query's hi and lo terms (two
      // products into one accumulator).
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        intx4 raw[4][2];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int h = 0; h < 2; ++h)
            raw[j][h] = *reinterpret_cast<const intx4*>(kslot + (kb ^ ((8 * m + h) << 4)) + j * 1024);
        const intx8 qhi = {qf[4 * m].x, qf[4 * m].y, qf[4 * m].z, qf[4 * m].w,
                           qf[4 * m + 1].x, qf[4 * m + 1].y, qf[4 * m + 1].z, qf[4 * m + 1].w};
        const intx8 qlo = {qf[4 * m + 2].x, qf[4 * m + 2].y, qf[4 * m + 2].z, qf[4 * m + 2].w,
                           qf[4 * m + 3].x, qf[4 * m + 3].y, qf[4 * m + 3].z, qf[4 * m + 3].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const intx8 a = {raw[j][0].x, raw[j][0].y, raw[j][0].z, raw[j][0].w,
                           raw[j][1].x, raw[j][1].y, raw[j][1].z, raw[j][1].w};
          st[0][j] = mfma_e4m3_16x16x128(a, qhi, st[0][j]);
          st[0][j] = mfma_e4m3_16x16x128(a, qlo, st[0][j]);
        }
        // Per product m: the first row's two reads, then two products
        // behind each further row's reads.
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int j = 1; j < 4; ++j) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      }
    } else if constexpr (kK8) {
      intx4 raw[kD / 64][4];
      intx4 qv[kD / 64][kTps][2];   // token pairs: Q fragments read back per K tile
#pragma unroll
      for (int u = 0; u < kD / 64; ++u) {
        if constexpr (kTps == 2) {
#pragma unroll
          for (int tk = 0; tk < kTps; ++tk) {
            qv[u][tk][0] = qfrag(tk, 2 * u);
            qv[u][tk][1] = qfrag(tk, 2 * u + 1);
          }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
          raw[u][j] = *reinterpret_cast<const intx4*>(kslot + (kb ^ (u << 6)) + j * 1024);
      }
#pragma unroll
      for (int u = 0; u < kD / 64; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // Each K operand is widened once and feeds every token's product.
          const intx4 k_lo = e4m3x8_to_bf16(raw[u][j].x, raw[u][j].y);
          const intx4 k_hi = e4m3x8_to_bf16(raw[u][j].z, raw[u][j].w);
#pragma unroll
          for (int tk = 0; tk < kTps; ++tk) {
            st[tk][j] = mfma_bf16_16x16x32(k_lo, kTps == 1 ? qfrag(0, 2 * u) : qv[u][tk][0], st[tk][j]);
            st[tk][j] = mfma_bf16_16x16x32(k_hi, kTps == 1 ? qfrag(0, 2 * u + 1) : qv[u][tk][1], st[tk][j]);
          }
        }
      if constexpr (kTps == 2) {
        // Per step u: four Q and four K reads feed sixteen products; one
        // step of reads runs ahead.
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
        for (int u = 1; u < kD / 64; ++u) {
          __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
      } else {
        __builtin_amdgcn_sched_group_barrier(0x100, kAhead8, 0);
#pragma unroll
        for (int i = 0; i < 16 - kAhead8; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * kAhead8, 0);
      }
    } else {
      intx4 a[kD / 32][4];
      intx4 qv[kD / 32][kTps];   // token pairs: Q fragments read back per K tile
#pragma unroll
      for (int c = 0; c < kD / 32; ++c) {
        if constexpr (kTps == 2) {
#pragma unroll
          for (int tk = 0; tk < kTps; ++tk) qv[c][tk] = qfrag(tk, c);
        }
        const uint32_t a_off = kb ^ (c << 6);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          a[c][j] = *reinterpret_cast<const intx4*>(kslot + a_off + ((j >> 1) * 32 + (j & 1) * 4) * 512);
      }
#pragma unroll
      for (int c = 0; c < kD / 32; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int tk = 0; tk < kTps; ++tk)
            st[tk][j] = mfma_bf16_16x16x32(a[c][j], kTps == 1 ? qfrag(0, c) : qv[c][tk], st[tk][j]);
      // Software pipeline: operands of kAhead products in flight ahead of
      // the matrix unit (the other wave on this SIMD is a loader).  Token
      // pairs: per chunk c, two Q and four K reads feed eight products; two
      // chunks of reads run ahead.
      if constexpr (kTps == 2) {
        __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
        for (int c = 1; c < kD / 32; ++c) {
          __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
      } else {
        __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
        for (int i = 0; i < 32 - kAhead; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, kAhead, 0);
      }
    }
    // Lane values: tile j, element i is key key0 + 8q4 + 32(j/2) + 4(j%2) + i
    // (FP8: key0 + 16q4 + 4j + i); those in [lo, Lq) are attended.  A page
    // wholly inside [lo, Lq) (every page but the first and last of a slot)
    // takes the branch without masks.
#pragma unroll
    for (int tk = 0; tk < kTps; ++tk) {
      float sv[4][4];
      const float qs = kE4m3 ? qk_scale * q_descale[tk] : qk_scale;   // (E4M3 products: the query's 2^-e)
      const bool interior = key0 >= lo && key0 + kPage <= Lq[tk];   // uniform
      if (interior) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) sv[j][i] = st[tk][j][i] * qs;
      } else {
        const int ebase = key0 + (kMap16 ? 16 : 8) * q4;
        const int e_lo = lo - ebase, e_hi = Lq[tk] - ebase;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int e = kMap16 ? 4 * j + i : 32 * (j >> 1) + 4 * (j & 1) + i;
            sv[j][i] = (e >= e_lo && e < e_hi) ? st[tk][j][i] * qs : kNegInf;
          }
      }
      float mx = fmaxf(fmaxf(sv[0][0], sv[0][1]), fmaxf(sv[0][2], sv[0][3]));
#pragma unroll
      for (int j = 1; j < 4; ++j)
        mx = fmaxf(mx, fmaxf(fmaxf(sv[j][0], sv[j][1]), fmaxf(sv[j][2], sv[j][3])));
      mx = wave_max_xor16_32(mx);
      // Lazy max: keep the old reference unless this tile exceeds it by > 2^8.
      const bool move = mx > m_run[tk] + kLazyRescale;
      const float m_new = move ? mx : m_run[tk];
      if (__any(move && m_run[tk] != kNegInf)) {
        const float alpha = fast_exp2(m_run[tk] - m_new);   // 1 where the max stays
        l_run[tk] *= alpha;
#pragma unroll
        for (int ct = 0; ct < kD / 16; ++ct) acc[tk][ct] *= alpha;
      }
      m_run[tk] = m_new;
      // p = 2^(s - m); a head with no attended key yet (m = -inf, only on a
      // masked page) gets p = 0 instead of 2^NaN.
      const float m_sub = m_new == kNegInf ? 0.f : m_new;
      float psum = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sv[j][i] = fast_exp2(sv[j][i] - m_sub);
          psum += sv[j][i];
        }
      l_run[tk] += psum;
      // P^T B operands: keys 32s + 8q4 .. +7 (FP8: 16q4 + 8s .. +7) come
      // from tiles 2s (first four) and 2s + 1 (last four).
#pragma unroll
      for (int s = 0; s < 2; ++s)
        pb[tk][s] = intx4{(int)pack_bf16x2(sv[2 * s][0], sv[2 * s][1]), (int)pack_bf16x2(sv[2 * s][2], sv[2 * s][3]),
                          (int)pack_bf16x2(sv[2 * s + 1][0], sv[2 * s + 1][1]),
                          (int)pack_bf16x2(sv[2 * s + 1][2], sv[2 * s + 1][3])};
    }
  };

  auto v_phase = [&]() __attribute__((always_inline)) {
    if constexpr (kV8) {
      intx4 raw[kD / 16];
#pragma unroll
      for (int ct = 0; ct < kD / 16; ++ct) raw[ct] = *reinterpret_cast<const intx4*>(vslot + vfrag0 + ct * 1024);
#pragma unroll
      for (int ct = 0; ct < kD / 16; ++ct) {
        const intx4 v_lo = e4m3x8_to_bf16(raw[ct].x, raw[ct].y);
        const intx4 v_hi = e4m3x8_to_bf16(raw[ct].z, raw[ct].w);
#pragma unroll
        for (int tk = 0; tk < kTps; ++tk) {
          acc[tk][ct] = mfma_bf16_16x16x32(v_lo, pb[tk][0], acc[tk][ct]);
          acc[tk][ct] = mfma_bf16_16x16x32(v_hi, pb[tk][1], acc[tk][ct]);
        }
      }
      if constexpr (kTps == 1) {
        __builtin_amdgcn_sched_group_barrier(0x100, kAhead8, 0);
#pragma unroll
        for (int i = 0; i < 16 - kAhead8; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * kAhead8, 0);
      }
      return;
    }
    intx4 a[2][kD / 16];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int ct = 0; ct < kD / 16; ++ct)
        a[s][ct] = *reinterpret_cast<const intx4*>(vslot + (s ? vfrag1 : vfrag0) + ct * 2048);
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int ct = 0; ct < kD / 16; ++ct)
#pragma unroll
        for (int tk = 0; tk < kTps; ++tk) acc[tk][ct] = mfma_bf16_16x16x32(a[s][ct], pb[tk][s], acc[tk][ct]);
    // Each V^T read feeds one product per token.
    __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
    for (int i = 0; i < 32 - kAhead; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, kTps, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kTps * kAhead, 0);
  };

  if constexpr (kBal) {
    // Pieces back to back.  The tiles of one slot are consecutive pages, so
    // a piece runs from its first tile up to the slot's last page or the end
    // of the workgroup's range; the loaders stream straight across piece
    // boundaries.  A new piece starts a fresh state on its query.  Piece 0
    // of workgroup w is partial w, its last piece partial G + w (G
    // workgroups); the pieces between are whole slots.
    for (int t = 0, piece = 0; t < nt; ++piece) {
      const int info = readfirstlane(tile_pg[t]);
      const int slot = info >> 20, page0 = info & 0xfffff;
      L = readfirstlane(bal_len[slot]);
      const int pages = (L + kPage - 1) / kPage;
      const int t_stop = min(nt, t + max(pages - page0, 1));
      if (piece > 0) {
        b = slot;
        load_q(b);
        reset_state();
      }
      set_query_keys(L);
      const bool whole = page0 == 0 && t_stop - t == pages;
      for (int key0 = page0 * kPage; t < t_stop; ++t, key0 += kPage) {
        lds_barrier();   // K tile visible
        k_phase(key0);
        lds_barrier();   // V^T tile visible
        v_phase();
      }
      store_result(whole, (piece > 0 ? (int64_t)gridDim.x : 0) + wl);
    }
    return;
  }
  for (int t = 0; t < nt; ++t) {
    lds_barrier();   // K tile t visible
    k_phase((t_begin + t) * kPage);
    lds_barrier();   // V^T tile t visible
    v_phase();
  }
  }   // compute waves
  }   // !empty

  // ---- finish: the output, or this split's partial for the merge ----
  if (loader) return;
  store_result(p.splits == 1, (int64_t)bg * p.splits + split);
}

}  // namespace

// FP8 tiles in LDS: K stays 8-bit, V^T is widened by the loaders (the
// compute waves widen every K operand they read, four times per tile; the
// loaders widen each V^T code once).
constexpr bool kFp8K8 = true, kFp8V8 = false;

template <int kTps>
void launch_mqa_t(const DecodeParams& p, bool fp8, bool dense, hipStream_t stream) {
  const dim3 block(256 + kLoaders);
  const dim3 grid(p.splits, p.batch * p.hkv);
  if (p.balanced) {
    // One workgroup per range of the batch's pages: as many as the split
    // plan would use (the kernel leaves extra ones idle for short batches).
    const dim3 grid1(p.splits * p.batch * p.hkv);
    if (fp8)
      hipLaunchKernelGGL((mqa_decode_kernel<true, true, kFp8K8, kFp8V8, true, kTps>), grid1, block, 0, stream, p);
    else
      hipLaunchKernelGGL((mqa_decode_kernel<true, false, false, false, true, kTps>), grid1, block, 0, stream, p);
  } else if (fp8) {
    if (dense)
      hipLaunchKernelGGL((mqa_decode_kernel<true, true, kFp8K8, kFp8V8, false, kTps>), grid, block, 0, stream, p);
    else if constexpr (kTps == 1)
      hipLaunchKernelGGL((mqa_decode_kernel<false, true, kFp8K8, kFp8V8, false, 1>), grid, block, 0, stream, p);
  } else {
    if (dense)
      hipLaunchKernelGGL((mqa_decode_kernel<true, false, false, false, false, kTps>), grid, block, 0, stream, p);
    else if constexpr (kTps == 1)
      hipLaunchKernelGGL((mqa_decode_kernel<false, false, false, false, false, 1>), grid, block, 0, stream, p);
  }
}

hipError_t launch_mqa(const DecodeParams& p, bool fp8, hipStream_t stream) {
  const bool dense = p.window == 0;
  if (p.balanced && (!dense || p.hkv != 1 || !p.block_table || p.batch > kMaxBalancedSlots ||
                     p.chunk_tiles > kMaxBalancedTiles || p.max_blocks > (1 << 20)))
    return hipErrorInvalidValue;
  // Token pairs: one KV head, dense, 128 query rows per slot.
  if (p.tps == 2) {
    if (!dense || p.hkv != 1 || p.hq != 2 * kG) return hipErrorInvalidValue;
    launch_mqa_t<2>(p, fp8, dense, stream);
  } else {
    if (p.tps != 1 || p.hq != kG * p.hkv) return hipErrorInvalidValue;
    launch_mqa_t<1>(p, fp8, dense, stream);
  }
  return hipGetLastError();
}

int mqa_max_chunk_tiles() { return kMaxChunkTiles; }

}  // namespace mfa

// Device helpers for gfx950 (CDNA4): MFMA wrappers, bf16/FP8 conversion,
// LDS-DMA loads, wave reductions.  Wave size is 64 throughout.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mfa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(4))) float floatx4;
typedef __attribute__((ext_vector_type(2))) float floatx2;
typedef __attribute__((ext_vector_type(4))) int intx4;
typedef __attribute__((ext_vector_type(2))) int intx2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();

// D(16x16 fp32) += A(16x32 bf16) * B(32x16 bf16).  Operand layout (lane l,
// wave64): A row = l % 16, B column = l % 16, both hold the 8 consecutive
// K-indices 8*(l/16) .. 8*(l/16)+7.  Result: lane l holds D[4*(l/16)+i][l%16],
// i = 0..3.
__device__ __forceinline__ floatx4 mfma_bf16_16x16x32(intx4 a, intx4 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

typedef __attribute__((ext_vector_type(8))) int intx8;

// D(16x16 fp32) += A(16x128 E4M3) * B(128x16 E4M3) on the gfx950 8-bit
// matrix unit (unit block scales: exponent code 127 = 2^0).  Lane l holds
// row (A) / column (B) l % 16 and 32 K-indices; byte i of lane group l / 16
// in A meets byte i of the same lane group in B, so any assignment of K
// indices to (l / 16, i) shared by both operands gives the same product.
// Result: lane l holds D[4*(l/16)+i][l%16], i = 0..3.
__device__ __forceinline__ floatx4 mfma_e4m3_16x16x128(intx8 a, intx8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Round-to-nearest-even fp32 -> bf16 of two values packed low/high.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo_to_f32(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi_to_f32(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// Exact widening of four OCP E4M3FN bytes (one dword) to four bf16 (two
// dwords).  Every E4M3 value is representable in bf16, so the hardware
// conversion (fp8 -> fp32, then fp32 -> bf16) is exact.
__device__ __forceinline__ intx2 e4m3x4_to_bf16x4(uint32_t w) {
  floatx2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  floatx2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  intx2 r;
  r.x = (int)pack_bf16x2(a.x, a.y);
  r.y = (int)pack_bf16x2(b.x, b.y);
  return r;
}

// A cache block id from the block table, kept inside the pool: ids outside
// [0, num_blocks) (a caller error, or table entries past a slot's end that
// are fetched ahead of time) read block 0 instead of faulting.
__device__ __forceinline__ int pool_block(int blk, int64_t num_blocks) {
  return (int64_t)(uint32_t)blk < num_blocks ? blk : 0;
}

// A slot length kept inside [0, max_blocks * 64] (a longer or negative
// length is a caller error; clamping keeps every table and cache read in
// bounds).
__device__ __forceinline__ int slot_len(int L, int max_blocks) {
  return min(max(L, 0), max_blocks * 64);
}

// Query slot s of a call with p.tq query tokens per cached sequence, p.tps
// of them per slot: its cached sequence (table row, length entry), and the
// keys its last token attends: the sequence's length, clamped as above, less
// the tokens that follow it (never below 0).
template <class P>
__device__ __forceinline__ int seq_of(const P& p, int s) {
  return p.tq == p.tps ? s : s / (p.tq / p.tps);
}
template <class P>
__device__ __forceinline__ int query_len(const P& p, int s) {
  if (p.tq == 1) return slot_len(p.ctx_lens[s], p.max_blocks);
  const int per_seq = p.tq / p.tps;
  const int seq = s / per_seq;
  const int last = (s - seq * per_seq) * p.tps + p.tps - 1;
  return max(slot_len(p.ctx_lens[seq], p.max_blocks) - (p.tq - 1 - last), 0);
}
// The same without control flow, for per-lane slots: the compiler waits for
// every earlier load of the wave where the branches of the form above join
// (tq = 1 implies tps = 1, where the general form reduces to the length).
template <class P>
__device__ __forceinline__ int query_len_flat(const P& p, int s) {
  const int per_seq = p.tq / p.tps;
  const int seq = s / per_seq;
  const int last = (s - seq * per_seq) * p.tps + p.tps - 1;
  return max(slot_len(p.ctx_lens[seq], p.max_blocks) - (p.tq - 1 - last), 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 16-byte global -> LDS copy without a register round trip
// (global_load_lds_dwordx4).  Lane l of the wave writes lds_base + 16*l;
// lds_base must be wave-uniform.  Issued through inline asm on purpose: the
// compiler's own wait insertion for LDS DMA cannot tell ring slots apart and
// would drain every in-flight copy before each LDS read.  Callers therefore
// own the synchronisation: wait_vmcnt<N>() for their own copies, then a
// workgroup barrier before other waves read the slot.
__device__ __forceinline__ void dma16(const void* gptr, const void* lds_base) {
  const uint32_t lds = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds_base;
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gptr), "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory", "m0");
}

// The same copy, non-temporal: for streamed data that no later load of the
// kernel reuses.  (A per-group attention kernel streamed 12% faster this way
// at one workgroup per CU.)
__device__ __forceinline__ void dma16_nt(const void* gptr, const void* lds_base) {
  const uint32_t lds = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds_base;
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt"
               :
               : "v"(gptr), "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory", "m0");
}

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ float wave_max_xor16_32(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

__device__ __forceinline__ float wave_sum_xor16_32(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

__device__ __forceinline__ int readfirstlane(int x) { return __builtin_amdgcn_readfirstlane(x); }

// XCD-major number of launch slot x of a 1-D grid of n workgroups: slots go
// round-robin over the 8 XCDs, so slot x runs on XCD x % 8 and gets number
// (x % 8) * (n / 8) + x / 8; numbers k * n/8 .. (k+1) * n/8 - 1 share XCD k.
// (Identity when n is not a multiple of 8.)
__device__ __forceinline__ int xcd_major(int x, int n) {
  return (n & 7) ? x : (x & 7) * (n >> 3) + (x >> 3);
}

}  // namespace mfa

// Parameter blocks shared by the host launchers and the decode kernels.
// Plain C++ (no HIP types) so the host-side planning code can include it.
#pragma once

#include <stdint.h>

namespace mfa {

constexpr int kPage = 64;          // tokens per cache block (one kernel tile)

// One decode-attention launch.  Element strides are in elements of the KV
// storage type.  For a paged cache the K/V tile of (slot b, page t, group g)
// starts at   k + block * k_block_stride + g * k_head_stride
//             v + block * v_block_stride + g * v_head_stride
// with block = block_table[b * max_blocks + t]; for a contiguous cache the
// block index is replaced by (b * max_blocks + t) for K and the V tile starts
// at v + b * v_seq_stride + g * v_head_stride + t * v_tile_stride.  Inside a
// V tile, keys 8c .. 8c + 7 of channel ch (16 contiguous bytes in bf16) start
// at ch * v_row_stride + c * v_chunk_stride: (64, 8) for channel-major
// blocks [d][64], (8, 8 d) for blocks cut into 8-token sub-blocks [8][d][8].
// Query slot s holds tps consecutive query tokens of cached sequence
// s / (tq / tps) (block-table row, length, contiguous cache slot).  With
// tq > 1 the tq tokens are the last tq cached keys of their sequence and
// token t attends the first L - (tq - 1 - t) keys (causal among the new
// tokens); a slot's length is that of its last token.
struct DecodeParams {
  const void* q;              // [B, Hq, d]  (B = batch query slots)
  const void* k;
  const void* v;
  const int32_t* block_table; // nullptr: contiguous
  const int32_t* ctx_lens;    // [B]
  const float* k_scale;       // [Hkv] (FP8) or nullptr
  const float* v_scale;
  void* out;                  // [B, Hq, d]
  float* part_o;              // [B*Hkv, splits, G, d]   (splits > 1)
  int32_t part_bf16;          // 1: part_o holds bf16 values (uint16_t), else fp32
  float* part_ml;             // [B*Hkv, splits, G, 2]   (splits > 1)
  // Balanced partition (MQA, paged, dense): the batch's pages are cut into
  // equal ranges, one per workgroup of a 1-D grid of G; partials then live
  // at rows w (the workgroup's first range piece) and G + w (its last), and
  // unit_desc[b] = {first workgroup, its piece is that workgroup's first (1)
  // or last (0), last workgroup, 0} tells the merge where slot b's pieces are.
  int32_t balanced;
  int32_t* unit_desc;         // [B] int4
  float scale;                // logit scale
  int32_t batch;              // query slots: cached sequences x tq
  int32_t tq;                 // query tokens per cached sequence (>= 1)
  int32_t tps;                // query tokens per slot: 1, or 2 (pairs, hq = 2 x 64 rows)
  int32_t hq;
  int32_t hkv;
  int32_t max_blocks;         // block-table row length / capacity in blocks
  int64_t num_blocks;         // blocks in the paged pool (ids are clamped into it)
  int32_t window;             // 0 = dense
  int32_t splits;             // >= 1
  int32_t chunk_tiles;        // 32-key tiles per split
  int32_t out_f32;            // 1: out is fp32, else bf16
  int64_t k_block_stride;
  int64_t k_head_stride;
  int64_t k_row_stride;       // elements between consecutive keys
  int64_t v_block_stride;
  int64_t v_head_stride;
  int64_t v_row_stride;       // elements between consecutive channels
  int64_t v_seq_stride;       // contiguous V: elements between slots
  int64_t v_chunk_stride;     // elements between consecutive 8-key runs of a channel
  int64_t v_tile_stride;      // contiguous V: elements between consecutive 64-key tiles
};

// One KV-append launch (layouts as for DecodeParams with block_table set,
// or the contiguous layouts when it is null).
struct AppendParams {
  const void* k_new;          // [B, Hkv, d]
  const void* v_new;
  void* k_cache;
  void* v_cache;
  const int32_t* block_table; // nullptr: contiguous
  int32_t* ctx_lens;          // [B], read and advanced
  const float* k_scale;       // [Hkv] (FP8) or nullptr
  const float* v_scale;
  const int32_t* active;      // [B] or nullptr
  int32_t batch;
  int32_t hkv;
  int32_t head_dim;
  int32_t max_blocks;
  int64_t num_blocks;
  int32_t v_sub8;             // 1: V blocks cut into 8-token sub-blocks [8][d][8]
};

}  // namespace mfa

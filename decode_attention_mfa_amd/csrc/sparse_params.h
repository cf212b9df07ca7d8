// Launch parameters of the Step-5 sparse global attention kernels (block
// summaries, top-512 selection, attention over the selected blocks).  Shapes
// are the Step-5 layer's: 64 query heads in 4 KV groups of width 192, an
// indexer of 4 groups x 4 search heads x 256 proxy coordinates, 8-token
// blocks, 512 selected blocks.
#pragma once

#include <cstdint>

#include "kernel_params.h"

namespace mfa {

constexpr int kSparseBlock = 8;        // tokens per historical block
constexpr int kSparseBudget = 512;     // historical blocks selected per (request, group)
constexpr int kSparseGroups = 4;       // provider groups = KV groups
constexpr int kSparseHeads = 4;        // search heads per group
constexpr int kSparseWidth = 256;      // proxy coordinates
constexpr int kSparseMaxCand = 4096;   // candidate blocks per request at most (32768 tokens)
constexpr int kSparseMaxTiles = (kSparseBudget + 1 + 7) / 8;   // 64-key tiles of one (request, group)

struct SparseParams {
  // Attention over the selected tokens: q [B, 64, 192], paged K/V in the
  // GQA layout, block_table, ctx_lens, out, split partials and strides.
  DecodeParams dp;
  const int32_t* sel;       // [B, 4, 512] selected block ids, ascending
  const int32_t* nsel;      // [B, 4] selected blocks
  // Indexer.
  const void* q_idx;        // [B, 4, 4, 256] bf16
  const float* w;           // [B, 4, 4] signed search-head weights
  const uint8_t* summ;      // [B, cap8, 256] E4M3 codes of the block summaries
  uint8_t* summ_out;        // the same array, written by the summary kernel
  const void* k_idx;        // [B, cap, 256] bf16 proxy keys
  const void* z;            // [B, cap, 256] bf16 compression logits
  int32_t cap8;             // summaries per request (cap / 8)
  int32_t new_tokens;       // > 0: summarise only the blocks the last new_tokens tokens completed
  float* scores;            // [B, 4, cap8] fp32 scores (workspace)
  int32_t* sel_out;         // selection outputs
  int32_t* nsel_out;
};

}  // namespace mfa

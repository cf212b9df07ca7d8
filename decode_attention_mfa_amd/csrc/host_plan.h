// Host-side validation and launch planning for the decode entry points.
// Plain C++ with no HIP calls, so every error path can be exercised on a
// machine without a GPU.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/mfa_decode.h"

namespace mfa {

enum class DecodePath : int {
  kMqaShared = 0,   // 64 heads per KV head, d = 256, bf16: shared-tile MFMA kernel
  kGqaSplitKeys = 1,// 16 heads per KV head, d in {192, 256}, bf16: key-split MFMA kernel
  kF32 = 2,         // fp32 storage: vector-ALU kernel
};

struct DecodePlan {
  DecodePath path;
  int32_t group;          // Hq / Hkv
  int32_t splits;         // >= 1
  int32_t chunk_pages;    // 64-key pages per split
  int32_t pages_cap;      // most pages one slot can touch
  size_t part_o_offset;   // bytes into the workspace
  size_t part_ml_offset;
  // Paged calls split the batch's actual pages evenly over splits * B
  // workgroups instead (MQA, dense, heuristic split count): room for two
  // partials per workgroup and one int4 piece descriptor per slot.
  bool balanced;
  size_t unit_desc_offset;
  size_t workspace_bytes; // 0 when splits == 1
};

// Largest chunk a split may cover (block ids cached per workgroup).
constexpr int32_t kMaxChunkPages = 2048;
// Largest query-head count and forced split count a descriptor may carry.
constexpr int32_t kMaxQueryHeads = 1024;
constexpr int32_t kMaxForcedSplits = 16384;
// Heuristic split counts: splitting must take at least this many bf16 K/V
// bytes off each workgroup's share, else the call runs unsplit (measured on
// MI355X: 384 KB saved per workgroup lost to the merge, 512 KB won).
constexpr int64_t kMinSplitSavedBytes = 448 * 1024;
// Workspace regions are aligned to this many bytes.
constexpr size_t kWorkspaceAlign = 256;
// Balanced partition limits: one scan lane per slot (a 512-thread
// workgroup) and at most this many pages per workgroup (piece list in LDS).
constexpr int32_t kMaxBalancedSlots = 512;
constexpr int32_t kMaxBalancedChunk = 512;
// Query tokens per cached sequence a multi-token call takes at most (the
// speculative / MTP verify widths the pages discuss are 2 to a few).
constexpr int32_t kMaxQueryTokens = 16;


// Validate sizes and dtypes (no pointers).  `mqa_entry` applies the MQA
// entry's extra rule Hkv == 1.
mfa_status validate_decode_desc(const mfa_decode_desc* d, int32_t window, bool mqa_entry);

// Validate the pointer arguments of a call whose descriptor is valid.
mfa_status validate_decode_ptrs(const mfa_decode_desc* d, const void* q, const void* k_cache,
                                const void* v_cache, const int32_t* ctx_lens,
                                const float* k_scale, const float* v_scale, const void* out,
                                float scale);

// Path, split count and workspace layout for a valid descriptor.  num_cus is
// only used when desc->num_splits == 0.
// rows_per_head: query rows per (slot, query head) of the descriptor, 2 when
// each slot carries a pair of query tokens (the partials double).
DecodePlan plan_decode(const mfa_decode_desc* d, int32_t window, int32_t num_cus,
                       int32_t rows_per_head = 1);

mfa_status validate_query_proj_desc(const mfa_query_proj_desc* d);

// Validate a KV-append descriptor and its pointers (nothing dereferenced).
mfa_status validate_kv_append(const mfa_kv_append_desc* d, const void* k_new, const void* v_new,
                              const void* k_cache, const void* v_cache, const int32_t* ctx_lens,
                              const float* k_scale, const float* v_scale);

// Upper bound of the down projection's split-K factor (the norm kernel sums
// at most this many partials per element).
constexpr int kMaxQueryKSplits = 8;

struct QueryProjPlan {
  int32_t k_splits;        // split-K factor of the down projection
  size_t y_partial_offset; // fp32 [k_splits, batch, rank]
  size_t r_offset;         // bf16 [batch, rank]
  size_t workspace_bytes;
};

QueryProjPlan plan_query_proj(const mfa_query_proj_desc* d);

}  // namespace mfa

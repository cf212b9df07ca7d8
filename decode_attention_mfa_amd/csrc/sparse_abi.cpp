// C-ABI entry points of the Step-5 sparse global attention (see
// include/mfa_decode.h).  Host validation, then kernels enqueued on the
// caller's stream: no allocation, no synchronisation, no device reads.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>

#include "../../include/mfa_decode.h"
#include "sparse_params.h"

namespace mfa {
hipError_t launch_sparse_summary(const SparseParams& p, hipStream_t stream);
hipError_t launch_sparse_select(const SparseParams& p, hipStream_t stream);
hipError_t launch_sparse_attention(const SparseParams& p, hipStream_t stream);
}  // namespace mfa

namespace {

constexpr size_t kAlign = 256;
constexpr int kHq = 64, kHkv = 4, kD = 192;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

mfa_status validate(const mfa_sparse_desc* d) {
  if (!d) return MFA_ERR_NULL;
  if (d->out_dtype != MFA_BF16 && d->out_dtype != MFA_F32) return MFA_ERR_DTYPE;
  if (d->batch < 0 || d->batch > 16383 || d->max_blocks_per_seq <= 0 ||
      d->max_blocks_per_seq > mfa::kSparseMaxCand / 8 || d->num_blocks < 0 || d->num_splits < 0 ||
      d->num_splits > mfa::kSparseMaxTiles)
    return MFA_ERR_SHAPE;
  return MFA_OK;
}

// Splits of one (request, group)'s at most 65 tiles: one workgroup per
// compute unit at least (256 units), chunks of >= 8 tiles.
int32_t plan_splits(const mfa_sparse_desc* d) {
  if (d->num_splits > 0) return d->num_splits;
  const int units = std::max(1, d->batch * kHkv);
  const int want = (256 + units - 1) / units;
  const int chunk = std::max(8, (mfa::kSparseMaxTiles + want - 1) / want);
  return (mfa::kSparseMaxTiles + chunk - 1) / chunk;
}

struct Plan {
  int32_t splits, chunk;
  size_t part_o, part_ml;
  size_t attn_bytes;   // the attention's split partials
  size_t bytes;        // the workspace: partials or the selection's scores
};

Plan plan(const mfa_sparse_desc* d) {
  Plan pl{};
  pl.splits = plan_splits(d);
  pl.chunk = (mfa::kSparseMaxTiles + pl.splits - 1) / pl.splits;
  if (pl.splits > 1) {
    const size_t rows = (size_t)d->batch * kHkv * pl.splits * 16;
    pl.part_o = 0;
    pl.part_ml = align_up(rows * kD * sizeof(float), kAlign);
    pl.attn_bytes = align_up(pl.part_ml + rows * 2 * sizeof(float), kAlign);
  }
  // The selection's scores [B, 4, cap8] fp32 share the workspace.
  const size_t score_bytes =
      align_up((size_t)d->batch * kHkv * d->max_blocks_per_seq * 8 * sizeof(float), kAlign);
  pl.bytes = std::max(pl.attn_bytes, score_bytes);
  return pl;
}

mfa::SparseParams base_params(const mfa_sparse_desc* d, const int32_t* ctx_lens) {
  mfa::SparseParams p{};
  p.dp.ctx_lens = ctx_lens;
  p.dp.batch = d->batch;
  p.dp.tq = 1;
  p.dp.tps = 1;
  p.dp.hq = kHq;
  p.dp.hkv = kHkv;
  p.dp.max_blocks = d->max_blocks_per_seq;
  p.dp.num_blocks = d->num_blocks;
  p.cap8 = d->max_blocks_per_seq * 8;
  return p;
}

// new_tokens == 0: every complete block; > 0: the blocks the last new_tokens
// tokens of each request completed.
mfa_status summarize(const mfa_sparse_desc* desc, const void* k_idx, const void* z,
                     const int32_t* ctx_lens, int32_t new_tokens, uint8_t* summaries,
                     mfa_stream_t stream) {
  const mfa_status st = validate(desc);
  if (st != MFA_OK || desc->batch == 0) return st;
  if (!k_idx || !z || !ctx_lens || !summaries) return MFA_ERR_NULL;
  if (!aligned16(k_idx) || !aligned16(z) || !aligned16(summaries)) return MFA_ERR_ALIGN;
  mfa::SparseParams p = base_params(desc, ctx_lens);
  p.k_idx = k_idx;
  p.z = z;
  p.summ_out = summaries;
  p.new_tokens = new_tokens;
  return mfa::launch_sparse_summary(p, reinterpret_cast<hipStream_t>(stream)) == hipSuccess
             ? MFA_OK : MFA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

mfa_status mfa_sparse_summarize(const mfa_sparse_desc* desc, const void* k_idx, const void* z,
                                const int32_t* ctx_lens, uint8_t* summaries, mfa_stream_t stream) {
  return summarize(desc, k_idx, z, ctx_lens, 0, summaries, stream);
}

mfa_status mfa_sparse_summarize_new(const mfa_sparse_desc* desc, const void* k_idx,
                                    const void* z, const int32_t* ctx_lens, int32_t new_tokens,
                                    uint8_t* summaries, mfa_stream_t stream) {
  const mfa_status st = validate(desc);
  if (st != MFA_OK) return st;
  if (new_tokens < 1 || (int64_t)new_tokens > (int64_t)desc->max_blocks_per_seq * 64)
    return MFA_ERR_ARG;
  return summarize(desc, k_idx, z, ctx_lens, new_tokens, summaries, stream);
}

mfa_status mfa_sparse_select(const mfa_sparse_desc* desc, const void* q_idx, const float* w,
                             const uint8_t* summaries, const int32_t* ctx_lens, int32_t* selected,
                             int32_t* num_selected, void* workspace, size_t workspace_bytes,
                             mfa_stream_t stream) {
  const mfa_status st = validate(desc);
  if (st != MFA_OK || desc->batch == 0) return st;
  if (!q_idx || !w || !summaries || !ctx_lens || !selected || !num_selected) return MFA_ERR_NULL;
  if (!aligned16(q_idx) || !aligned16(summaries)) return MFA_ERR_ALIGN;
  const Plan pl = plan(desc);
  if (!workspace || workspace_bytes < pl.bytes) return MFA_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign) return MFA_ERR_ALIGN;
  mfa::SparseParams p = base_params(desc, ctx_lens);
  p.scores = static_cast<float*>(workspace);
  p.q_idx = q_idx;
  p.w = w;
  p.summ = summaries;
  p.sel_out = selected;
  p.nsel_out = num_selected;
  return mfa::launch_sparse_select(p, reinterpret_cast<hipStream_t>(stream)) == hipSuccess
             ? MFA_OK : MFA_ERR_LAUNCH;
}

mfa_status mfa_sparse_attention(const mfa_sparse_desc* desc, const void* q, const void* k_cache,
                                const void* v_cache, const int32_t* block_table,
                                const int32_t* ctx_lens, const int32_t* selected,
                                const int32_t* num_selected, void* out, float scale,
                                void* workspace, size_t workspace_bytes, mfa_stream_t stream) {
  const mfa_status st = validate(desc);
  if (st != MFA_OK || desc->batch == 0) return st;
  if (!q || !k_cache || !v_cache || !block_table || !ctx_lens || !selected || !num_selected || !out)
    return MFA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return MFA_ERR_ALIGN;
  if (!std::isfinite(scale)) return MFA_ERR_ARG;
  if (desc->num_blocks <= 0) return MFA_ERR_SHAPE;
  const Plan pl = plan(desc);
  if (pl.attn_bytes > 0 && (!workspace || workspace_bytes < pl.attn_bytes)) return MFA_ERR_WORKSPACE;
  if (workspace && (reinterpret_cast<uintptr_t>(workspace) % kAlign)) return MFA_ERR_ALIGN;
  mfa::SparseParams p = base_params(desc, ctx_lens);
  mfa::DecodeParams& dp = p.dp;
  dp.q = q;
  dp.k = k_cache;
  dp.v = v_cache;
  dp.block_table = block_table;
  dp.out = out;
  dp.out_f32 = desc->out_dtype == MFA_F32;
  dp.scale = scale;
  dp.splits = pl.splits;
  dp.chunk_tiles = pl.chunk;
  if (pl.splits > 1) {
    dp.part_o = reinterpret_cast<float*>(static_cast<char*>(workspace) + pl.part_o);
    dp.part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + pl.part_ml);
  }
  dp.k_block_stride = (int64_t)kHkv * 64 * kD;
  dp.k_head_stride = (int64_t)64 * kD;
  dp.k_row_stride = kD;
  // V^T in 8-token sub-blocks: [num_blocks, 4, 8, 192, 8].
  dp.v_block_stride = (int64_t)kHkv * kD * 64;
  dp.v_head_stride = (int64_t)kD * 64;
  dp.v_row_stride = 8;
  p.sel = selected;
  p.nsel = num_selected;
  return mfa::launch_sparse_attention(p, reinterpret_cast<hipStream_t>(stream)) == hipSuccess
             ? MFA_OK : MFA_ERR_LAUNCH;
}

size_t mfa_sparse_workspace_size(const mfa_sparse_desc* desc) {
  if (validate(desc) != MFA_OK) return 0;
  return plan(desc).bytes;
}

}  // extern "C"

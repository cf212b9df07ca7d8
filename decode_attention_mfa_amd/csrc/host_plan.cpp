// Host-side validation and launch planning (no HIP calls).
#include "host_plan.h"

#include <cmath>

#include "kernel_params.h"

namespace mfa {
namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool is_dtype(int32_t v) { return v == MFA_F32 || v == MFA_BF16 || v == MFA_FP8_E4M3; }

// Which kernel serves (group, d, kv dtype); -1 if none.
int path_for(int32_t group, int32_t d, int32_t kv) {
  if (kv == MFA_F32) return (d > 0 && d <= 256 && d % 4 == 0) ? (int)DecodePath::kF32 : -1;
  if (group == 64 && d == 256) return (int)DecodePath::kMqaShared;
  if (group == 16 && (d == 192 || d == 256)) return (int)DecodePath::kGqaSplitKeys;
  return -1;
}

// FP8 storage: the shared-tile MQA kernel and the per-group kernel read E4M3
// codes (each widens them to bf16 MFMA operands itself); the fp32 path does not.
bool fp8_supported(int path) {
  return path == (int)DecodePath::kMqaShared || path == (int)DecodePath::kGqaSplitKeys;
}

}  // namespace

mfa_status validate_decode_desc(const mfa_decode_desc* d, int32_t window, bool mqa_entry) {
  if (!d) return MFA_ERR_NULL;
  if (!is_dtype(d->q_dtype) || !is_dtype(d->kv_dtype) || !is_dtype(d->out_dtype))
    return MFA_ERR_DTYPE;
  if (d->kv_dtype == MFA_F32) {
    if (d->q_dtype != MFA_F32 || d->out_dtype != MFA_F32) return MFA_ERR_DTYPE;
  } else {
    if (d->q_dtype != MFA_BF16) return MFA_ERR_DTYPE;
    if (d->out_dtype == MFA_FP8_E4M3) return MFA_ERR_DTYPE;
  }
  if (d->batch < 0 || d->num_q_heads <= 0 || d->num_kv_heads <= 0 || d->head_dim <= 0)
    return MFA_ERR_SHAPE;
  if (d->num_q_heads % d->num_kv_heads != 0) return MFA_ERR_SHAPE;
  if (d->page_size != kPage) return MFA_ERR_SHAPE;
  if (d->max_blocks_per_seq <= 0 || d->num_splits < 0 || d->num_blocks < 0) return MFA_ERR_SHAPE;
  // Upper bounds that keep the workspace arithmetic (rows x d x 4 bytes, in
  // 64-bit) far from overflow for any accepted shape.
  if (d->num_q_heads > kMaxQueryHeads || d->num_splits > kMaxForcedSplits) return MFA_ERR_SHAPE;
  if (mqa_entry && d->num_kv_heads != 1) return MFA_ERR_SHAPE;
  // One grid row per (slot, KV head) and one workgroup per (slot, head) on
  // the fp32 path: stay inside the 65535 limit of a grid's y dimension.
  if ((int64_t)d->batch * d->num_kv_heads > 65535 || d->batch > 65535) return MFA_ERR_SHAPE;
  const int path = path_for(d->num_q_heads / d->num_kv_heads, d->head_dim, d->kv_dtype);
  if (path < 0) return MFA_ERR_SHAPE;
  if (d->kv_dtype == MFA_FP8_E4M3 && !fp8_supported(path)) return MFA_ERR_DTYPE;
  if (window < 0) return MFA_ERR_ARG;
  // Element offsets are formed in 64-bit; keep per-slot sizes in 32-bit range.
  if ((int64_t)d->max_blocks_per_seq * kPage > INT32_MAX) return MFA_ERR_SHAPE;
  return MFA_OK;
}

mfa_status validate_decode_ptrs(const mfa_decode_desc* d, const void* q, const void* k_cache,
                                const void* v_cache, const int32_t* ctx_lens,
                                const float* k_scale, const float* v_scale, const void* out,
                                float scale) {
  if (!q || !k_cache || !v_cache || !ctx_lens || !out) return MFA_ERR_NULL;
  if (d->kv_dtype == MFA_FP8_E4M3 && (!k_scale || !v_scale)) return MFA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return MFA_ERR_ALIGN;
  if (!std::isfinite(scale)) return MFA_ERR_ARG;
  return MFA_OK;
}

DecodePlan plan_decode(const mfa_decode_desc* d, int32_t window, int32_t num_cus,
                       int32_t rows_per_head) {
  DecodePlan pl{};
  const int32_t group = d->num_q_heads / d->num_kv_heads;
  pl.path = (DecodePath)path_for(group, d->head_dim, d->kv_dtype);
  pl.group = group;
  int64_t cap = d->max_blocks_per_seq;
  if (window > 0) cap = std::min<int64_t>(cap, ceil_div(window, kPage) + 1);
  pl.pages_cap = (int32_t)cap;

  int64_t splits = 1;
  if (pl.path == DecodePath::kF32) {
    splits = 1;
  } else if (d->num_splits > 0) {
    splits = std::min<int64_t>(d->num_splits, cap);
  } else {
    // One wave of workgroups (one resident per compute unit) at least, with
    // chunks of >= 4 pages (256 keys) so the pipeline prologue is amortised.
    const int64_t units = std::max<int64_t>(1, (int64_t)d->batch * d->num_kv_heads);
    const int64_t cus = std::max<int32_t>(1, num_cus);
    const int64_t want = ceil_div(cus, units);
    const int64_t chunk = std::max<int64_t>(4, ceil_div(cap, want));
    splits = ceil_div(cap, chunk);
    // A split adds the merge kernel and the boundary before it (~4-5 us on
    // MI355X); it pays only when it takes enough work off each workgroup.
    // Work is counted as bf16 K/V bytes per page (FP8 tiles cost about as
    // much compute-wave time as bf16 ones), doubled for two-token slots.
    const int64_t saved = (cap - ceil_div(cap, splits)) * 2 * kPage * d->head_dim * 2 * rows_per_head;
    if (splits > 1 && saved < kMinSplitSavedBytes) splits = 1;
  }
  int64_t chunk = ceil_div(cap, splits);
  // A split caches its block ids (the fp32 kernel walks the table itself and
  // never splits).
  if (pl.path != DecodePath::kF32 && chunk > kMaxChunkPages) chunk = kMaxChunkPages;
  splits = ceil_div(cap, chunk);
  pl.splits = (int32_t)splits;
  pl.chunk_pages = (int32_t)chunk;

  // Lengths live on the device, so a ragged batch cannot be planned here;
  // with the heuristic split count, MQA dense calls let the kernel cut the
  // batch's actual pages evenly instead (paged caches only, decided at the
  // call).
  pl.balanced = pl.splits > 1 && pl.path == DecodePath::kMqaShared && d->num_splits == 0 &&
                window == 0 && d->num_kv_heads == 1 && d->batch <= kMaxBalancedSlots &&
                pl.chunk_pages <= kMaxBalancedChunk && d->max_blocks_per_seq <= (1 << 20);
  if (pl.splits > 1) {
    size_t rows = (size_t)d->batch * d->num_kv_heads * pl.splits * group * rows_per_head;
    if (pl.balanced) rows *= 2;   // two partials per workgroup
    pl.part_o_offset = 0;
    pl.part_ml_offset = align_up(pl.part_o_offset + rows * d->head_dim * sizeof(float), kWorkspaceAlign);
    pl.unit_desc_offset = align_up(pl.part_ml_offset + rows * 2 * sizeof(float), kWorkspaceAlign);
    const size_t desc_bytes = pl.balanced ? (size_t)d->batch * 4 * sizeof(int32_t) : 0;
    pl.workspace_bytes = align_up(pl.unit_desc_offset + desc_bytes, kWorkspaceAlign);
  }
  return pl;
}

mfa_status validate_query_proj_desc(const mfa_query_proj_desc* d) {
  if (!d) return MFA_ERR_NULL;
  if (d->out_dtype != MFA_BF16 && d->out_dtype != MFA_F32) return MFA_ERR_DTYPE;
  if (d->batch < 0 || d->hidden <= 0 || d->rank <= 0 || d->num_heads <= 0 || d->head_dim <= 0)
    return MFA_ERR_SHAPE;
  if (d->hidden % 64 || d->rank % 64 || d->rank > 4096) return MFA_ERR_SHAPE;
  if (((int64_t)d->num_heads * d->head_dim) % 64) return MFA_ERR_SHAPE;
  if (!(d->eps >= 0.f) || !std::isfinite(d->eps)) return MFA_ERR_ARG;
  return MFA_OK;
}

mfa_status validate_kv_append(const mfa_kv_append_desc* d, const void* k_new, const void* v_new,
                              const void* k_cache, const void* v_cache, const int32_t* ctx_lens,
                              const float* k_scale, const float* v_scale) {
  if (!d) return MFA_ERR_NULL;
  const bool combo = (d->new_dtype == MFA_BF16 && (d->kv_dtype == MFA_BF16 || d->kv_dtype == MFA_FP8_E4M3)) ||
                     (d->new_dtype == MFA_F32 && d->kv_dtype == MFA_F32);
  if (!combo) return MFA_ERR_DTYPE;
  if (d->batch < 0 || d->num_kv_heads < 1 || d->head_dim < 4 || d->head_dim > 256 ||
      d->head_dim % 4 || d->page_size != kPage || d->max_blocks_per_seq < 1)
    return MFA_ERR_SHAPE;
  if (d->batch == 0) return MFA_OK;
  if (!k_new || !v_new || !k_cache || !v_cache || !ctx_lens) return MFA_ERR_NULL;
  if (d->kv_dtype == MFA_FP8_E4M3 && (!k_scale || !v_scale)) return MFA_ERR_NULL;
  const uintptr_t elem = d->kv_dtype == MFA_F32 ? 4 : d->kv_dtype == MFA_BF16 ? 2 : 1;
  const uintptr_t new_elem = d->new_dtype == MFA_F32 ? 4 : 2;
  if ((reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new)) % new_elem ||
      (reinterpret_cast<uintptr_t>(k_cache) | reinterpret_cast<uintptr_t>(v_cache)) % elem ||
      reinterpret_cast<uintptr_t>(ctx_lens) % 4)
    return MFA_ERR_ALIGN;
  return MFA_OK;
}

QueryProjPlan plan_query_proj(const mfa_query_proj_desc* d) {
  QueryProjPlan pl{};
  // Split the hidden (K) dimension of the down projection so that it fills
  // the device even at small batch; chunks stay multiples of 64.
  const int64_t kchunks = d->hidden / 64;
  int64_t ks = std::min<int64_t>(kMaxQueryKSplits, kchunks);
  while (kchunks % ks) --ks;
  pl.k_splits = (int32_t)ks;
  pl.y_partial_offset = 0;
  const size_t ybytes = (size_t)ks * d->batch * d->rank * sizeof(float);
  pl.r_offset = align_up(ybytes, kWorkspaceAlign);
  pl.workspace_bytes = align_up(pl.r_offset + (size_t)d->batch * d->rank * 2, kWorkspaceAlign);
  return pl;
}

}  // namespace mfa

// C-ABI entry points of the MFA decode library (see include/mfa_decode.h).
// Each call validates on the host, then only enqueues kernels on the caller's
// stream: no allocation, no synchronisation, no device reads on the host.
#include <hip/hip_runtime.h>

#include <atomic>
#include <climits>

#include "host_plan.h"
#include "kernel_params.h"

namespace mfa {
hipError_t launch_mqa(const DecodeParams& p, bool fp8, hipStream_t stream);
hipError_t launch_gqa(const DecodeParams& p, int d, bool fp8, hipStream_t stream);
hipError_t launch_f32(const DecodeParams& p, int d, hipStream_t stream);
hipError_t launch_combine(const DecodeParams& p, int group, int d, hipStream_t stream);
hipError_t launch_kv_append(const AppendParams& p, int new_dtype, int kv_dtype, hipStream_t stream);
int stream_read_threads();
hipError_t launch_stream_read(const void* src, int64_t bytes, int32_t* sink, int workgroups,
                              hipStream_t stream);
mfa_status query_proj_enqueue(const mfa_query_proj_desc* d, const QueryProjPlan& pl,
                              const void* x, const void* w_down, const void* w_up,
                              const float* gain, void* q_out, void* workspace,
                              hipStream_t stream);
}  // namespace mfa

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

// Compute units of the current device, cached per device (-1 on error).
int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -1;
  if (dev < kMaxDevices) {
    const int cached = g_cu_count[dev].load(std::memory_order_relaxed);
    if (cached > 0) return cached;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return -1;
  if (dev < kMaxDevices) g_cu_count[dev].store(n, std::memory_order_relaxed);
  return n;
}

mfa::DecodeParams make_params(const mfa_decode_desc* d, const mfa::DecodePlan& pl, const void* q,
                              const void* k_cache, const void* v_cache,
                              const int32_t* block_table, const int32_t* ctx_lens,
                              const float* k_scale, const float* v_scale, void* out, float scale,
                              int32_t window, void* workspace, int32_t v_layout = 0) {
  using mfa::kPage;
  mfa::DecodeParams p{};
  p.q = q;
  p.k = k_cache;
  p.v = v_cache;
  p.block_table = block_table;
  p.ctx_lens = ctx_lens;
  p.k_scale = d->kv_dtype == MFA_FP8_E4M3 ? k_scale : nullptr;
  p.v_scale = d->kv_dtype == MFA_FP8_E4M3 ? v_scale : nullptr;
  p.out = out;
  if (pl.splits > 1) {
    p.part_o = reinterpret_cast<float*>(static_cast<char*>(workspace) + pl.part_o_offset);
    p.part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + pl.part_ml_offset);
    if (pl.balanced && block_table) {
      p.balanced = 1;
      p.unit_desc = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + pl.unit_desc_offset);
    }
  }
  p.scale = scale;
  p.batch = d->batch;
  p.tq = 1;
  p.tps = 1;
  p.hq = d->num_q_heads;
  p.hkv = d->num_kv_heads;
  p.max_blocks = d->max_blocks_per_seq;
  p.num_blocks = d->num_blocks;
  p.window = window;
  p.splits = pl.splits;
  p.chunk_tiles = pl.chunk_pages;
  p.out_f32 = d->out_dtype == MFA_F32;
  // A bf16 result needs no more than bf16 partials from the shared-tile
  // kernel (half the partial traffic); an fp32 result keeps fp32 partials.
  p.part_bf16 = pl.path == mfa::DecodePath::kMqaShared && !p.out_f32;
  const int64_t hd = d->head_dim, hkv = d->num_kv_heads;
  if (block_table) {
    p.k_block_stride = hkv * kPage * hd;
    p.k_head_stride = kPage * hd;
    p.k_row_stride = hd;
    p.v_block_stride = hkv * hd * kPage;
    p.v_head_stride = hd * kPage;
    p.v_row_stride = kPage;
    p.v_seq_stride = 0;
    p.v_chunk_stride = 8;
    if (v_layout == MFA_V_SUBBLOCK8) {   // [blocks, Hkv, 8, d, 8]
      p.v_row_stride = 8;
      p.v_chunk_stride = 8 * hd;
    }
  } else {
    const int64_t cap = (int64_t)d->max_blocks_per_seq * kPage;
    p.k_block_stride = kPage * hkv * hd;
    p.k_head_stride = hd;
    p.k_row_stride = hkv * hd;
    p.v_block_stride = 0;
    p.v_head_stride = hd * cap;
    p.v_row_stride = cap;
    p.v_seq_stride = hkv * hd * cap;
    p.v_chunk_stride = 8;
    p.v_tile_stride = kPage;
    if (v_layout == MFA_V_SUBBLOCK8) {   // [B, Hkv, cap / 8, d, 8]
      p.v_row_stride = 8;
      p.v_chunk_stride = 8 * hd;
      p.v_tile_stride = kPage * hd;
    }
  }
  return p;
}

// Descriptor of the query slots of a call with tq query tokens per cached
// sequence.  An even tq > 1 runs batch * tq / 2 slots of two tokens each (one
// K/V read per pair, 2 x Hq query rows per slot); an odd one batch * tq
// single-token slots.  The kernels map a slot back to its sequence and give
// each token its own length.  tq > 1 is built for the shared-KV MQA path.
mfa_status query_slot_desc(const mfa_decode_desc* d, int32_t tq, int32_t window, bool mqa_entry,
                           mfa_decode_desc* vd, int32_t* tps) {
  mfa_status st = mfa::validate_decode_desc(d, window, mqa_entry);
  if (st != MFA_OK) return st;
  if (tq < 1 || tq > mfa::kMaxQueryTokens || (int64_t)d->batch * tq > (int64_t)INT32_MAX)
    return MFA_ERR_SHAPE;
  *tps = (tq % 2 == 0) ? 2 : 1;
  *vd = *d;
  vd->batch = d->batch * (tq / *tps);
  // The query slots, not the sequences, set the grid: apply the size rules
  // (the 65535 limit of a grid's y dimension among them) to them again.
  st = mfa::validate_decode_desc(vd, window, mqa_entry);
  if (st != MFA_OK) return st;
  if (tq > 1 && mfa::plan_decode(vd, window, 1).path != mfa::DecodePath::kMqaShared)
    return MFA_ERR_SHAPE;
  return MFA_OK;
}

// phase: 0 = the whole call, 1 = the attention kernel only, 2 = the merge only.
mfa_status decode_impl(const mfa_decode_desc* d0, int32_t tq, const void* q, const void* k_cache,
                       const void* v_cache, const int32_t* block_table, const int32_t* ctx_lens,
                       const float* k_scale, const float* v_scale, void* out, float scale,
                       int32_t window, void* workspace, size_t workspace_bytes,
                       mfa_stream_t stream, bool mqa_entry, int phase = 0,
                       int32_t v_layout = MFA_V_CHANNEL_MAJOR) {
  if (v_layout != MFA_V_CHANNEL_MAJOR && v_layout != MFA_V_SUBBLOCK8) return MFA_ERR_ARG;
  mfa_decode_desc vd;
  int32_t tps = 1;
  mfa_status st = query_slot_desc(d0, tq, window, mqa_entry, &vd, &tps);
  if (st != MFA_OK) return st;
  const mfa_decode_desc* d = &vd;
  if (d->batch == 0) return MFA_OK;
  st = mfa::validate_decode_ptrs(d, q, k_cache, v_cache, ctx_lens, k_scale, v_scale, out, scale);
  if (st != MFA_OK) return st;
  if (workspace && (reinterpret_cast<uintptr_t>(workspace) % mfa::kWorkspaceAlign))
    return MFA_ERR_ALIGN;
  if (block_table && d->num_blocks <= 0) return MFA_ERR_SHAPE;   // a paged call needs a pool
  int cus = 0;
  if (d->num_splits == 0) {
    cus = device_cu_count();
    if (cus <= 0) return MFA_ERR_LAUNCH;
  }
  const mfa::DecodePlan pl = mfa::plan_decode(d, window, cus, tps);
  // Sub-blocked V is read by the per-group bf16 path only.
  if (v_layout == MFA_V_SUBBLOCK8 && pl.path != mfa::DecodePath::kGqaSplitKeys) return MFA_ERR_SHAPE;
  if (v_layout == MFA_V_SUBBLOCK8 && d->kv_dtype != MFA_BF16) return MFA_ERR_DTYPE;
  if (pl.workspace_bytes > 0 && (!workspace || workspace_bytes < pl.workspace_bytes))
    return MFA_ERR_WORKSPACE;

  mfa::DecodeParams p = make_params(d, pl, q, k_cache, v_cache, block_table, ctx_lens, k_scale,
                                    v_scale, out, scale, window, workspace, v_layout);
  p.tq = tq;
  p.tps = tps;
  p.hq = d->num_q_heads * tps;   // query rows per slot
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (phase != 2) switch (pl.path) {
    case mfa::DecodePath::kMqaShared:
      e = mfa::launch_mqa(p, d->kv_dtype == MFA_FP8_E4M3, s);
      break;
    case mfa::DecodePath::kGqaSplitKeys:
      e = mfa::launch_gqa(p, d->head_dim, d->kv_dtype == MFA_FP8_E4M3, s);
      break;
    case mfa::DecodePath::kF32:
      e = mfa::launch_f32(p, d->head_dim, s);
      break;
  }
  if (e != hipSuccess) return MFA_ERR_LAUNCH;
  if (phase != 1 && pl.splits > 1 && pl.path != mfa::DecodePath::kF32) {
    e = mfa::launch_combine(p, pl.group * tps, d->head_dim, s);
    if (e != hipSuccess) return MFA_ERR_LAUNCH;
  }
  return MFA_OK;
}

}  // namespace

namespace mfa {
// The MQA decode call of mfa_decode_attention, for the library's other entry
// points (the allocation-free variant in noalloc.hip).
mfa_status decode_mqa_entry(const mfa_decode_desc* desc, const void* q, const void* k_cache,
                            const void* v_cache, const int32_t* block_table,
                            const int32_t* ctx_lens, const float* k_scale, const float* v_scale,
                            void* out, float scale, void* workspace, size_t workspace_bytes,
                            mfa_stream_t stream) {
  return decode_impl(desc, 1, q, k_cache, v_cache, block_table, ctx_lens, k_scale, v_scale, out,
                     scale, 0, workspace, workspace_bytes, stream, /*mqa_entry=*/true);
}
}  // namespace mfa

extern "C" {

mfa_status mfa_decode_attention(const mfa_decode_desc* desc, const void* q, const void* k_cache,
                                const void* v_cache, const int32_t* block_table,
                                const int32_t* ctx_lens, const float* k_scale,
                                const float* v_scale, void* out, float scale, void* workspace,
                                size_t workspace_bytes, mfa_stream_t stream) {
  return decode_impl(desc, 1, q, k_cache, v_cache, block_table, ctx_lens, k_scale, v_scale, out,
                     scale, 0, workspace, workspace_bytes, stream, /*mqa_entry=*/true);
}

mfa_status mfa_decode_attention_phase(const mfa_decode_desc* desc, const void* q,
                                      const void* k_cache, const void* v_cache,
                                      const int32_t* block_table, const int32_t* ctx_lens,
                                      const float* k_scale, const float* v_scale, void* out,
                                      float scale, void* workspace, size_t workspace_bytes,
                                      int32_t phase, mfa_stream_t stream) {
  if (phase != 1 && phase != 2) return MFA_ERR_ARG;
  return decode_impl(desc, 1, q, k_cache, v_cache, block_table, ctx_lens, k_scale, v_scale, out,
                     scale, 0, workspace, workspace_bytes, stream, /*mqa_entry=*/true, phase);
}

mfa_status mfa_decode_attention_mtp(const mfa_decode_desc* desc, int32_t num_query_tokens,
                                    const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* block_table, const int32_t* ctx_lens,
                                    const float* k_scale, const float* v_scale, void* out,
                                    float scale, void* workspace, size_t workspace_bytes,
                                    mfa_stream_t stream) {
  return decode_impl(desc, num_query_tokens, q, k_cache, v_cache, block_table, ctx_lens, k_scale,
                     v_scale, out, scale, 0, workspace, workspace_bytes, stream,
                     /*mqa_entry=*/true);
}

size_t mfa_decode_mtp_workspace_size(const mfa_decode_desc* desc, int32_t num_query_tokens) {
  mfa_decode_desc vd;
  int32_t tps = 1;
  if (query_slot_desc(desc, num_query_tokens, 0, true, &vd, &tps) != MFA_OK) return 0;
  int cus = 0;
  if (vd.num_splits == 0) {
    cus = device_cu_count();
    if (cus <= 0) return 0;
  }
  return mfa::plan_decode(&vd, 0, cus, tps).workspace_bytes;
}

mfa_status mfa_decode_attention_gqa(const mfa_decode_desc* desc, const void* q,
                                    const void* k_cache, const void* v_cache,
                                    const int32_t* block_table, const int32_t* ctx_lens,
                                    const float* k_scale, const float* v_scale, void* out,
                                    float scale, int32_t window, void* workspace,
                                    size_t workspace_bytes, mfa_stream_t stream) {
  return decode_impl(desc, 1, q, k_cache, v_cache, block_table, ctx_lens, k_scale, v_scale, out,
                     scale, window, workspace, workspace_bytes, stream, /*mqa_entry=*/false);
}

mfa_status mfa_decode_attention_gqa_layout(const mfa_decode_desc* desc, const void* q,
                                           const void* k_cache, const void* v_cache,
                                           const int32_t* block_table, const int32_t* ctx_lens,
                                           const float* k_scale, const float* v_scale, void* out,
                                           float scale, int32_t window, int32_t v_layout,
                                           void* workspace, size_t workspace_bytes,
                                           mfa_stream_t stream) {
  return decode_impl(desc, 1, q, k_cache, v_cache, block_table, ctx_lens, k_scale, v_scale, out,
                     scale, window, workspace, workspace_bytes, stream, /*mqa_entry=*/false,
                     /*phase=*/0, v_layout);
}

size_t mfa_decode_workspace_size(const mfa_decode_desc* desc, int32_t window) {
  if (mfa::validate_decode_desc(desc, window, false) != MFA_OK) return 0;
  int cus = 0;
  if (desc->num_splits == 0) {
    cus = device_cu_count();
    if (cus <= 0) return 0;
  }
  return mfa::plan_decode(desc, window, cus).workspace_bytes;
}

int32_t mfa_decode_plan_splits(const mfa_decode_desc* desc, int32_t window, int32_t num_cus) {
  if (mfa::validate_decode_desc(desc, window, false) != MFA_OK) return 0;
  return mfa::plan_decode(desc, window, num_cus > 0 ? num_cus : 1).splits;
}

mfa_status mfa_kv_append_layout(const mfa_kv_append_desc* desc, const void* k_new,
                                const void* v_new, void* k_cache, void* v_cache,
                                const int32_t* block_table, int32_t* ctx_lens,
                                const float* k_scale, const float* v_scale, const int32_t* active,
                                int32_t v_layout, mfa_stream_t stream) {
  if (v_layout != MFA_V_CHANNEL_MAJOR && v_layout != MFA_V_SUBBLOCK8) return MFA_ERR_ARG;
  mfa_status st = mfa::validate_kv_append(desc, k_new, v_new, k_cache, v_cache, ctx_lens, k_scale,
                                          v_scale);
  if (st != MFA_OK) return st;
  // Sub-blocked V is the bf16 layout of the per-group and sparse paths.
  if (v_layout == MFA_V_SUBBLOCK8 && desc->kv_dtype != MFA_BF16) return MFA_ERR_DTYPE;
  if (desc->batch == 0) return MFA_OK;
  if (block_table && desc->num_blocks <= 0) return MFA_ERR_SHAPE;   // a paged call needs a pool
  mfa::AppendParams p{};
  p.k_new = k_new;
  p.v_new = v_new;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_table = block_table;
  p.ctx_lens = ctx_lens;
  p.k_scale = desc->kv_dtype == MFA_FP8_E4M3 ? k_scale : nullptr;
  p.v_scale = desc->kv_dtype == MFA_FP8_E4M3 ? v_scale : nullptr;
  p.active = active;
  p.batch = desc->batch;
  p.hkv = desc->num_kv_heads;
  p.head_dim = desc->head_dim;
  p.max_blocks = desc->max_blocks_per_seq;
  p.num_blocks = desc->num_blocks;
  p.v_sub8 = v_layout == MFA_V_SUBBLOCK8;
  const hipError_t e = mfa::launch_kv_append(p, desc->new_dtype, desc->kv_dtype,
                                             reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? MFA_OK : MFA_ERR_LAUNCH;
}

mfa_status mfa_kv_append(const mfa_kv_append_desc* desc, const void* k_new, const void* v_new,
                         void* k_cache, void* v_cache, const int32_t* block_table,
                         int32_t* ctx_lens, const float* k_scale, const float* v_scale,
                         const int32_t* active, mfa_stream_t stream) {
  return mfa_kv_append_layout(desc, k_new, v_new, k_cache, v_cache, block_table, ctx_lens,
                              k_scale, v_scale, active, MFA_V_CHANNEL_MAJOR, stream);
}

mfa_status mfa_query_proj(const mfa_query_proj_desc* desc, const void* x, const void* w_qdown,
                          const void* w_qup, const float* gain, void* q_out, void* workspace,
                          size_t workspace_bytes, mfa_stream_t stream) {
  mfa_status st = mfa::validate_query_proj_desc(desc);
  if (st != MFA_OK) return st;
  if (desc->batch == 0) return MFA_OK;
  if (!x || !w_qdown || !w_qup || !q_out) return MFA_ERR_NULL;
  const uintptr_t mis = reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(w_qdown) |
                        reinterpret_cast<uintptr_t>(w_qup) | reinterpret_cast<uintptr_t>(q_out);
  if (mis & 15u) return MFA_ERR_ALIGN;
  const mfa::QueryProjPlan pl = mfa::plan_query_proj(desc);
  if (!workspace || workspace_bytes < pl.workspace_bytes) return MFA_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) % mfa::kWorkspaceAlign) return MFA_ERR_ALIGN;
  return mfa::query_proj_enqueue(desc, pl, x, w_qdown, w_qup, gain, q_out, workspace,
                                 reinterpret_cast<hipStream_t>(stream));
}

size_t mfa_query_proj_workspace_size(const mfa_query_proj_desc* desc) {
  if (mfa::validate_query_proj_desc(desc) != MFA_OK) return 0;
  return mfa::plan_query_proj(desc).workspace_bytes;
}

mfa_status mfa_stream_read(const void* src, size_t bytes, int32_t* sink, size_t sink_len,
                           mfa_stream_t stream) {
  if (!src || !sink) return MFA_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(src) & 15u) return MFA_ERR_ALIGN;
  if (bytes == 0 || bytes % 16 || bytes > ((size_t)1 << 40)) return MFA_ERR_SHAPE;
  const int wgs = device_cu_count();
  if (wgs <= 0) return MFA_ERR_LAUNCH;
  if (sink_len < (size_t)wgs * (size_t)mfa::stream_read_threads()) return MFA_ERR_SHAPE;
  return mfa::launch_stream_read(src, (int64_t)bytes, sink, wgs, reinterpret_cast<hipStream_t>(stream)) ==
                 hipSuccess
             ? MFA_OK
             : MFA_ERR_LAUNCH;
}

const char* mfa_status_string(mfa_status s) {
  switch (s) {
    case MFA_OK: return "ok";
    case MFA_ERR_NULL: return "a required pointer is NULL";
    case MFA_ERR_DTYPE: return "unsupported dtype or dtype combination";
    case MFA_ERR_SHAPE: return "sizes inconsistent or outside the supported set";
    case MFA_ERR_ALIGN: return "pointer not 16-byte aligned (workspace: 256-byte)";
    case MFA_ERR_ARG: return "invalid argument (negative window or non-finite scale)";
    case MFA_ERR_WORKSPACE: return "workspace missing or too small";
    case MFA_ERR_LAUNCH: return "HIP runtime refused a launch";
  }
  return "unknown status";
}

int32_t mfa_abi_version(void) { return MFA_ABI_VERSION; }

}  // extern "C"

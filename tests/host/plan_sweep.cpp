// Host-side sweep of the decode library's validation and launch planning
// (decode_attention_mfa_amd/csrc/host_plan.cpp), built with AddressSanitizer
// and UndefinedBehaviorSanitizer by tests/test_host_sanitizers.py.  Every
// descriptor of a grid of edge values goes through the validators; every one
// they accept is planned, and the plan's invariants are checked:
//   splits >= 1, 1 <= chunk <= the chunk limit, the chunks cover the slot's
//   pages without an empty one, workspace regions aligned and in order, and
//   no workspace unless the call splits.
// Exit status 0 when every check holds; the sanitizers abort on any
// out-of-bounds access, signed overflow or other undefined behaviour.
#include <cstdint>
#include <cstdio>
#include <algorithm>
#include <cstdlib>
#include <vector>

#include "host_plan.h"

namespace {

int failures = 0;

void check(bool ok, const char* what, const mfa_decode_desc& d, int32_t window) {
  if (ok) return;
  if (++failures <= 20)
    std::fprintf(stderr,
                 "FAIL %s: batch=%d hq=%d hkv=%d d=%d max_blocks=%d num_blocks=%lld splits=%d "
                 "kv=%d window=%d\n",
                 what, d.batch, d.num_q_heads, d.num_kv_heads, d.head_dim, d.max_blocks_per_seq,
                 (long long)d.num_blocks, d.num_splits, d.kv_dtype, window);
}

}  // namespace

int main() {
  const int32_t batches[] = {0, 1, 2, 63, 64, 65, 255, 256, 511, 512, 513, 65535, 65536,
                             INT32_MAX, -1};
  const int32_t heads[][2] = {{64, 1}, {64, 4}, {32, 2}, {128, 2}, {64, 0}, {0, 1}, {63, 4},
                              {8, 8}, {INT32_MAX, 1}};
  const int32_t dims[] = {256, 192, 128, 4, 3, 0, 260, INT32_MAX};
  const int32_t max_blocks[] = {1, 2, 63, 64, 512, 513, 2048, 2049, 4096, 1 << 20,
                                (1 << 20) + 1, INT32_MAX / 64, INT32_MAX / 64 + 1, INT32_MAX, 0,
                                -1};
  const int32_t splits[] = {0, 1, 2, 3, 7, 100, 4096, INT32_MAX, -1};
  const int32_t windows[] = {0, 1, 511, 512, 4096, INT32_MAX, -1};
  const int32_t dtypes[][3] = {{MFA_BF16, MFA_BF16, MFA_BF16}, {MFA_BF16, MFA_FP8_E4M3, MFA_BF16},
                               {MFA_BF16, MFA_BF16, MFA_F32}, {MFA_F32, MFA_F32, MFA_F32},
                               {MFA_F32, MFA_BF16, MFA_BF16}, {MFA_BF16, MFA_FP8_E4M3, MFA_FP8_E4M3},
                               {7, MFA_BF16, MFA_BF16}};
  const int32_t cus[] = {1, 80, 256, 304};
  long planned = 0, refused = 0;
  for (int32_t b : batches)
    for (const auto& h : heads)
      for (int32_t hd : dims)
        for (int32_t mb : max_blocks)
          for (int32_t sp : splits)
            for (int32_t w : windows)
              for (const auto& dt : dtypes) {
                mfa_decode_desc d{};
                d.batch = b;
                d.num_q_heads = h[0];
                d.num_kv_heads = h[1];
                d.head_dim = hd;
                d.page_size = 64;
                d.max_blocks_per_seq = mb;
                d.num_blocks = (int64_t)(b > 0 ? b : 1) * (mb > 0 ? mb : 1);
                d.q_dtype = dt[0];
                d.kv_dtype = dt[1];
                d.out_dtype = dt[2];
                d.num_splits = sp;
                for (bool mqa : {false, true}) {
                  if (mfa::validate_decode_desc(&d, w, mqa) != MFA_OK) {
                    ++refused;
                    continue;
                  }
                  check(!mqa || d.num_kv_heads == 1, "mqa entry took Hkv != 1", d, w);
                  for (int32_t c : cus)
                    for (int32_t rows : {1, 2}) {
                      const mfa::DecodePlan pl = mfa::plan_decode(&d, w, c, rows);
                      ++planned;
                      check(pl.splits >= 1, "splits >= 1", d, w);
                      check(pl.chunk_pages >= 1 && (pl.path == mfa::DecodePath::kF32 ||
                                                    pl.chunk_pages <= mfa::kMaxChunkPages),
                            "chunk within limits", d, w);
                      check(pl.path != mfa::DecodePath::kF32 || pl.splits == 1,
                            "the fp32 path never splits", d, w);
                      check(pl.pages_cap >= 1 && pl.pages_cap <= d.max_blocks_per_seq,
                            "pages_cap within the table", d, w);
                      check((int64_t)pl.splits * pl.chunk_pages >= pl.pages_cap,
                            "chunks cover the pages", d, w);
                      check((int64_t)(pl.splits - 1) * pl.chunk_pages < pl.pages_cap,
                            "no empty chunk", d, w);
                      // A forced count holds unless its chunks would pass the
                      // per-split page limit; then it is the least count that fits.
                      const int64_t least = ((int64_t)pl.pages_cap + mfa::kMaxChunkPages - 1) /
                                            mfa::kMaxChunkPages;
                      check(d.num_splits <= 0 ||
                                pl.splits <= std::max<int64_t>(d.num_splits, least),
                            "forced count is an upper bound", d, w);
                      if (pl.splits == 1) {
                        check(pl.workspace_bytes == 0, "no workspace unsplit", d, w);
                      } else {
                        check(pl.part_ml_offset % mfa::kWorkspaceAlign == 0 &&
                                  pl.unit_desc_offset % mfa::kWorkspaceAlign == 0 &&
                                  pl.workspace_bytes % mfa::kWorkspaceAlign == 0,
                              "aligned regions", d, w);
                        check(pl.part_o_offset <= pl.part_ml_offset &&
                                  pl.part_ml_offset <= pl.unit_desc_offset &&
                                  pl.unit_desc_offset <= pl.workspace_bytes,
                              "ordered regions", d, w);
                        const size_t rows_all = (size_t)d.batch * d.num_kv_heads * pl.splits *
                                                pl.group * rows * (pl.balanced ? 2 : 1);
                        check(pl.part_ml_offset >= rows_all * d.head_dim * sizeof(float),
                              "partials fit", d, w);
                      }
                      check(!pl.balanced || (w == 0 && d.num_kv_heads == 1 && d.num_splits == 0),
                            "balanced cut only for dense MQA with the heuristic", d, w);
                    }
                }
                // The pointer checks never dereference: fake aligned and
                // misaligned addresses exercise every branch.
                const void* a = reinterpret_cast<const void*>(0x10000);
                const void* mis = reinterpret_cast<const void*>(0x10004);
                const int32_t* ai = reinterpret_cast<const int32_t*>(0x10000);
                const float* af = reinterpret_cast<const float*>(0x10000);
                if (mfa::validate_decode_desc(&d, 0, false) == MFA_OK) {
                  check(mfa::validate_decode_ptrs(&d, a, a, a, ai, af, af, const_cast<void*>(a),
                                                  0.0625f) == MFA_OK, "aligned ok", d, 0);
                  check(mfa::validate_decode_ptrs(&d, mis, a, a, ai, af, af, const_cast<void*>(a),
                                                  0.0625f) == MFA_ERR_ALIGN, "misaligned q", d, 0);
                  check(mfa::validate_decode_ptrs(&d, a, a, a, nullptr, af, af,
                                                  const_cast<void*>(a), 0.0625f) == MFA_ERR_NULL,
                        "null lens", d, 0);
                }
              }
  // Query path and KV append descriptors.
  for (int32_t b : batches)
    for (int32_t hidden : {64, 7168, 100, 0, INT32_MAX - 63})
      for (int32_t rank : {64, 2048, 4096, 4160, 0, 63})
        for (int32_t nh : {64, 1, 0, 3}) {
          mfa_query_proj_desc q{};
          q.batch = b;
          q.hidden = hidden;
          q.rank = rank;
          q.num_heads = nh;
          q.head_dim = 256;
          q.eps = 1e-6f;
          q.out_dtype = MFA_BF16;
          if (mfa::validate_query_proj_desc(&q) != MFA_OK) continue;
          const mfa::QueryProjPlan pl = mfa::plan_query_proj(&q);
          if (!(pl.k_splits >= 1 && (hidden / 64) % pl.k_splits == 0 &&
                pl.r_offset % mfa::kWorkspaceAlign == 0 && pl.workspace_bytes >= pl.r_offset)) {
            ++failures;
            std::fprintf(stderr, "FAIL query plan batch=%d hidden=%d rank=%d\n", b, hidden, rank);
          }
        }
  for (int32_t b : batches)
    for (int32_t hd : {4, 192, 256, 260, 2, 0})
      for (int32_t mb : {1, 64, 0, INT32_MAX}) {
        mfa_kv_append_desc a{};
        a.batch = b;
        a.num_kv_heads = 1;
        a.head_dim = hd;
        a.page_size = 64;
        a.max_blocks_per_seq = mb;
        a.num_blocks = 16;
        a.new_dtype = MFA_BF16;
        a.kv_dtype = MFA_FP8_E4M3;
        const void* p = reinterpret_cast<const void*>(0x10000);
        const float* f = reinterpret_cast<const float*>(0x10000);
        (void)mfa::validate_kv_append(&a, p, p, p, p, reinterpret_cast<const int32_t*>(0x10000),
                                      f, f);
        (void)mfa::validate_kv_append(&a, p, p, p, p, reinterpret_cast<const int32_t*>(0x10000),
                                      nullptr, f);
      }
  std::printf("planned %ld descriptors, refused %ld, failures %d\n", planned, refused, failures);
  return failures == 0 ? 0 : 1;
}

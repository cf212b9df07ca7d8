/*
 * mfa_decode.h -- C ABI of the MI355X (gfx950) MFA decode-attention library.
 *
 * What the library computes
 *   One decode step of Multi-matrix Factorization Attention (MFA): every slot
 *   of the batch contributes one new query token with Hq = 64 heads of width
 *   d = 256, and all heads attend to ONE shared K head and ONE shared V head
 *   over the slot's whole cache ("Step-3 is Large yet Affordable",
 *   section 2 "Step-3 model card", Table 1).  For head h and slot b with
 *   L = ctx_lens[b] keys:
 *       s_j   = scale * <q[b,h,:], K_j>             j in [lo, L)
 *       out   = sum_j softmax(s)_j * V_j
 *   with lo = 0 (dense) or max(0, L - window) for a sliding window that counts
 *   the current token ("Step-5-Preview: Sparse GQA, Indexer und
 *   KV-Speicher", backbone table and the attention equation of section
 *   "Die eigentliche Attention liest weiterhin originale K/V", which also
 *   gives the GQA head-to-group map g(h) = floor(h / (Hq/Hkv))).
 *   L counts the token appended in this step (duck-llm chapter 7, section
 *   7.6: the decode kernel must see cached_len + 1).
 *
 * Cache layouts (P = page_size = 64 tokens per block; d contiguous for K,
 * tokens contiguous for V -- V blocks are channel-major so that a 16-byte
 * load gives 8 consecutive keys of one channel, the operand shape of the
 * PV matrix product):
 *   paged       K: [num_blocks, Hkv, P, d]      V: [num_blocks, Hkv, d, P]
 *               logical position j of slot b is row j % P of block
 *               block_table[b * max_blocks_per_seq + j / P]
 *   contiguous  (block_table == NULL)
 *               K: [B, cap, Hkv, d]             V: [B, Hkv, d, cap]
 *               with cap = max_blocks_per_seq * P
 *   Rows at positions >= L inside a slot's last block may hold anything,
 *   NaN included: they never reach the result.  Block-table entries past the
 *   last block a slot uses do not affect the result either, but the kernels
 *   may read them ahead of the length (prefetch and speculation): they must
 *   be readable memory, and whatever they hold is clamped into the pool
 *   before any cache access (callers pad with -1, which reads block 0).
 *
 * Ownership, streams, graphs
 *   The caller owns every buffer (device memory for all data pointers).  The
 *   library allocates nothing during a call, keeps no pointer after it
 *   returns, reads no device data on the host and never synchronises: a call
 *   only validates its arguments on the host and enqueues kernels on
 *   `stream` (NULL = the null stream).  ctx_lens and the block table are read
 *   by the kernels when they execute, so a captured graph replays correctly
 *   after the caller updates them in place (the graph-state hazards of
 *   duck-llm chapter 7, section 7.5).
 *
 * Errors
 *   Problems detectable on the host return a non-zero mfa_status and enqueue
 *   nothing.  Device-side contract violations (a block id outside the pool,
 *   L > max_blocks_per_seq * P, L < 0) give unspecified values for that
 *   slot but never an out-of-bounds access: ids outside [0, num_blocks)
 *   read block 0 and lengths are clamped into [0, max_blocks_per_seq * P].
 */
#ifndef MFA_DECODE_H
#define MFA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MFA_ABI_VERSION 1

/* A hipStream_t (struct ihipStream_t*).  NULL means the null stream. */
struct ihipStream_t;
typedef struct ihipStream_t* mfa_stream_t;

typedef enum mfa_status {
  MFA_OK = 0,
  MFA_ERR_NULL = 1,        /* a required pointer is NULL                         */
  MFA_ERR_DTYPE = 2,       /* unsupported dtype or dtype combination             */
  MFA_ERR_SHAPE = 3,       /* sizes inconsistent or outside the supported set    */
  MFA_ERR_ALIGN = 4,       /* a data pointer is not 16-byte aligned              */
  MFA_ERR_ARG = 5,         /* other invalid argument (negative window, bad scale)*/
  MFA_ERR_WORKSPACE = 6,   /* workspace missing or smaller than required         */
  MFA_ERR_LAUNCH = 7       /* the HIP runtime refused a launch                   */
} mfa_status;

typedef enum mfa_dtype {
  MFA_F32 = 0,             /* IEEE binary32                                      */
  MFA_BF16 = 1,            /* bfloat16                                           */
  MFA_FP8_E4M3 = 2         /* OCP FP8 E4M3FN (bias 7, max 448, 0x7F/0xFF NaN)    */
} mfa_dtype;

/*
 * Shape and type of one decode-attention call.
 *   batch               B >= 0 slots (B == 0 enqueues nothing)
 *   num_q_heads         Hq, at most 1024
 *   num_kv_heads        Hkv, Hq % Hkv == 0
 *   head_dim            d
 *   page_size           tokens per cache block; must be 64
 *   max_blocks_per_seq  paged: length (= row stride) of each block-table row;
 *                       contiguous: cache capacity / 64
 *   num_blocks          paged: blocks in each pool (>= 1; block ids are
 *                       clamped into it); contiguous: ignored
 *   q_dtype, kv_dtype, out_dtype
 *                       supported: kv BF16 or FP8_E4M3 with q BF16 and out
 *                       BF16 or F32; kv F32 with q F32 and out F32
 *   num_splits          0 = choose with the library's heuristic
 *                       (mfa_decode_plan_splits); > 0 forces that many splits
 *                       of each slot's key range (at most the slot's pages,
 *                       and at least enough that no split covers more than
 *                       2048 pages, the block ids one split caches); at
 *                       most 16384.  With 0, a paged dense MQA
 *                       call (Hkv == 1, B <= 512, at most 512 pages per
 *                       split) instead spreads the batch's actual pages
 *                       evenly over the same number of workgroups, reading
 *                       ctx_lens on the device (ragged batches keep every
 *                       compute unit busy); results then depend on the
 *                       lengths only, and are bit-identical across runs.
 * Supported (Hq/Hkv, d): (64, 256) on the shared-tile MFMA path (MQA);
 * (16, 192), (16, 256) on the per-group MFMA path (GQA); any Hq/Hkv and any
 * d <= 256 that is a multiple of 4 with F32 storage.  Both MFMA paths read
 * BF16 or FP8_E4M3 caches (one fp32 scale per KV head).
 */
typedef struct mfa_decode_desc {
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t page_size;
  int32_t max_blocks_per_seq;
  int64_t num_blocks;
  int32_t q_dtype;
  int32_t kv_dtype;
  int32_t out_dtype;
  int32_t num_splits;
} mfa_decode_desc;

/*
 * MFA decode attention (the MQA case, Hkv == 1, dense).
 *   q            [B, Hq, d]            q_dtype, contiguous
 *   k_cache      K pool / static cache (layouts above), kv_dtype
 *   v_cache      V pool / static cache (layouts above), kv_dtype
 *   block_table  [B, max_blocks_per_seq] int32 physical block ids, or NULL
 *                for a contiguous cache
 *   ctx_lens     [B] int32, keys per slot including the current token
 *   k_scale      FP8 only: [Hkv] fp32 per-KV-head dequantisation scales
 *   v_scale      (stored value = code * scale); NULL otherwise
 *   out          [B, Hq, d]            out_dtype, written in full
 *                (a slot with L == 0 gets zeros)
 *   scale        logit scale, finite (1/sqrt(d) for both pages' models)
 *   workspace    device scratch of at least mfa_decode_workspace_size(desc,0)
 *                bytes, 256-byte aligned; may be NULL when that size is 0.
 *                Calls that share a workspace must be ordered on one stream.
 * All data pointers must be 16-byte aligned.
 * Returns MFA_ERR_SHAPE when num_kv_heads != 1.
 */
mfa_status mfa_decode_attention(const mfa_decode_desc* desc, const void* q,
                                const void* k_cache, const void* v_cache,
                                const int32_t* block_table, const int32_t* ctx_lens,
                                const float* k_scale, const float* v_scale, void* out,
                                float scale, void* workspace, size_t workspace_bytes,
                                mfa_stream_t stream);

/*
 * mfa_decode_attention in its two launches, for callers that place work
 * between them or time them apart: phase 1 enqueues the attention kernel
 * (the split partials go to the workspace; with one split it writes out),
 * phase 2 enqueues the merge of those partials into out (nothing with one
 * split).  Arguments as mfa_decode_attention, identical for both phases and
 * the same device; phase 2 must follow phase 1 on the stream with the
 * workspace untouched in between.  Other phase values return MFA_ERR_ARG.
 */
mfa_status mfa_decode_attention_phase(const mfa_decode_desc* desc, const void* q,
                                      const void* k_cache, const void* v_cache,
                                      const int32_t* block_table, const int32_t* ctx_lens,
                                      const float* k_scale, const float* v_scale, void* out,
                                      float scale, void* workspace, size_t workspace_bytes,
                                      int32_t phase, mfa_stream_t stream);

/*
 * mfa_decode_attention for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation and kernels, with the split partials in
 * a library-owned device array of MFA_NOALLOC_SCRATCH_BYTES per GPU instead
 * of a caller workspace.  The call allocates and frees nothing.  Arguments as
 * mfa_decode_attention, less the workspace.  Returns MFA_ERR_WORKSPACE when
 * the call would need more than the array (mfa_decode_workspace_size(desc,
 * 0) > MFA_NOALLOC_SCRATCH_BYTES; e.g. forced split counts on large
 * batches), and MFA_ERR_LAUNCH if the array's device address cannot be
 * obtained.  Every call on one GPU shares that GPU's array: calls that
 * overlap on one GPU (several streams, several host threads) race and must
 * be serialised by the caller.  The array holds the last call's partials
 * until the process ends; no call needs it cleared.
 */
#define MFA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

mfa_status mfa_decode_attention_noalloc(const mfa_decode_desc* desc, const void* q,
                                        const void* k_cache, const void* v_cache,
                                        const int32_t* block_table, const int32_t* ctx_lens,
                                        const float* k_scale, const float* v_scale, void* out,
                                        float scale, mfa_stream_t stream);

/*
 * Multi-token queries per slot (MTP / speculative verification, "Step-3 is
 * Large yet Affordable", section 5.2: MTP raises the attention's arithmetic
 * intensity).  Each cached sequence b has num_query_tokens = Tq new query
 * tokens, already appended: they are its last Tq cached keys, and token t
 * attends keys [0, L_b - (Tq - 1 - t)), causal among the new tokens (a
 * token with no key left gets zeros).  desc->batch counts sequences.
 *   q            [B, Tq, Hq, d]        q_dtype, contiguous
 *   out          [B, Tq, Hq, d]        out_dtype, written in full
 *   ctx_lens     [B] int32, keys per sequence including all Tq new tokens
 * Everything else as mfa_decode_attention (Hkv == 1, dense), with the
 * workspace of mfa_decode_mtp_workspace_size(desc, Tq).  Built on the shared
 * K/V path: bf16 or FP8 E4M3 caches, Hq = 64, d = 256; other shapes, or
 * Tq outside [1, 16], return MFA_ERR_SHAPE.  Tq == 1 is mfa_decode_attention.
 */
mfa_status mfa_decode_attention_mtp(const mfa_decode_desc* desc, int32_t num_query_tokens,
                                    const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* block_table, const int32_t* ctx_lens,
                                    const float* k_scale, const float* v_scale, void* out,
                                    float scale, void* workspace, size_t workspace_bytes,
                                    mfa_stream_t stream);

/* Workspace bytes of mfa_decode_attention_mtp with this descriptor and Tq
 * (0 for an invalid descriptor); device queries as mfa_decode_workspace_size. */
size_t mfa_decode_mtp_workspace_size(const mfa_decode_desc* desc, int32_t num_query_tokens);

/*
 * GQA / sliding-window variant: as mfa_decode_attention, for any supported
 * Hkv (head h reads KV group floor(h / (Hq/Hkv))) and window >= 0
 * (0 = dense; W > 0 attends to keys [max(0, L - W), L - 1]).
 */
mfa_status mfa_decode_attention_gqa(const mfa_decode_desc* desc, const void* q,
                                    const void* k_cache, const void* v_cache,
                                    const int32_t* block_table, const int32_t* ctx_lens,
                                    const float* k_scale, const float* v_scale, void* out,
                                    float scale, int32_t window, void* workspace,
                                    size_t workspace_bytes, mfa_stream_t stream);

/*
 * Layouts of a V pool, for the entries that take a v_layout argument.
 *   MFA_V_CHANNEL_MAJOR  paged [num_blocks, Hkv, d, 64], contiguous
 *                        [B, Hkv, d, cap] (the layout of every other entry)
 *   MFA_V_SUBBLOCK8      paged [num_blocks, Hkv, 8, d, 8], contiguous
 *                        [B, Hkv, cap/8, d, 8]: token j of a 64-token block
 *                        sits in 8-token sub-block j / 8 at column j % 8
 *                        (the V layout of mfa_sparse_attention)
 * Both keep the 8 tokens of one channel in 16 contiguous bytes (bf16).
 */
typedef enum mfa_v_layout {
  MFA_V_CHANNEL_MAJOR = 0,
  MFA_V_SUBBLOCK8 = 1
} mfa_v_layout;

/*
 * mfa_decode_attention_gqa with the V pool in layout v_layout.  With
 * MFA_V_SUBBLOCK8 one cache of the Step-5 global layer (K [num_blocks, 4, 64,
 * 192], V [num_blocks, 4, 8, 192, 8]) serves this dense call, the sparse
 * call mfa_sparse_attention and the append mfa_kv_append_layout: the dense
 * global layer and the sparse path attend to the same original K/V
 * ("Step-5-Preview: Sparse GQA, Indexer und KV-Speicher", section "Die
 * eigentliche Attention liest weiterhin originale K/V").  The result is
 * bit-identical to the channel-major call on the same values.
 * MFA_V_SUBBLOCK8 is read by the per-group bf16 path only ((Hq/Hkv, d) =
 * (16, 192) or (16, 256)); other shapes return MFA_ERR_SHAPE and an E4M3
 * cache MFA_ERR_DTYPE.  Other v_layout values return MFA_ERR_ARG.
 */
mfa_status mfa_decode_attention_gqa_layout(const mfa_decode_desc* desc, const void* q,
                                           const void* k_cache, const void* v_cache,
                                           const int32_t* block_table, const int32_t* ctx_lens,
                                           const float* k_scale, const float* v_scale, void* out,
                                           float scale, int32_t window, int32_t v_layout,
                                           void* workspace, size_t workspace_bytes,
                                           mfa_stream_t stream);

/* Workspace bytes a call with this descriptor and window needs (0 when every
 * slot fits one split; room for the even page partition when num_splits is 0
 * and the call may use it).  Pure host arithmetic: no HIP call is made when
 * desc->num_splits > 0; otherwise the current device's compute-unit count is
 * queried once and cached. */
size_t mfa_decode_workspace_size(const mfa_decode_desc* desc, int32_t window);

/* The split heuristic (host integers only): how many chunks each slot's key
 * range is cut into, given the device's compute-unit count.  Aims for
 * B * Hkv * splits at or above one wave of workgroups on `num_cus` compute
 * units, with chunks at least 256 keys long, and runs unsplit (1) when the
 * split would take less than 448 KB of bf16-sized K/V off each workgroup
 * (the merge kernel would cost more than it saves).  Returns >= 1, or 0 if
 * desc is NULL or invalid. */
int32_t mfa_decode_plan_splits(const mfa_decode_desc* desc, int32_t window, int32_t num_cus);

/*
 * KV append with a device-owned length counter: the step just before decode
 * attention in a decode loop (duck-llm chapter 7, section 7.6: the decode
 * context kernel writes the new token's K/V and owns the active length, which
 * then counts the token; section 7.5: state that lives on the device keeps a
 * captured graph valid from step to step).
 *   batch               B >= 0 slots (B == 0 enqueues nothing)
 *   num_kv_heads        Hkv >= 1
 *   head_dim            d, 4 <= d <= 256, multiple of 4
 *   page_size           must be 64
 *   max_blocks_per_seq  paged: length (= row stride) of each block-table row;
 *                       contiguous: cache capacity / 64
 *   num_blocks          paged: blocks in each pool (>= 1); contiguous: ignored
 *   new_dtype           dtype of k_new / v_new: BF16 for BF16 or FP8_E4M3
 *                       caches, F32 for F32 caches
 *   kv_dtype            cache dtype: BF16, FP8_E4M3 or F32
 */
typedef struct mfa_kv_append_desc {
  int32_t batch;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t page_size;
  int32_t max_blocks_per_seq;
  int64_t num_blocks;
  int32_t new_dtype;
  int32_t kv_dtype;
} mfa_kv_append_desc;

/*
 * For every slot b, with pos = ctx_lens[b] read on the device:
 *   K row pos of slot b, head g    <- k_new[b, g, :]
 *   V column pos of slot b, head g <- v_new[b, g, :]
 *   ctx_lens[b]                    <- pos + 1
 * where row pos lives in block block_table[b, pos / 64] at row pos % 64
 * (paged) or at position pos of slot b (contiguous), in the cache layouts of
 * mfa_decode_attention (V channel-major).  BF16 and F32 values are copied
 * bit for bit.  FP8: code = E4M3FN(x / scale) with the quotient taken in
 * fp32, rounded to the nearest code (ties to the even code) and saturated to
 * +-448; NaN stays NaN.
 *   k_new, v_new   [B, Hkv, d] new_dtype, contiguous
 *   k_cache, v_cache, block_table   as for mfa_decode_attention (block_table
 *                  NULL: contiguous cache)
 *   ctx_lens       [B] int32 on the device: read, then advanced by one
 *   k_scale, v_scale   FP8 only: [Hkv] fp32 scales (stored = code * scale);
 *                  NULL otherwise
 *   active         NULL (every slot appends) or [B] int32, 0 = skip the slot
 * A slot is left untouched (nothing written, length unchanged) when it is
 * inactive, when pos < 0 or pos >= max_blocks_per_seq * 64, or (paged) when
 * its block id lies outside [0, num_blocks).  One kernel is enqueued on
 * `stream`; no allocation, no synchronisation, nothing read on the host, so
 * the call can be captured in a graph together with the decode call.  Calls
 * that share ctx_lens must be ordered on one stream.  Data pointers must be
 * aligned to their element size.
 */
mfa_status mfa_kv_append(const mfa_kv_append_desc* desc, const void* k_new, const void* v_new,
                         void* k_cache, void* v_cache, const int32_t* block_table,
                         int32_t* ctx_lens, const float* k_scale, const float* v_scale,
                         const int32_t* active, mfa_stream_t stream);

/*
 * mfa_kv_append with the V pool in layout v_layout (mfa_v_layout): the new
 * token's V column goes to sub-block pos % 64 / 8, column pos % 8 under
 * MFA_V_SUBBLOCK8, which needs a BF16 cache (other dtypes return
 * MFA_ERR_DTYPE); other v_layout values return MFA_ERR_ARG.  Values are
 * copied bit for bit, as by mfa_kv_append.
 */
mfa_status mfa_kv_append_layout(const mfa_kv_append_desc* desc, const void* k_new,
                                const void* v_new, void* k_cache, void* v_cache,
                                const int32_t* block_table, int32_t* ctx_lens,
                                const float* k_scale, const float* v_scale, const int32_t* active,
                                int32_t v_layout, mfa_stream_t stream);

/*
 * Low-rank MFA query path ("Step-3 is Large yet Affordable", section 2):
 *     y = x W_qdown^T;  r = y / sqrt(mean(y^2) + eps) * gain;  q = r W_qup^T
 * and q is viewed as [B, num_heads, head_dim] (head h = output columns
 * h*head_dim .. h*head_dim + head_dim - 1).
 *   x        [batch, hidden]                      bf16, row-major
 *   w_qdown  [rank, hidden]                       bf16, row-major ("out, in")
 *   w_qup    [num_heads * head_dim, rank]         bf16, row-major ("out, in")
 *   gain     [rank] fp32, or NULL for unit gain
 *   q_out    [batch, num_heads * head_dim]        out_dtype (BF16 or F32)
 *   workspace >= mfa_query_proj_workspace_size(desc) bytes, 256-byte aligned
 * Supported: hidden % 64 == 0, rank % 64 == 0, rank <= 4096,
 * (num_heads * head_dim) % 64 == 0.
 */
typedef struct mfa_query_proj_desc {
  int32_t batch;
  int32_t hidden;
  int32_t rank;
  int32_t num_heads;
  int32_t head_dim;
  float eps;
  int32_t out_dtype;
} mfa_query_proj_desc;

mfa_status mfa_query_proj(const mfa_query_proj_desc* desc, const void* x, const void* w_qdown,
                          const void* w_qup, const float* gain, void* q_out, void* workspace,
                          size_t workspace_bytes, mfa_stream_t stream);

size_t mfa_query_proj_workspace_size(const mfa_query_proj_desc* desc);

/*
 * Step-5 sparse global attention for one decode token per request
 * ("Step-5-Preview: Sparse GQA, Indexer und KV-Speicher", the indexer and
 * attention sections).  Shapes are the Step-5 layer's: 64 query heads in 4 KV
 * groups of width 192 (bf16, paged like mfa_decode_attention_gqa), an indexer
 * of 4 provider groups x 4 search heads x 256 proxy coordinates, 8-token
 * blocks and 512 selected blocks.  The decode token of request b sits at
 * t = L - 1, L = ctx_lens[b] (counting it).  Three calls:
 *   mfa_sparse_summarize  block summaries c[r] of the complete blocks
 *   mfa_sparse_select     weighted-ReLU scores and the causal top-512
 *   mfa_sparse_attention  softmax attention over the selected original K/V
 */
typedef struct mfa_sparse_desc {
  int32_t batch;               /* requests B                                     */
  int32_t max_blocks_per_seq;  /* 64-token pages per request (<= 512: 32K tokens)*/
  int64_t num_blocks;          /* blocks in the paged K/V pool                   */
  int32_t out_dtype;           /* MFA_BF16 or MFA_F32                            */
  int32_t num_splits;          /* 0 = heuristic, else forced (1..65)             */
} mfa_sparse_desc;

/*
 * Summaries of every complete block r < floor(L / 8) of each request:
 * c[r, d] = sum_j softmax_j(z[8r + j, d]) k_idx[8r + j, d] over the block's 8
 * tokens, per coordinate d, in fp32, rounded to bf16 and stored as the
 * nearest E4M3FN code (ties to even, saturating).
 *   k_idx, z    [B, max_blocks_per_seq * 64, 256] bf16 proxy keys and
 *               compression logits, token-major
 *   summaries   [B, max_blocks_per_seq * 8, 256] uint8 E4M3 codes; entries of
 *               incomplete or absent blocks are left as they are
 */
mfa_status mfa_sparse_summarize(const mfa_sparse_desc* desc, const void* k_idx, const void* z,
                                const int32_t* ctx_lens, uint8_t* summaries, mfa_stream_t stream);

/*
 * Summaries of only the blocks that the last new_tokens tokens of each
 * request completed: blocks r with floor((L - new_tokens) / 8) <= r <
 * floor(L / 8), L = ctx_lens[b] read on the device (so a captured graph stays
 * valid as the lengths advance).  Each is computed exactly as by
 * mfa_sparse_summarize; every other entry of `summaries` is left as it is.
 * Decode summarises a block when its eighth token arrives ("Step-5-Preview:
 * Sparse GQA, Indexer und KV-Speicher", section "Acht Tokens ergeben einen
 * Such-Key"): a decode loop calls this with new_tokens = 1 after each
 * append, and with Tq after appending Tq tokens.  new_tokens outside
 * [1, max_blocks_per_seq * 64] returns MFA_ERR_ARG.
 */
mfa_status mfa_sparse_summarize_new(const mfa_sparse_desc* desc, const void* k_idx,
                                    const void* z, const int32_t* ctx_lens, int32_t new_tokens,
                                    uint8_t* summaries, mfa_stream_t stream);

/*
 * Scores s[g, r] = sum_h w[g, h] ReLU(Q8(q_idx[g, h]) . c[r]) for the
 * candidate blocks r < floor(t / 8), Q8 the E4M3 rounding (fp32 sums), and
 * per group the 512 highest, equal scores to the lower block id.
 *   q_idx          [B, 4, 4, 256] bf16 search queries
 *   w              [B, 4, 4] fp32 signed search-head weights (prescale included)
 *   summaries      as written by mfa_sparse_summarize
 *   selected       [B, 4, 512] int32: the selected block ids, ascending
 *   num_selected   [B, 4] int32: min(candidates, 512)
 *   workspace      at least mfa_sparse_workspace_size(desc) bytes, 256-byte
 *                  aligned (the fp32 scores); the same workspace serves
 *                  mfa_sparse_attention when both are ordered on one stream
 */
mfa_status mfa_sparse_select(const mfa_sparse_desc* desc, const void* q_idx, const float* w,
                             const uint8_t* summaries, const int32_t* ctx_lens, int32_t* selected,
                             int32_t* num_selected, void* workspace, size_t workspace_bytes,
                             mfa_stream_t stream);

/*
 * out[b, h] = softmax attention of q[b, h] over J[t, g(h)]: the tokens of the
 * selected blocks and of the current block up to t, g(h) = floor(h / 16).
 *   q            [B, 64, 192] bf16
 *   k_cache      [num_blocks, 4, 64, 192] bf16 (as the GQA entry)
 *   v_cache      [num_blocks, 4, 8, 192, 8] bf16: V^T per 8-token sub-block
 *                (token j of a block: sub-block (j % 64) / 8, column j % 8),
 *                so a selected block's V is one contiguous 3 KB read
 *   block_table  [B, max_blocks_per_seq] int32
 *   selected, num_selected   as written by mfa_sparse_select (ids outside the
 *                candidates are clamped into them; counts into [0, 512])
 *   out          [B, 64, 192] out_dtype; a request with L == 0 gets zeros
 *   workspace    at least mfa_sparse_workspace_size(desc) bytes, 256-aligned
 */
mfa_status mfa_sparse_attention(const mfa_sparse_desc* desc, const void* q, const void* k_cache,
                                const void* v_cache, const int32_t* block_table,
                                const int32_t* ctx_lens, const int32_t* selected,
                                const int32_t* num_selected, void* out, float scale,
                                void* workspace, size_t workspace_bytes, mfa_stream_t stream);

/* Workspace bytes of mfa_sparse_select and mfa_sparse_attention (the larger
 * of the scores and the attention's split partials; 0 for a bad desc). */
size_t mfa_sparse_workspace_size(const mfa_sparse_desc* desc);

/*
 * Read-rate reference (measurement only; not part of a decode call).  Reads
 * the `bytes` bytes at `src` once, the way the decode kernels stream their
 * tiles: 16-byte non-temporal loads, the buffer cut into one contiguous
 * range per workgroup, one workgroup of 512 threads per compute unit.  Timed
 * over a decode call's byte count, it gives the read rate a kernel with no
 * other work reaches on this device: a practical reference below the
 * published HBM peak for the memory-bound MFA decode ("Step-3 is Large yet
 * Affordable", section 5.1), not a bound (a kernel with more bytes in flight
 * can match or pass it).
 *   src       device memory, 16-byte aligned; bytes > 0, a multiple of 16
 *   sink      int32 [sink_len] device memory; sink_len >= num_cus * 512,
 *             where num_cus is the current device's compute-unit count.
 *             Thread t of workgroup w writes sink[512 w + t] = the XOR of
 *             every 32-bit word it read, so the XOR of sink[0 .. 512 num_cus)
 *             equals the XOR of all 32-bit words of the buffer.
 * Enqueues one kernel on `stream`; errors as for the decode calls (NULL
 * pointers MFA_ERR_NULL, misaligned src MFA_ERR_ALIGN, sizes MFA_ERR_SHAPE).
 */
mfa_status mfa_stream_read(const void* src, size_t bytes, int32_t* sink, size_t sink_len,
                           mfa_stream_t stream);

/* Static, never-NULL description of a status code. */
const char* mfa_status_string(mfa_status status);

/* MFA_ABI_VERSION of the built library. */
int32_t mfa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MFA_DECODE_H */

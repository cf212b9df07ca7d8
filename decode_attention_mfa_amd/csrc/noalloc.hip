// mfa_decode_attention without a caller workspace, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc): the split partials live in a file-scope
// device array, one per GPU, held until the process ends.
//
// The array's name in host code is a host-side stand-in, not a device
// address.  Its device address is looked up once per device, with that
// device current, by hipGetSymbolAddress, and only that pointer is handed to
// the kernels.  Every call on a GPU shares that GPU's array: calls that
// overlap on one GPU race.  Nothing in it needs clearing between calls:
// every value a call reads from it (split partials, piece descriptors) is
// written earlier in the same call.
#include <hip/hip_runtime.h>

#include <mutex>

#include "host_plan.h"

namespace mfa {
mfa_status decode_mqa_entry(const mfa_decode_desc* desc, const void* q, const void* k_cache,
                            const void* v_cache, const int32_t* block_table,
                            const int32_t* ctx_lens, const float* k_scale, const float* v_scale,
                            void* out, float scale, void* workspace, size_t workspace_bytes,
                            mfa_stream_t stream);
}  // namespace mfa

namespace {

constexpr size_t kScratchBytes = (size_t)64 << 20;   // MFA_NOALLOC_SCRATCH_BYTES
static_assert(kScratchBytes == MFA_NOALLOC_SCRATCH_BYTES, "header and library agree on the limit");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];   // device address of scratch, per device (null: not looked up)

// This device's copy of the array (nullptr on a HIP error).
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" mfa_status mfa_decode_attention_noalloc(const mfa_decode_desc* desc, const void* q,
                                                   const void* k_cache, const void* v_cache,
                                                   const int32_t* block_table,
                                                   const int32_t* ctx_lens, const float* k_scale,
                                                   const float* v_scale, void* out, float scale,
                                                   mfa_stream_t stream) {
  // Host-side checks first (nothing enqueued, no HIP call on an invalid
  // descriptor); a workspace larger than the array is refused.
  mfa_status st = mfa::validate_decode_desc(desc, 0, /*mqa_entry=*/true);
  if (st != MFA_OK) return st;
  if (desc->batch == 0) return MFA_OK;
  if (mfa_decode_workspace_size(desc, 0) > kScratchBytes) return MFA_ERR_WORKSPACE;
  void* ws = device_scratch();
  if (!ws) return MFA_ERR_LAUNCH;
  return mfa::decode_mqa_entry(desc, q, k_cache, v_cache, block_table, ctx_lens, k_scale, v_scale,
                               out, scale, ws, kScratchBytes, stream);
}

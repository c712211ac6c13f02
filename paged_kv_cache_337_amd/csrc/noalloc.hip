// pa_decode_noalloc: pa_decode on a static device scratch, for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid allocation).
//
// The decode path's workspace -- work list, per-sequence partition counts,
// shared groups and float32 partition states -- lives in `scratch`, a
// file-scope device array of kScratchBytes.  Every device the library runs
// this entry point on holds its own copy of the array until the process ends.
// In host code the name `scratch` is only a stand-in for the device symbol:
// the array's device address is asked for once per device, with that device
// current, and that address is what the kernels receive.  All calls on one
// device share the array and it keeps the last call's contents; nothing in it
// needs to start at zero (the plan kernel writes every field the decode and
// merge kernels read).  Calls that overlap on one device race.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "api_internal.hpp"
#include "pa.h"

namespace {

constexpr size_t kScratchBytes = size_t{128} << 20;  // 128 MiB per device
constexpr int kMaxDevices = 64;

static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each device (NULL: not asked yet)

// Device address of the scratch on the current device, asked for on the first
// call made with that device current.
int current_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return pa::set_error(PA_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return pa::set_error(PA_ERR_UNSUPPORTED, "device " + std::to_string(dev) + " beyond the scratch table");
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return pa::set_error(PA_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return PA_OK;
}

}  // namespace

extern "C" {

size_t pa_decode_noalloc_scratch_bytes(void) { return kScratchBytes; }

int pa_decode_noalloc(const pa_pool* pool, int layer, const void* q, int num_seqs, int num_q_heads,
                      const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens,
                      int max_context_len, float scale, int partition_tokens, void* out, void* stream) {
  if (!pool) return pa::set_error(PA_ERR_INVALID_ARG, "pool is NULL");
  void* ws = nullptr;
  const int rc = current_scratch(&ws);
  if (rc != PA_OK) return rc;
  return pa::decode_call(pool, layer, q, num_seqs, num_q_heads, block_tables, max_blocks_per_seq, context_lens,
                         max_context_len, scale, partition_tokens, ws, kScratchBytes, out, stream, true);
}

}  // extern "C"

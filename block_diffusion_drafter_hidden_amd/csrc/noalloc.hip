// dflash_draft_block without a workspace argument: the draft step's scratch (residual
// stream, q / block K / V, attention partials, SwiGLU output, argmax partials, k-split
// partials) lives in one file-scope device array instead, for callers that cannot
// allocate device memory.  The array's device address is looked up once per device and
// handed to the kernels like any workspace; host code never passes the array's name.
#include <hip/hip_runtime.h>

#include <mutex>

#include "dflash.h"

namespace {

constexpr size_t kScratchBytes = DFLASH_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void* g_scratch[kMaxDevices];   // device address of `scratch` on each device, once looked up

// The scratch address on the current device (looked up on the first call there).
dflash_status scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DFLASH_ERR_HIP;
  std::lock_guard<std::mutex> hold(g_lock);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DFLASH_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return DFLASH_OK;
}

}  // namespace

extern "C" {

size_t dflash_noalloc_scratch_bytes(void) { return kScratchBytes; }

dflash_status dflash_draft_block_noalloc(const dflash_config* cfg, const void* packed,
                                         const void* embed, const dflash_kv_cache* cache,
                                         const int32_t* anchor_ids, int32_t batch,
                                         int32_t* draft_ids, float* top2_gap,
                                         float* logits_out, hipStream_t stream) {
  if (!cfg || !cache || batch <= 0) return DFLASH_ERR_INVALID_ARG;
  // Sizes beyond the array are refused before anything is looked up or launched.
  const size_t need = dflash_workspace_size(cfg, batch, 0, cache->max_pages_per_seq * 16);
  if (need == 0) return DFLASH_ERR_INVALID_ARG;
  if (need > kScratchBytes) return DFLASH_ERR_WORKSPACE;
  void* ws = nullptr;
  const dflash_status st = scratch_on_current_device(&ws);
  if (st != DFLASH_OK) return st;
  return dflash_draft_block(cfg, packed, embed, cache, anchor_ids, batch, draft_ids, top2_gap,
                            logits_out, ws, kScratchBytes, stream);
}

}  // extern "C"

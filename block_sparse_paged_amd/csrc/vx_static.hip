// The decode step for callers that cannot allocate device memory: code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
// vx_sparse_decode_step_static is vx_sparse_decode_step with the workspace
// taken from a file-scope device array instead of the caller.
//
// In host code the array's name is only a host-side stand-in: its device
// address is looked up once per device with hipGetSymbolAddress (each GPU
// holds its own copy of the array) and only that address is handed to the
// kernels.  Nothing here allocates: no hipMalloc, no hipFree, no library
// routine that allocates.
#include <hip/hip_runtime.h>

#include <mutex>

#include "vx.h"
#include "vx_internal.h"

namespace {

constexpr size_t kScratchBytes = VX_STATIC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

// Workspace of every vx_sparse_decode_step_static call on this device (the
// five benchmark workloads need at most 17 MB).  Held until the process ends.
__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of the current device's `scratch`, looked up on the first
// call with that device current.
vx_status scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return VX_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return VX_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return VX_OK;
}

}  // namespace

extern "C" {

vx_status vx_sparse_decode_step_static(const vx_paged_kv* kv, const vx_batch* batch,
                                       const void* q, int32_t topk, int32_t n_bos, int32_t n_eos,
                                       int32_t update_completed, float sm_scale, int32_t* sel,
                                       void* out, float* lse, hipStream_t stream) {
  if (topk < 0 || n_bos < 0 || n_eos < 1 || (long long)topk + n_bos + n_eos > 0x7fffffffLL)
    return VX_ERR_INVALID_ARGUMENT;
  size_t need = 0;
  vx_status st = vx_workspace_size(VX_OP_DECODE_STEP, kv, batch, topk + n_bos + n_eos, &need);
  if (st != VX_OK) return st;
  if (need > kScratchBytes) return VX_ERR_WORKSPACE_TOO_SMALL;
  if (batch->batch == 0)      // nothing to launch: leave the device untouched
    return vx_sparse_decode_step(kv, batch, q, topk, n_bos, n_eos, update_completed, sm_scale,
                                 sel, out, lse, nullptr, 0, stream);
  void* ws = nullptr;
  if ((st = scratch_ptr(&ws)) != VX_OK) return st;
  return vx_sparse_decode_step(kv, batch, q, topk, n_bos, n_eos, update_completed, sm_scale, sel,
                               out, lse, ws, kScratchBytes, stream);
}

}  // extern "C"

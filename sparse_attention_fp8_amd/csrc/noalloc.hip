// dsa_forward_noalloc: the whole path with its scratch in a fixed device array.
//
// dsa_forward takes its scratch (chunk scores, selected positions, the split
// partials of the decode attention) from a caller-provided workspace.  Callers that
// cannot allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation) use this variant instead: the scratch is the
// file-scope array below, kScratchBytes long, which every GPU the library runs on
// holds until the process ends.  The kernels are those of dsa_forward.
#include <hip/hip_runtime.h>

#include <mutex>

#include "dsa.h"
#include "dsa_internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;   // 64 MiB per device
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// Device address of each GPU's copy of `scratch`.  In host code the array's name is
// only a stand-in for the device symbol, so kernels are always given the address
// that hipGetSymbolAddress reports for the current device.
std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices] = {};

hipError_t scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

dsa_status dsa_forward_noalloc(const dsa_rows* rows, const dsa_dims* dims, const void* q_idx,
                               const float* q_scale, const float* w, const void* k_idx,
                               const float* k_scale, const void* q, const void* latent,
                               float softmax_scale, void* out, float* lse, int32_t* indices_out,
                               int32_t chunk_rows, void* stream) {
  // a call whose arguments are invalid reports that (size 0) through dsa_forward
  const size_t need = dsa_forward_workspace_size(rows, dims, chunk_rows);
  if (need > kScratchBytes)
    return dsa::set_error(DSA_E_WORKSPACE,
                          "dsa_forward_noalloc needs %zu scratch bytes; its fixed scratch holds "
                          "%zu (use fewer rows per chunk, or dsa_forward with a workspace)",
                          need, kScratchBytes);
  void* ptr = nullptr;
  const hipError_t err = scratch_of_current_device(&ptr);
  if (err != hipSuccess)
    return dsa::set_error(DSA_E_HIP, "scratch address: %s", hipGetErrorString(err));
  return dsa_forward(rows, dims, q_idx, q_scale, w, k_idx, k_scale, q, latent, softmax_scale, out,
                     lse, indices_out, chunk_rows, ptr, kScratchBytes, stream);
}

}  // extern "C"

// dv_layer_step_noalloc: dv_layer_step with its scratch memory in a fixed device array of
// the library instead of a caller workspace, for callers that cannot allocate device memory
// (code under stream capture, tight serving loops, harnesses that forbid allocation).
//
// The array `scratch` is a file-scope device variable: the loader places one copy in every
// GPU's memory when the library's code object is loaded there, and it stays until the
// process ends. In host code its name is only a host-side stand-in; the device address of
// each GPU's copy comes from hipGetSymbolAddress, taken once per device (with that device
// current) and kept in a fixed table, and only that address is ever handed to kernels.
//
// Every call on one GPU shares that GPU's copy, which keeps the last call's contents: calls
// that overlap on one GPU (two streams, two host threads, one stream captured while another
// runs) race on it. The layer step needs nothing in its scratch to start at zero (it writes
// everything it reads), so no clearing is done.
#include <mutex>

#include "dejavu_hip.h"
#include "dv_kernels.h"

namespace {

constexpr size_t kScratchBytes = DV_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_setup_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` on each GPU (null: not set up yet)

// The current device's copy of `scratch`, looked up on the first call on that device.
dv_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return dv::record_error(DV_ERR_HIP, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return dv::record_error(DV_ERR_HIP, "device ordinal beyond the scratch table");
  std::lock_guard<std::mutex> lk(g_setup_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return dv::record_error(DV_ERR_HIP, e != hipSuccess ? hipGetErrorString(e) : "scratch has no device address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DV_OK;
}

}  // namespace

extern "C" dv_status dv_layer_step_noalloc(const dv_dims* dims, const dv_layer* layer, const dv_predictor* pred,
                                           const float* x, const float* x_pred, int32_t B, int32_t k, int32_t kh,
                                           const int32_t* idx_in, const int32_t* heads_in, void* k_cache,
                                           void* v_cache, int32_t t_past, float* x_out, int32_t* idx_out,
                                           int32_t* heads_out, hipStream_t stream) {
  // Sizes beyond the array are refused before any HIP call. Invalid arguments size to 0 and
  // are reported by dv_layer_step's own checks, which run before it touches the scratch.
  const size_t need = dv_workspace_bytes(dims, B, k, kh);
  if (need > kScratchBytes)
    return dv::record_error(DV_ERR_WORKSPACE,
                            "dv_layer_step_noalloc: this shape and batch need more scratch than the library's "
                            "fixed DV_NOALLOC_SCRATCH_BYTES array; use dv_layer_step with a workspace");
  void* ws = nullptr;
  if (need > 0) {
    const dv_status s = scratch_of_current_device(&ws);
    if (s != DV_OK) return s;
  }
  return dv_layer_step(dims, layer, pred, x, x_pred, B, k, kh, idx_in, heads_in, k_cache, v_cache, t_past, x_out,
                       idx_out, heads_out, ws, ws != nullptr ? kScratchBytes : 0, stream);
}

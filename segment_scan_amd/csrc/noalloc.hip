// noalloc.hip -- the seam step for callers that cannot allocate device memory.
//
// hypic_seam_step_noalloc is hypic_seam_step with its workspace (the delta
// family's per-window records) taken from a fixed device array of this library
// instead of a caller buffer.  The array is a file-scope __device__ variable:
// every GPU the library runs on holds its own copy from the code object's load
// until the process ends, at an address known only on the device, so the host
// asks for it once per device with hipGetSymbolAddress and passes that address
// -- never the array's name, which in host code is only a stand-in -- to the
// kernels.  Nothing here allocates or frees memory.
#include "../../include/hypic.h"

#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.h"

namespace {

constexpr size_t kScratchBytes = (size_t)64 << 20;  // HYPIC_NOALLOC_SCRATCH_BYTES
static_assert(kScratchBytes == HYPIC_NOALLOC_SCRATCH_BYTES, "header and library agree on the scratch size");

__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];  // device address of `scratch` on each device, once looked up

// Address of this device's copy of the array (current device), or NULL with *err set.
void* scratch_ptr(hipError_t* err) {
  int dev = -1;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace

extern "C" hypic_status hypic_seam_step_noalloc(hypic_family fam, int n_seg, int w, int n_chain, int d_k,
                                                 int d_v, const hypic_tokens* seam, const hypic_cpairs* body,
                                                 float* S_run, float* o_out, const hypic_pairs* window_out,
                                                 void* stream) {
  size_t need = 0;
  hypic_status st = hypic_seam_step_workspace_size(fam, n_seg, w, n_chain, d_k, d_v, &need);
  if (st != HYPIC_OK) return st;
  if (need > kScratchBytes)
    return hypic::report_error(HYPIC_E_INVALID,
                               "hypic_seam_step_noalloc: the window records need %zu bytes, more than the %zu "
                               "of the library's fixed scratch (fewer segments or chains per call)",
                               need, kScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    hipError_t e = hipSuccess;
    ws = scratch_ptr(&e);
    if (!ws)
      return hypic::report_error(HYPIC_E_HIP, "hypic_seam_step_noalloc: scratch address: %s", hipGetErrorString(e));
  }
  return hypic_seam_step(fam, n_seg, w, n_chain, d_k, d_v, seam, body, S_run, o_out, window_out, ws,
                         need > 0 ? kScratchBytes : 0, stream);
}

// omq_lwc_backward_noalloc: the weight-side straight-through backward with its
// partial buffers in a fixed device array instead of a caller workspace, for
// callers that cannot allocate device memory.
//
// The array lives in the library's device code object: every GPU the library runs
// on holds its own copy, at its own address, until the process ends.  Host code
// never passes the array's name to a kernel (on the host that name is a stand-in,
// not a device address): the device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and kept.
#include "api_util.h"

#include <mutex>

using namespace omq;

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;   // 64 MiB per device
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// the current device's address of the array (looked up on its first use there)
int scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return OMQ_E_HIP;
  if (dev < 0 || dev >= kMaxDevices) return OMQ_E_UNIMPLEMENTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return OMQ_E_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return OMQ_OK;
}

}  // namespace

extern "C" {

size_t omq_noalloc_scratch_bytes(void) { return kScratchBytes; }

int omq_lwc_backward_noalloc(const float* gW_hat, const void* W, int w_dt, int64_t c_out,
                             int64_t c_in, int64_t group, int n_bits, const float* a_gamma,
                             const float* a_beta, const float* s, const float* h, const float* z,
                             const int32_t* arg_max, const int32_t* arg_min,
                             const float* dy_colsum, float* g_a_gamma, float* g_a_beta,
                             float* g_s, float* g_delta, void* stream) {
  if (c_out < 0 || c_in <= 0) return OMQ_E_SHAPE;
  // the partials this shape needs must fit the fixed array
  if (omq_lwc_backward_workspace_size(c_out, c_in) > kScratchBytes) return OMQ_E_WORKSPACE;
  void* ws = nullptr;
  const int rc = scratch_ptr(&ws);
  if (rc) return rc;
  // every partial and record is written before it is read: nothing to clear
  return omq_lwc_backward(gW_hat, W, w_dt, c_out, c_in, group, n_bits, a_gamma, a_beta, s, h,
                          z, arg_max, arg_min, dy_colsum, g_a_gamma, g_a_beta, g_s, g_delta, ws,
                          kScratchBytes, stream);
}

}  // extern "C"

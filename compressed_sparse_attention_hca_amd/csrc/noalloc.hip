// csa_fwd_noalloc: the fused CSA layer with its workspace in a static device array, for
// callers that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid allocation).  The kernels are those of csa_fwd;
// only the workspace differs.
//
// `scratch` is a file-scope device array, so the loader gives each GPU its own copy
// when the library's code object is loaded there, and it lives until the process
// ends.  In host code its name stands for a host-side shadow, not a device address:
// the device address is looked up once per device with hipGetSymbolAddress (with that
// device current) and that pointer is what the kernels receive.  Every call on one
// GPU shares that GPU's copy, and the workspace needs no clearing (every kernel writes
// the part it later reads), so calls that overlap on one GPU race: a caller keeps them
// on one stream or orders them.
#include <hip/hip_runtime.h>

#include <mutex>

#include "csa.h"
#include "validate.hpp"

namespace {

// The workspace of the headline shape (CSA, B = 1, S = 65536, D = 512 in bf16,
// top-512 with the FP8 indexer or the indexer prologue) is 210 MiB; 256 MiB covers it
// with room for the alignment of its regions.
constexpr size_t kScratchBytes = size_t(256) << 20;
static_assert(kScratchBytes == CSA_NOALLOC_SCRATCH_BYTES, "header and library agree on the size");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// Device address of this GPU's copy of `scratch`, looked up on the first call there.
csa_status_t scratch_for(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) {
    csa::set_error("device %d is beyond the %d devices the static workspace table holds", dev, kMaxDevices);
    return CSA_ERR_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
    void* ptr = nullptr;
    if (e == hipSuccess) e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    const hipError_t e2 = (cur >= 0 && cur != dev) ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess || e2 != hipSuccess || !ptr) {
      csa::set_error("static workspace lookup on device %d: %s", dev,
                     hipGetErrorString(e != hipSuccess ? e : e2));
      return CSA_ERR_HIP;
    }
    g_ptr[dev] = ptr;
  }
  *out = g_ptr[dev];
  return CSA_OK;
}

}  // namespace

extern "C" csa_status_t csa_fwd_noalloc(const csa_params_t* p, const csa_inputs_t* in, void* o, void* stream) {
  // invalid params (their status and message) and empty batches: csa_fwd needs no
  // workspace to report or to do nothing
  const size_t need = csa_workspace_bytes(p, CSA_OP_CSA_FWD);
  if (need == 0) return csa_fwd(p, in, o, nullptr, 0, stream);
  if (need > kScratchBytes) {
    csa::set_error("this shape needs %zu bytes of workspace; the static workspace holds %zu "
                   "(use csa_fwd with a caller workspace)", need, kScratchBytes);
    return CSA_ERR_WORKSPACE;
  }
  hipDevice_t dev = 0;
  const hipError_t e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev);
  if (e != hipSuccess) {
    csa::set_error("device of the stream: %s", hipGetErrorString(e));
    return CSA_ERR_HIP;
  }
  void* ws = nullptr;
  const csa_status_t s = scratch_for((int)dev, &ws);
  if (s != CSA_OK) return s;
  return csa_fwd(p, in, o, ws, kScratchBytes, stream);
}

// noalloc.hip - qgemm_noalloc: the qgemm_ex computation for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc).  It runs the same kernels as
// qgemm_ex; the only difference is where the split-K partials live: a fixed
// array in each device's copy of the code object instead of a workspace that
// the library allocates or the caller passes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <vector>

#include "../../include/qgemm.h"
#include "internal.h"

namespace qg {

// The fp32 split-K partials of qgemm_noalloc.  On the host the name `scratch`
// only stands in for the symbol; host code uses the per-device address that
// hipGetSymbolAddress returns, never the name itself.
static __device__ __align__(256) uint8_t scratch[QGEMM_NOALLOC_SCRATCH_BYTES];

static std::mutex g_scratch_mutex;
static std::vector<void*> g_scratch_ptr;   // device address of `scratch`, per device

// Address of this device's `scratch`, looked up once per device with that
// device current (each device holds its own copy at its own address).
static int scratch_address(int dev, void** out) {
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if ((int)g_scratch_ptr.size() <= dev) g_scratch_ptr.resize(dev + 1, nullptr);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const int st = hip_status(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
    if (st != QG_OK) {
      clear_pending_error();
      return st;
    }
    if (!ptr) return QG_E_DEVICE;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return QG_OK;
}

}  // namespace qg

using namespace qg;

extern "C" int qgemm_noalloc(const uint16_t* x, int ldx, const uint32_t* packed,
                             const uint16_t* scales, const uint16_t* zeros,
                             const uint16_t* residual, int ldr, int M, int N, int K, int group,
                             int fmt, uint16_t* y, int ldy, void* stream) {
  const Call c{x, ldx, packed, scales, zeros, residual, ldr, M, N, K, group, fmt, y, ldy};
  Plan p;
  int st = validate_call(c, &p);
  if (st != QG_OK) return st;
  if (p.ws_bytes() > QGEMM_NOALLOC_SCRATCH_BYTES) return QG_E_WORKSPACE;
  if (M == 0 || N == 0) return QG_OK;   // no-op, no HIP call
  int dev = 0;
  st = current_device(&dev);
  if (st != QG_OK) return st;
  st = call_pointers_ok(c);
  if (st != QG_OK) return st;
  void* ws = nullptr;
  if (p.ws_bytes() > 0) {
    st = scratch_address(dev, &ws);
    if (st != QG_OK) return st;
  }
  // the partials are written in full by every split before the reduce reads
  // them, so nothing in `scratch` needs clearing between calls
  return launch_call(c, p, reinterpret_cast<float*>(ws), stream);
}

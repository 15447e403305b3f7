// ld_latent_decode_noalloc: the decode step for callers that cannot allocate device memory (code
// under graph capture, tight serving loops, harnesses that forbid allocation).  It is
// ld_latent_decode with the workspace taken from a fixed device array of this library instead of a
// caller buffer.  See include/latent_decode.h.
#include <hip/hip_runtime.h>

#include <mutex>

#include "ld_internal.h"

// The workspace of every ld_latent_decode_noalloc call on a device: the split partials, the plan
// arrays and the combine counters.  Each device holds its own copy for as long as the process
// lives.  Host code never passes `scratch` itself (on the host it is only a stand-in symbol): the
// device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) char scratch[LD_NOALLOC_SCRATCH_BYTES];

namespace {

struct DeviceScratch {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
DeviceScratch g_scratch[ld::kMaxDevices];

// Device address of `scratch` on the current device (looked up on the first call on that device).
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= ld::kMaxDevices) return hipErrorInvalidDevice;
  DeviceScratch& d = g_scratch[dev];
  std::call_once(d.once, [&d] {
    void* p = nullptr;
    d.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    d.ptr = p;
  });
  *out = d.ptr;
  return d.err;
}

}  // namespace

extern "C" int32_t ld_latent_decode_noalloc(const ld_problem* p, const void* q_latent, const void* q_rope,
                                           const ld_kv_cache* cache, const int32_t* block_table,
                                           const int32_t* seq_lens, void* out, float* lse, void* stream) {
  // the problem must fit the fixed array; sizes are checked before anything touches the device
  size_t need = 0;
  const int32_t st = ld_workspace_size(p, &need);
  if (st != LD_OK) return st;
  if (need > (size_t)LD_NOALLOC_SCRATCH_BYTES) return LD_ERR_WORKSPACE_TOO_SMALL;
  if (p->batch == 0) return LD_OK;
  void* ws = nullptr;
  if (scratch_address(&ws) != hipSuccess || ws == nullptr) return LD_ERR_HIP;
  return ld_latent_decode(p, q_latent, q_rope, cache, block_table, seq_lens, out, lse, ws,
                          (size_t)LD_NOALLOC_SCRATCH_BYTES, stream);
}

// osdn_forward_noalloc: the OSDN forward with the library's own static device
// scratch in place of a caller workspace, for callers that cannot allocate
// (work captured into HIP graphs, tight serving loops, harnesses that forbid
// hipMalloc). The scratch is a file-scope device array: every device the
// library runs on holds one copy, from module load until the process ends.
// Its device address is looked up once per device, on the first call made
// with that device current, and kept; the array's name is never passed to a
// kernel or a copy (in host code it is only a stand-in for the symbol).
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/osdn.h"

namespace {

static __device__ __align__(256) unsigned char scratch[OSDN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

struct ScratchTable {
  std::mutex mu;
  void* ptr[kMaxDevices] = {};
};

ScratchTable& table() {
  static ScratchTable t;
  return t;
}

// Device address of this device's scratch (nullptr if the runtime fails).
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  ScratchTable& t = table();
  std::lock_guard<std::mutex> g(t.mu);
  if (!t.ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    t.ptr[dev] = p;
  }
  return t.ptr[dev];
}

}  // namespace

extern "C" int osdn_forward_noalloc(int B, int H, int T, int Dk, int Dv,
                                    int chunk, int dtype, const void* q,
                                    const void* k, const void* v,
                                    const float* beta, const float* r,
                                    float eta, const float* d0, const float* S0,
                                    float scale, void* o, float* S_T,
                                    float* d_T, float* rho, float* q_geo,
                                    void* stream) {
  if (B < 0 || H < 0 || T < 0) return OSDN_ERR_BAD_DIMS;
  if (!osdn_forward_supported(Dk, Dv, chunk, dtype)) return OSDN_ERR_UNSUPPORTED;
  const size_t need = osdn_forward_workspace_bytes(B, H, T, Dk, Dv, chunk, dtype);
  if (need > (size_t)OSDN_NOALLOC_SCRATCH_BYTES) return OSDN_ERR_WORKSPACE;
  if ((size_t)B * H == 0) return OSDN_OK;  // nothing to do, no device touched
  void* ws = nullptr;
  if (need > 0) {
    ws = scratch_ptr();
    if (!ws) return OSDN_ERR_HIP;
  }
  return osdn_forward(B, H, T, Dk, Dv, chunk, dtype, q, k, v, beta, r, eta, d0,
                      S0, scale, o, S_T, d_T, rho, q_geo, ws,
                      (size_t)OSDN_NOALLOC_SCRATCH_BYTES, stream);
}

// Static device scratch of the allocation-free step entry point.
//
// orthrus_step_noalloc stages its step metadata and its decode-attention
// partial results here instead of in buffers it would otherwise grow with
// hipMalloc.  The array is a file-scope __device__ object: every device the
// library runs on holds its own copy, at its own address, from module load
// until the process ends.  Host code never passes the array's name to a
// kernel or a copy (on the host that name is only a stand-in for the
// device symbol); it uses the address hipGetSymbolAddress returns for the
// device, resolved once per device when an engine is created there.
#include <hip/hip_runtime.h>

#include <mutex>

#include "orthrus_internal.h"

namespace orthrus {

static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
void *g_addr[MAX_DEVICES] = {};
}  // namespace

int noalloc_scratch_init(int device) {
  if (device < 0 || device >= MAX_DEVICES) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_addr[device]) return (int)hipSuccess;
  int cur = -1;
  hipError_t r = hipGetDevice(&cur);
  if (r != hipSuccess) return (int)r;
  if (cur != device) return (int)hipErrorInvalidDevice;  // the caller makes `device` current
  void *p = nullptr;
  r = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (r != hipSuccess) return (int)r;
  if (!p) return (int)hipErrorInvalidSymbol;
  g_addr[device] = p;
  return (int)hipSuccess;
}

void *noalloc_scratch(int device) {
  if (device < 0 || device >= MAX_DEVICES) return nullptr;
  std::lock_guard<std::mutex> lk(g_mu);
  return g_addr[device];
}

}  // namespace orthrus

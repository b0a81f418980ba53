// Static device scratch for kla_chunk_fwd_noalloc: the prefill workspace (chunk
// records, and on the scan path the segment maps and start states) for callers that
// cannot allocate device memory.
//
// The buffer is a file-scope device array, so every GPU the library runs on holds
// its own copy, of KLA_NOALLOC_SCRATCH_BYTES, from the loading of this code object
// until the process ends. In host code the array's name is only a host-side handle:
// its device address on the current device comes from hipGetSymbolAddress, looked up
// once per device (with that device current) on the entry point's first call there
// and kept. Kernels receive that address, never the name.
#include <mutex>

#include "kla.h"
#include "kla_launch.h"

namespace kla {
namespace {

static __device__ __align__(256) uint8_t scratch[KLA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 64;
std::once_flag g_once[kMaxScratchDevices];
void* g_addr[kMaxScratchDevices] = {};
hipError_t g_err[kMaxScratchDevices] = {};

}  // namespace

hipError_t scratch_buffer(void** addr, size_t* bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    const hipError_t err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_err[dev] = err;
    if (err == hipSuccess) g_addr[dev] = p;
  });
  if (g_err[dev] != hipSuccess) return g_err[dev];
  if (!g_addr[dev]) return hipErrorNotInitialized;
  *addr = g_addr[dev];
  *bytes = sizeof scratch;
  return hipSuccess;
}

}  // namespace kla

// Library-owned scratch for the entry point that allocates nothing
// (gqa_decode_attn_noalloc): the split partials of the attention call live in
// a file-scope device array instead of a caller-supplied workspace.
//
// Each GPU the library runs on holds its own copy of `scratch` for the life of
// the process.  In host code the array's name is only a host-side stand-in,
// so its device address is looked up once per device (with that device
// current) through hipGetSymbolAddress and cached; kernels receive that
// address, never the name.  Every call on one GPU shares that GPU's copy:
// calls that may overlap on one GPU race on it.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/decode_attn.h"
#include "kernels.h"

namespace da {
namespace {

constexpr size_t kScratchBytes = DA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_lock;
void* g_ptr[kMaxDevices] = {};

}  // namespace

size_t noalloc_scratch_bytes() { return kScratchBytes; }

int noalloc_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return (int)err;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> guard(g_lock);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return (int)err;
    if (p == nullptr) return (int)hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return 0;
}

}  // namespace da

// The library's static split-T scratch: device memory for the decode kernel's
// split records, ready flags and status word that callers unable to allocate
// device memory use instead of a workspace of their own.
//
// The array below is a file-scope device variable, so each GPU the library
// runs on holds its own copy, from the first use of the library's code on that
// GPU until the process ends.  Host code never passes the array's name to a
// kernel (in host code that name is a stand-in, not a device address): the
// first call on each device, with that device current, resolves the device
// address with hipGetSymbolAddress, keeps it per device and zero-fills the
// status word and the ready flags with a fill kernel on the caller's stream
// (no memset node, so the call may be captured into a graph).  Every later
// call on that device uses the resolved address.  Calls on one device share
// the array: calls that overlap in time race.
#include <algorithm>
#include <mutex>
#include <vector>

#include "common.hpp"

namespace gqa {

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

__global__ void zero_words_kernel(uint32_t* p, int64_t n) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = 0u;
}

std::mutex g_mu;
std::vector<void*> g_ptr;   // resolved address per device (nullptr until set up)

}  // namespace

hipError_t static_scratch(int64_t zero_bytes, hipStream_t s, void** out) {
  *out = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_mu);
  if (static_cast<int>(g_ptr.size()) <= dev) g_ptr.resize(dev + 1, nullptr);
  if (!g_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    const int64_t words = (zero_bytes + 3) / 4;
    hipLaunchKernelGGL(zero_words_kernel, dim3(static_cast<unsigned>(std::min<int64_t>(1024, (words + 255) / 256))),
                       dim3(256), 0, s, static_cast<uint32_t*>(ptr), words);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    g_ptr[dev] = ptr;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace gqa

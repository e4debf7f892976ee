// Device memory of the allocation-free entry point (muon_ns_batched_noalloc):
// the workspace is this file-scope array, one copy per GPU the library runs
// on, held until the process ends.  In host code `scratch` names a host-side
// stand-in, not device memory: host code uses only the address that
// hipGetSymbolAddress returns for the current device, looked up once per
// device and kept.
#include <cstring>
#include <map>
#include <mutex>

#include "muon_internal.hpp"
#include "muon_mi355x.h"

namespace muon {

namespace {

static __device__ __align__(256) unsigned char scratch[MUON_NOALLOC_MAX_WORKSPACE];

std::mutex g_scratch_mu;
std::map<int, char*> g_scratch_base;

// Bytes carried by one launch of the copy kernel, as its arguments.
constexpr uint32_t kPutChunk = 2048;
struct PutChunk {
  unsigned char bytes[kPutChunk];
};

__global__ __launch_bounds__(kThreads) void k_put_bytes(PutChunk c, unsigned char* dst,
                                                        uint32_t n) {
  for (uint32_t i = threadIdx.x; i < n; i += kThreads) dst[i] = c.bytes[i];
}

}  // namespace

hipError_t noalloc_scratch(char** base) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  auto it = g_scratch_base.find(dev);
  if (it != g_scratch_base.end()) {
    *base = it->second;
    return hipSuccess;
  }
  void* p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  if (p == nullptr) return hipErrorInvalidSymbol;
  g_scratch_base[dev] = static_cast<char*>(p);
  *base = static_cast<char*>(p);
  return hipSuccess;
}

hipError_t launch_put_bytes(const void* src, size_t n, void* dst, hipStream_t s) {
  const unsigned char* from = static_cast<const unsigned char*>(src);
  unsigned char* to = static_cast<unsigned char*>(dst);
  PutChunk c;
  for (size_t off = 0; off < n; off += kPutChunk) {
    const uint32_t len = static_cast<uint32_t>(n - off < kPutChunk ? n - off : kPutChunk);
    std::memcpy(c.bytes, from + off, len);
    hipLaunchKernelGGL(k_put_bytes, dim3(1), dim3(kThreads), 0, s, c, to + off, len);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace muon

// A plain HBM stream with the access pattern of the momentum pass, as the
// yardstick for the bandwidth-bound kernels: every block moves 4 KiB of each
// input to each output, 16-byte vectors, lane-contiguous (vector v of the
// block's chunk goes to thread v % 256), all of a block's loads issued before
// its first store (one 16-byte vector per thread and stream: of the shapes
// tried, 1 to 8 vectors per thread, one-shot or grid-stride, the fastest
// plain stream).  With as many outputs as inputs, output k receives input k;
// with two inputs and one output, the output is their bitwise XOR (so that
// both are read); with one input and two outputs, both receive it.
#include "device_common.hpp"
#include "muon_mi355x.h"

namespace muon {

namespace {

constexpr int kStreamVecs = 1;  // 16-byte vectors per thread and stream: 4 KiB per block
constexpr size_t kStreamChunk = static_cast<size_t>(kStreamVecs) * kThreads * 16;

template <int NIN, int NOUT, bool NT>
__global__ __launch_bounds__(kThreads) void k_hbm_stream(const char* in0, const char* in1,
                                                         char* out0, char* out1) {
  const size_t base = static_cast<size_t>(blockIdx.x) * kStreamChunk + threadIdx.x * 16;
  const char* in[2] = {in0, in1};
  char* out[2] = {out0, out1};
  u32x4_t v[NIN][kStreamVecs];
#pragma unroll
  for (int s = 0; s < NIN; ++s)
#pragma unroll
    for (int i = 0; i < kStreamVecs; ++i) {
      const char* p = in[s] + base + static_cast<size_t>(i) * kThreads * 16;
      v[s][i] = NT ? ld16_nt(p) : ld16(p);
    }
  if constexpr (NIN == 2 && NOUT == 1) {
#pragma unroll
    for (int i = 0; i < kStreamVecs; ++i) v[0][i] ^= v[1][i];
  }
#pragma unroll
  for (int s = 0; s < NOUT; ++s)
#pragma unroll
    for (int i = 0; i < kStreamVecs; ++i) {
      char* p = out[s] + base + static_cast<size_t>(i) * kThreads * 16;
      if (NT)
        st16_nt(p, v[s % NIN][i]);
      else
        st16(p, v[s % NIN][i]);
    }
}

template <int NIN, int NOUT>
void launch_stream(dim3 grid, hipStream_t s, bool nt, const char* i0, const char* i1, char* o0,
                   char* o1) {
  if (nt)
    hipLaunchKernelGGL((k_hbm_stream<NIN, NOUT, true>), grid, dim3(kThreads), 0, s, i0, i1, o0, o1);
  else
    hipLaunchKernelGGL((k_hbm_stream<NIN, NOUT, false>), grid, dim3(kThreads), 0, s, i0, i1, o0, o1);
}

}  // namespace

}  // namespace muon

using namespace muon;

extern "C" int32_t muon_hbm_stream(int32_t n_in, const void* const* in, int32_t n_out,
                                   void* const* out, size_t bytes, int32_t nontemporal,
                                   void* stream) {
  if (n_in < 1 || n_in > 2 || n_out < 1 || n_out > 2 || in == nullptr || out == nullptr)
    return MUON_ERR_INVALID_ARG;
  if (bytes == 0) return MUON_OK;
  if (bytes % 16384 != 0 || bytes / kStreamChunk > 0x7fffffffu) return MUON_ERR_INVALID_ARG;
  for (int k = 0; k < n_in; ++k)
    if (in[k] == nullptr || (reinterpret_cast<uintptr_t>(in[k]) & 15u) != 0)
      return MUON_ERR_INVALID_ARG;
  for (int k = 0; k < n_out; ++k)
    if (out[k] == nullptr || (reinterpret_cast<uintptr_t>(out[k]) & 15u) != 0)
      return MUON_ERR_INVALID_ARG;
  const dim3 grid(static_cast<uint32_t>(bytes / kStreamChunk));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const char* i0 = static_cast<const char*>(in[0]);
  const char* i1 = static_cast<const char*>(in[n_in > 1 ? 1 : 0]);
  char* o0 = static_cast<char*>(out[0]);
  char* o1 = static_cast<char*>(out[n_out > 1 ? 1 : 0]);
  const bool nt = nontemporal != 0;
  if (n_in == 1 && n_out == 1) launch_stream<1, 1>(grid, s, nt, i0, i1, o0, o1);
  else if (n_in == 1) launch_stream<1, 2>(grid, s, nt, i0, i1, o0, o1);
  else if (n_out == 1) launch_stream<2, 1>(grid, s, nt, i0, i1, o0, o1);
  else launch_stream<2, 2>(grid, s, nt, i0, i1, o0, o1);
  return hipGetLastError() == hipSuccess ? MUON_OK : MUON_ERR_HIP;
}

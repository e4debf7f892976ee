// Device helpers shared by the kernels: element types, bf16 rounding,
// deterministic reductions, batch/tile lookup and the XCD-aware block order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "muon_internal.hpp"

namespace muon {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))  // LDS pointers, for the transposing reads

// Storage types: bf16 is carried as its raw 16 bits.
struct bf16_tag {};

template <typename T> struct Elt;

template <> struct Elt<uint16_t> {
  static constexpr int kVec = 8;  // elements per 16-byte vector
  static __device__ __forceinline__ float to_f32(uint16_t v) {
    return __uint_as_float(static_cast<uint32_t>(v) << 16);
  }
  // Round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
  static __device__ __forceinline__ uint16_t from_f32(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
  }
  // from_f32(lo) | from_f32(hi) << 16 in one packed conversion (the same
  // rounding; written element by element it took four instructions).
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const f32x2_t f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
  }
};

template <> struct Elt<float> {
  static constexpr int kVec = 4;
  static __device__ __forceinline__ float to_f32(float v) { return v; }
  static __device__ __forceinline__ float from_f32(float f) { return f; }
};

// Unpack / pack one 16-byte vector of T into / from fp32 values.
template <typename T>
__device__ __forceinline__ void vec_to_f32(const u32x4_t& v, float* out) {
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(v[i] << 16);
      out[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(v[i]);
  }
}

template <typename T>
__device__ __forceinline__ u32x4_t f32_to_vec(const float* in) {
  u32x4_t v;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = Elt<uint16_t>::pack2(in[2 * i], in[2 * i + 1]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __float_as_uint(in[i]);
  }
  return v;
}

// 16-byte loads and stores of global memory.  The pointers come from
// descriptors and are generic; naming the global address space makes these
// global_load/global_store instructions, which wait on vmcnt alone (a flat
// access would also hold lgkmcnt, and so every later wait for an LDS read).
#define GLOBAL_AS __attribute__((address_space(1)))
__device__ __forceinline__ u32x4_t ld16(const void* p) {
  return *(const GLOBAL_AS u32x4_t*)(p);
}
__device__ __forceinline__ void st16(void* p, const u32x4_t& v) {
  *(GLOBAL_AS u32x4_t*)(p) = v;
}
// The same with the nontemporal hint, for data that one call reads or writes
// once (the momentum pass's G, M and M').
__device__ __forceinline__ u32x4_t ld16_nt(const void* p) {
  return __builtin_nontemporal_load((const GLOBAL_AS u32x4_t*)(p));
}
__device__ __forceinline__ void st16_nt(void* p, const u32x4_t& v) {
  __builtin_nontemporal_store(v, (GLOBAL_AS u32x4_t*)(p));
}

// Sum over a wavefront of 64 lanes with a fixed butterfly order (deterministic).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Sum over a block of kThreads threads; every thread gets the result.
template <typename F>
__device__ __forceinline__ F block_sum(F v, F* scratch /* kThreads/64 entries */) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) scratch[wave] = v;
  __syncthreads();
  F t = 0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) t += scratch[w];
  __syncthreads();
  return t;
}

// The ping-pong iterate buffer `which` (0 or 1) of a matrix.  A select rather
// than an index, so that a descriptor held by a kernel stays in registers.
__device__ __forceinline__ void* iterate(const MatDesc& d, int which) {
  return which ? d.x[1] : d.x[0];
}

// A value from a table that no kernel writes while it runs (the descriptors,
// the block prefixes), read through the constant address space.  The matrix-
// core kernels write memory before they read these tables (the atomics of a
// tile claim); through a generic pointer the compiler then no longer proves the
// table unchanged and loads it into vector registers instead of scalar ones,
// which made the wide product kernel spill 82 registers inside its K loop.
template <typename T>
__device__ __forceinline__ T load_const(const T* p) {
  static_assert(sizeof(T) % 4 == 0, "whole dwords");
  using CU32 = const __attribute__((address_space(4))) uint32_t;
  CU32* q = (CU32*)(p);
  uint32_t w[sizeof(T) / 4];
#pragma unroll
  for (int i = 0; i < static_cast<int>(sizeof(T) / 4); ++i) w[i] = q[i];
  T v;
  __builtin_memcpy(&v, w, sizeof(T));
  return v;
}

// Index j with prefix[j] <= b < prefix[j+1] (b < prefix[batch]); exactly one
// interval holds b, and empty intervals never match.  Up to kLocateScan
// matrices the whole block finds it at once: every thread tests a few
// intervals in parallel (one round of independent loads) and the owner
// publishes j through `slot` in LDS, instead of a binary search's chain of
// dependent loads at the start of every block.  Larger batches, where that
// scan would cost every block `batch` loads, take the binary search (every
// thread the same one: no LDS).  batch is uniform, so the whole block takes
// the same branch.
constexpr int kLocateScan = 2048;
__device__ __forceinline__ int locate_matrix(const int32_t* prefix, int batch, int32_t b,
                                             int* slot) {
  if (batch > kLocateScan) {
    int lo = 0, hi = batch;  // prefix[lo] <= b < prefix[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (load_const(prefix + mid) <= b)
        lo = mid;
      else
        hi = mid;
    }
    return lo;
  }
  for (int k = threadIdx.x; k < batch; k += blockDim.x)
    if (prefix[k] <= b && b < prefix[k + 1]) *slot = k;
  __syncthreads();
  return *slot;
}

// Slab layout of every workspace matrix (the iterate X, A and B): a padded
// matrix with `ncols` columns is cut into slabs of kSlabRows x kSlabCols
// elements, each stored contiguously and row-major; the slabs of one band of
// kSlabRows rows follow each other.  A K-slice of 32 columns of a 256-row
// band is then one contiguous run of memory, which is what the matrix-core
// kernels stream into LDS.
constexpr int kSlabRows = kTile;  // 256
constexpr int kSlabCols = 32;
__device__ __forceinline__ int64_t slab_off(int64_t r, int64_t c, int64_t ncols) {
  return ((r / kSlabRows) * (ncols / kSlabCols) + c / kSlabCols) * (kSlabRows * kSlabCols) +
         (r % kSlabRows) * kSlabCols + (c % kSlabCols);
}
// Offset of (r0 + q, c0 + cc) from (r0, c0), for r0 a multiple of kSlabRows,
// c0 a multiple of kSlabCols, 0 <= q < kSlabRows and cc >= 0: the same band,
// slab cc / kSlabCols after c0's.  Unsigned 32-bit shifts and masks only.  The
// matrix-core epilogues add it to their tile's origin, slab_off(r0, c0, ncols),
// which is uniform over the workgroup; computing slab_off per store (signed
// 64-bit division and products) cost about 40 VALU instructions per 16-byte
// store and most of the epilogue's time.
__device__ __forceinline__ uint32_t slab_local(uint32_t q, uint32_t cc) {
  return (cc / kSlabCols) * (kSlabRows * kSlabCols) + q * kSlabCols + (cc % kSlabCols);
}

// Workgroups are dealt round-robin to the 8 XCDs of the chip (block b runs on
// XCD b % 8).  Renumber them so that each XCD receives one contiguous range of
// logical blocks, of equal length: neighbouring tiles, which share operands,
// then share an L2.
__device__ __forceinline__ int32_t xcd_remap(int32_t b, int32_t n) {
  const int32_t xcd = b % kXcd, local = b / kXcd;
  const int32_t per = n / kXcd, rem = n % kXcd;
  return xcd * per + (xcd < rem ? xcd : rem) + local;
}

}  // namespace muon

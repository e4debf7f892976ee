// Block-scaled e4m3 copies of the iterate, A and B for the e4m3 steps.
//
// Every 32 consecutive elements of a row (along the side the next product
// contracts over) share one power-of-two scale 2^e, the smallest that brings
// the block's largest magnitude to at most 448 (e4m3's largest value), so no
// element saturates; each element x is stored as the e4m3 rounding (to nearest
// even) of x * 2^-e.  The layout (F8 layout, muon_internal.hpp) keeps a bf16
// slab's geometry: 256 rows x 64 columns, one 16 KiB run per K slice of a band.
#include "device_common.hpp"

namespace muon {

namespace {

// Byte offset of element (r, c) of a matrix with `ncols` columns in the F8 layout.
__device__ __forceinline__ int64_t f8_off(int64_t r, int64_t c, int64_t ncols) {
  return ((r / kTile) * (ncols / 64) + c / 64) * (kTile * 64) + (r % kTile) * 64 + (c % 64);
}

// Byte offset, from the scales' base, of the scale of row r's block holding column c.
__device__ __forceinline__ int64_t f8_scale_off(int64_t r, int64_t c, int64_t ncols) {
  const int64_t slab = (r / kTile) * (ncols / 64) + c / 64;
  const int rl = static_cast<int>(r % kTile), kb = static_cast<int>((c % 64) / 32);
  return slab * 512 + 4 * (32 * (2 * (rl / 128) + kb) + rl % 32) + (rl / 32) % 4;
}

// Exponent e of a block's scale: the smallest with amax <= 448 * 2^e.  With
// amax = m * 2^E, 1 <= m < 2, and 448 = 1.75 * 2^8: e = E - 8 when m <= 1.75
// (mantissa field <= 0x600000), else E - 7.  Clamped to [-127, 126], so that
// both 2^-e (a normal float) and the E8M0 byte e + 127 exist; a zero or
// subnormal block takes -127 (its elements then stay below 4 after scaling).
__device__ __forceinline__ int block_exp(float amax) {
  const uint32_t b = __float_as_uint(amax);
  const int field = static_cast<int>((b >> 23) & 255);
  if (field == 0) return -127;
  const int e = field - 127 - 8 + ((b & 0x7fffffu) > 0x600000u ? 1 : 0);
  return e < -127 ? -127 : (e > 126 ? 126 : e);
}

__device__ __forceinline__ float pow2(int k) {  // 2^k for k in [-126, 127]
  return __uint_as_float(static_cast<uint32_t>(k + 127) << 23);
}

// 16 values, already scaled, as 16 e4m3 bytes (round to nearest even), in order.
__device__ __forceinline__ u32x4_t pack16_e4m3(const float* v) {
  u32x4_t w;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int x = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * i], v[4 * i + 1], 0, false);
    x = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * i + 2], v[4 * i + 3], x, true);
    w[i] = static_cast<uint32_t>(x);
  }
  return w;
}

// Quantizes the 16 values of this thread (half of a block of 32; the other
// half is on lane ^ 1), stores them at `data` and, from the even lane of the
// pair, the block's scale at `scale`.
__device__ __forceinline__ void quant16(const float* v, uint8_t* data, uint8_t* scale, bool even) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
  const int e = block_exp(amax);
  const float inv = pow2(-e);
  float s[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) s[i] = v[i] * inv;
  st16(data, pack16_e4m3(s));
  if (even) *scale = static_cast<uint8_t>(e + 127);
}

}  // namespace

// One block per kQ8Tile x kQ8Tile tile of the source (bf16, slab layout): thread
// t holds row t / 4, columns 16 (t % 4) .. + 15 of the tile, which it
// quantizes along the row into buffer 0.  TRANSPOSE (the iterate only): the
// tile also goes through LDS, and thread t quantizes column t / 4, rows
// 16 (t % 4) .. + 15, into row t / 4 of X^T in buffer 1.
template <bool TRANSPOSE>
__global__ __launch_bounds__(kThreads) void k_quant8(LaunchCtx c, int32_t src, int32_t cur) {
  __shared__ float tile[TRANSPOSE ? kQ8Tile : 1][kQ8Tile + 1];
  __shared__ int slot;
  const int32_t* pre = c.prefix + (src == Q8_X ? PH_Q8X : PH_Q8S) * (c.batch + 1);
  const int32_t b = blockIdx.x;
  const int j = __builtin_amdgcn_readfirstlane(locate_matrix(pre, c.batch, b, &slot));
  const MatDesc& d = c.desc[j];
  const int32_t t = b - pre[j];
  const int64_t ncols = src == Q8_X ? d.l_pad : d.s_pad;
  const int32_t tpr = static_cast<int32_t>(ncols / kQ8Tile);
  const int64_t r0 = static_cast<int64_t>(t / tpr) * kQ8Tile;
  const int64_t c0 = static_cast<int64_t>(t % tpr) * kQ8Tile;
  const uint16_t* m = static_cast<const uint16_t*>(src == Q8_X ? iterate(d, cur)
                                                   : src == Q8_A ? d.gram : d.poly);
  const int row = threadIdx.x >> 2, q = threadIdx.x & 3;
  const bool even = (q & 1) == 0;
  // 16 consecutive columns inside one 32-column slab: 32 contiguous bytes
  float v[16];
  {
    const uint16_t* p = m + slab_off(r0 + row, c0 + 16 * q, ncols);
    vec_to_f32<uint16_t>(ld16(p), v);
    vec_to_f32<uint16_t>(ld16(p + 8), v + 8);
  }
  const int64_t cap = static_cast<int64_t>(d.s_pad) * d.l_pad;  // data bytes of an e4m3 buffer
  uint8_t* f0 = reinterpret_cast<uint8_t*>(f8_buffer(d, 0));
  quant16(v, f0 + f8_off(r0 + row, c0 + 16 * q, ncols),
          f0 + cap + f8_scale_off(r0 + row, c0 + 16 * q, ncols), even);
  if constexpr (TRANSPOSE) {
#pragma unroll
    for (int i = 0; i < 16; ++i) tile[row][16 * q + i] = v[i];
    __syncthreads();
    float w[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) w[i] = tile[16 * q + i][row];
    // X^T is l_pad x s_pad: its row c0 + row, columns r0 + 16 q ..
    uint8_t* f1 = reinterpret_cast<uint8_t*>(f8_buffer(d, 1));
    quant16(w, f1 + f8_off(c0 + row, r0 + 16 * q, d.s_pad),
            f1 + cap + f8_scale_off(c0 + row, r0 + 16 * q, d.s_pad), even);
  }
}

hipError_t launch_quant8(const LaunchCtx& c, int32_t nblocks, int32_t src, int32_t cur) {
  if (nblocks <= 0) return hipSuccess;
  if (src == Q8_X)
    hipLaunchKernelGGL((k_quant8<true>), dim3(nblocks), dim3(kThreads), 0, c.stream, c, src, cur);
  else
    hipLaunchKernelGGL((k_quant8<false>), dim3(nblocks), dim3(kThreads), 0, c.stream, c, src, cur);
  return hipGetLastError();
}

}  // namespace muon

// Fused AdamW step over a ragged batch of flat tensors (the parameters that
// Muon does not cover: norms, routers, embeddings).
//
// Per element, in fp32 (p and g stored as T, the moments m and v as fp32):
//   p <- p * (1 - lr * wd)
//   m <- beta1 * m + (1 - beta1) * g
//   v <- beta2 * v + (1 - beta2) * g^2
//   p <- p - (lr / (1 - beta1^t)) * m / (sqrt(v) / sqrt(1 - beta2^t) + eps)
// Bandwidth-bound: each block reads its whole span (p, g, m, v) before the
// first store.  Blocks find their tensor through the prefix table in one round
// of loads, as the other elementwise kernels do.
#include "device_common.hpp"

namespace muon {

namespace {

constexpr int kAdamVec = 8;    // elements per thread and iteration
constexpr int kAdamIters = 4;  // iterations per block

template <typename T>
__device__ __forceinline__ void load8(const T* p, float* v) {
  if constexpr (sizeof(T) == 2) {
    vec_to_f32<T>(ld16(p), v);
  } else {
    vec_to_f32<T>(ld16(p), v);
    vec_to_f32<T>(ld16(p + 4), v + 4);
  }
}

template <typename T>
__device__ __forceinline__ void store8(T* p, const float* v) {
  if constexpr (sizeof(T) == 2) {
    st16(p, f32_to_vec<T>(v));
  } else {
    st16(p, f32_to_vec<T>(v));
    st16(p + 4, f32_to_vec<T>(v + 4));
  }
}

__device__ __forceinline__ void adamw_update(const AdamParams& a, float& p, float g, float& m,
                                             float& v) {
  p *= a.decay;
  m = a.beta1 * m + a.one_minus_beta1 * g;
  v = a.beta2 * v + a.one_minus_beta2 * (g * g);
  const float denom = sqrtf(v) * a.inv_bc2_sqrt + a.eps;
  p -= a.step_size * (m / denom);
}

template <typename T>
__global__ __launch_bounds__(kThreads) void k_adamw(AdamCtx c, AdamParams a) {
  __shared__ int slot;
  constexpr int64_t kSpan = static_cast<int64_t>(kThreads) * kAdamVec * kAdamIters;
  const int32_t b = blockIdx.x;
  const int j = __builtin_amdgcn_readfirstlane(locate_matrix(c.prefix, c.batch, b, &slot));
  const AdamDesc& d = c.desc[j];
  const int64_t numel = d.numel;
  const int64_t base = static_cast<int64_t>(b - c.prefix[j]) * kSpan;
  T* __restrict__ pp = static_cast<T*>(d.p) + base;
  const T* __restrict__ gp = static_cast<const T*>(d.g) + base;
  float* __restrict__ mp = d.m + base;
  float* __restrict__ vp = d.v + base;
  if (base + kSpan <= numel) {
    float p[kAdamIters][kAdamVec], g[kAdamIters][kAdamVec], m[kAdamIters][kAdamVec],
        v[kAdamIters][kAdamVec];
#pragma unroll
    for (int it = 0; it < kAdamIters; ++it) {
      const int64_t off = (static_cast<int64_t>(it) * kThreads + threadIdx.x) * kAdamVec;
      load8<T>(pp + off, p[it]);
      load8<T>(gp + off, g[it]);
      load8<float>(mp + off, m[it]);
      load8<float>(vp + off, v[it]);
    }
#pragma unroll
    for (int it = 0; it < kAdamIters; ++it) {
      const int64_t off = (static_cast<int64_t>(it) * kThreads + threadIdx.x) * kAdamVec;
#pragma unroll
      for (int e = 0; e < kAdamVec; ++e) adamw_update(a, p[it][e], g[it][e], m[it][e], v[it][e]);
      store8<T>(pp + off, p[it]);
      store8<float>(mp + off, m[it]);
      store8<float>(vp + off, v[it]);
    }
  } else {
    // the tensor's last, partial span: element by element
    const int64_t n = numel - base;
    for (int64_t i = threadIdx.x; i < n; i += kThreads) {
      float p = Elt<T>::to_f32(pp[i]);
      float m = mp[i], v = vp[i];
      adamw_update(a, p, Elt<T>::to_f32(gp[i]), m, v);
      pp[i] = Elt<T>::from_f32(p);
      mp[i] = m;
      vp[i] = v;
    }
  }
}

}  // namespace

int64_t adamw_blocks(int64_t numel) {
  const int64_t span = static_cast<int64_t>(kThreads) * kAdamVec * kAdamIters;
  return (numel + span - 1) / span;
}

hipError_t launch_adamw(const AdamCtx& c, int32_t nblocks, bool is_bf16, const AdamParams& a) {
  if (nblocks <= 0) return hipSuccess;
  if (is_bf16)
    hipLaunchKernelGGL(k_adamw<uint16_t>, dim3(nblocks), dim3(kThreads), 0, c.stream, c, a);
  else
    hipLaunchKernelGGL(k_adamw<float>, dim3(nblocks), dim3(kThreads), 0, c.stream, c, a);
  return hipGetLastError();
}

}  // namespace muon

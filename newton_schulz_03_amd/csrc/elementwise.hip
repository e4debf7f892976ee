// Bandwidth-bound kernels of the Muon step:
//   k_reduce     momentum M' = beta*M + G (step) and per-block sums of U^2; with the
//                momentum in host memory it also leaves a device copy of the new momentum
//   k_finalize   1 / (||U||_F + eps) per matrix from those partials
//   k_normalize  X0 = U / (||U||_F + eps) in the wide orientation, zero padded
//   k_finish     W' = W - lr*sqrt(max(1,rows/cols))*O (step) or out = O (orthogonalize only)
// All of them read and write whole 16-byte vectors along rows, so every
// wavefront touches contiguous runs of memory, and each block issues all of its
// loads before it waits on any of them: what keeps HBM busy is the number of
// bytes in flight.  The norm is deterministic: each reduce block writes one
// partial, and one finalize block per matrix sums them in a fixed order.
#include "device_common.hpp"

namespace muon {

namespace {

template <typename T>
struct URow {
  // Loads 16 consecutive elements of U from user row `r`, starting at column c0,
  // with zeros beyond the row.  U is x (orthogonalize only), M' (step), or
  // G + beta*M' (Nesterov step).
  static __device__ __forceinline__ void load(const MatDesc& d, const ElemParams& p, int64_t r,
                                              int64_t c0, float* u) {
    constexpr int V = Elt<T>::kVec;
    const int64_t cols = d.cols;
    const int64_t rowoff = r * cols;
#pragma unroll
    for (int q = 0; q < 16 / V; ++q) {
      const int64_t col = c0 + q * V;
      float* o = u + q * V;
      if (d.vec_ok && col + V <= cols) {
        const int64_t off = rowoff + col;
        if (p.mode == MODE_NS) {
          vec_to_f32<T>(ld16(static_cast<const T*>(d.src) + off), o);
        } else {
          vec_to_f32<T>(ld16(static_cast<const T*>(d.u_src) + off), o);
          if (p.nesterov) {
            float g[V];
            vec_to_f32<T>(ld16(static_cast<const T*>(d.src) + off), g);
#pragma unroll
            for (int e = 0; e < V; ++e) o[e] = g[e] + p.beta * o[e];
          }
        }
      } else {
#pragma unroll
        for (int e = 0; e < V; ++e) {
          float v = 0.f;
          if (col + e < cols) {
            const int64_t off = rowoff + col + e;
            if (p.mode == MODE_NS) {
              v = Elt<T>::to_f32(static_cast<const T*>(d.src)[off]);
            } else {
              v = Elt<T>::to_f32(static_cast<const T*>(d.u_src)[off]);
              if (p.nesterov) v = Elt<T>::to_f32(static_cast<const T*>(d.src)[off]) + p.beta * v;
            }
          }
          o[e] = v;
        }
      }
    }
  }
};

}  // namespace

// ---------------------------------------------------------------------------
// k_reduce: one block per kThreads*V*kReduceIters elements of one matrix.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kThreads) void k_reduce(LaunchCtx c, ElemParams p) {
  __shared__ float scratch[kThreads / 64];
  __shared__ int slot;
  constexpr int V = Elt<T>::kVec;
  constexpr int64_t kSpan = static_cast<int64_t>(kThreads) * V * kReduceIters;
  const int32_t* pre = c.prefix + PH_REDUCE * (c.batch + 1);
  const int32_t b = blockIdx.x;
  const int j = __builtin_amdgcn_readfirstlane(locate_matrix(pre, c.batch, b, &slot));
  const MatDesc& d = c.desc[j];
  const int64_t numel = d.numel;
  const int64_t base = static_cast<int64_t>(b - pre[j]) * kSpan;
  float acc = 0.f;
  if (base + kSpan <= numel) {
    // a whole span: all loads go out before the first store
    const T* __restrict__ src = static_cast<const T*>(d.src) + base;
    if (p.mode == MODE_NS) {
      u32x4_t xv[kReduceIters];
#pragma unroll
      for (int it = 0; it < kReduceIters; ++it)
        xv[it] = ld16(src + (static_cast<int64_t>(it) * kThreads + threadIdx.x) * V);
#pragma unroll
      for (int it = 0; it < kReduceIters; ++it) {
        float u[V];
        vec_to_f32<T>(xv[it], u);
#pragma unroll
        for (int e = 0; e < V; ++e) acc += u[e] * u[e];
      }
    } else {
      T* __restrict__ mom = static_cast<T*>(d.mom) + base;
      T* __restrict__ copy = d.mom_copy ? static_cast<T*>(d.mom_copy) + base : nullptr;
      u32x4_t gv[kReduceIters], mv[kReduceIters];
#pragma unroll
      for (int it = 0; it < kReduceIters; ++it) {
        const int64_t off = (static_cast<int64_t>(it) * kThreads + threadIdx.x) * V;
        gv[it] = ld16(src + off);
        mv[it] = ld16(mom + off);
      }
#pragma unroll
      for (int it = 0; it < kReduceIters; ++it) {
        const int64_t off = (static_cast<int64_t>(it) * kThreads + threadIdx.x) * V;
        float g[V], m[V], mn[V], mr[V];
        vec_to_f32<T>(gv[it], g);
        vec_to_f32<T>(mv[it], m);
#pragma unroll
        for (int e = 0; e < V; ++e) mn[e] = p.beta * m[e] + g[e];
        const u32x4_t packed = f32_to_vec<T>(mn);
        st16(mom + off, packed);
        if (copy) st16(copy + off, packed);
        vec_to_f32<T>(packed, mr);  // U is formed from the stored (rounded) M', as later kernels do
#pragma unroll
        for (int e = 0; e < V; ++e) {
          const float u = p.nesterov ? g[e] + p.beta * mr[e] : mr[e];
          acc += u * u;
        }
      }
    }
  } else {
    // the matrix's last, partial span
#pragma unroll 1
    for (int it = 0; it < kReduceIters; ++it) {
      const int64_t off = base + (static_cast<int64_t>(it) * kThreads + threadIdx.x) * V;
      if (off >= numel) break;
      const int n = (off + V <= numel) ? V : static_cast<int>(numel - off);
      float u[V];
      if (p.mode == MODE_NS) {
        if (n == V) {
          vec_to_f32<T>(ld16(static_cast<const T*>(d.src) + off), u);
        } else {
          for (int e = 0; e < V; ++e)
            u[e] = e < n ? Elt<T>::to_f32(static_cast<const T*>(d.src)[off + e]) : 0.f;
        }
      } else {
        float g[V], m[V];
        T* mp = static_cast<T*>(d.mom) + off;
        const T* gp = static_cast<const T*>(d.src) + off;
        if (n == V) {
          vec_to_f32<T>(ld16(gp), g);
          vec_to_f32<T>(ld16(mp), m);
        } else {
          for (int e = 0; e < V; ++e) {
            g[e] = e < n ? Elt<T>::to_f32(gp[e]) : 0.f;
            m[e] = e < n ? Elt<T>::to_f32(mp[e]) : 0.f;
          }
        }
        float mn[V];
#pragma unroll
        for (int e = 0; e < V; ++e) mn[e] = p.beta * m[e] + g[e];
        u32x4_t packed = f32_to_vec<T>(mn);
        float mr[V];
        vec_to_f32<T>(packed, mr);
        T* cp = d.mom_copy ? static_cast<T*>(d.mom_copy) + off : nullptr;
        if (n == V) {
          st16(mp, packed);
          if (cp) st16(cp, packed);
        } else {
          for (int e = 0; e < n; ++e) mp[e] = Elt<T>::from_f32(mn[e]);
          if (cp)
            for (int e = 0; e < n; ++e) cp[e] = Elt<T>::from_f32(mn[e]);
        }
#pragma unroll
        for (int e = 0; e < V; ++e) u[e] = p.nesterov ? g[e] + p.beta * mr[e] : mr[e];
      }
#pragma unroll
      for (int e = 0; e < V; ++e) acc += u[e] * u[e];
    }
  }
  const float total = block_sum(acc, scratch);
  if (threadIdx.x == 0) c.partials[b] = total;
}

// ---------------------------------------------------------------------------
// k_finalize: block j sums matrix j's partials in a fixed order (double), then
// stores 1 / (sqrt(sum) + eps).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_finalize(LaunchCtx c, ElemParams p) {
  __shared__ double scratch[kThreads / 64];
  const int j = blockIdx.x;
  const int32_t* pre = c.prefix + PH_REDUCE * (c.batch + 1);
  double s = 0.0;
  for (int32_t k = pre[j] + threadIdx.x; k < pre[j + 1]; k += kThreads) s += c.partials[k];
  s = block_sum(s, scratch);
  if (threadIdx.x == 0)
    c.inv_norm[j] = static_cast<float>(1.0 / (sqrt(s) + static_cast<double>(p.eps)));
}

// ---------------------------------------------------------------------------
// k_normalize: one block per 64x64 tile of the padded wide iterate X0.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kThreads) void k_normalize(LaunchCtx c, ElemParams p) {
  __shared__ float tile[kEwTile][kEwTile + 1];
  __shared__ int slot;
  constexpr int V = Elt<T>::kVec;
  const int32_t* pre = c.prefix + PH_NORMALIZE * (c.batch + 1);
  const int32_t b = blockIdx.x;
  const int j = __builtin_amdgcn_readfirstlane(locate_matrix(pre, c.batch, b, &slot));
  const MatDesc& d = c.desc[j];
  const int32_t t = b - pre[j];
  const int32_t tpr = d.l_pad / kEwTile;
  const int64_t i0 = static_cast<int64_t>(t / tpr) * kEwTile;  // wide rows
  const int64_t j0 = static_cast<int64_t>(t % tpr) * kEwTile;  // wide cols
  const int rr = threadIdx.x >> 2, cc = (threadIdx.x & 3) * 16;
  float u[16];
  if (!d.tall) {
    if (i0 + rr < d.s) {
      URow<T>::load(d, p, i0 + rr, j0 + cc, u);
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) u[e] = 0.f;
    }
    const float inv = c.inv_norm[j];
#pragma unroll
    for (int e = 0; e < 16; ++e) u[e] *= inv;
  } else {
    // wide X0[i][jw] = U[jw][i]: stage the user tile (rows j0.., cols i0..) through LDS
    if (j0 + rr < d.l) {
      URow<T>::load(d, p, j0 + rr, i0 + cc, u);
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) u[e] = 0.f;
    }
    const float inv = c.inv_norm[j];
#pragma unroll
    for (int e = 0; e < 16; ++e) tile[rr][cc + e] = u[e] * inv;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 16; ++e) u[e] = tile[cc + e][rr];
  }
  // 16 consecutive columns starting at a multiple of 16 stay inside one slab row
  T* x0 = static_cast<T*>(iterate(d, 0)) + slab_off(i0 + rr, j0 + cc, d.l_pad);
#pragma unroll
  for (int q = 0; q < 16 / V; ++q) st16(x0 + q * V, f32_to_vec<T>(u + q * V));
}

// ---------------------------------------------------------------------------
// k_finish: one block per 64x64 tile of the user-shaped output.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kThreads) void k_finish(LaunchCtx c, ElemParams p) {
  __shared__ float tile[kEwTile][kEwTile + 1];
  __shared__ int slot;
  constexpr int V = Elt<T>::kVec;
  const int32_t* pre = c.prefix + PH_FINISH * (c.batch + 1);
  const int32_t b = blockIdx.x;
  const int j = __builtin_amdgcn_readfirstlane(locate_matrix(pre, c.batch, b, &slot));
  const MatDesc& d = c.desc[j];
  const int32_t t = b - pre[j];
  const int32_t tpr = static_cast<int32_t>((d.cols + kEwTile - 1) / kEwTile);
  const int64_t r0 = static_cast<int64_t>(t / tpr) * kEwTile;  // user rows
  const int64_t c0 = static_cast<int64_t>(t % tpr) * kEwTile;  // user cols
  const int rr = threadIdx.x >> 2, cc = (threadIdx.x & 3) * 16;
  const T* X = static_cast<const T*>(iterate(d, p.cur));
  const int64_t r = r0 + rr;
  const int64_t cols = d.cols;
  T* dst = static_cast<T*>(d.dst) + r * cols;
  // W first: its loads do not wait for the iterate's
  const bool vec_row = d.vec_ok && c0 + cc + 16 <= cols && r < d.rows;
  u32x4_t wv[16 / V];
  if (p.mode == MODE_STEP && vec_row) {
#pragma unroll
    for (int q = 0; q < 16 / V; ++q) wv[q] = ld16(dst + c0 + cc + q * V);
  }
  float o[16];
  if (!d.tall) {
    const T* src = X + slab_off(r0 + rr, c0 + cc, d.l_pad);  // inside the padded buffer
#pragma unroll
    for (int q = 0; q < 16 / V; ++q) vec_to_f32<T>(ld16(src + q * V), o + q * V);
  } else {
    // O[r][c] = X[c][r]: stage the wide tile (rows c0.., cols r0..) through LDS
    const T* src = X + slab_off(c0 + rr, r0 + cc, d.l_pad);
    float v[16];
#pragma unroll
    for (int q = 0; q < 16 / V; ++q) vec_to_f32<T>(ld16(src + q * V), v + q * V);
#pragma unroll
    for (int e = 0; e < 16; ++e) tile[rr][cc + e] = v[e];
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 16; ++e) o[e] = tile[cc + e][rr];
  }
  if (r >= d.rows) return;
  const float step = p.lr * d.scale;
  if (vec_row) {
#pragma unroll
    for (int q = 0; q < 16 / V; ++q) {
      float* oq = o + q * V;
      if (p.mode == MODE_STEP) {
        float w[V];
        vec_to_f32<T>(wv[q], w);
#pragma unroll
        for (int e = 0; e < V; ++e) oq[e] = w[e] - step * oq[e];
      }
      st16(dst + c0 + cc + q * V, f32_to_vec<T>(oq));
    }
    return;
  }
#pragma unroll
  for (int q = 0; q < 16 / V; ++q) {
    const int64_t col = c0 + cc + q * V;
    float* oq = o + q * V;
    if (d.vec_ok && col + V <= cols) {
      if (p.mode == MODE_STEP) {
        float w[V];
        vec_to_f32<T>(ld16(dst + col), w);
#pragma unroll
        for (int e = 0; e < V; ++e) oq[e] = w[e] - step * oq[e];
      }
      st16(dst + col, f32_to_vec<T>(oq));
    } else {
      for (int e = 0; e < V; ++e) {
        if (col + e >= cols) break;
        float v = oq[e];
        if (p.mode == MODE_STEP) v = Elt<T>::to_f32(dst[col + e]) - step * v;
        dst[col + e] = Elt<T>::from_f32(v);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Launchers.
// ---------------------------------------------------------------------------
hipError_t launch_reduce(const LaunchCtx& c, int32_t nblocks, bool is_bf16, const ElemParams& p) {
  if (nblocks <= 0) return hipSuccess;
  if (is_bf16)
    hipLaunchKernelGGL(k_reduce<uint16_t>, dim3(nblocks), dim3(kThreads), 0, c.stream, c, p);
  else
    hipLaunchKernelGGL(k_reduce<float>, dim3(nblocks), dim3(kThreads), 0, c.stream, c, p);
  return hipGetLastError();
}

hipError_t launch_finalize(const LaunchCtx& c, const ElemParams& p) {
  if (c.batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_finalize, dim3(c.batch), dim3(kThreads), 0, c.stream, c, p);
  return hipGetLastError();
}

hipError_t launch_normalize(const LaunchCtx& c, int32_t nblocks, bool is_bf16, const ElemParams& p) {
  if (nblocks <= 0) return hipSuccess;
  if (is_bf16)
    hipLaunchKernelGGL(k_normalize<uint16_t>, dim3(nblocks), dim3(kThreads), 0, c.stream, c, p);
  else
    hipLaunchKernelGGL(k_normalize<float>, dim3(nblocks), dim3(kThreads), 0, c.stream, c, p);
  return hipGetLastError();
}

hipError_t launch_finish(const LaunchCtx& c, int32_t nblocks, bool is_bf16, const ElemParams& p) {
  if (nblocks <= 0) return hipSuccess;
  if (is_bf16)
    hipLaunchKernelGGL(k_finish<uint16_t>, dim3(nblocks), dim3(kThreads), 0, c.stream, c, p);
  else
    hipLaunchKernelGGL(k_finish<float>, dim3(nblocks), dim3(kThreads), 0, c.stream, c, p);
  return hipGetLastError();
}

}  // namespace muon

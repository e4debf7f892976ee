// Bandwidth-bound kernels of the Muon step:
//   k_prepare    momentum M' = beta*M + G (step) in the user's matrix, U = M' (or
//                G + beta*M', Nesterov; x when only orthogonalizing) written once
//                into the wide iterate, zero padded, and per-block sums of U^2
//   k_finalize   1 / (||U||_F + eps) per matrix from those partials
//   k_finish     W' = W - lr*sqrt(max(1,rows/cols))*O (step) or out = O (orthogonalize only)
// The iterate holds U itself, not X0 = U / (||U||_F + eps): the first Gram and
// the first product take the factor into the scale they store with (the
// finish pass, when there are no iterations), so U is read from HBM once.
// Every kernel reads and writes whole 16-byte vectors along rows, so every
// wavefront touches contiguous runs of memory, and each block issues all of its
// loads before it waits on any of them: what keeps HBM busy is the number of
// bytes in flight.  The norm is deterministic: each prepare block writes one
// partial, and one finalize block per matrix sums them in a fixed order.
#include "device_common.hpp"

namespace muon {

namespace {

// One 16-byte vector (V elements) of the user's matrix: the loads, then M', U
// and the momentum store.
template <typename T>
struct UVec {
  static constexpr int V = Elt<T>::kVec;
  u32x4_t a, m;  // G (or x) and M
  bool full;     // the whole vector lies in the matrix, 16-byte aligned

  __device__ __forceinline__ void load(const MatDesc& d, const ElemParams& p, int64_t r,
                                       int64_t c0) {
    full = r < d.rows && d.vec_ok && c0 + V <= d.cols;
    if (!full) return;
    const int64_t off = r * d.cols + c0;
    // read once: nontemporal (measured: the pass 3% faster on 96 x 2048x6144)
    a = ld16_nt(static_cast<const T*>(d.src) + off);
    if (p.mode == MODE_STEP) m = ld16_nt(static_cast<const T*>(d.mom) + off);
  }

  // u <- U over the vector (zeros outside the matrix); stores M' (step).  U is
  // formed from the stored, rounded M', as the oracle's bf16 reading has it.
  __device__ __forceinline__ void finish(const MatDesc& d, const ElemParams& p, int64_t r,
                                         int64_t c0, float* u) const {
    if (full) {
      if (p.mode == MODE_NS) {
        vec_to_f32<T>(a, u);
        return;
      }
      float g[V], mo[V], mn[V];
      vec_to_f32<T>(a, g);
      vec_to_f32<T>(m, mo);
#pragma unroll
      for (int e = 0; e < V; ++e) mn[e] = p.beta * mo[e] + g[e];
      const u32x4_t packed = f32_to_vec<T>(mn);
      st16_nt(static_cast<T*>(d.mom) + r * d.cols + c0, packed);  // not read again this call
      vec_to_f32<T>(packed, u);
      if (p.nesterov) {
#pragma unroll
        for (int e = 0; e < V; ++e) u[e] = g[e] + p.beta * u[e];
      }
      return;
    }
    // an edge vector: element by element, clipped to the shape
#pragma unroll
    for (int e = 0; e < V; ++e) u[e] = 0.f;
    if (r >= d.rows) return;
    const int64_t off = r * d.cols;
    const T* src = static_cast<const T*>(d.src) + off;
    T* mom = static_cast<T*>(d.mom) + off;
#pragma unroll 1
    for (int e = 0; e < V && c0 + e < d.cols; ++e) {
      const float g = Elt<T>::to_f32(src[c0 + e]);
      if (p.mode == MODE_NS) {
        u[e] = g;
        continue;
      }
      const T stored = Elt<T>::from_f32(p.beta * Elt<T>::to_f32(mom[c0 + e]) + g);
      mom[c0 + e] = stored;
      const float mr = Elt<T>::to_f32(stored);
      u[e] = p.nesterov ? g + p.beta * mr : mr;
    }
  }
};

}  // namespace

// ---------------------------------------------------------------------------
// k_prepare: one block per tile of the padded wide iterate: kPrepWideRows x
// 256 for a wide matrix; kPrepTallS x kPrepTallL (short side x long side,
// 128 x 128) for a tall one, which is read as the user's kPrepTallL x
// kPrepTallS tile (rows of 256 bytes) and transposed through LDS.  Each
// thread moves 16-byte vectors v = it * 256 + threadIdx.x of the tile in
// row-major order, so every load and store instruction of a wave covers whole
// rows of the tile: contiguous runs of memory.  The transpose holds U already
// rounded to T (the iterate's element type).
// ---------------------------------------------------------------------------
namespace {

// Loads, momentum and U for the tile's kVecs vectors per thread; returns the
// thread's sum of squares.  The tile is read as rows of vpr vectors starting
// at the user's (r0, c0).
template <typename T, int kVecs>
__device__ __forceinline__ float prepare_vectors(const MatDesc& d, const ElemParams& p, int64_t r0,
                                                 int64_t c0, int vpr, u32x4_t* up) {
  constexpr int V = Elt<T>::kVec;
  UVec<T> uv[kVecs];
#pragma unroll
  for (int it = 0; it < kVecs; ++it) {
    const int v = it * kThreads + threadIdx.x;
    uv[it].load(d, p, r0 + v / vpr, c0 + (v % vpr) * V);
  }
  float acc = 0.f;
#pragma unroll
  for (int it = 0; it < kVecs; ++it) {
    const int v = it * kThreads + threadIdx.x;
    float u[V];
    uv[it].finish(d, p, r0 + v / vpr, c0 + (v % vpr) * V, u);
#pragma unroll
    for (int e = 0; e < V; ++e) acc += u[e] * u[e];
    up[it] = f32_to_vec<T>(u);
  }
  return acc;
}

}  // namespace

template <typename T>
__global__ __launch_bounds__(kThreads) void k_prepare(LaunchCtx c, ElemParams p) {
  constexpr int V = Elt<T>::kVec;
  constexpr int kTallRows = kPrepTallL, kTallCols = kPrepTallS;  // the user's tile of a tall matrix
  constexpr int kVecsTall = kTallRows * kTallCols / V / kThreads;   // 8 (bf16) or 16 (fp32)
  constexpr int kVecsWide = kPrepWideRows * kWideTileCols / V / kThreads;
  constexpr int kPitch = kTallCols + 4 / static_cast<int>(sizeof(T));  // one 4-byte word of padding
  __shared__ __attribute__((aligned(16))) T tile[kTallRows][kPitch];
  __shared__ float scratch[kThreads / 64];
  __shared__ int slot;
  const int32_t* pre = c.prefix + PH_PREPARE * (c.batch + 1);
  const int32_t b = blockIdx.x;
  const int j = __builtin_amdgcn_readfirstlane(locate_matrix(pre, c.batch, b, &slot));
  const MatDesc& d = c.desc[j];
  const int32_t t = b - pre[j];
  T* xu = static_cast<T*>(iterate(d, 0));  // the first iterate buffer, holding U
  float acc;
  if (!d.tall) {
    // the user's rows are the iterate's: read and write the same vectors
    const int32_t tpr = d.l_pad / kWideTileCols;
    const int64_t i0 = static_cast<int64_t>(t / tpr) * kPrepWideRows;
    const int64_t j0 = static_cast<int64_t>(t % tpr) * kWideTileCols;
    constexpr int vpr = kWideTileCols / V;
    u32x4_t up[kVecsWide];
    acc = prepare_vectors<T, kVecsWide>(d, p, i0, j0, vpr, up);
    // V consecutive columns starting at a multiple of V stay inside one slab row
#pragma unroll
    for (int it = 0; it < kVecsWide; ++it) {
      const int v = it * kThreads + threadIdx.x;
      st16(xu + slab_off(i0 + v / vpr, j0 + (v % vpr) * V, d.l_pad), up[it]);
    }
  } else {
    const int32_t tpr = d.l_pad / kTallRows;
    const int64_t i0 = static_cast<int64_t>(t / tpr) * kTallCols;  // wide rows (short side)
    const int64_t j0 = static_cast<int64_t>(t % tpr) * kTallRows;  // wide cols (long side)
    constexpr int vpr = kTallCols / V;
    union Packed {
      u32x4_t v;
      T e[V];
    } up[kVecsTall];
    acc = prepare_vectors<T, kVecsTall>(d, p, j0, i0, vpr, &up[0].v);
#pragma unroll
    for (int it = 0; it < kVecsTall; ++it) {
      const int v = it * kThreads + threadIdx.x;
      const int row = v / vpr, col = (v % vpr) * V;
#pragma unroll
      for (int e = 0; e < V; ++e) tile[row][col + e] = up[it].e[e];
    }
    __syncthreads();
    // the wide tile is kTallCols x kTallRows: vector v covers wide row v / wvpr,
    // columns (v % wvpr) * V + 0..V-1, i.e. user rows of the tile at user column row
    constexpr int wvpr = kTallRows / V;
#pragma unroll
    for (int it = 0; it < kVecsTall; ++it) {
      const int v = it * kThreads + threadIdx.x;
      const int wrow = v / wvpr, wcol = (v % wvpr) * V;
      Packed o;
#pragma unroll
      for (int e = 0; e < V; ++e) o.e[e] = tile[wcol + e][wrow];
      st16(xu + slab_off(i0 + wrow, j0 + wcol, d.l_pad), o.v);
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
  const int32_t* pre = c.prefix + PH_PREPARE * (c.batch + 1);
  double s = 0.0;
  for (int32_t k = pre[j] + threadIdx.x; k < pre[j + 1]; k += kThreads) s += c.partials[k];
  s = block_sum(s, scratch);
  if (threadIdx.x == 0)
    c.inv_norm[j] = static_cast<float>(1.0 / (sqrt(s) + static_cast<double>(p.eps)));
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
  if (p.scale_x) {
    const float f = c.inv_norm[j];  // the iterate is U itself: O = X0 = f * U
#pragma unroll
    for (int e = 0; e < 16; ++e) o[e] *= f;
  }
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
hipError_t launch_prepare(const LaunchCtx& c, int32_t nblocks, bool is_bf16, const ElemParams& p) {
  if (nblocks <= 0) return hipSuccess;
  if (is_bf16)
    hipLaunchKernelGGL(k_prepare<uint16_t>, dim3(nblocks), dim3(kThreads), 0, c.stream, c, p);
  else
    hipLaunchKernelGGL(k_prepare<float>, dim3(nblocks), dim3(kThreads), 0, c.stream, c, p);
  return hipGetLastError();
}

hipError_t launch_finalize(const LaunchCtx& c, const ElemParams& p) {
  if (c.batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_finalize, dim3(c.batch), dim3(kThreads), 0, c.stream, c, p);
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

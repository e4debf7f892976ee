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
// 256 x 64) for a tall one, which is read as the user's kPrepTallL x
// kPrepTallS tile (bf16 rows of 512 bytes, as a wide tile's) and transposed
// through LDS.  (Tiles of 128 x 128, rows of 256 bytes, ran the pass at 0.66
// of the HBM peak against 0.72 for wide matrices.)  Each
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

// The bf16 tall tile (the user's kPrepTallL x kPrepTallS = 64 x 256, rows of
// 512 bytes) into the wide iterate, transposed through LDS.  Each thread's 8
// vectors go in as whole 16-byte row pieces (thread vector v: user row v / 32,
// chunk v % 32).  They come out with gfx950's transposing LDS read
// (ds_read_b64_tr_b16): a 16-lane group reads 4 user rows x 16 user columns
// (lanes 4r .. 4r + 3 take row r, 4 columns each) and lane j receives column j
// of the 4 rows.  Two such reads give a lane 8 consecutive user rows of one
// user column: one 16-byte vector of an iterate row.  Wave instruction I
// (0..31) covers user columns 16 (I % 16) + 0..15 and user rows 32 (I / 16) +
// 0..31: 16 iterate rows x 64 contiguous bytes of one slab.  Chunk k of user
// row r sits at chunk k ^ (2 (r & 3) + 8 ((r >> 3) & 1)), so that the 4 rows x
// 32 bytes of a group, and the two groups of a 32-lane half, fall on distinct
// banks.
__device__ __forceinline__ int tall_chunk(int row, int k) {
  return k ^ (2 * (row & 3) + 8 * ((row >> 3) & 1));
}

__device__ __forceinline__ void transpose_tall_bf16(char* lds, const u32x4_t* up, uint16_t* xu,
                                                    int64_t i0, int64_t j0, int64_t l_pad) {
  constexpr int kRowB = kPrepTallS * 2;       // 512 bytes
  constexpr int kChunks = kRowB / 16;         // 32 per user row
  constexpr int kColBlocks = kPrepTallS / 16;  // 16 blocks of 16 user columns
  constexpr int kNv = kPrepTallL * kPrepTallS / (8 * kThreads);  // vectors per thread
  static_assert(kNv * 8 * kThreads == kPrepTallL * kPrepTallS && kPrepTallL % 32 == 0,
                "whole vectors per thread; whole 32-row blocks");
#pragma unroll
  for (int it = 0; it < kNv; ++it) {
    const int v = it * kThreads + threadIdx.x;
    const int row = v / kChunks;
    *reinterpret_cast<u32x4_t*>(lds + row * kRowB + (tall_chunk(row, v % kChunks) << 4)) = up[it];
  }
  __syncthreads();
  uint16_t* const org = xu + slab_off(i0, j0, l_pad);  // the tile's origin (uniform)
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, rr = (lane >> 2) & 3, qq = lane & 3, j = lane & 15;
#pragma unroll
  for (int k = 0; k < kNv; ++k) {
    const int I = kNv * wave + k;
    const int wb = I % kColBlocks, cb = I / kColBlocks;
    u32x4_t o;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = 32 * cb + 8 * g + 4 * h + rr;
      const char* a = lds + row * kRowB + (tall_chunk(row, 2 * wb + (qq >> 1)) << 4) + 8 * (qq & 1);
      const s16x4_t x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4_t*)(a));
      const u32x2_t xv = __builtin_bit_cast(u32x2_t, x);
      o[2 * h] = xv[0];
      o[2 * h + 1] = xv[1];
    }
    // iterate row i0 + 16 wb + j (a user column), columns j0 + 32 cb + 8 g .. + 7 (user
    // rows); the tile's rows lie in one band of the slab layout
    st16_nt(org + slab_local(16 * wb + j, 32 * cb + 8 * g), o);
  }
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
  const int32_t per = c.per[PH_PREPARE];  // a uniform batch: the matrix by one division
  const int j = per > 0 ? b / per : __builtin_amdgcn_readfirstlane(locate_matrix(pre, c.batch, b, &slot));
  const MatDesc& d = c.desc[j];
  const int32_t t = per > 0 ? b - j * per : b - pre[j];
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
    // V consecutive columns starting at a multiple of V stay inside one slab row,
    // and the tile's rows inside one band.
    // Nontemporal: U is far larger than the caches, and the first Gram reads it
    // back from HBM (measured: the pass 1.5% faster than with cached stores).
    T* const org = xu + slab_off(i0, j0, d.l_pad);
#pragma unroll
    for (int it = 0; it < kVecsWide; ++it) {
      const int v = it * kThreads + threadIdx.x;
      st16_nt(org + slab_local(v / vpr, (v % vpr) * V), up[it]);
    }
  } else {
    // consecutive blocks take neighbouring column strips of the same user rows,
    // so that together they read whole user rows (measured: in the other order,
    // strips of one column across all rows, the pass ran 4% slower)
    const int32_t tps = d.s_pad / kTallCols;
    const int64_t i0 = static_cast<int64_t>(t % tps) * kTallCols;  // wide rows (short side)
    const int64_t j0 = static_cast<int64_t>(t / tps) * kTallRows;  // wide cols (long side)
    constexpr int vpr = kTallCols / V;
    union Packed {
      u32x4_t v;
      T e[V];
    } up[kVecsTall];
    acc = prepare_vectors<T, kVecsTall>(d, p, j0, i0, vpr, &up[0].v);
    if constexpr (sizeof(T) == 2) {
      transpose_tall_bf16(reinterpret_cast<char*>(&tile[0][0]), &up[0].v, xu, i0, j0, d.l_pad);
      const float total = block_sum(acc, scratch);
      if (threadIdx.x == 0) c.partials[b] = total;
      return;
    }
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
    T* const org = xu + slab_off(i0, j0, d.l_pad);  // the tile's rows lie in one band
#pragma unroll
    for (int it = 0; it < kVecsTall; ++it) {
      const int v = it * kThreads + threadIdx.x;
      const int wrow = v / wvpr, wcol = (v % wvpr) * V;
      Packed o;
#pragma unroll
      for (int e = 0; e < V; ++e) o.e[e] = tile[wcol + e][wrow];
      st16_nt(org + slab_local(wrow, wcol), o.v);
    }
  }
  const float total = block_sum(acc, scratch);
  if (threadIdx.x == 0) c.partials[b] = total;
}

// ---------------------------------------------------------------------------
// k_finalize: block j sums matrix j's partials in a fixed order (double), then
// stores 1 / (sqrt(sum) + eps).  Block 0 also zeroes both sets of claim
// counters, ahead of the call's first matrix-core launch.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_finalize(LaunchCtx c, ElemParams p) {
  __shared__ double scratch[kThreads / 64];
  const int j = blockIdx.x;
  if (j == 0 && threadIdx.x < 2 * kSchedInts) {
    int32_t* set = threadIdx.x < kSchedInts ? c.sched : c.sched_next;
    __hip_atomic_store(set + (threadIdx.x % kSchedInts), 0, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
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

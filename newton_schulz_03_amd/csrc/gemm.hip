// Matrix-core kernels of the Newton-Schulz iteration, on the padded wide
// iterate X (s_pad x l_pad, row-major):
//   GRAM  A = X X^T          upper-triangle tiles only, each stored twice (mirror)
//   POLY  B = b A + c A A    A is symmetric, so A A = A A^T: same form as GRAM
//   PROD  X' = a X + alpha Q X   with Q = B (or A when c == 0)
//
// One 256x256 output tile per workgroup of 4 wavefronts (2x2, 128x128 each),
// K staged through LDS 128 bytes at a time (64 bf16 or 32 fp32), double
// buffered so that one barrier per K slice suffices.  Every operand is held in
// LDS as rows of K ("K-major"), which is what a lane of the matrix core wants:
// 8 consecutive bf16 of K per lane for v_mfma_f32_32x32x16_bf16 (4 fp32 feed
// four v_mfma_f32_32x32x2_f32).  X, read as the right operand of Q X, is
// K-major in memory only along its columns; its 8x8 (4x4) blocks are
// transposed in registers on the way into LDS.  LDS rows are XOR-swizzled in
// 16-byte chunks so that both the row-wise fills and the fragment reads spread
// over the banks.
#include "device_common.hpp"

namespace muon {

namespace {

constexpr int kRowBytes = 128;                 // bytes of K per LDS row per stage
constexpr int kRowsPerOp = kTile;              // 256 rows per operand
constexpr int kOpBytes = kRowsPerOp * kRowBytes;  // 32 KiB
constexpr int kStageBytes = 2 * kOpBytes;         // P and Q operands
constexpr int kLdsBytes = 2 * kStageBytes;        // two stages: 128 KiB

enum GemmMode : int { GM_GRAM = 0, GM_POLY = 1, GM_PROD = 2 };

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kRowBytes + ((chunk ^ ((row ^ (row >> 3)) & 7)) << 4);
}

__device__ __forceinline__ u32x4_t lds_ld16(const char* lds, int off) {
  return *reinterpret_cast<const u32x4_t*>(lds + off);
}
__device__ __forceinline__ void lds_st16(char* lds, int off, const u32x4_t& v) {
  *reinterpret_cast<u32x4_t*>(lds + off) = v;
}

// 256 rows x 128 bytes of a row-major matrix whose rows are K: thread t moves
// chunk (t & 7) of rows (t >> 3) + 32u, u = 0..7.
template <typename T>
struct KMajorTile {
  static constexpr int V = Elt<T>::kVec;
  u32x4_t r[8];
  __device__ __forceinline__ void load(const T* rows, int64_t ld, int64_t k0) {
    const int c = threadIdx.x & 7, r0 = threadIdx.x >> 3;
    const T* p = rows + static_cast<int64_t>(r0) * ld + k0 + c * V;
#pragma unroll
    for (int u = 0; u < 8; ++u) r[u] = ld16(p + static_cast<int64_t>(32 * u) * ld);
  }
  __device__ __forceinline__ void store(char* lds) const {
    const int c = threadIdx.x & 7, r0 = threadIdx.x >> 3;
#pragma unroll
    for (int u = 0; u < 8; ++u) lds_st16(lds, swz(r0 + 32 * u, c), r[u]);
  }
};

// A slab of BK rows (K) x 256 columns (N) of a row-major matrix, stored in LDS
// transposed as 256 rows of K.  Moved in V x V blocks (V = elements per 16 B).
template <typename T>
struct MNMajorTile {
  static constexpr int V = Elt<T>::kVec;
  static constexpr int BK = kRowBytes / sizeof(T);
  static constexpr int NB = kRowsPerOp / V;      // blocks along N
  static constexpr int KB = BK / V;              // blocks along K (8)
  static constexpr int PER = NB * KB / kThreads;  // blocks per thread: 1 (bf16), 2 (fp32)
  u32x4_t r[PER][V];
  __device__ __forceinline__ void load(const T* cols, int64_t ld, int64_t k0) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int q = threadIdx.x + kThreads * p;
      const int nb = q % NB, kb = q / NB;
      const T* src = cols + (k0 + kb * V) * ld + nb * V;
#pragma unroll
      for (int e = 0; e < V; ++e) r[p][e] = ld16(src + static_cast<int64_t>(e) * ld);
    }
  }
  __device__ __forceinline__ void store(char* lds) const {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int q = threadIdx.x + kThreads * p;
      const int nb = q % NB, kb = q / NB;
#pragma unroll
      for (int i = 0; i < V; ++i) {
        u32x4_t o;
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int dw = 0; dw < 4; ++dw) {
            const uint32_t lo = r[p][2 * dw][i >> 1], hi = r[p][2 * dw + 1][i >> 1];
            o[dw] = (i & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
          }
        } else {
#pragma unroll
          for (int dw = 0; dw < 4; ++dw) o[dw] = r[p][dw][i];
        }
        lds_st16(lds, swz(nb * V + i, kb), o);
      }
    }
  }
};

// acc += P_frag * Q_frag over one 16-byte chunk of K per lane.
template <typename T>
__device__ __forceinline__ void mfma_chunk(f32x16_t& acc, const u32x4_t& p, const u32x4_t& q) {
  if constexpr (sizeof(T) == 2) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, p),
                                                   __builtin_bit_cast(bf16x8_t, q), acc, 0, 0, 0);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(p[e]), __uint_as_float(q[e]), acc,
                                                 0, 0, 0);
  }
}

template <typename T>
__device__ __forceinline__ void load4(const T* p, float* v) {
  if constexpr (sizeof(T) == 2) {
    const u32x2_t w = *reinterpret_cast<const u32x2_t*>(p);
    v[0] = __uint_as_float(w[0] << 16);
    v[1] = __uint_as_float(w[0] & 0xffff0000u);
    v[2] = __uint_as_float(w[1] << 16);
    v[3] = __uint_as_float(w[1] & 0xffff0000u);
  } else {
    const u32x4_t w = ld16(p);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = __uint_as_float(w[e]);
  }
}

template <typename T>
__device__ __forceinline__ void store4(T* p, const float* v) {
  if constexpr (sizeof(T) == 2) {
    u32x2_t w;
    w[0] = static_cast<uint32_t>(Elt<uint16_t>::from_f32(v[0])) |
           (static_cast<uint32_t>(Elt<uint16_t>::from_f32(v[1])) << 16);
    w[1] = static_cast<uint32_t>(Elt<uint16_t>::from_f32(v[2])) |
           (static_cast<uint32_t>(Elt<uint16_t>::from_f32(v[3])) << 16);
    *reinterpret_cast<u32x2_t*>(p) = w;
  } else {
    u32x4_t w;
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = __float_as_uint(v[e]);
    st16(p, w);
  }
}

// Upper-triangle tile (ti <= tj) number t of a T x T tile grid, row by row.
__device__ __forceinline__ void sym_tile(int32_t t, int32_t T, int32_t& ti, int32_t& tj) {
  int32_t i = 0;
  while (t >= T - i) {
    t -= T - i;
    ++i;
  }
  ti = i;
  tj = i + t;
}

}  // namespace

template <typename T, int MODE>
__global__ __launch_bounds__(kThreads, 1) void k_gemm(LaunchCtx c, int32_t cur, float a,
                                                      float alpha, float beta_c, int32_t use_poly) {
  __shared__ __attribute__((aligned(16))) char smem[kLdsBytes];
  constexpr int BK = kRowBytes / sizeof(T);

  const int32_t b = xcd_remap(static_cast<int32_t>(blockIdx.x), static_cast<int32_t>(gridDim.x));
  const int32_t* pre = c.prefix + (MODE == GM_PROD ? PH_PROD : PH_SYM) * (c.batch + 1);
  const int j = find_matrix(pre, c.batch, b);
  const MatDesc& d = c.desc[j];
  const int32_t t = b - pre[j];
  const int32_t ts = d.s_pad / kTile;
  int32_t ti, tj;
  if constexpr (MODE == GM_PROD) {
    ti = t % ts;  // tile row along the short side, fastest: neighbours share X columns
    tj = t / ts;
  } else {
    sym_tile(t, ts, ti, tj);
  }
  const int64_t s_pad = d.s_pad, l_pad = d.l_pad;
  const T* Xc = static_cast<const T*>(d.x[cur]);

  // Operand P (MFMA rows, index p) and Q (MFMA columns, index q): D[p][q] = sum_k P[p][k] Q[q][k].
  const T* p_base;
  const T* q_base;
  int64_t p_ld, q_ld, K;
  if constexpr (MODE == GM_GRAM) {
    p_base = Xc + ti * kTile * l_pad;  p_ld = l_pad;
    q_base = Xc + tj * kTile * l_pad;  q_ld = l_pad;
    K = l_pad;
  } else if constexpr (MODE == GM_POLY) {
    const T* A = static_cast<const T*>(d.gram);
    p_base = A + ti * kTile * s_pad;  p_ld = s_pad;
    q_base = A + tj * kTile * s_pad;  q_ld = s_pad;
    K = s_pad;
  } else {
    // P = columns tj of X (transposed on the way into LDS), Q = rows ti of B (or A)
    const T* Q = static_cast<const T*>(use_poly ? d.poly : d.gram);
    p_base = Xc + tj * kTile;  p_ld = l_pad;
    q_base = Q + ti * kTile * s_pad;  q_ld = s_pad;
    K = s_pad;
  }

  using PTile = typename std::conditional<MODE == GM_PROD, MNMajorTile<T>, KMajorTile<T>>::type;
  PTile pt;
  KMajorTile<T> qt;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, lh = lane >> 5;

  f32x16_t acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[mi][ni][e] = 0.f;

  const int nk = static_cast<int>(K / BK);
  pt.load(p_base, p_ld, 0);
  qt.load(q_base, q_ld, 0);
  pt.store(smem);
  qt.store(smem + kOpBytes);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    char* stage = smem + (kt & 1) * kStageBytes;
    const bool more = kt + 1 < nk;
    if (more) {
      pt.load(p_base, p_ld, static_cast<int64_t>(kt + 1) * BK);
      qt.load(q_base, q_ld, static_cast<int64_t>(kt + 1) * BK);
    }
    const char* P = stage;
    const char* Q = stage + kOpBytes;
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {
      const int chunk = 2 * sub + lh;
      u32x4_t pf[4], qf[4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) pf[mi] = lds_ld16(P, swz(wm * 128 + mi * 32 + lr, chunk));
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) qf[ni] = lds_ld16(Q, swz(wn * 128 + ni * 32 + lr, chunk));
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) mfma_chunk<T>(acc[mi][ni], pf[mi], qf[ni]);
    }
    if (more) {
      char* next = smem + ((kt + 1) & 1) * kStageBytes;
      pt.store(next);
      qt.store(next + kOpBytes);
    }
    __syncthreads();
  }

  // Epilogue.  Lane (lr, lh) holds D[p0 + e][q] for e = 0..3, with
  // p0 = wm*128 + mi*32 + 8g + 4lh and q = wn*128 + ni*32 + lr, in acc[mi][ni][4g + e].
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int p0 = wm * 128 + mi * 32 + 8 * g + 4 * lh;
        const int q = wn * 128 + ni * 32 + lr;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[mi][ni][4 * g + e];
        if constexpr (MODE == GM_PROD) {
          // D[p][q] = (Q X)[ti*256 + q][tj*256 + p]
          const int64_t row = static_cast<int64_t>(ti) * kTile + q;
          const int64_t col = static_cast<int64_t>(tj) * kTile + p0;
          float x[4];
          load4<T>(Xc + row * l_pad + col, x);
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = a * x[e] + alpha * v[e];
          store4<T>(static_cast<T*>(d.x[cur ^ 1]) + row * l_pad + col, v);
        } else {
          T* out = static_cast<T*>(MODE == GM_GRAM ? d.gram : d.poly);
          const int64_t rq = static_cast<int64_t>(tj) * kTile + q;   // mirror row
          const int64_t cp = static_cast<int64_t>(ti) * kTile + p0;  // mirror col
          if constexpr (MODE == GM_POLY) {
            // A[ti*256+p][tj*256+q] = A[tj*256+q][ti*256+p]: A is stored symmetric
            float av[4];
            load4<T>(static_cast<const T*>(d.gram) + rq * s_pad + cp, av);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = alpha * av[e] + beta_c * v[e];
          }
          float r[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) r[e] = Elt<T>::to_f32(Elt<T>::from_f32(v[e]));
          store4<T>(out + rq * s_pad + cp, r);
          if (ti != tj) {
#pragma unroll
            for (int e = 0; e < 4; ++e) out[(cp + e) * s_pad + rq] = Elt<T>::from_f32(r[e]);
          }
        }
      }
    }
  }
}

hipError_t launch_gram(const LaunchCtx& c, int32_t nblocks, bool is_bf16, int32_t cur) {
  if (nblocks <= 0) return hipSuccess;
  if (is_bf16)
    hipLaunchKernelGGL((k_gemm<uint16_t, GM_GRAM>), dim3(nblocks), dim3(kThreads), 0, c.stream, c,
                       cur, 0.f, 0.f, 0.f, 0);
  else
    hipLaunchKernelGGL((k_gemm<float, GM_GRAM>), dim3(nblocks), dim3(kThreads), 0, c.stream, c, cur,
                       0.f, 0.f, 0.f, 0);
  return hipGetLastError();
}

hipError_t launch_poly(const LaunchCtx& c, int32_t nblocks, bool is_bf16, float b, float cc) {
  if (nblocks <= 0) return hipSuccess;
  if (is_bf16)
    hipLaunchKernelGGL((k_gemm<uint16_t, GM_POLY>), dim3(nblocks), dim3(kThreads), 0, c.stream, c,
                       0, 0.f, b, cc, 0);
  else
    hipLaunchKernelGGL((k_gemm<float, GM_POLY>), dim3(nblocks), dim3(kThreads), 0, c.stream, c, 0,
                       0.f, b, cc, 0);
  return hipGetLastError();
}

hipError_t launch_prod(const LaunchCtx& c, int32_t nblocks, bool is_bf16, int32_t cur, float a,
                       float alpha, bool use_poly) {
  if (nblocks <= 0) return hipSuccess;
  if (is_bf16)
    hipLaunchKernelGGL((k_gemm<uint16_t, GM_PROD>), dim3(nblocks), dim3(kThreads), 0, c.stream, c,
                       cur, a, alpha, 0.f, use_poly ? 1 : 0);
  else
    hipLaunchKernelGGL((k_gemm<float, GM_PROD>), dim3(nblocks), dim3(kThreads), 0, c.stream, c, cur,
                       a, alpha, 0.f, use_poly ? 1 : 0);
  return hipGetLastError();
}

}  // namespace muon

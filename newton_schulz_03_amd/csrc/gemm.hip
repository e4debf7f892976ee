// Matrix-core kernels of the Newton-Schulz iteration, fp32 mode, on the padded
// wide iterate X (s_pad x l_pad, row-major).  (bf16 runs the pipelined kernel
// of gemm_bf16.hip; the tile decode and epilogues are shared.)
//   GRAM  A = X X^T          upper-triangle tiles only, each stored twice (mirror)
//   POLY  B = b A + c A A    A is symmetric, so A A = A A^T: same form as GRAM
//   PROD  X' = a X + alpha Q X   with Q = B (or A when c == 0)
//
// One 256x256 output tile per workgroup of 4 wavefronts (2x2, 128x128 each),
// K staged through LDS 128 bytes (32 fp32) at a time, double buffered so that
// one barrier per K slice suffices.  Every operand is held in LDS as rows of K
// ("K-major"), which is what a lane of the matrix core wants: 4 consecutive
// fp32 of K per lane feed four v_mfma_f32_32x32x2_f32.  X, read as the right
// operand of Q X, is K-major in memory only along its columns; its 4x4 blocks
// are transposed in registers on the way into LDS.  LDS rows are XOR-swizzled in
// 16-byte chunks so that both the row-wise fills and the fragment reads spread
// over the banks.
#include "gemm_common.hpp"

namespace muon {

namespace {

constexpr int kRowBytes = 128;                 // bytes of K per LDS row per stage
constexpr int kRowsPerOp = kTile;              // 256 rows per operand
constexpr int kOpBytes = kRowsPerOp * kRowBytes;  // 32 KiB
constexpr int kStageBytes = 2 * kOpBytes;         // P and Q operands
constexpr int kLdsBytes = 2 * kStageBytes;        // two stages: 128 KiB

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
  // rows [row0, row0 + 256) of a slab-layout matrix with ld columns, columns [k0, k0 + BK)
  __device__ __forceinline__ void load(const T* m, int64_t row0, int64_t ld, int64_t k0) {
    const int c = threadIdx.x & 7, r0 = threadIdx.x >> 3;
#pragma unroll
    for (int u = 0; u < 8; ++u) r[u] = ld16(m + slab_off(row0 + r0 + 32 * u, k0 + c * V, ld));
  }
  __device__ __forceinline__ void store(char* lds) const {
    const int c = threadIdx.x & 7, r0 = threadIdx.x >> 3;
#pragma unroll
    for (int u = 0; u < 8; ++u) lds_st16(lds, swz(r0 + 32 * u, c), r[u]);
  }
};

// A slab of BK rows (K) x 256 columns (N) of a row-major fp32 matrix, stored in
// LDS transposed as 256 rows of K.  Moved in 4 x 4 blocks (16 B per row).
template <typename T>
struct MNMajorTile {
  static_assert(sizeof(T) == 4, "fp32 only: bf16 runs the kernels of gemm_bf16.hip");
  static constexpr int V = Elt<T>::kVec;
  static constexpr int BK = kRowBytes / sizeof(T);
  static constexpr int NB = kRowsPerOp / V;      // blocks along N
  static constexpr int KB = BK / V;              // blocks along K (8)
  static constexpr int PER = NB * KB / kThreads;  // blocks per thread: 2
  u32x4_t r[PER][V];
  // rows [k0, k0 + BK) x columns [n0, n0 + 256) of a slab-layout matrix with ld columns
  __device__ __forceinline__ void load(const T* m, int64_t n0, int64_t ld, int64_t k0) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int q = threadIdx.x + kThreads * p;
      const int nb = q % NB, kb = q / NB;
#pragma unroll
      for (int e = 0; e < V; ++e) r[p][e] = ld16(m + slab_off(k0 + kb * V + e, n0 + nb * V, ld));
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
#pragma unroll
        for (int dw = 0; dw < 4; ++dw) o[dw] = r[p][dw][i];
        lds_st16(lds, swz(nb * V + i, kb), o);
      }
    }
  }
};

// acc += P_frag * Q_frag over one 16-byte chunk of K (4 fp32) per lane.
__device__ __forceinline__ void mfma_chunk(f32x16_t& acc, const u32x4_t& p, const u32x4_t& q) {
#pragma unroll
  for (int e = 0; e < 4; ++e)
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(p[e]), __uint_as_float(q[e]), acc,
                                               0, 0, 0);
}

}  // namespace

template <typename T, int MODE>
__global__ __launch_bounds__(kThreads, 1) void k_gemm_staged(LaunchCtx c, GemmArgs g) {
  __shared__ __attribute__((aligned(16))) char smem[kLdsBytes];
  constexpr int BK = kRowBytes / sizeof(T);

  __shared__ int slot, claimed;
  const int32_t t = claim_tile(g.split, c, &claimed);
  if (t < 0) return;  // the whole block
  const TileRef tr = decode_tile<MODE>(c, t, &slot);
  const MatDesc& d = tr.d;
  const int32_t ti = tr.ti, tj = tr.tj;
  const int64_t s_pad = d.s_pad, l_pad = d.l_pad;
  const T* Xc = static_cast<const T*>(iterate(d, g.cur));

  // Operand P (MFMA rows, index p) and Q (MFMA columns, index q): D[p][q] = sum_k P[p][k] Q[q][k].
  // p_at / q_at: first row (K-major) or first column (MN-major) of the tile's operand.
  const T* p_m;
  const T* q_m;
  int64_t p_at, q_at, p_ld, q_ld, K;
  if constexpr (MODE == GM_GRAM) {
    p_m = Xc;  p_at = ti * kTile;  p_ld = l_pad;
    q_m = Xc;  q_at = tj * kTile;  q_ld = l_pad;
    K = l_pad;
  } else if constexpr (MODE == GM_POLY) {
    const T* A = static_cast<const T*>(d.gram);
    p_m = A;  p_at = ti * kTile;  p_ld = s_pad;
    q_m = A;  q_at = tj * kTile;  q_ld = s_pad;
    K = s_pad;
  } else {
    // P = columns tj of X (transposed on the way into LDS), Q = rows ti of B (or A)
    p_m = Xc;  p_at = tj * kTile;  p_ld = l_pad;
    q_m = static_cast<const T*>(g.use_poly ? d.poly : d.gram);  q_at = ti * kTile;  q_ld = s_pad;
    K = s_pad;
  }

  using PTile = typename std::conditional<MODE == GM_PROD, MNMajorTile<T>, KMajorTile<T>>::type;
  PTile pt;
  KMajorTile<T> qt;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, lh = lane >> 5;

  f32x16_t acc[4][4];
  zero_acc(acc);

  const int nk = static_cast<int>(K / BK);
  pt.load(p_m, p_at, p_ld, 0);
  qt.load(q_m, q_at, q_ld, 0);
  pt.store(smem);
  qt.store(smem + kOpBytes);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    char* stage = smem + (kt & 1) * kStageBytes;
    const bool more = kt + 1 < nk;
    if (more) {
      pt.load(p_m, p_at, p_ld, static_cast<int64_t>(kt + 1) * BK);
      qt.load(q_m, q_at, q_ld, static_cast<int64_t>(kt + 1) * BK);
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
        for (int ni = 0; ni < 4; ++ni) mfma_chunk(acc[mi][ni], pf[mi], qf[ni]);
    }
    if (more) {
      char* next = smem + ((kt + 1) & 1) * kStageBytes;
      pt.store(next);
      qt.store(next + kOpBytes);
    }
    __syncthreads();
  }
  gemm_store<T, MODE, true>(acc, tr, g, norm_factor<MODE>(c, g, tr));
}

namespace {

// The tiles that sp splits.  bf16 launches under a CU budget (c.max_blocks
// workgroups, fewer than one per tile) loop over the tiles instead.
template <int MODE>
hipError_t launch_mode(const LaunchCtx& c, const XcdSplit& sp, bool is_bf16, GemmArgs g) {
  const int32_t ntiles = sp.lo[kXcd];
  if (ntiles <= 0) return hipSuccess;
  g.ntiles = ntiles;
  g.split = sp;
  if (is_bf16) {
    const bool loop = c.max_blocks > 0 && c.max_blocks < sp.grid;
    const int32_t grid = !loop ? sp.grid : c.max_blocks < ntiles ? c.max_blocks : ntiles;
    return launch_gemm_bf16(MODE, c, grid, loop, g);
  }
  hipLaunchKernelGGL((k_gemm_staged<float, MODE>), dim3(sp.grid), dim3(kThreads), 0, c.stream, c,
                     g);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gram(const LaunchCtx& c, const XcdSplit& sp, bool is_bf16, int32_t cur,
                       float out_scale, bool first) {
  GemmArgs g{cur, 0.f, out_scale, 0, FIN_NONE, 0.f, first ? 1 : 0, 0, {}};
  return launch_mode<GM_GRAM>(c, sp, is_bf16, g);
}

hipError_t launch_poly(const LaunchCtx& c, const XcdSplit& sp, bool is_bf16, float b, float cc) {
  GemmArgs g{0, b / cc, cc, 0, FIN_NONE, 0.f, 0, 0, {}};
  return launch_mode<GM_POLY>(c, sp, is_bf16, g);
}

hipError_t launch_prod(const LaunchCtx& c, const XcdSplit& sp, bool is_bf16, int32_t cur, float a,
                       bool use_poly, bool first, int32_t finish, float lr) {
  if (finish != FIN_NONE && !is_bf16) return hipErrorInvalidValue;  // fp32 keeps the finish kernel
  GemmArgs g{cur, a, 1.f, use_poly ? 1 : 0, finish, lr, first ? 1 : 0, 0, {}};
  return launch_mode<GM_PROD>(c, sp, is_bf16, g);
}

}  // namespace muon

// Shared pieces of the matrix-core kernels: tile decode and epilogues.
//
// Every kernel computes one 256x256 tile D[p][q] = sum_k P[p][k] Q[q][k] with
// 4 wavefronts in a 2x2 grid (128x128 each) of v_mfma 32x32 blocks.  Lane
// (lr = lane % 32, lh = lane / 32) of wave (wm, wn) holds, in acc[mi][ni][4g+e],
//   D[p0 + e][q]  with  p0 = wm*128 + mi*32 + 8g + 4lh,  q = wn*128 + ni*32 + lr.
//
//   GRAM  P = Q = rows of X          D = (X X^T) tile (ti, tj), ti <= tj
//   POLY  P = Q = rows of A          D = (A A) tile (ti, tj), ti <= tj
//   PROD  P = columns tj of X, Q = rows ti of B (or A):  D[p][q] = (B X)[ti*256+q][tj*256+p]
#pragma once

#include "device_common.hpp"

namespace muon {

enum GemmMode : int { GM_GRAM = 0, GM_POLY = 1, GM_PROD = 2 };

// What each kernel accumulates and stores (s = init_scale):
//   GRAM  acc = X X^T,            A  = out_scale * acc   (out_scale = b when c = 0, else 1)
//   POLY  acc = A A + s A,        B  = c * acc = b A + c A A   (s = b/c)
//   PROD  acc = Q X + s X,        X' = acc                     (s = a)
// In the first iteration X holds U = (||U||_F + eps) X0, so the Gram stores
// f^2 * out_scale * acc and the product f * acc, f = 1 / (||U||_F + eps)
// (norm_factor); the iteration then runs on X0 exactly as written above.
// The s-multiple of the source tile is added inside the K loop by the bf16
// kernel (matrix cores, see gemm_bf16.hip) and at store time by the fp32 one.
// The last product of a call can hand its result straight to the user's
// matrix instead of the workspace (bf16 kernel): FIN_STEP writes
// W - lr * scale * X', FIN_NS writes X' to the output.
enum FinishMode : int { FIN_NONE = 0, FIN_STEP = 1, FIN_NS = 2 };

struct GemmArgs {
  int32_t cur;        // X buffer holding the current iterate
  float init_scale;   // POLY: b/c;  PROD: a
  float out_scale;    // GRAM: 1 or b;  POLY: c;  PROD: 1
  int32_t use_poly;   // PROD: Q = B (1) or A (0)
  int32_t finish;     // PROD: FinishMode
  float lr;           // PROD with FIN_STEP: learning rate
  int32_t first;      // GRAM, PROD: X[cur] holds U; scale by f^2 (GRAM) or f (PROD), f = inv_norm
  int32_t ntiles;     // tiles of the launch
  XcdSplit split;     // one tile per workgroup: which tile workgroup b takes (claim_tile)
};

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
    w[0] = Elt<uint16_t>::pack2(v[0], v[1]);
    w[1] = Elt<uint16_t>::pack2(v[2], v[3]);
    *reinterpret_cast<u32x2_t*>(p) = w;
  } else {
    u32x4_t w;
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = __float_as_uint(v[e]);
    st16(p, w);
  }
}

// Tile orders that keep the operand bands of concurrently running tiles few:
// the tile rows are taken kTileGroup at a time, so a round of neighbouring
// tiles (one XCD's 32 CUs) reads about 8 row bands and 4 column bands, not 24
// row bands and 1 column band of a 24 x 24 grid.

constexpr int32_t kTileGroup = 8;

// Product tile number t of a ts x tl grid: in a group of kTileGroup tile rows,
// rows run fastest.  With ts <= kTileGroup this is row-fastest order overall.
__host__ __device__ __forceinline__ void prod_tile(int32_t t, int32_t ts, int32_t tl, int32_t& ti,
                                                   int32_t& tj) {
  const int32_t per_group = kTileGroup * tl;
  const int32_t grp = t / per_group, first = grp * kTileGroup;
  const int32_t g = ts - first < kTileGroup ? ts - first : kTileGroup;
  const int32_t r = t - grp * per_group;
  ti = first + r % g;
  tj = r / g;
}

// Upper-triangle tile (ti <= tj) number t of a T x T tile grid.  Bands of
// kTileGroup tile rows in order; in a band of g rows starting at row a, first
// the g x g triangle without its diagonal, column by column (column a + d holds
// rows a .. a + d - 1), then the g diagonal tiles in a row, then the columns
// right of the triangle, g rows each.
//
// Why the diagonal tiles are consecutive: an XCD dispatches its workgroups in
// order, and its k-th goes to shader engine k mod 4, whether or not that engine
// has a free CU.  A diagonal tile forms 36 of the 64 blocks and finishes early;
// scattered among longer tiles, they free CUs on one engine while the next
// workgroup in order waits for a CU on another, and the free CUs idle meanwhile.
// Four consecutive workgroups land on the four engines, so a run of diagonal
// tiles gives every engine the same mix of short and long tiles.
__host__ __device__ __forceinline__ void sym_tile(int32_t t, int32_t T, int32_t& ti, int32_t& tj) {
  int32_t a = 0;
  for (;;) {
    const int32_t g = T - a < kTileGroup ? T - a : kTileGroup;
    const int32_t off = g * (g - 1) / 2;  // off-diagonal tiles of the triangle
    const int32_t tri = off + g;
    const int32_t band = tri + g * (T - a - g);
    if (t < band) {
      if (t < off) {
        // column a + d holds triangle tiles d (d - 1) / 2 .. d (d + 1) / 2 - 1
        int32_t d = 1;
        while ((d + 1) * d / 2 <= t) ++d;
        ti = a + (t - d * (d - 1) / 2);
        tj = a + d;
      } else if (t < tri) {
        ti = tj = a + (t - off);
      } else {
        const int32_t r = t - tri;
        ti = a + r % g;
        tj = a + g + r / g;
      }
      return;
    }
    t -= band;
    a += kTileGroup;
  }
}

struct TileRef {
  MatDesc d;  // a register copy: the epilogue's stores cannot alias it
  int32_t mat;  // index of the matrix in the batch
  int32_t ti, tj;
};

// Extra factor of the stored result (see the table at GemmArgs): f^2 for the
// first Gram, f for the first product, 1 otherwise.
template <int MODE>
__device__ __forceinline__ float norm_factor(const LaunchCtx& c, const GemmArgs& g,
                                             const TileRef& tr) {
  if (MODE == GM_POLY || !g.first) return 1.f;
  const float f = c.inv_norm[tr.mat];
  return MODE == GM_GRAM ? f * f : f;
}

// XCD x's range [lo, hi) and the start of its pool [dyn, hi) (an unrolled
// select: no dynamic index into the kernel argument).
__host__ __device__ __forceinline__ void xcd_range(const XcdSplit& s, int32_t x, int32_t& lo,
                                                   int32_t& dyn, int32_t& hi) {
  lo = s.lo[0];
  dyn = s.dyn[0];
  hi = s.lo[1];
#pragma unroll
  for (int i = 1; i < kXcd; ++i) {
    if (x == i) {
      lo = s.lo[i];
      dyn = s.dyn[i];
      hi = s.lo[i + 1];
    }
  }
}

// Statically dealt tile of workgroup b: b runs on XCD x = b % 8 and takes the
// (b / 8)-th tile of that XCD's range, unless it lies in the range's pool; -1
// otherwise (the workgroup then claims a pool tile, or finds none left).
__host__ __device__ __forceinline__ int32_t split_tile(const XcdSplit& s, int32_t b) {
  const int32_t x = b % kXcd, k = b / kXcd;
  int32_t lo, dyn, hi;
  xcd_range(s, x, lo, dyn, hi);
  return lo + k < dyn ? lo + k : -1;
}

// Workgroup 0 of a matrix-core launch zeroes the next launch's claim counters
// (the previous launch's set, which no workgroup uses any more).
__device__ __forceinline__ void zero_next_sched(const LaunchCtx& c) {
  if (blockIdx.x == 0 && threadIdx.x < kSchedInts)
    __hip_atomic_store(c.sched_next + threadIdx.x, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The tile of this workgroup, or -1.  Called by the whole block (the branch
// depends on blockIdx.x only); lds is one int of LDS.
//
// A workgroup past the static part of its XCD's range claims a pool tile.
//
// Single queue (s.norder > 0): one increment of counter kXcd; the old value k
// names the k-th entry of the queue, or nothing once k >= s.norder.
//
// Per-XCD pools: wave 0 increments its own XCD's counter: the old value k
// hands out the k-th tile of that pool.  Once that pool is empty, the wave
// reads all eight counters and claims from the pool with the most tiles left,
// and repeats while some pool has tiles.
//
// Every increment returns a distinct value, so each pool tile goes to exactly
// one workgroup.  A workgroup gives up only after finding every pool (or the
// queue) empty.  The grid holds at least as many claiming workgroups as pool
// tiles.  So every tile is taken exactly once.  A failed per-XCD claim means
// that pool emptied after it was read, and it is never picked again: at most
// kXcd failures, so the loop ends.
__device__ __forceinline__ int32_t claim_tile(const XcdSplit& s, const LaunchCtx& c, int* lds) {
  const int32_t b = static_cast<int32_t>(blockIdx.x);
  zero_next_sched(c);
  const int32_t t0 = split_tile(s, b);
  if (t0 >= 0 || s.pool == 0) return t0;
  if (s.norder > 0) {
    if (threadIdx.x == 0) {
      const int32_t k = atomicAdd(c.sched + kXcd, 1);
      *lds = k < s.norder ? c.orders[s.order_off + k] : -1;
    }
  } else if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int32_t t = -1;
    auto claim = [&](int32_t y) {  // lane 0: one increment of pool y's counter
      if (lane == 0) {
        int32_t lo, dyn, hi;
        xcd_range(s, y, lo, dyn, hi);
        if (dyn < hi) {
          const int32_t k = atomicAdd(c.sched + y, 1);
          if (k < hi - dyn) t = dyn + k;
        }
      }
      t = __shfl(t, 0);
    };
    claim(b % kXcd);
    for (int round = 0; t < 0 && round <= kXcd; ++round) {
      // key = (tiles left) * 8 + (7 - y) on lane y < 8: the largest names the
      // pool with the most tiles left (the lowest y on a tie)
      int32_t key = -(1 << 30);
      if (lane < kXcd) {
        int32_t lo, dyn, hi;
        xcd_range(s, lane, lo, dyn, hi);
        const int32_t taken =
            __hip_atomic_load(c.sched + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        key = (hi - dyn - taken) * kXcd + (kXcd - 1 - lane);
      }
#pragma unroll
      for (int m = 1; m < kXcd; m <<= 1) key = max(key, __shfl_xor(key, m));
      key = __shfl(key, 0);
      if (key < kXcd) break;  // no pool has a tile left
      claim(kXcd - 1 - (key & (kXcd - 1)));
    }
    if (lane == 0) *lds = t;
  }
  __syncthreads();
  // uniform: without readfirstlane the tile and everything derived from it
  // (matrix, tile row and column, addresses) would sit in vector registers,
  // and the product kernels spill
  return __builtin_amdgcn_readfirstlane(*lds);
}

// Tile number b of the launch -> (matrix, tile) for the symmetric phases (GRAM,
// POLY) or the product.  Called by the whole block: the matrix is located
// cooperatively, through `slot` in LDS.
template <int MODE>
__device__ __forceinline__ TileRef decode_tile(const LaunchCtx& c, int32_t b, int* slot) {
  constexpr int ph = MODE == GM_PROD ? PH_PROD : PH_SYM;
  const int32_t* pre = c.prefix + ph * (c.batch + 1);
  // a uniform batch: the matrix by one division, without the prefix table's
  // loads and the lookup's barrier on the tile's way to its first loads
  const int32_t per = c.per[ph];
  const int j = per > 0 ? b / per : __builtin_amdgcn_readfirstlane(locate_matrix(pre, c.batch, b, slot));
  TileRef r;
  r.d = load_const(c.desc + j);
  r.mat = j;
  const int32_t t = per > 0 ? b - j * per : b - load_const(pre + j);
  const int32_t ts = r.d.s_pad / kTile;
  if constexpr (MODE == GM_PROD) {
    prod_tile(t, ts, r.d.l_pad / kTile, r.ti, r.tj);
  } else {
    sym_tile(t, ts, r.ti, r.tj);
  }
  return r;
}

// Per-lane coordinates of the accumulator layout described above.
struct LanePos {
  int64_t row0, col0;  // PROD: output row (ti*256 + q0) and column (tj*256 + p0) of acc[0][0][0]
  int64_t rq0, cp0;    // GRAM/POLY: the mirror position (row tj*256 + q0, column ti*256 + p0)
};

__device__ __forceinline__ LanePos lane_pos(const TileRef& tr) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, lh = lane >> 5;
  LanePos lp;
  lp.row0 = static_cast<int64_t>(tr.ti) * kTile + wn * 128 + lr;
  lp.col0 = static_cast<int64_t>(tr.tj) * kTile + wm * 128 + 4 * lh;
  lp.rq0 = static_cast<int64_t>(tr.tj) * kTile + wn * 128 + lr;
  lp.cp0 = static_cast<int64_t>(tr.ti) * kTile + wm * 128 + 4 * lh;
  return lp;
}

__device__ __forceinline__ void zero_acc(f32x16_t (&acc)[4][4]) {
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[mi][ni][e] = 0.f;
}

// Stores the finished tile.  With ADD_TERM the accumulated sum does not yet
// hold the init_scale multiple of the source tile (X for the product, A for
// the polynomial); it is read and added here, one row of blocks at a time.
template <typename T, int MODE, bool ADD_TERM>
__device__ __forceinline__ void gemm_store(const f32x16_t (&acc)[4][4], const TileRef& tr,
                                           const GemmArgs& g, float nf) {
  const LanePos lp = lane_pos(tr);
  const int64_t s_pad = tr.d.s_pad, l_pad = tr.d.l_pad;
  if constexpr (MODE == GM_PROD) {
    const T* __restrict__ xin = static_cast<const T*>(iterate(tr.d, g.cur));
    T* __restrict__ xout = static_cast<T*>(iterate(tr.d, g.cur ^ 1));
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      float x[4][4][4];
      if constexpr (ADD_TERM) {
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
#pragma unroll
          for (int gg = 0; gg < 4; ++gg)
            load4<T>(xin + slab_off(lp.row0 + ni * 32, lp.col0 + mi * 32 + 8 * gg, l_pad), x[ni][gg]);
      }
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[e] = acc[mi][ni][4 * gg + e];
            if constexpr (ADD_TERM) v[e] += g.init_scale * x[ni][gg][e];
            v[e] *= nf;
          }
          store4<T>(xout + slab_off(lp.row0 + ni * 32, lp.col0 + mi * 32 + 8 * gg, l_pad), v);
        }
    }
  } else {
    // D[p][q] = S[ti*256 + p][tj*256 + q] of the symmetric result S; the lane's
    // four consecutive p are contiguous in row (tj*256 + q) of S (the mirror).
    T* __restrict__ out = static_cast<T*>(MODE == GM_GRAM ? tr.d.gram : tr.d.poly);
    const T* __restrict__ gram = static_cast<const T*>(tr.d.gram);
    const bool offdiag = tr.ti != tr.tj;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      float av[4][4][4];
      if constexpr (ADD_TERM && MODE == GM_POLY) {
        // A[ti*256+p][tj*256+q] = A[tj*256+q][ti*256+p]: A is stored symmetric
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
#pragma unroll
          for (int gg = 0; gg < 4; ++gg)
            load4<T>(gram + slab_off(lp.rq0 + ni * 32, lp.cp0 + mi * 32 + 8 * gg, s_pad), av[ni][gg]);
      }
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float t = acc[mi][ni][4 * gg + e];
            if constexpr (ADD_TERM && MODE == GM_POLY) t += g.init_scale * av[ni][gg][e];
            v[e] = g.out_scale * nf * t;
          }
          const int64_t rq = lp.rq0 + ni * 32, cp = lp.cp0 + mi * 32 + 8 * gg;
          store4<T>(out + slab_off(rq, cp, s_pad), v);
          if (offdiag) {
#pragma unroll
            for (int e = 0; e < 4; ++e) out[slab_off(cp + e, rq, s_pad)] = Elt<T>::from_f32(v[e]);
          }
        }
    }
  }
}

// Launches of the bf16 pipelined kernels (gemm_bf16.hip): g.split.grid
// workgroups of one tile each, or (loop) nblocks < g.ntiles workgroups that
// loop over the tiles.
hipError_t launch_gemm_bf16(int mode, const LaunchCtx& c, int32_t nblocks, bool loop,
                            const GemmArgs& g);

}  // namespace muon

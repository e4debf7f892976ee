// Matrix-core products on block-scaled e4m3 operands, for the e4m3 steps (gfx950).
//
// The tiles (256 x 256, four waves of 128 x 128), the LDS ring of 4 stages,
// the direct-to-LDS loads with hand-counted waits and the staged tile store
// are the bf16 kernel's (gemm_pipeline.hpp).  What differs:
//  * A stage row holds 64 e4m3 K values in the bf16 row's 64 bytes, so one
//    stage is one K step of v_mfma_scale_f32_32x32x64_f8f6f4: twice the K of a
//    bf16 stage, at twice the matrix-core rate per cycle.
//  * Both operands are K-major (the product reads X^T), each in the F8 layout
//    (muon_internal.hpp), and every stage also carries the two operands'
//    block scales, 512 bytes each (one dword-per-lane load per wave: waves 0-1
//    the P scales, waves 2-3 the Q scales).
//  * Lane (r, h) of a 32-row fragment holds 16 values of the row's first
//    32-value block and 16 of its second: chunks h and 2 + h of the 64-byte
//    row, the two chunks the bf16 kernel reads for its two K halves, at the
//    same swizzled offsets.  The lane supplies the scale of its row's block h;
//    one dword holds the scales of the lane's four fragment rows, and op_sel
//    picks the byte for each MFMA.
//  * The a X (product) and (b/c) A (A^2) terms are added to the fp32
//    accumulators in the epilogue, read from the bf16 X and A.
// Per slice: the first half's 8 MFMAs go out with the P and scale loads of
// slice kt+3; after the wait for slice kt+1 and one barrier, the second half's
// 8 MFMAs go out with the Q loads of slice kt+3 and the reads of slice kt+1's
// fragments into the other fragment set.
#include <utility>

#include "gemm_pipeline.hpp"

namespace muon {

namespace {

constexpr int SCB = 512;                   // scale bytes per operand and stage
constexpr int STAGE8 = 2 * OPB + 2 * SCB;  // 33 KiB: P data, Q data, P scales, Q scales
constexpr int LDS8 = NST * STAGE8;         // 132 KiB
constexpr int LOADS8 = 2 * LPO + 1;        // loads per wave and stage: P, then scales, then Q
static_assert(LDS8 >= kTile * MNROW, "the tile store stages a whole 256 x 256 bf16 tile in the ring");
static_assert(LDS8 + 1024 <= 160 * 1024, "LDS of a CU");

typedef int32_t i32x8_t __attribute__((ext_vector_type(8)));

// One dword per lane straight into LDS (lane i's 4 bytes at lds_addr + 4 i),
// counted by hand like lds_dma16.
__device__ __forceinline__ void lds_dma4(uint32_t lds_addr, int32_t voff, i32x4_t rsrc) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}

// This wave's quarter of a stage's scales: 256 bytes of one operand's 512.
struct ScaleStream {
  const char* base;  // the operand band's scales at slice 0, plus this wave's half (uniform)
  int32_t lds;       // LDS byte offset within a stage

  __device__ __forceinline__ void issue(int ks, uint32_t stage_lds, int lane) const {
    const uint64_t b = reinterpret_cast<uint64_t>(base) + static_cast<uint64_t>(ks) * SCB;
    i32x4_t r;
    r[0] = __builtin_amdgcn_readfirstlane(static_cast<int32_t>(b & 0xffffffffu));
    r[1] = __builtin_amdgcn_readfirstlane(static_cast<int32_t>((b >> 32) & 0xffffu));
    r[2] = 256;  // exactly the bytes this load reads
    r[3] = 0x00020000;
    lds_dma4(__builtin_amdgcn_readfirstlane(stage_lds + lds), 4 * lane, r);
  }
};

struct Frags8 {
  i32x8_t p[4];    // P fragments: rows 32 mi + r of the wave's 128; dwords 0-3 chunk h, 4-7 chunk 2 + h
  i32x8_t q[4];
  int32_t sp, sq;  // scale dwords: byte mi (ni) is the scale of fragment row mi (ni), block h
};

// Half h (dwords 4h .. 4h + 3) of a fragment from one 16-byte LDS read.
__device__ __forceinline__ void set_half(i32x8_t& f, int h, const u32x4_t& v) {
#pragma unroll
  for (int k = 0; k < 4; ++k) f[4 * h + k] = static_cast<int32_t>(v[k]);
}

// Adds the init_scale multiple of the source tile to the accumulators (lane
// layout of gemm_common.hpp): PROD  a X[ti*256 + q][tj*256 + p];
// POLY  (b/c) A[ti*256 + p][tj*256 + q], read as A[tj*256 + q][ti*256 + p] (A is
// stored symmetric).  Four consecutive p are contiguous in a row of the slab.
template <int MODE>
__device__ __forceinline__ void add_term(f32x16_t (&acc)[4][4], const TileRef& tr,
                                         const GemmArgs& g) {
  const LanePos lp = lane_pos(tr);
  const uint16_t* src = static_cast<const uint16_t*>(MODE == GM_PROD ? iterate(tr.d, g.cur)
                                                                      : tr.d.gram);
  const int64_t ld = MODE == GM_PROD ? tr.d.l_pad : tr.d.s_pad;
  const int64_t r0 = MODE == GM_PROD ? lp.row0 : lp.rq0;
  const int64_t c0 = MODE == GM_PROD ? lp.col0 : lp.cp0;
  // the tile's origin (uniform) and this lane's offsets within the tile
  const int64_t tr0 = static_cast<int64_t>(MODE == GM_PROD ? tr.ti : tr.tj) * kTile;
  const int64_t tc0 = static_cast<int64_t>(MODE == GM_PROD ? tr.tj : tr.ti) * kTile;
  const uint16_t* const org = src + slab_off(tr0, tc0, ld);
  const int q0 = static_cast<int>(r0 - tr0), p0 = static_cast<int>(c0 - tc0);
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    float x[4][4][4];
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg)
        load4<uint16_t>(org + slab_local(q0 + ni * 32, p0 + mi * 32 + 8 * gg), x[ni][gg]);
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[mi][ni][4 * gg + e] += g.init_scale * x[ni][gg][e];
  }
}

// One output tile (tile number t of the launch), as gemm_tile in gemm_bf16.hip.
//   GRAM  P = Q = rows of X (buffer 0), K = l_pad
//   POLY  P = Q = rows of A (buffer 0), K = s_pad
//   PROD  P = rows tj of X^T (buffer 1), Q = rows ti of B (buffer 0), K = s_pad
template <int MODE, bool FIRST>
__device__ __forceinline__ void gemm_tile_f8(const LaunchCtx& c, const GemmArgs& g, int32_t t,
                                             char* smem, int* slot) {
  const TileRef tr = decode_tile<MODE>(c, t, slot);
  const MatDesc& d = tr.d;
  const int64_t cap = static_cast<int64_t>(d.s_pad) * d.l_pad;  // scales follow the data
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, lh = lane >> 5;

  const char* pm = f8_buffer(d, MODE == GM_PROD ? 1 : 0);
  const char* qm = f8_buffer(d, 0);
  const int64_t kcols = MODE == GM_GRAM ? d.l_pad : d.s_pad;  // K of both operands
  const int64_t pband = MODE == GM_PROD ? tr.tj : tr.ti;
  const int64_t qband = MODE == GM_PROD ? tr.ti : tr.tj;
  // a 64-column e4m3 slab has the bytes of a 32-column bf16 slab
  const Stream sp = kmajor_stream(reinterpret_cast<const uint16_t*>(pm), pband, kcols / 2, wave, lane);
  const Stream sq = kmajor_stream(reinterpret_cast<const uint16_t*>(qm), qband, kcols / 2, wave, lane);
  const int64_t spb = kcols / 64;  // slabs per band
  ScaleStream ss;
  {
    const bool q_op = (wave >> 1) != 0;
    ss.base = (q_op ? qm : pm) + cap + (q_op ? qband : pband) * spb * SCB + (wave & 1) * 256;
    ss.lds = 2 * OPB + (wave >> 1) * SCB + (wave & 1) * 256;
  }
  const int nk = static_cast<int>(kcols / 64);

  // Per-lane offsets within a stage: the bf16 kernel's fragment offsets for
  // its K halves 0 and 1 are this lane's chunks h and 2 + h.
  int32_t qoff[2], poff[2];
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    const int sw = ((2 * sub + lh) ^ kkey(lr)) << 4;
    qoff[sub] = OPB + (wn * 128 + lr) * KROW + sw;
    poff[sub] = (wm * 128 + lr) * KROW + sw;
  }
  const int32_t psc = 2 * OPB + 4 * (32 * (2 * wm + lh) + lr);
  const int32_t qsc = 2 * OPB + SCB + 4 * (32 * (2 * wn + lh) + lr);

  // Fragment reads in the order the MFMAs consume them: the scales, P[0],
  // Q[0..3], then P[1..3]; two 16-byte reads per fragment.
  constexpr int NREAD8 = 18;
  auto read_op = [&](Frags8& f, const char* stage, int i) {
    if (i == 0) {
      f.sp = *reinterpret_cast<const int32_t*>(stage + psc);
    } else if (i == 1) {
      f.sq = *reinterpret_cast<const int32_t*>(stage + qsc);
    } else if (i < 4) {
      set_half(f.p[0], i - 2, lds16(stage + poff[i - 2]));
    } else if (i < 12) {
      const int ni = (i - 4) >> 1, h = (i - 4) & 1;
      set_half(f.q[ni], h, lds16(stage + qoff[h] + ni * 32 * KROW));
    } else {
      const int mi = 1 + ((i - 12) >> 1), h = (i - 12) & 1;
      set_half(f.p[mi], h, lds16(stage + poff[h] + mi * 32 * KROW));
    }
  };

  f32x16_t acc[4][4];
  zero_acc(acc);

  const uint32_t ring = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((LDS_AS char*)smem));

  // Prologue: slices 0..NST-2 requested (P, scales, Q each), slice 0 awaited.
  // Slice indices past the end are clamped to the last slice: those loads
  // refill a stage nobody reads again and keep the count in flight constant.
#pragma unroll
  for (int s = 0; s < NST - 1; ++s) {
    const int ks = s < nk ? s : nk - 1;
    sp.issue(ks, ring + s * STAGE8);
    ss.issue(ks, ring + s * STAGE8, lane);
    sq.issue(ks, ring + s * STAGE8 + OPB);
  }
  wait_vm<(NST - 2) * LOADS8>();
  __syncthreads();

  Frags8 f0, f1;
#pragma unroll
  for (int i = 0; i < NREAD8; ++i) read_op(f0, smem, i);

  // Slice kt on fragments fa (stage kt), reading stage kt+1 into fb.
  auto slice = [&](int kt, Frags8& fa, Frags8& fb) {
    const int ks = kt + NST - 1 < nk ? kt + NST - 1 : nk - 1;
    const uint32_t fill = ring + ((kt + NST - 1) & (NST - 1)) * STAGE8;
    const i32x4_t rp = sp.rsrc(ks);
    static_for(
        [&](auto I) {
          constexpr int i = decltype(I)::value;
          if constexpr ((i & 1) == 0) sp.issue_one(rp, fill, i >> 1);
          if constexpr (i == 7) ss.issue(ks, fill, lane);
          acc[i >> 2][i & 3] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              fa.p[i >> 2], fa.q[i & 3], acc[i >> 2][i & 3], 0, 0, i >> 2, fa.sp,
              i & 3, fa.sq);
          __builtin_amdgcn_sched_barrier(0);
        },
        std::make_integer_sequence<int, 8>{});
    // slice kt+1 has landed once only slice kt+2 and the P and scale loads of
    // kt+NST-1 remain
    wait_vm<(NST - 3) * LOADS8 + LPO + 1>();
    wait_lgkm0();  // this wave's reads of stage kt+NST-1's previous slice are done
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    const i32x4_t rq = sq.rsrc(ks);
    const char* next = smem + ((kt + 1) & (NST - 1)) * STAGE8;
    static_for(
        [&](auto I) {
          constexpr int i = 8 + decltype(I)::value;
          constexpr int j = decltype(I)::value;
          if constexpr ((j & 1) == 0) sq.issue_one(rq, fill + OPB, j >> 1);
          // 18 reads over 8 MFMAs: three in the first two, two in the rest
          constexpr int r0 = j < 2 ? 3 * j : 6 + 2 * (j - 2);
          constexpr int r1 = j < 2 ? 3 * j + 3 : 6 + 2 * (j - 1);
#pragma unroll
          for (int r = r0; r < r1; ++r) read_op(fb, next, r);
          acc[i >> 2][i & 3] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              fa.p[i >> 2], fa.q[i & 3], acc[i >> 2][i & 3], 0, 0, i >> 2, fa.sp,
              i & 3, fa.sq);
          __builtin_amdgcn_sched_barrier(0);
        },
        std::make_integer_sequence<int, 8>{});
  };
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    slice(kt, f0, f1);
    slice(kt + 1, f1, f0);
  }
  if (kt < nk) slice(kt, f0, f1);  // its reads of the next stage are in bounds and unused
  wait_vm<0>();  // no load may still target LDS: the ring is reused for the store
  __syncthreads();
  if constexpr (MODE != GM_GRAM) add_term<MODE>(acc, tr, g);
  const float nf = MODE == GM_PROD ? (FIRST ? c.inv_norm[tr.mat] : 1.f) : norm_factor<MODE>(c, g, tr);
  store_tile_lds<MODE>(acc, tr, g, nf, smem, wave, lane, static_cast<int>(threadIdx.x));
}

}  // namespace

// One block per CU, one tile per block (claim_tile: XCD ranges of equal work).
template <int MODE, bool FIRST>
__global__ __launch_bounds__(kThreads, 1) void k_gemm_f8(LaunchCtx c, GemmArgs g) {
  __shared__ __attribute__((aligned(1024))) char smem[LDS8];
  __shared__ int slot, claimed;
  const int32_t t = claim_tile(g.split, c, &claimed);
  if (t < 0) return;  // the whole block
  gemm_tile_f8<MODE, FIRST>(c, g, t, smem, &slot);
}

namespace {

template <int MODE, bool FIRST>
hipError_t launch_f8(const LaunchCtx& c, const XcdSplit& sp, GemmArgs g) {
  const int32_t ntiles = sp.lo[kXcd];
  if (ntiles <= 0) return hipSuccess;
  g.ntiles = ntiles;
  g.split = sp;
  hipLaunchKernelGGL((k_gemm_f8<MODE, FIRST>), dim3(sp.grid), dim3(kThreads), 0, c.stream, c, g);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gram8(const LaunchCtx& c, const XcdSplit& sp, float out_scale, bool first) {
  const GemmArgs g{0, 0.f, out_scale, 0, FIN_NONE, 0.f, first ? 1 : 0, 0, {}};
  return launch_f8<GM_GRAM, false>(c, sp, g);
}

hipError_t launch_poly8(const LaunchCtx& c, const XcdSplit& sp, float b, float cc) {
  const GemmArgs g{0, b / cc, cc, 0, FIN_NONE, 0.f, 0, 0, {}};
  return launch_f8<GM_POLY, false>(c, sp, g);
}

hipError_t launch_prod8(const LaunchCtx& c, const XcdSplit& sp, int32_t cur, float a, bool first) {
  const GemmArgs g{cur, a, 1.f, 1, FIN_NONE, 0.f, first ? 1 : 0, 0, {}};
  return first ? launch_f8<GM_PROD, true>(c, sp, g) : launch_f8<GM_PROD, false>(c, sp, g);
}

}  // namespace muon

// Pipelined bf16 matrix-core kernel of the Newton-Schulz iteration (gfx950).
//
// Same three products and tile layout as the fp32 path (see gemm_common.hpp);
// what differs is how operands reach the matrix cores:
//
//  * Global -> LDS without registers: buffer_load_dwordx4 ... lds writes each
//    lane's 16 bytes straight into LDS (lane i at base + 16 i).  The LDS layout
//    is therefore chosen by permuting which global chunk each lane fetches.
//  * A ring of 4 LDS stages of 32 K-values (P and Q tiles of 256 x 32 bf16,
//    32 KiB per stage, 128 KiB in all): k-slice j is requested while slice
//    j-3 is consumed, and one barrier per slice suffices.
//  * Workspace matrices are stored in 256 x 32 slabs, so each slice of a
//    K-major operand (rows of X, A or B) is one contiguous 16 KiB slab and each
//    load instruction reads 1 KiB of consecutive bytes.  In LDS the slab keeps
//    its 64-byte rows, their four 16-byte chunks XOR-swizzled by
//    ((row >> 2) ^ (row >> 3)) & 3 so that the fragment reads do not collide.
//  * The MN-major operand of the product (X read along its columns) arrives as
//    8 pieces of 32 rows x 64 bytes (one per slab), chunks swizzled by
//    2 ((row >> 1) & 1); fragments are assembled with ds_read_b64_tr_b16, whose
//    16-lane groups read a 4 x 16 block and hand each lane one column.
//  * Fragments are software-pipelined across the slice boundary: the reads of
//    the next slice's first half overlap the MFMAs of this slice's second half.
#include "gemm_pipeline.hpp"

namespace muon {

// ---------------------------------------------------------------------------
// Per-workgroup timeline of the bf16 matrix-core launches, for scheduling
// analysis.  Compiled in only with -DMUON_TILE_TRACE, a separate build of the
// library (libmuon_mi355x_tiletrace.so); in the default build these functions
// are empty and the kernels are unchanged.  Each launch kind writes its own
// slot (0 Gram, 1 A^2, 2 wide product, 3 square product), so the last launch
// of each kind in a call remains.  Per workgroup (kTraceWords values): its
// start and end on the 100 MHz real-time counter, its tile (or -1) with the
// hardware ids of the CU it ran on (HW_ID: CU and shader engine; XCC_ID: the
// XCD), and, for off-diagonal tiles, the moments its K loop began (first
// slice in LDS, after the barrier) and ended (last MFMA issued and every load
// landed, after the barrier): prologue, K loop and epilogue of each tile; and
// the starts of its slices 8 and nk - 8, which split the K loop into its
// first 8 slices, the middle and the last 8.
[[maybe_unused]] constexpr int kTraceSlots = 4;
[[maybe_unused]] constexpr int kTraceBlocks = 65536;
[[maybe_unused]] constexpr int kTraceWords = 7;  // start, end, ids, K loop start and end, slices 8 and nk-8
#ifdef MUON_TILE_TRACE
__device__ unsigned long long g_tile_trace[kTraceSlots * kTraceBlocks * kTraceWords];
#endif

__device__ __forceinline__ void trace_start(int slot) {
#ifdef MUON_TILE_TRACE
  if (threadIdx.x == 0 && blockIdx.x < kTraceBlocks)
    g_tile_trace[(slot * kTraceBlocks + blockIdx.x) * kTraceWords] = __builtin_amdgcn_s_memrealtime();
#else
  (void)slot;
#endif
}

// word 3: the K loop begins, 4: it has ended, 5 and 6: slices 8 and nk - 8
// begin (single-tile kernels only)
__device__ __forceinline__ void trace_phase(int slot, int word) {
#ifdef MUON_TILE_TRACE
  if (threadIdx.x == 0 && blockIdx.x < kTraceBlocks)
    g_tile_trace[(slot * kTraceBlocks + blockIdx.x) * kTraceWords + word] =
        __builtin_amdgcn_s_memrealtime();
#else
  (void)slot;
  (void)word;
#endif
}

__device__ __forceinline__ void trace_end(int slot, int32_t tile) {
#ifdef MUON_TILE_TRACE
  if (threadIdx.x == 0 && blockIdx.x < kTraceBlocks) {
    unsigned long long* r = g_tile_trace + (slot * kTraceBlocks + blockIdx.x) * kTraceWords;
    r[1] = __builtin_amdgcn_s_memrealtime();
    const uint32_t hw_id = __builtin_amdgcn_s_getreg((31 << 11) | 4);  // HW_REG_HW_ID, 32 bits
    const uint32_t xcc_id = __builtin_amdgcn_s_getreg((3 << 11) | 20);  // HW_REG_XCC_ID, 4 bits
    r[2] = (static_cast<unsigned long long>(hw_id) << 32) |
           (static_cast<unsigned long long>(xcc_id & 15u) << 24) |
           (static_cast<uint32_t>(tile + 1) & 0xFFFFFFu);
  }
#else
  (void)slot;
  (void)tile;
#endif
}

namespace {

// Piece u of this thread (tid = 64 wave + lane) in the final store: user row
// (within the tile) and first of 8 user columns, and the 8 elements of T it
// carries.  A wide matrix takes rows of T, a tall one columns of T (its rows).
template <bool TALL>
struct FinalPiece {
  static __device__ __forceinline__ int row(int u, int wave, int lane, int tid) {
    return TALL ? 16 * ((32 * wave + u) >> 3) + (lane & 15) : (tid >> 5) + 8 * u;
  }
  static __device__ __forceinline__ int col(int u, int wave, int lane, int tid) {
    return TALL ? 8 * (4 * ((32 * wave + u) & 7) + (lane >> 4)) : 8 * (tid & 31);
  }
  static __device__ __forceinline__ u32x4_t tile(const char* smem, int u, int wave, int lane,
                                                 int tid) {
    if constexpr (TALL) {
      return read_tile_column(smem, 32 * wave + u, lane);
    } else {
      const int q = (tid >> 5) + 8 * u, c = tid & 31;
      return *reinterpret_cast<const u32x4_t*>(smem + q * MNROW + ((c ^ (q & 31)) << 4));
    }
  }
};

// A tile wholly inside the user's matrix, whose rows are whole 16-byte vectors:
// the W pieces are loaded ahead in two halves, so that their latency hides
// behind the staging and behind the first half's stores.
template <bool TALL>
__device__ __forceinline__ void store_final_interior(const f32x16_t (&acc)[4][4], float nf,
                                                     uint16_t* base, int64_t cols, bool upd,
                                                     float step, char* smem, int wave, int lane,
                                                     int tid) {
  using P = FinalPiece<TALL>;
  u32x4_t w[32];
  if (upd) {
#pragma unroll
    for (int u = 0; u < 16; ++u)
      w[u] = ld16(base + P::row(u, wave, lane, tid) * cols + P::col(u, wave, lane, tid));
  }
  stage_tile(acc, nf, smem, wave, lane);
  if (upd) {
#pragma unroll
    for (int u = 16; u < 32; ++u)
      w[u] = ld16(base + P::row(u, wave, lane, tid) * cols + P::col(u, wave, lane, tid));
  }
#pragma unroll
  for (int u = 0; u < 32; ++u) {
    u32x4_t v = P::tile(smem, u, wave, lane, tid);
    if (upd) {
      float x[8], wf[8];
      vec_to_f32<uint16_t>(v, x);
      vec_to_f32<uint16_t>(w[u], wf);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = wf[e] - step * x[e];
      v = f32_to_vec<uint16_t>(x);
    }
    st16(base + P::row(u, wave, lane, tid) * cols + P::col(u, wave, lane, tid), v);
  }
}

// A tile on the matrix's edge: element by element where the 16-byte vector
// does not fit, every piece clipped to the shape.
template <bool TALL>
__device__ __forceinline__ void store_final_edge(const f32x16_t (&acc)[4][4], float nf,
                                                 const MatDesc& d, int64_t ur0, int64_t uc0,
                                                 bool upd, float step, char* smem, int wave,
                                                 int lane, int tid) {
  using P = FinalPiece<TALL>;
  uint16_t* __restrict__ out = static_cast<uint16_t*>(d.dst);
  const int64_t rows = d.rows, cols = d.cols;
  stage_tile(acc, nf, smem, wave, lane);
#pragma unroll 1
  for (int u = 0; u < 32; ++u) {
    const int64_t r = ur0 + P::row(u, wave, lane, tid), c = uc0 + P::col(u, wave, lane, tid);
    const u32x4_t xv = P::tile(smem, u, wave, lane, tid);
    if (r >= rows || c >= cols) continue;
    float x[8];
    vec_to_f32<uint16_t>(xv, x);
    uint16_t* o = out + r * cols + c;
    if (d.vec_ok && c + 8 <= cols) {
      if (upd) {
        float wf[8];
        vec_to_f32<uint16_t>(ld16(o), wf);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = wf[e] - step * x[e];
      }
      st16(o, f32_to_vec<uint16_t>(x));
    } else {
#pragma unroll 1
      for (int e = 0; e < 8 && c + e < cols; ++e)
        o[e] = Elt<uint16_t>::from_f32(upd ? Elt<uint16_t>::to_f32(o[e]) - step * x[e] : x[e]);
    }
  }
}

// The last product of a call: the user's matrix receives W - lr * scale * X'
// (FIN_STEP) or X' (FIN_NS), in its own orientation and clipped to its shape,
// and the iterate is not stored.  T[q][p] = X'[ti*256 + q][tj*256 + p] is
// staged in LDS as for the iterate.
__device__ __forceinline__ void store_final(const f32x16_t (&acc)[4][4], const TileRef& tr,
                                            const GemmArgs& g, float nf, char* smem, int wave,
                                            int lane, int tid) {
  const MatDesc& d = tr.d;
  const bool tall = d.tall != 0;
  const bool upd = g.finish == FIN_STEP;
  const float step = g.lr * d.scale;
  const int64_t ur0 = static_cast<int64_t>(tall ? tr.tj : tr.ti) * kTile;  // user rows of the tile
  const int64_t uc0 = static_cast<int64_t>(tall ? tr.ti : tr.tj) * kTile;  // user columns
  const bool interior = d.vec_ok && ur0 + kTile <= d.rows && uc0 + kTile <= d.cols;
  uint16_t* base = static_cast<uint16_t*>(d.dst) + ur0 * d.cols + uc0;
  if (interior) {
    if (tall)
      store_final_interior<true>(acc, nf, base, d.cols, upd, step, smem, wave, lane, tid);
    else
      store_final_interior<false>(acc, nf, base, d.cols, upd, step, smem, wave, lane, tid);
  } else {
    if (tall)
      store_final_edge<true>(acc, nf, d, ur0, uc0, upd, step, smem, wave, lane, tid);
    else
      store_final_edge<false>(acc, nf, d, ur0, uc0, upd, step, smem, wave, lane, tid);
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// Diagonal tiles of the symmetric products (GRAM and POLY with ti == tj).  P
// and Q are the same 256 rows, so only P is streamed into the ring (4 loads per
// thread and slice, two in each half), and only the 36 blocks of 32 x 32 on or
// above the block diagonal are formed, 9 per wave: wave W takes block rows W
// and 7 - W, blocks (W, W..7) and (7 - W, 7 - W..7), from the fragments of
// blocks W..7 alone (P and Q fragments are the same).  A full tile spends 64
// MFMAs per wave and K step on 16 blocks; this spends 9 on 9.  Every block takes
// the same MFMAs in the same order as in a full tile, the (b/c) A term of POLY
// included, so the blocks on and above the diagonal are bit-identical to a full
// tile's.  The blocks below are stored as the mirrors of those above, so the
// stored A and B are exactly symmetric.
template <int W>
struct DiagWave {
  static constexpr int kFrags = 8 - W;  // fragments of blocks W..7
  static constexpr int kBlocks = 9;
  static constexpr int row(int i) { return i < 8 - W ? W : 7 - W; }
  static constexpr int col(int i) { return i < 8 - W ? W + i : 7 - W + (i - (8 - W)); }
};

template <int MODE, int W>
__device__ __forceinline__ void diag_wave(const LaunchCtx& c, const GemmArgs& g, const TileRef& tr,
                                          char* smem, int lane) {
  using DW = DiagWave<W>;
  constexpr int NF = DW::kFrags;
  const int64_t s_pad = tr.d.s_pad, l_pad = tr.d.l_pad;
  const uint16_t* src = MODE == GM_GRAM ? static_cast<const uint16_t*>(iterate(tr.d, g.cur))
                                        : static_cast<const uint16_t*>(tr.d.gram);
  const int64_t K = MODE == GM_GRAM ? l_pad : s_pad;
  const Stream sp = kmajor_stream(src, tr.ti, K, W, lane);
  const int nk = static_cast<int>(K / BK);
  const int lr = lane & 31, lh = lane >> 5;
  int32_t base[2];
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) base[sub] = lr * KROW + (((2 * sub + lh) ^ kkey(lr)) << 4);

  f32x16_t acc[DW::kBlocks];
#pragma unroll
  for (int i = 0; i < DW::kBlocks; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[i][e] = 0.f;

  // the (b/c) A term (POLY): see gemm_tile
  const __bf16 s_hi = static_cast<__bf16>(g.init_scale);
  const __bf16 s_lo = static_cast<__bf16>(g.init_scale - static_cast<float>(s_hi));
  auto ident = [&](int h, __bf16 v) {
    bf16x8_t r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = lr == 16 * h + 8 * lh + e ? v : static_cast<__bf16>(0.f);
    return r;
  };
  // term MFMAs of block row R (a compile-time row; -1: none), in column order
  auto term_op = [&](const u32x4_t (&f)[NF], int h, auto R) {
    constexpr int r = decltype(R)::value;
    if constexpr (MODE == GM_POLY && r >= 0) {
      const bf16x8_t id[2] = {ident(h, s_hi), ident(h, s_lo)};
      static_for<DW::kBlocks>([&](auto I) {
        constexpr int i = decltype(I)::value;
        if constexpr (DW::row(i) == r) {
#pragma unroll
          for (int part = 0; part < 2; ++part)
            acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                id[part], __builtin_bit_cast(bf16x8_t, f[DW::col(i) - W]), acc[i], 0, 0, 0);
        }
      });
    }
  };
  auto mfma_op = [&](const u32x4_t (&f)[NF], auto I) {
    constexpr int i = decltype(I)::value;
    acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
        __builtin_bit_cast(bf16x8_t, f[DW::row(i) - W]), __builtin_bit_cast(bf16x8_t, f[DW::col(i) - W]),
        acc[i], 0, 0, 0);
  };

  const uint32_t ring = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((LDS_AS char*)smem));
  // prologue: slices 0..NST-2 (clamped as in gemm_tile), wait for slice 0
#pragma unroll
  for (int st = 0; st < NST - 1; ++st) sp.issue(st < nk ? st : nk - 1, ring + st * STAGEB);
  wait_vm<(NST - 2) * LPO>();
  __syncthreads();
  u32x4_t f0[NF], f1[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) f0[f] = lds16(smem + base[0] + (W + f) * 32 * KROW);

  auto slice = [&](int kt, auto R) {
    const char* stage = smem + (kt & (NST - 1)) * STAGEB;
    const int ks = kt + NST - 1 < nk ? kt + NST - 1 : nk - 1;
    const uint32_t fill = ring + ((kt + NST - 1) & (NST - 1)) * STAGEB;
    const i32x4_t rp = sp.rsrc(ks);
    term_op(f0, 0, R);
    __builtin_amdgcn_sched_barrier(0);
    static_for<DW::kBlocks>([&](auto I) {
      constexpr int i = decltype(I)::value;
      if constexpr (i == 0 || i == 4) sp.issue_one(rp, fill, i / 4);
      if constexpr (i < NF) f1[i] = lds16(stage + base[1] + (W + i) * 32 * KROW);
      mfma_op(f0, I);
      __builtin_amdgcn_sched_barrier(0);
    });
    // slice kt+1 has landed once only slice kt+2 and half of kt+NST-1 remain
    wait_vm<(NST - 3) * LPO + LPO / 2>();
    wait_lgkm0();
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    const char* next = smem + ((kt + 1) & (NST - 1)) * STAGEB;
    term_op(f1, 1, R);
    __builtin_amdgcn_sched_barrier(0);
    static_for<DW::kBlocks>([&](auto I) {
      constexpr int i = decltype(I)::value;
      if constexpr (i == 0 || i == 4) sp.issue_one(rp, fill, 2 + i / 4);
      if constexpr (i < NF) f0[i] = lds16(next + base[0] + (W + i) * 32 * KROW);
      mfma_op(f1, I);
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  using NoTerm = std::integral_constant<int, -1>;
  if constexpr (MODE == GM_GRAM) {
    for (int kt = 0; kt < nk; ++kt) slice(kt, NoTerm{});
  } else {
    // the term slices of block rows W and 7 - W (both < nk)
    const int r0 = 8 * tr.ti + W, r1 = 8 * tr.ti + 7 - W;
    for (int kt = 0; kt < r0; ++kt) slice(kt, NoTerm{});
    slice(r0, std::integral_constant<int, W>{});
    for (int kt = r0 + 1; kt < r1; ++kt) slice(kt, NoTerm{});
    slice(r1, std::integral_constant<int, 7 - W>{});
    for (int kt = r1 + 1; kt < nk; ++kt) slice(kt, NoTerm{});
  }
  wait_vm<0>();  // no load may still target LDS: the ring is reused for the store
  __syncthreads();

  // T[q][p] = S[ti*256 + p][ti*256 + q] for the formed blocks (p's block <= q's),
  // staged as in stage_tile
  const float scale = g.out_scale * norm_factor<MODE>(c, g, tr);
  static_for<DW::kBlocks>([&](auto I) {
    constexpr int i = decltype(I)::value;
    const int q = 32 * DW::col(i) + lr;
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) {
      const int ch = 4 * DW::row(i) + gg;
      u32x2_t w;
      w[0] = Elt<uint16_t>::pack2(scale * acc[i][4 * gg + 0], scale * acc[i][4 * gg + 1]);
      w[1] = Elt<uint16_t>::pack2(scale * acc[i][4 * gg + 2], scale * acc[i][4 * gg + 3]);
      *reinterpret_cast<u32x2_t*>(smem + q * MNROW + ((ch ^ (q & 31)) << 4) + 8 * lh) = w;
    }
  });
}

// The store of a diagonal tile: rows of T where p's block <= q's block go to
// S[ti*256 + q][ti*256 + p] (on and below the diagonal), columns of T where
// p's block < q's block to S[ti*256 + p][ti*256 + q] (above it).
template <int MODE>
__device__ __forceinline__ void diag_store(const TileRef& tr, char* smem, int wave, int lane,
                                           int tid) {
  uint16_t* dst = static_cast<uint16_t*>(MODE == GM_GRAM ? tr.d.gram : tr.d.poly);
  const int64_t ld = tr.d.s_pad, o = static_cast<int64_t>(tr.ti) * kTile;
  uint16_t* const org = dst + slab_off(o, o, ld);  // the tile's origin (uniform)
  const int t = tid, ch = t & 31;
#pragma unroll 8
  for (int u = 0; u < 32; ++u) {
    const int q = (t >> 5) + 8 * u;
    if ((ch >> 2) <= (q >> 5)) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(smem + q * MNROW + ((ch ^ (q & 31)) << 4));
      st16_nt(org + slab_local(q, 8 * ch), v);  // as in store_tile_lds
    }
  }
  const int grp = lane >> 4, j = lane & 15;
#pragma unroll 1
  for (int ub = 0; ub < 4; ++ub) {  // I & 7 = m constant, as in store_tile_lds
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int I = 32 * wave + 8 * ub + m;
      const int pb = I >> 3, cq = 4 * (I & 7) + grp;
      if ((pb >> 1) < (cq >> 2))
        st16_nt(org + slab_local(16 * pb + j, 8 * cq), read_tile_column(smem, I, lane));
    }
  }
}

template <int MODE>
__device__ __forceinline__ void diag_tile(const LaunchCtx& c, const GemmArgs& g, const TileRef& tr,
                                          char* smem, int lane, int tid) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  switch (wave) {
    case 0: diag_wave<MODE, 0>(c, g, tr, smem, lane); break;
    case 1: diag_wave<MODE, 1>(c, g, tr, smem, lane); break;
    case 2: diag_wave<MODE, 2>(c, g, tr, smem, lane); break;
    default: diag_wave<MODE, 3>(c, g, tr, smem, lane); break;
  }
  __syncthreads();
  diag_store<MODE>(tr, smem, wave, lane, tid);
}

// One output tile (tile number t of the launch).  FINAL (products only): the last product
// of a call, storing with store_final.  FIRST (products only): the first product of a
// call, whose iterate is still U, scaled by the norm factor as it is stored.
template <int MODE, bool FINAL, bool FIRST, bool LOOP>
__device__ __forceinline__ void gemm_tile(const LaunchCtx& c, const GemmArgs& g, int32_t t,
                                          char* smem, int* slot) {
  const TileRef tr = decode_tile<MODE>(c, t, slot);
  const MatDesc& d = tr.d;
  const int64_t s_pad = d.s_pad, l_pad = d.l_pad;
  const uint16_t* Xc = static_cast<const uint16_t*>(iterate(d, g.cur));

  // LOOP: the lane index passes through an empty asm, so that the per-lane
  // offsets and identity fragments derived from it are formed anew for every
  // tile instead of being hoisted out of the tile loop and held live through
  // the epilogue (which made the looping kernels spill more).  The epilogues
  // take the thread index as tid, formed from that lane, for the same reason:
  // their per-thread store addresses, from threadIdx.x itself, were hoisted and
  // spilled (67 values stored before the tile loop, 98 reloads per tile).
  int lane = threadIdx.x & 63;
  if constexpr (LOOP) asm volatile("" : "+v"(lane));
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tid = LOOP ? 64 * wave + lane : static_cast<int>(threadIdx.x);
  if constexpr (MODE != GM_PROD) {
    if (tr.ti == tr.tj) {
      diag_tile<MODE>(c, g, tr, smem, lane, tid);
      return;
    }
  }
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, lh = lane >> 5;

  Stream sp, sq;
  int64_t K;
  if constexpr (MODE == GM_GRAM) {
    K = l_pad;
    sp = kmajor_stream(Xc, tr.ti, l_pad, wave, lane);
    sq = kmajor_stream(Xc, tr.tj, l_pad, wave, lane);
  } else if constexpr (MODE == GM_POLY) {
    K = s_pad;
    const uint16_t* A = static_cast<const uint16_t*>(d.gram);
    sp = kmajor_stream(A, tr.ti, s_pad, wave, lane);
    sq = kmajor_stream(A, tr.tj, s_pad, wave, lane);
  } else {
    K = s_pad;
    const uint16_t* Q = static_cast<const uint16_t*>(g.use_poly ? d.poly : d.gram);
    sp = mnmajor_stream<LPO>(Xc, tr.tj, l_pad, wave, lane);
    sq = kmajor_stream(Q, tr.ti, s_pad, wave, lane);
  }
  const int nk = static_cast<int>(K / BK);

  // Per-lane fragment offsets within a stage.
  //  K-major: row (base + 32x + lr), chunk (2 sub + lh) ^ kkey(lr)   [kkey(base + 32x + lr) = kkey(lr)]
  int32_t qoff[2], poff[2];
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    const int sw = ((2 * sub + lh) ^ kkey(lr)) << 4;
    qoff[sub] = OPB + (wn * 128 + lr) * KROW + sw;
    poff[sub] = (wm * 128 + lr) * KROW + sw;
  }
  //  MN-major (product): 16-lane group gq, source row r, column quad qq.  The
  //  lane points at row 8 (gq >> 1) + r (+ 16 sub + 4 h) of slab piece 4 wm + mi,
  //  columns 16 (gq & 1) + 4 qq .. + 3.
  int32_t moff0;
  {
    const int gq = lane >> 4, r = (lane >> 2) & 3, qq = lane & 3;
    const int c = 2 * (gq & 1) + (qq >> 1);
    moff0 = 4 * wm * (32 * KROW) + (8 * (gq >> 1) + r) * KROW + ((c ^ (2 * ((r >> 1) & 1))) << 4) +
            8 * (qq & 1);
  }

  // Fragment reads, numbered in the order the MFMAs below consume them:
  // P[0] first (two transposed halves in the product), then Q[0..3], then P[1..3].
  constexpr int NREAD = MODE == GM_PROD ? 12 : 8;
  auto read_op = [&](Frags& f, const char* stage, int sub, int i) {
    if constexpr (MODE == GM_PROD) {
      if (i < 2) {
        const char* base = stage + moff0 + (16 * sub + 4 * i) * KROW;
        const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4_t*)(base));
        const u32x2_t u = __builtin_bit_cast(u32x2_t, v);
        f.p[0][2 * i] = u[0];
        f.p[0][2 * i + 1] = u[1];
      } else if (i < 6) {
        f.q[i - 2] = lds16(stage + qoff[sub] + (i - 2) * 32 * KROW);
      } else {
        const int mi = 1 + (i - 6) / 2, h = (i - 6) % 2;
        const char* base = stage + moff0 + mi * (32 * KROW) + (16 * sub + 4 * h) * KROW;
        const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4_t*)(base));
        const u32x2_t u = __builtin_bit_cast(u32x2_t, v);
        f.p[mi][2 * h] = u[0];
        f.p[mi][2 * h + 1] = u[1];
      }
    } else {
      if (i == 0) {
        f.p[0] = lds16(stage + poff[sub]);
      } else if (i < 5) {
        f.q[i - 1] = lds16(stage + qoff[sub] + (i - 1) * 32 * KROW);
      } else {
        f.p[i - 4] = lds16(stage + poff[sub] + (i - 4) * 32 * KROW);
      }
    }
  };

  f32x16_t acc[4][4];
  zero_acc(acc);

  // The s-multiple of the source tile (PROD: a X; POLY: (b/c) A) comes from the
  // matrix cores.  In the slice that streams the needed rows, the fragments
  // already in registers times a scaled identity give exactly that term:
  //   PROD  sum_k X[32kt+k][p] * (s d(q,k))  = s X[32kt+q][p]   (identity as the Q operand)
  //   POLY  sum_k (s d(p,k)) * A[tj*256+q][32kt+k] = s A[ti*256+p][tj*256+q]   (as P)
  // s is split into bf16 hi + lo parts, so the term is exact to ~1e-5.  The
  // identity fragment of K-half h: lane l, element e is nonzero iff
  // (l & 31) == 16h + 8(l >> 5) + e.
  const __bf16 s_hi = static_cast<__bf16>(g.init_scale);
  const __bf16 s_lo = static_cast<__bf16>(g.init_scale - static_cast<float>(s_hi));
  auto ident = [&](int h, __bf16 v) {
    bf16x8_t r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = lr == 16 * h + 8 * lh + e ? v : static_cast<__bf16>(0.f);
    return r;
  };
  // Term MFMAs for block R of this wave (R is a compile-time constant; -1: none).
  auto term_op = [&](const Frags& f, int h, auto R) {
    constexpr int r = decltype(R)::value;
    if constexpr (MODE != GM_GRAM && r >= 0) {
      const bf16x8_t id[2] = {ident(h, s_hi), ident(h, s_lo)};
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int part = 0; part < 2; ++part) {
          if constexpr (MODE == GM_PROD)
            acc[x][r] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8_t, f.p[x]), id[part], acc[x][r], 0, 0, 0);
          else
            acc[r][x] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                id[part], __builtin_bit_cast(bf16x8_t, f.q[x]), acc[r][x], 0, 0, 0);
        }
    }
  };

  auto mfma_op = [&](const Frags& f, int i) {
    const int mi = i >> 2, ni = i & 3;
    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, f.p[mi]),
                                                          __builtin_bit_cast(bf16x8_t, f.q[ni]),
                                                          acc[mi][ni], 0, 0, 0);
  };

  // LDS byte address of the ring (the low 32 bits of an LDS pointer are its offset).
  const uint32_t ring = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((LDS_AS char*)smem));

  // Prologue: request slices 0..NST-2, wait for slice 0.  Slice indices past the
  // end are clamped to the last slice: the extra loads refill a stage nobody
  // reads again and keep the count of loads in flight the same every iteration.
#pragma unroll
  for (int s = 0; s < NST - 1; ++s) {
    const int ks = s < nk ? s : nk - 1;
    sp.issue(ks, ring + s * STAGEB);
    sq.issue(ks, ring + s * STAGEB + OPB);
  }
  wait_vm<(NST - 2) * 2 * LPO>();
  __syncthreads();
  if constexpr (!LOOP) trace_phase(MODE == GM_PROD ? 3 : MODE, 3);

  Frags f0, f1;
#pragma unroll
  for (int i = 0; i < NREAD; ++i) read_op(f0, smem, 0, i);

  // One K-slice.  Each half is 16 steps of {memory op(s), one MFMA}, fenced so
  // that the compiler keeps the interleaving: the MFMA pipe stays fed while the
  // reads for the next half-slice and the loads for a later stage go out behind
  // it.  The last slice runs the same body: its reads of the next stage and its
  // (clamped) loads are in bounds and simply unused.
  // Slice kt: stage kt is read; stage kt+NST-1 (the one slice kt-1 used) is
  // refilled with slice kt+NST-1, its P loads in the first half and its Q loads
  // in the second, so that the address path sees one load every few MFMAs.
  // A term slice issues its term MFMAs first in each half, while only that
  // half's fragments are live (after the half's products, both fragment sets
  // would be, and the wide kernel, which adds its terms in the same order,
  // would spill).
  auto slice = [&](int kt, auto R) {
    if constexpr (!LOOP) {
      if (kt == 8) trace_phase(MODE == GM_PROD ? 3 : MODE, 5);
      if (kt == nk - 8) trace_phase(MODE == GM_PROD ? 3 : MODE, 6);
    }
    const int st = kt & (NST - 1);
    const char* stage = smem + st * STAGEB;
    const int ks = kt + NST - 1 < nk ? kt + NST - 1 : nk - 1;
    const uint32_t fill = ring + ((kt + NST - 1) & (NST - 1)) * STAGEB;
    const i32x4_t rp = sp.rsrc(ks);
    term_op(f0, 0, R);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if ((i & 3) == 0) sp.issue_one(rp, fill, i >> 2);
      if (i < NREAD) read_op(f1, stage, 1, i);
      mfma_op(f0, i);
      __builtin_amdgcn_sched_barrier(0);
    }
    // slice kt+1 has landed once only slice kt+2 and the P half of kt+NST-1 remain
    wait_vm<(NST - 3) * 2 * LPO + LPO>();
    wait_lgkm0();  // this wave's reads of `stage` are done before the next refill
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    const i32x4_t rq = sq.rsrc(ks);
    const char* next = smem + ((kt + 1) & (NST - 1)) * STAGEB;
    term_op(f1, 1, R);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if ((i & 3) == 0) sq.issue_one(rq, fill + OPB, i >> 2);
      if (i < NREAD) read_op(f0, next, 0, i);
      mfma_op(f1, i);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  using NoTerm = std::integral_constant<int, -1>;
  if constexpr (MODE == GM_GRAM) {
    for (int kt = 0; kt < nk; ++kt) slice(kt, NoTerm{});
  } else {
    // slices rel0 .. rel0+3 carry the s-multiple term for blocks 0..3 (rel0 + 3 < nk)
    const int rel0 = __builtin_amdgcn_readfirstlane(8 * tr.ti + 4 * (MODE == GM_PROD ? wn : wm));
    for (int kt = 0; kt < rel0; ++kt) slice(kt, NoTerm{});
    slice(rel0 + 0, std::integral_constant<int, 0>{});
    slice(rel0 + 1, std::integral_constant<int, 1>{});
    slice(rel0 + 2, std::integral_constant<int, 2>{});
    slice(rel0 + 3, std::integral_constant<int, 3>{});
    for (int kt = rel0 + 4; kt < nk; ++kt) slice(kt, NoTerm{});
  }
  wait_vm<0>();  // no load may still target LDS: the ring is reused for the store
  __syncthreads();
  if constexpr (!LOOP) trace_phase(MODE == GM_PROD ? 3 : MODE, 4);
  // the norm factor: a product takes it only in its FIRST instantiation, so
  // every other product stages with an exact 1 (no multiply)
  const float nf = MODE == GM_PROD ? (FIRST ? c.inv_norm[tr.mat] : 1.f) : norm_factor<MODE>(c, g, tr);
  if constexpr (FINAL)
    store_final(acc, tr, g, nf, smem, wave, lane, tid);
  else
    store_tile_lds<MODE>(acc, tr, g, nf, smem, wave, lane, tid);
}

// ---------------------------------------------------------------------------
// Wide product tiles: 256 rows of B (q) x 384 columns of X (p).
//
// Per K slice such a tile streams 40 KiB for 6.3 MFLOP, where a 256 x 256 tile
// streams 32 KiB for 4.2 MFLOP: 17% fewer operand bytes per flop, and the
// per-slice barrier and waits are spread over 1.5x the matrix-core work.  The
// four waves keep a 2 x 2 grid of 192 (p) x 128 (q) blocks, 24 accumulator
// blocks of 32 x 32 and 384 fp32 registers per lane.  The compiler places MFMA
// accumulators in AGPRs only (256 per lane), so p-blocks 0..3 stay ordinary
// MFMAs on AGPRs (acc) and p-blocks 4..5 are inline VGPR-form MFMAs (accv).
// The main loop needs fewer than 100 other VGPRs.
//   Hazards of the inline MFMAs: their A/B operands come from LDS reads, which
//   the compiler guards with lgkmcnt waits like any other use; the MFMAs into
//   one block are at least 6 MFMAs apart; the zeroing of accv and the
//   epilogue's reads of it are separated from the MFMAs by mfma_guard.
// LDS: a 4-stage ring of 40 KiB stages (the X slice, 24 KiB, then the B slice),
// all 160 KiB of the CU.  The tile is stored through LDS in two halves of
// 256 x 192.  Every output element takes the same MFMAs in the same order as
// in the 256 x 256 kernel, so the results are bit-identical.
constexpr int LPW = kTileW * KROW / (kThreads * 16);  // loads per thread and slice, X slice (6)
constexpr int OPBW = kTileW * KROW;                   // 24 KiB: the X slice of a stage
constexpr int STAGEW = OPBW + OPB;                    // 40 KiB
constexpr int LDSW = NST * STAGEW;                    // 160 KiB
constexpr int WROW = kTileW;                          // bytes of a staged half-tile row (192 bf16)
static_assert(LPW == 6 && LDSW == 163840, "wide tile geometry");
static_assert(kTile * WROW <= LDSW, "a staged half tile fits in the ring");

// d += a b on VGPR accumulators.
__device__ __forceinline__ void mfma_v(f32x16_t& d, const u32x4_t& a, const u32x4_t& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}

// Wait states between the inline MFMAs and any other write or read of their
// accumulators (the compiler does not look inside inline assembly).
__device__ __forceinline__ void mfma_guard(f32x16_t (&v)[2][4]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+v"(v[0][0]), "+v"(v[0][1]), "+v"(v[0][2]), "+v"(v[0][3]), "+v"(v[1][0]),
                 "+v"(v[1][1]), "+v"(v[1][2]), "+v"(v[1][3]));
}

// Tile number b of a wide product launch -> (matrix, tile), as decode_tile.
__device__ __forceinline__ TileRef decode_wide(const LaunchCtx& c, int32_t b, int* slot) {
  const int32_t* pre = c.prefix + PH_PRODW * (c.batch + 1);
  const int32_t per = c.per[PH_PRODW];  // as in decode_tile
  const int j = per > 0 ? b / per : __builtin_amdgcn_readfirstlane(locate_matrix(pre, c.batch, b, slot));
  TileRef r;
  r.d = load_const(c.desc + j);
  r.mat = j;
  prod_tile(per > 0 ? b - j * per : b - load_const(pre + j), r.d.s_pad / kTile,
            r.d.l_pad / kTileW, r.ti, r.tj);
  return r;
}

// Stores X'[ti*256 + q][tj*384 + p] = nf * acc (bf16) into the other iterate
// buffer, through LDS in halves h = 0, 1.  Half h holds p-blocks 3h .. 3h+2 of
// every wave: columns tj*384 + 192 wm + 96 h + (0 .. 95), wm = 0, 1.  A staged
// half is 256 rows of 192 values (24 chunks of 16 bytes); chunk c of row q is
// kept at c ^ ((q >> 1) & 7), so that both the staging writes and the reads
// below spread over all banks.  It goes out in units of 16 rows x one
// 32-column slab, 1 KiB of consecutive bytes in the slab layout, one unit per
// wave instruction.
__device__ __forceinline__ void store_wide(const f32x16_t (&acc)[4][4], const f32x16_t (&accv)[2][4],
                                           const TileRef& tr, const GemmArgs& g, float nf,
                                           char* smem, int wave, int lane) {
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, lh = lane >> 5;
  uint16_t* __restrict__ dst = static_cast<uint16_t*>(iterate(tr.d, g.cur ^ 1));
  const int64_t ld = tr.d.l_pad;
  const int64_t r0 = static_cast<int64_t>(tr.ti) * kTile;
  const int64_t cw = static_cast<int64_t>(tr.tj) * kTileW;
  uint16_t* const org = dst + slab_off(r0, cw, ld);  // the tile's origin (uniform)
  // p-block 3h + ml of this wave (its four q-blocks) into the staged half
  auto stage_mi = [&](const f32x16_t (&a)[4], int ml) {
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        const int q = wn * 128 + ni * 32 + lr;
        const int c = 12 * wm + 4 * ml + gg;
        u32x2_t w;
        w[0] = Elt<uint16_t>::pack2(nf * a[ni][4 * gg + 0], nf * a[ni][4 * gg + 1]);
        w[1] = Elt<uint16_t>::pack2(nf * a[ni][4 * gg + 2], nf * a[ni][4 * gg + 3]);
        *reinterpret_cast<u32x2_t*>(smem + q * WROW + ((c ^ ((q >> 1) & 7)) << 4) + 8 * lh) = w;
      }
  };
  auto store_half = [&](int h) {
#pragma unroll 1
    for (int k = 0; k < 4; ++k) {
      // units 24 wave + 6 k + gs: slab gs of the half, rows 16 (4 wave + k) ..; the
      // six LDS reads go out before the six stores, so that their latencies overlap
      const int q = 16 * (4 * wave + k) + (lane & 15);
      u32x4_t val[6];
#pragma unroll
      for (int gs = 0; gs < 6; ++gs) {
        const int c = 4 * gs + (lane >> 4);
        val[gs] = *reinterpret_cast<const u32x4_t*>(smem + q * WROW + ((c ^ ((q >> 1) & 7)) << 4));
      }
#pragma unroll
      for (int gs = 0; gs < 6; ++gs) {
        const int col = 192 * (gs / 3) + 96 * h + 32 * (gs % 3) + 8 * (lane >> 4);  // in the tile
        st16(org + slab_local(q, col), val[gs]);
      }
    }
  };
  stage_mi(acc[0], 0);
  stage_mi(acc[1], 1);
  stage_mi(acc[2], 2);
  __syncthreads();
  store_half(0);
  __syncthreads();  // every wave has read half 0 before half 1 overwrites it
  stage_mi(acc[3], 0);
  stage_mi(accv[0], 1);
  stage_mi(accv[1], 2);
  __syncthreads();
  store_half(1);
}

// One wide product tile (tile number t of the launch): X' = a X + Q X into the
// other iterate buffer, scaled by the norm factor in the FIRST product.  The
// pipeline is gemm_tile's (ring, waits, fragment order, fused a X term) with
// six p-blocks per wave instead of four.
template <bool FIRST>
__device__ __forceinline__ void gemm_tile_wide(const LaunchCtx& c, const GemmArgs& g, int32_t t,
                                               char* smem, int* slot) {
  const TileRef tr = decode_wide(c, t, slot);
  const MatDesc& d = tr.d;
  const int64_t s_pad = d.s_pad, l_pad = d.l_pad;
  const uint16_t* Xc = static_cast<const uint16_t*>(iterate(d, g.cur));
  const uint16_t* Q = static_cast<const uint16_t*>(g.use_poly ? d.poly : d.gram);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, lh = lane >> 5;

  const StreamT<LPW> sp = mnmajor_stream<LPW>(Xc, tr.tj, l_pad, wave, lane);
  const Stream sq = kmajor_stream(Q, tr.ti, s_pad, wave, lane);
  const int nk = static_cast<int>(s_pad / BK);

  // Fragment offsets within a stage, as in gemm_tile; the X slice comes first.
  int32_t qoff[2];
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    const int sw = ((2 * sub + lh) ^ kkey(lr)) << 4;
    qoff[sub] = OPBW + (wn * 128 + lr) * KROW + sw;
  }
  int32_t moff0;
  {
    const int gq = lane >> 4, r = (lane >> 2) & 3, qq = lane & 3;
    const int cc = 2 * (gq & 1) + (qq >> 1);
    moff0 = 6 * wm * (32 * KROW) + (8 * (gq >> 1) + r) * KROW +
            ((cc ^ (2 * ((r >> 1) & 1))) << 4) + 8 * (qq & 1);
  }

  struct FragsW {
    u32x4_t p[6];
    u32x4_t q[4];
  };
  // Reads in the order the MFMAs consume them: P[0] (two transposed halves),
  // Q[0..3], then P[1..5].
  constexpr int NREADW = 16;
  auto read_op = [&](FragsW& f, const char* stage, int sub, int i) {
    if (i >= 2 && i < 6) {
      f.q[i - 2] = lds16(stage + qoff[sub] + (i - 2) * 32 * KROW);
    } else {
      const int mi = i < 2 ? 0 : 1 + (i - 6) / 2, h = i < 2 ? i : (i - 6) % 2;
      const char* base = stage + moff0 + mi * (32 * KROW) + (16 * sub + 4 * h) * KROW;
      const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4_t*)(base));
      const u32x2_t u = __builtin_bit_cast(u32x2_t, v);
      f.p[mi][2 * h] = u[0];
      f.p[mi][2 * h + 1] = u[1];
    }
  };

  f32x16_t acc[4][4];
  zero_acc(acc);
  f32x16_t accv[2][4];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int e = 0; e < 16; ++e) accv[mi][ni][e] = 0.f;
  mfma_guard(accv);

  auto mma = [&](int mi, int ni, const u32x4_t& a, const u32x4_t& b) {
    if (mi < 4)
      acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          __builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), acc[mi][ni], 0, 0, 0);
    else
      mfma_v(accv[mi - 4][ni], a, b);
  };
  auto mfma_op = [&](const FragsW& f, int i) { mma(i >> 2, i & 3, f.p[i >> 2], f.q[i & 3]); };

  // The a X term, as in gemm_tile: the X fragments times a scaled identity, in
  // hi and lo bf16 parts (all hi parts first, so that no two MFMAs into one
  // block follow each other).
  const __bf16 s_hi = static_cast<__bf16>(g.init_scale);
  const __bf16 s_lo = static_cast<__bf16>(g.init_scale - static_cast<float>(s_hi));
  auto ident = [&](int h, __bf16 v) {
    bf16x8_t r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = lr == 16 * h + 8 * lh + e ? v : static_cast<__bf16>(0.f);
    return r;
  };
  // The identity fragments are built by VALU instructions: the guard puts wait
  // states between them and the inline MFMAs that read them, and the fences
  // keep the twelve MFMAs in this order.
  auto term_op = [&](const FragsW& f, int h, auto R) {
    constexpr int r = decltype(R)::value;
    if constexpr (r >= 0) {
      u32x4_t id[2] = {__builtin_bit_cast(u32x4_t, ident(h, s_hi)),
                       __builtin_bit_cast(u32x4_t, ident(h, s_lo))};
      asm volatile("s_nop 4" : "+v"(id[0]), "+v"(id[1]));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int part = 0; part < 2; ++part)
#pragma unroll
        for (int x = 0; x < 6; ++x) {
          mma(x, r, f.p[x], id[part]);
          __builtin_amdgcn_sched_barrier(0);
        }
    }
  };

  const uint32_t ring = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((LDS_AS char*)smem));

  // Prologue: slices 0..NST-2 requested, slice 0 awaited (past the end: clamped).
#pragma unroll
  for (int s = 0; s < NST - 1; ++s) {
    const int ks = s < nk ? s : nk - 1;
    sp.issue(ks, ring + s * STAGEW);
    sq.issue(ks, ring + s * STAGEW + OPBW);
  }
  wait_vm<(NST - 2) * (LPW + LPO)>();
  __syncthreads();
  trace_phase(2, 3);

  FragsW f0, f1;
#pragma unroll
  for (int i = 0; i < NREADW; ++i) read_op(f0, smem, 0, i);

  // One K slice: 24 steps of {memory op(s), one MFMA} per half; the X-slice
  // loads of stage kt+NST-1 go out in the first half (one every 4 MFMAs), the
  // B-slice loads in the second (one every 6).  Term MFMAs come first in their
  // half, as in gemm_tile: issued after the products they spilled 8 dwords,
  // and every spill reload then waited for vmcnt(0), since the compiler cannot
  // count the loads in the inline assembly, draining the operand prefetch.
  auto slice = [&](int kt, auto R) {
    if (kt == 8) trace_phase(2, 5);
    if (kt == nk - 8) trace_phase(2, 6);
    const char* stage = smem + (kt & (NST - 1)) * STAGEW;
    const int ks = kt + NST - 1 < nk ? kt + NST - 1 : nk - 1;
    const uint32_t fill = ring + ((kt + NST - 1) & (NST - 1)) * STAGEW;
    const i32x4_t rp = sp.rsrc(ks);
    term_op(f0, 0, R);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 24; ++i) {
      if ((i & 3) == 0) sp.issue_one(rp, fill, i >> 2);
      if (i < NREADW) read_op(f1, stage, 1, i);
      mfma_op(f0, i);
      __builtin_amdgcn_sched_barrier(0);
    }
    // slice kt+1 has landed once only slice kt+2 and the X half of kt+NST-1 remain
    wait_vm<(NST - 3) * (LPW + LPO) + LPW>();
    wait_lgkm0();
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    const i32x4_t rq = sq.rsrc(ks);
    const char* next = smem + ((kt + 1) & (NST - 1)) * STAGEW;
    term_op(f1, 1, R);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 24; ++i) {
      if (i % 6 == 0) sq.issue_one(rq, fill + OPBW, i / 6);
      if (i < NREADW) read_op(f0, next, 0, i);
      mfma_op(f1, i);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  using NoTerm = std::integral_constant<int, -1>;
  const int rel0 = __builtin_amdgcn_readfirstlane(8 * tr.ti + 4 * wn);
  for (int kt = 0; kt < rel0; ++kt) slice(kt, NoTerm{});
  slice(rel0 + 0, std::integral_constant<int, 0>{});
  slice(rel0 + 1, std::integral_constant<int, 1>{});
  slice(rel0 + 2, std::integral_constant<int, 2>{});
  slice(rel0 + 3, std::integral_constant<int, 3>{});
  for (int kt = rel0 + 4; kt < nk; ++kt) slice(kt, NoTerm{});
  wait_vm<0>();
  __syncthreads();
  trace_phase(2, 4);
  mfma_guard(accv);
  const float nf = FIRST ? c.inv_norm[tr.mat] : 1.f;
  store_wide(acc, accv, tr, g, nf, smem, wave, lane);
}

// One block per CU, one tile per block, taken by claim_tile: the XCDs get
// ranges of equal work, the last tiles of each claimed at run time.  LOOP (a CU budget: fewer workgroups than tiles): a
// block takes tiles blockIdx.x, blockIdx.x + gridDim.x, ..., renumbered so that
// each XCD walks one contiguous range of equal length.  The loop is a separate
// instantiation: across tiles the compiler keeps tile-invariant values in
// registers, which the single-tile kernel cannot spare.
template <int MODE, bool FINAL, bool LOOP, bool FIRST>
__global__ __launch_bounds__(kThreads, 1) void k_gemm_bf16(LaunchCtx c, GemmArgs g) {
  __shared__ __attribute__((aligned(1024))) char smem[LDSB];
  __shared__ int slot;
  if constexpr (LOOP) {
    zero_next_sched(c);
    for (int32_t v = blockIdx.x; v < g.ntiles; v += gridDim.x) {
      gemm_tile<MODE, FINAL, FIRST, true>(c, g, xcd_remap(v, g.ntiles), smem, &slot);
      __syncthreads();  // every wave is done with LDS before the next tile's loads land there
    }
  } else {
    constexpr int kSlot = MODE == GM_PROD ? 3 : MODE;
    trace_start(kSlot);
    __shared__ int claimed;
    const int32_t t = claim_tile(g.split, c, &claimed);
    if (t >= 0) gemm_tile<MODE, FINAL, FIRST, false>(c, g, t, smem, &slot);
    trace_end(kSlot, t);
  }
}

template <int MODE, bool FINAL, bool FIRST>
void launch_one(const LaunchCtx& c, int32_t nblocks, bool loop, const GemmArgs& g) {
  if (loop)
    hipLaunchKernelGGL((k_gemm_bf16<MODE, FINAL, true, FIRST>), dim3(nblocks), dim3(kThreads), 0,
                       c.stream, c, g);
  else
    hipLaunchKernelGGL((k_gemm_bf16<MODE, FINAL, false, FIRST>), dim3(nblocks), dim3(kThreads), 0,
                       c.stream, c, g);
}

// Wide product tiles, one per workgroup (claim_tile).  The LDS slots of the
// claim and of the matrix lookup sit in the last ring stage, which the
// prologue leaves unfilled: every wave has read both before the first slice
// refills that stage.
template <bool FIRST>
__global__ __launch_bounds__(kThreads, 1) void k_gemm_bf16_wide(LaunchCtx c, GemmArgs g) {
  __shared__ __attribute__((aligned(1024))) char smem[LDSW];
  trace_start(2);
  int* slots = reinterpret_cast<int*>(smem + (NST - 1) * STAGEW);  // the lookup's, the claim's
  const int32_t t = claim_tile(g.split, c, slots + 1);
  if (t >= 0) gemm_tile_wide<FIRST>(c, g, t, smem, slots);  // the whole block
  trace_end(2, t);
}

template <bool FINAL>
void launch_prod_bf16(const LaunchCtx& c, int32_t nblocks, bool loop, const GemmArgs& g) {
  if (g.first)
    launch_one<GM_PROD, FINAL, true>(c, nblocks, loop, g);
  else
    launch_one<GM_PROD, FINAL, false>(c, nblocks, loop, g);
}

// g.split.grid workgroups of one tile each or, with loop, nblocks workgroups
// (fewer than g.ntiles) looping over the tiles.
hipError_t launch_gemm_bf16(int mode, const LaunchCtx& c, int32_t nblocks, bool loop,
                            const GemmArgs& g) {
  if (nblocks <= 0) return hipSuccess;
  switch (mode) {
    case GM_GRAM: launch_one<GM_GRAM, false, false>(c, nblocks, loop, g); break;
    case GM_POLY: launch_one<GM_POLY, false, false>(c, nblocks, loop, g); break;
    default:
      if (g.finish != FIN_NONE)
        launch_prod_bf16<true>(c, nblocks, loop, g);
      else
        launch_prod_bf16<false>(c, nblocks, loop, g);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_prod_wide(const LaunchCtx& c, const XcdSplit& sp, int32_t cur, float a,
                            bool use_poly, bool first) {
  const int32_t ntiles = sp.lo[kXcd];
  if (ntiles <= 0) return hipSuccess;
  const GemmArgs g{cur, a, 1.f, use_poly ? 1 : 0, FIN_NONE, 0.f, first ? 1 : 0, ntiles, sp};
  if (first)
    hipLaunchKernelGGL((k_gemm_bf16_wide<true>), dim3(sp.grid), dim3(kThreads), 0, c.stream, c, g);
  else
    hipLaunchKernelGGL((k_gemm_bf16_wide<false>), dim3(sp.grid), dim3(kThreads), 0, c.stream, c, g);
  return hipGetLastError();
}

}  // namespace muon

#ifdef MUON_TILE_TRACE
// Copies the timeline (kTraceSlots x kTraceBlocks x kTraceWords uint64) of the current
// device to host memory; bytes at most its size.  Exported by the timeline
// build only.  Returns a hipError_t code.
extern "C" int32_t muon_tile_trace_read(void* host, size_t bytes) {
  return static_cast<int32_t>(
      hipMemcpyFromSymbol(host, HIP_SYMBOL(muon::g_tile_trace), bytes, 0, hipMemcpyDeviceToHost));
}

// Zeroes the timeline of the current device (synchronously).
extern "C" int32_t muon_tile_trace_clear() {
  void* p = nullptr;
  hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(muon::g_tile_trace));
  if (e == hipSuccess) e = hipMemset(p, 0, sizeof(muon::g_tile_trace));
  if (e == hipSuccess) e = hipDeviceSynchronize();
  return static_cast<int32_t>(e);
}
#endif

// The operand pipeline shared by the matrix-core kernels (gemm_bf16.hip,
// gemm_f8.hip): the LDS ring of 256 x 64-byte K-major rows filled by
// direct-to-LDS loads with hand-counted waits, the swizzled fragment offsets,
// and the LDS-staged store of a finished 256 x 256 tile.  A bf16 stage holds
// 32 K values per row, an e4m3 stage 64 (the same 64 bytes).
#pragma once

#include "gemm_common.hpp"

namespace muon {

namespace {

constexpr int BK = 32;                      // K values per stage
constexpr int KROW = BK * 2;                // bytes of one K-major LDS row
constexpr int OPB = kTile * KROW;           // 16 KiB per operand per stage
constexpr int STAGEB = 2 * OPB;             // P then Q
constexpr int NST = 4;                      // stages in the ring
constexpr int LDSB = NST * STAGEB;          // 128 KiB
constexpr int LPO = OPB / (kThreads * 16);  // 16-byte loads per thread, operand and stage (4)
constexpr int MNROW = kTile * 2;            // bytes of one MN-major LDS row (256 columns)
static_assert(LDSB >= kTile * MNROW, "the tile store stages a whole 256 x 256 bf16 tile in the ring");


// Chunk key of a K-major LDS row.  It depends on row bits 2 and 3 only: with a
// key that varies with bit 1, gfx950 serves the fragment reads (ds_read_b128,
// lane l -> row l % 32) at half rate (measured with SQ_LDS_BANK_CONFLICT).
// Rows 32 x + r share the key of r, which the fragment offsets rely on.
__device__ __forceinline__ int kkey(int row) { return ((row >> 2) ^ (row >> 3)) & 3; }

// s_waitcnt on vmcnt only (gfx9 encoding: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[15:14]).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
}

typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));

// One 16-byte-per-lane load straight into LDS: lane i's data lands at
// lds_addr + 16 i.  Written as inline assembly so that the compiler does not
// guard every later LDS read with a full vmcnt wait; the kernel waits on vmcnt
// itself, counting the loads it has in flight.
__device__ __forceinline__ void lds_dma16(uint32_t lds_addr, int32_t voff, i32x4_t rsrc) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}

// One operand's stream of 256 x 32 (or, for the wide product's X, 32 x 384)
// tiles into the LDS ring, N 16-byte loads per thread and slice.  In the slab
// layout (slab_off in device_common.hpp) a K-major tile is one contiguous
// 16 KiB slab; the product's MN-major tile (32 rows of X x 64 N columns) is 2 N
// contiguous 2 KiB pieces, one per slab.
template <int N>
struct StreamT {
  const char* base;      // byte address at k-slice 0 (uniform)
  int64_t band_stride;   // MN-major: bytes between bands of 256 rows
  int32_t mn;            // 1: MN-major, 0: K-major
  int32_t voff[N];       // per-lane byte offsets, one per load instruction
  int32_t lds;           // LDS byte offset of this wave's first 1 KiB block, within the operand

  // Buffer resource for k-slice ks: base, stride 0, num_records (bytes), raw dword access.
  __device__ __forceinline__ i32x4_t rsrc(int ks) const {
    const uint64_t b = reinterpret_cast<uint64_t>(base) +
                       (mn ? static_cast<uint64_t>(ks >> 3) * band_stride +
                                 static_cast<uint64_t>(ks & 7) * (32 * KROW)
                           : static_cast<uint64_t>(ks) * OPB);
    i32x4_t r;
    r[0] = __builtin_amdgcn_readfirstlane(static_cast<int32_t>(b & 0xffffffffu));
    r[1] = __builtin_amdgcn_readfirstlane(static_cast<int32_t>((b >> 32) & 0xffffu));
    r[2] = mn ? (2 * N - 1) * OPB + 32 * KROW : OPB;  // exactly the bytes this slice reads
    r[3] = 0x00020000;
    return r;
  }
  __device__ __forceinline__ void issue_one(const i32x4_t& r, uint32_t stage_op_lds, int u) const {
    lds_dma16(__builtin_amdgcn_readfirstlane(stage_op_lds + lds + u * 1024), voff[u], r);
  }
  __device__ __forceinline__ void issue(int ks, uint32_t stage_op_lds) const {
    const i32x4_t r = rsrc(ks);
#pragma unroll
    for (int u = 0; u < N; ++u)
      lds_dma16(__builtin_amdgcn_readfirstlane(stage_op_lds + lds + u * 1024), voff[u], r);
  }
};
using Stream = StreamT<LPO>;

// Rows [256 band, 256 band + 256) of a slab-layout matrix with `ncols` columns.
// LDS: 256 rows of 64 bytes, chunk c of row r kept at c ^ kkey(r).
__device__ __forceinline__ Stream kmajor_stream(const uint16_t* m, int64_t band, int64_t ncols,
                                                int wave, int lane) {
  Stream s;
  s.base = reinterpret_cast<const char*>(m + band * (ncols / kSlabCols) * (kSlabRows * kSlabCols));
  s.band_stride = 0;
  s.mn = 0;
#pragma unroll
  for (int u = 0; u < LPO; ++u) {
    const int row = 16 * (LPO * wave + u) + (lane >> 2);
    const int c = (lane & 3) ^ kkey(row);
    s.voff[u] = row * KROW + c * 16;
  }
  s.lds = LPO * wave * 1024;
  return s;
}

// Columns [W tj, W tj + W) of a slab-layout matrix, W = 64 N (all its rows, 32
// per k-slice).  LDS: 2 N pieces (one per slab) of 32 rows x 64 bytes, chunk c
// of row r kept at c ^ (2 ((r >> 1) & 1)).
template <int N>
__device__ __forceinline__ StreamT<N> mnmajor_stream(const uint16_t* m, int64_t tj, int64_t ncols,
                                                     int wave, int lane) {
  StreamT<N> s;
  const int64_t slabs_per_band = ncols / kSlabCols;
  s.base = reinterpret_cast<const char*>(m + 2 * N * tj * (kSlabRows * kSlabCols));
  s.band_stride = slabs_per_band * OPB;
  s.mn = 1;
#pragma unroll
  for (int u = 0; u < N; ++u) {
    const int blk = N * wave + u;  // 1 KiB block: slab piece blk / 2, rows 16 (blk % 2) ..
    const int row = 16 * (blk & 1) + (lane >> 2);
    const int c = (lane & 3) ^ (2 * ((row >> 1) & 1));
    s.voff[u] = (blk >> 1) * OPB + row * KROW + c * 16;
  }
  s.lds = N * wave * 1024;
  return s;
}

struct Frags {
  u32x4_t p[4];
  u32x4_t q[4];
};

// body(integral_constant<int, i>) for each i of the sequence, or of 0 .. N-1:
// compile-time indices for register arrays and instruction operands.
template <typename F, int... Is>
__device__ __forceinline__ void static_for(F&& body, std::integer_sequence<int, Is...>) {
  (body(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& body) {
  static_for(static_cast<F&&>(body), std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ u32x4_t lds16(const char* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

__device__ __forceinline__ u32x4_t lds_tr(const char* p0, const char* p1) {
  const s16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4_t*)(p0));
  const s16x4_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4_t*)(p1));
  const u32x2_t ua = __builtin_bit_cast(u32x2_t, a), ub = __builtin_bit_cast(u32x2_t, b);
  u32x4_t r;
  r[0] = ua[0];
  r[1] = ua[1];
  r[2] = ub[0];
  r[3] = ub[1];
  return r;
}

// Stores the finished tile through LDS (the ring is idle once the K loop is
// done), so that global writes are whole 16-byte pieces of rows.
//   Tile T (256 x 256 bf16, 128 KiB) is laid out as rows of 512 bytes, row
//   index = the accumulator's q, 16-byte chunk c stored at c ^ (q & 31).
//   PROD       T[q][p] = X'[ti*256 + q][tj*256 + p]: rows go out as they are.
//   GRAM/POLY  T[q][p] = S[tj*256 + q][ti*256 + p] (the mirror); rows go out to
//              the mirror position, and for ti != tj the columns of T, read with
//              ds_read_b64_tr_b16, go out as rows of S[ti*256 + p][tj*256 + q].
// Accumulator tile -> T in LDS (bf16, scaled), then a barrier.
__device__ __forceinline__ void stage_tile(const f32x16_t (&acc)[4][4], float scale, char* smem,
                                           int wave, int lane) {
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, lh = lane >> 5;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        const int q = wn * 128 + ni * 32 + lr;
        const int c = 16 * wm + 4 * mi + gg;  // chunk of p0 = wm*128 + mi*32 + 8gg (+4lh)
        u32x2_t w;
        w[0] = Elt<uint16_t>::pack2(scale * acc[mi][ni][4 * gg + 0], scale * acc[mi][ni][4 * gg + 1]);
        w[1] = Elt<uint16_t>::pack2(scale * acc[mi][ni][4 * gg + 2], scale * acc[mi][ni][4 * gg + 3]);
        *reinterpret_cast<u32x2_t*>(smem + q * MNROW + ((c ^ (q & 31)) << 4) + 8 * lh) = w;
      }
  __syncthreads();
}

// Eight consecutive q of column p of T (two transposed reads), for the lanes
// of wave-instruction I: p = 16 (I >> 3) + (lane & 15), q = 8 (4 (I & 7) + lane / 16) + 0..7.
__device__ __forceinline__ u32x4_t read_tile_column(const char* smem, int I, int lane) {
  const int pb = I >> 3, cq = 4 * (I & 7) + (lane >> 4);
  const int r = (lane >> 2) & 3, qq = lane & 3;
  u32x4_t v;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int row = 8 * cq + 4 * h + r;
    const int chunk = 2 * pb + (qq >> 1);
    const char* a = smem + row * MNROW + ((chunk ^ (row & 31)) << 4) + 8 * (qq & 1);
    const s16x4_t x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4_t*)(a));
    const u32x2_t xu = __builtin_bit_cast(u32x2_t, x);
    v[2 * h] = xu[0];
    v[2 * h + 1] = xu[1];
  }
  return v;
}

template <int MODE>
__device__ __forceinline__ void store_tile_lds(const f32x16_t (&acc)[4][4], const TileRef& tr,
                                               const GemmArgs& g, float nf, char* smem, int wave,
                                               int lane, int tid) {
  stage_tile(acc, MODE == GM_PROD ? nf : g.out_scale * nf, smem, wave, lane);
  const int t = tid;  // threadIdx.x
  // Rows of T: thread t moves chunk (t & 31) of rows (t >> 5) + 8u.
  {
    uint16_t* dst;
    int64_t ld, r0, c0;
    if constexpr (MODE == GM_PROD) {
      dst = static_cast<uint16_t*>(iterate(tr.d, g.cur ^ 1));
      ld = tr.d.l_pad;
      r0 = static_cast<int64_t>(tr.ti) * kTile;
      c0 = static_cast<int64_t>(tr.tj) * kTile;
    } else {
      dst = static_cast<uint16_t*>(MODE == GM_GRAM ? tr.d.gram : tr.d.poly);
      ld = tr.d.s_pad;
      r0 = static_cast<int64_t>(tr.tj) * kTile;
      c0 = static_cast<int64_t>(tr.ti) * kTile;
    }
    uint16_t* const org = dst + slab_off(r0, c0, ld);  // the tile's origin (uniform)
    const int c = t & 31;
#pragma unroll 8
    for (int u = 0; u < 32; ++u) {
      const int q = (t >> 5) + 8 * u;
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(smem + q * MNROW + ((c ^ (q & 31)) << 4));
      // A and B go out with the nontemporal hint (measured: Gram and A^2
      // launches and the call 0.4% faster); the iterate without it (+0.8%)
      if constexpr (MODE == GM_PROD)
        st16(org + slab_local(q, 8 * c), v);
      else
        st16_nt(org + slab_local(q, 8 * c), v);
    }
  }
  if constexpr (MODE != GM_PROD) {
    if (tr.ti != tr.tj) {
      // Columns of T.  Wave instruction I = 32 wave + u covers p-block pb = I / 8
      // (16 columns) and q-chunks 4 (I % 8) + group; each lane gets 8 consecutive q
      // of one column p from two transposed reads.
      uint16_t* dst = static_cast<uint16_t*>(MODE == GM_GRAM ? tr.d.gram : tr.d.poly);
      const int64_t ld = tr.d.s_pad;
      const int64_t r0 = static_cast<int64_t>(tr.ti) * kTile;
      const int64_t c0 = static_cast<int64_t>(tr.tj) * kTile;
      uint16_t* const org = dst + slab_off(r0, c0, ld);
      const int grp = lane >> 4, j = lane & 15;
      // I = 32 wave + 8 ub + m: I & 7 = m is a constant of the unrolled inner
      // loop, so the LDS and global offsets that depend on it fold into
      // immediates (with a runtime u, the swizzle was recomputed per store).
#pragma unroll 1
      for (int ub = 0; ub < 4; ++ub) {
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const int I = 32 * wave + 8 * ub + m;
          const int pb = I >> 3, cq = 4 * (I & 7) + grp;
          st16_nt(org + slab_local(16 * pb + j, 8 * cq), read_tile_column(smem, I, lane));
        }
      }
    }
  }
}

}  // namespace

}  // namespace muon

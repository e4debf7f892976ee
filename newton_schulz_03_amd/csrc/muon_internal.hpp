// Internal definitions shared by the C ABI (host) and the kernels (device).
//
// Workspace layout, per call (offsets from the caller's 256-byte aligned base):
//   [table]     MatDesc[batch], then the phase prefix arrays int32[NPHASE][batch+1]
//   [inv]       float[batch]: 1 / (||U||_F + eps) per matrix
//   [partials]  float[prepare blocks]: per-block sums of squares (Frobenius norm)
//   per matrix  X ping, X pong: s_pad x l_pad;  A (Gram), B (polynomial): s_pad x s_pad
//               and, for calls with e4m3 steps (fp8_steps > 0), two e4m3 buffers of
//               s_pad * l_pad bytes plus one scale byte per 32 of them (F8 layout below)
// X ping starts out holding U itself; the first Gram and product scale by the
// norm factor.
// Every matrix is held in its wide orientation (short side first): a matrix
// with more rows than columns is transposed on the way in and back on the way
// out.  s_pad and l_pad round the short and long sides up to the GEMM tile
// (256); the padding holds zeros, which the iteration keeps at zero, so the
// product kernels need no bounds checks.  X, A and B are stored in slabs of
// 256 x 32 elements (see slab_off in device_common.hpp).
//
// F8 layout (e4m3 steps): an e4m3 copy of a matrix with `ncols` columns is held
// in slabs of 256 rows x 64 columns (16 KiB, the same bytes as a bf16 slab),
// each row's 64 values in two blocks of 32 with one power-of-two scale each
// (E8M0: 2^(byte - 127)).  The scales of slab k are the 512 bytes at
// scales + 512 k, where scales = data + s_pad * l_pad (the buffer's capacity);
// the scale of row r (within the slab's 256) and block kb is byte
// 4 * (32 * (2 * (r / 128) + kb) + r % 32) + (r / 32) % 4, so that one dword
// holds the four scales a matrix-core lane needs per 64-wide K step.
// Buffer 0 holds X (rows, blocks along the long side) for the Gram, then A,
// then B (rows, blocks along the short side); buffer 1 holds X^T (rows of X^T,
// blocks along X's short side) for the product.  Both follow B in the
// workspace (f8_buffer).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace muon {

constexpr int kTile = 256;          // GEMM output tile (both sides) and padding granularity
constexpr int kTileW = 384;         // columns of X in a wide product tile (256 rows of B x 384)
constexpr int kEwTile = 64;         // tile side of the finish kernel
constexpr int kPrepTallS = 256;     // prepare's tall tiles: kPrepTallS (short side) x kPrepTallL
constexpr int kPrepTallL = 64;      //   (long side) of the iterate, the user's kPrepTallL x kPrepTallS
constexpr int kPrepWideRows = 32;   // prepare's wide tiles: kPrepWideRows x 256
constexpr int kWideTileCols = 256;  // long-side width of prepare's wide tiles
constexpr int kThreads = 256;       // threads per block, every kernel
constexpr int kAlign = 256;         // workspace sub-buffer alignment
constexpr int kXcd = 8;             // XCDs of the chip: workgroup b runs on XCD b % 8

constexpr int kQ8Tile = 64;         // side of the e4m3 quantization tiles

enum Phase : int {
  PH_PREPARE = 0, PH_SYM = 1, PH_PROD = 2, PH_FINISH = 3, PH_PRODW = 4,
  PH_Q8X = 5,  // e4m3 quantization of the iterate: kQ8Tile x kQ8Tile tiles of s_pad x l_pad
  PH_Q8S = 6,  // e4m3 quantization of A or B: kQ8Tile x kQ8Tile tiles of s_pad x s_pad
  NPHASE = 7
};
enum Mode : int { MODE_NS = 0, MODE_STEP = 1 };

struct MatDesc {
  const void* src;   // NS: x;   STEP: g
  void* mom;         // STEP: m (updated in place); NS: unused
  void* dst;         // NS: out; STEP: w (updated in place)
  void* x[2];        // ping-pong iterate, s_pad x l_pad, wide orientation
  void* gram;        // A = X X^T, s_pad x s_pad
  void* poly;        // B = b A + c A^2, s_pad x s_pad; the e4m3 buffers follow it (f8_buffer)
  int64_t rows, cols, numel;  // user shape
  int32_t s, l;               // short and long side
  int32_t s_pad, l_pad;
  int32_t tall;               // rows > cols
  int32_t vec_ok;             // cols is a multiple of the 16-byte vector width
  float scale;                // sqrt(max(1, rows/cols))
  int32_t reserved;
};

// Tiles of one matrix-core launch, dealt to the XCDs in contiguous ranges cut
// so that every XCD gets about the same number of K slices to run, not the
// same number of tiles: in a ragged batch one tile can cost many times another.
// The last `pool` tiles of each range are not dealt in advance: workgroups
// claim them while the launch runs (claim_tile), so that an XCD that runs
// faster than the others ends by taking tiles off theirs.  When the tiles all
// cost the same, each XCD claims from its own pool first.  When they do not (a
// ragged batch), the pools form one queue, longest tiles first (`norder`
// entries of the order table from `order_off`), so that the launch ends with
// its shortest tiles.
struct XcdSplit {
  int32_t lo[kXcd + 1];  // XCD x owns tiles [lo[x], lo[x + 1]); lo[kXcd] = all tiles
  int32_t dyn[kXcd];     // its tiles [dyn[x], lo[x + 1]) are claimed at run time
  int32_t pool;          // the most tiles of one range claimed at run time (0: none)
  int32_t norder;        // > 0: the pools are claimed as one queue of this many tiles
  int32_t order_off;     // where that queue starts in the order table
  int32_t grid;          // kXcd * (the longest range + pool): the extra workgroups only claim
};

// Claim counters of the matrix-core launches: kSchedInts int32 per set, two
// sets used by alternate launches (counter x < kXcd: tiles claimed from XCD
// x's pool; counter kXcd: from the single queue).
constexpr int kSchedInts = 16;
// Entries of the order table per matrix-core launch kind (Gram, A^2, product,
// wide product): a ragged launch whose pools hold more tiles keeps per-XCD pools.
constexpr int kOrderCap = 2048;
constexpr int kOrderKinds = 4;

struct LaunchCtx {
  const MatDesc* desc;     // device copy of the descriptors
  const int32_t* prefix;   // device: NPHASE arrays of batch+1 block prefixes
  float* partials;         // device: per prepare-block sums of squares
  float* inv_norm;         // device: per matrix 1 / (||U||_F + eps)
  const int32_t* orders;   // device: the order table of the single claim queues
  int32_t* sched;          // device: this matrix-core launch's claim counters (zero at its start)
  int32_t* sched_next;     // device: the next one's, which this launch zeroes
  int32_t batch;
  int32_t max_blocks;      // matrix-core launches: most workgroups resident (0: one per tile)
  // per phase: the blocks of every matrix when all matrices have the same
  // number (then block b belongs to matrix b / per[ph]); 0 for a ragged batch
  int32_t per[NPHASE];
  hipStream_t stream;
};

struct ElemParams {
  int32_t mode;      // MODE_NS / MODE_STEP
  int32_t nesterov;
  float beta;
  float eps;
  float lr;
  int32_t cur;       // which X buffer holds the final iterate (finish)
  int32_t scale_x;   // finish: the iterate is still U (no iterations): scale by the norm factor
};

// Bytes of one e4m3 buffer of a matrix (s_pad * l_pad values and a scale byte
// per 32), and the address of buffer k (0 or 1), which follow B (bf16, s_pad^2)
// in the matrix's part of the workspace.
__host__ __device__ __forceinline__ size_t f8_buffer_bytes(int64_t s_pad, int64_t l_pad) {
  const size_t n = static_cast<size_t>(s_pad) * static_cast<size_t>(l_pad);
  return (n + n / 32 + kAlign - 1) / kAlign * kAlign;
}
__host__ __device__ __forceinline__ char* f8_buffer(const MatDesc& d, int k) {
  const size_t sb = (static_cast<size_t>(d.s_pad) * d.s_pad * 2 + kAlign - 1) / kAlign * kAlign;
  return static_cast<char*>(d.poly) + sb + k * f8_buffer_bytes(d.s_pad, d.l_pad);
}

// AdamW over a ragged batch of flat tensors.
struct AdamDesc {
  void* p;          // parameters (T), updated in place
  const void* g;    // gradients (T)
  float* m;         // first moment, fp32, updated in place
  float* v;         // second moment, fp32, updated in place
  int64_t numel;
};

struct AdamCtx {
  const AdamDesc* desc;    // device copy of the descriptors
  const int32_t* prefix;   // device: batch+1 block prefixes
  int32_t batch;
  hipStream_t stream;
};

struct AdamParams {
  float decay;            // 1 - lr * weight_decay
  float beta1, one_minus_beta1;
  float beta2, one_minus_beta2;
  float step_size;        // lr / (1 - beta1^t)
  float inv_bc2_sqrt;     // 1 / sqrt(1 - beta2^t)
  float eps;
};

int64_t adamw_blocks(int64_t numel);
hipError_t launch_adamw(const AdamCtx& c, int32_t nblocks, bool is_bf16, const AdamParams& a);

// Host launchers (one per kernel family).  is_bf16 selects the element type.
// Momentum (step), U into X ping and the per-block sums of U^2.
hipError_t launch_prepare(const LaunchCtx& c, int32_t nblocks, bool is_bf16, const ElemParams& p);
// One block per matrix: 1 / (||U||_F + eps) from the prepare partials, summed in a
// fixed order in double.
hipError_t launch_finalize(const LaunchCtx& c, const ElemParams& p);
hipError_t launch_finish(const LaunchCtx& c, int32_t nblocks, bool is_bf16, const ElemParams& p);
// The matrix-core launches run the tiles that `sp` splits (sp.lo[kXcd] of them).
// `first`: X[cur] still holds U, so the result takes the norm factor
// f = 1 / (||U||_F + eps) of its matrix (f^2 for the Gram).
// A = out_scale * X X^T  (out_scale = b when the polynomial has no A^2 term, else 1)
hipError_t launch_gram(const LaunchCtx& c, const XcdSplit& sp, bool is_bf16, int32_t cur,
                       float out_scale, bool first);
// B = b A + c A A  (c != 0)
hipError_t launch_poly(const LaunchCtx& c, const XcdSplit& sp, bool is_bf16, float b, float cc);
// X[next] = a X[cur] + Q X[cur] with Q = B (use_poly) or the already scaled A.
// finish != 0 (bf16 only): the last product of the call, whose result goes to
// the user's matrix (W - lr * scale * X', or the output) instead of X[next].
hipError_t launch_prod(const LaunchCtx& c, const XcdSplit& sp, bool is_bf16, int32_t cur,
                       float a, bool use_poly, bool first, int32_t finish = 0, float lr = 0.f);
// The same product into X[next], bf16 only, in tiles of 256 rows x kTileW
// columns (the PH_PRODW tiles that `sp` splits; every l_pad a multiple of
// kTileW).  Bit-identical to launch_prod: each output element accumulates the
// same MFMAs in the same order.
hipError_t launch_prod_wide(const LaunchCtx& c, const XcdSplit& sp, int32_t cur, float a,
                            bool use_poly, bool first);

// e4m3 steps.  launch_quant8: e4m3 copies with one power-of-two scale per 32
// elements along each row: Q8_X quantizes the iterate X[cur] into buffer 0
// (rows) and buffer 1 (rows of X^T); Q8_A / Q8_B quantize A / B into buffer 0.
enum Quant8Src : int { Q8_X = 0, Q8_A = 1, Q8_B = 2 };
hipError_t launch_quant8(const LaunchCtx& c, int32_t nblocks, int32_t src, int32_t cur);
// The matrix-core products on e4m3 operands (gemm_f8.hip), 256 x 256 tiles:
//   GRAM  A = out_scale * F0 F0^T                (F0: buffer 0; f^2 in the first step)
//   POLY  B = c * F0 F0^T + b * A                (F0 holds A; b A in fp32)
//   PROD  X[cur^1] = F1 F0^T + a X[cur]          (F0 holds B, or A when c = 0; F1 = X^T;
//                                                 f in the first step)
hipError_t launch_gram8(const LaunchCtx& c, const XcdSplit& sp, float out_scale, bool first);
hipError_t launch_poly8(const LaunchCtx& c, const XcdSplit& sp, float b, float cc);
hipError_t launch_prod8(const LaunchCtx& c, const XcdSplit& sp, int32_t cur, float a, bool first);

// The allocation-free entry point (noalloc_scratch.hip).  noalloc_scratch:
// the device address of the library's scratch array on the current device
// (MUON_NOALLOC_MAX_WORKSPACE bytes, looked up once per device).
// launch_put_bytes: enqueues kernels on `s` that write the n host bytes at
// src to dst, carrying them as kernel arguments (no staging memory).
hipError_t noalloc_scratch(char** base);
hipError_t launch_put_bytes(const void* src, size_t n, void* dst, hipStream_t s);

}  // namespace muon

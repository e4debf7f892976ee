// Internal definitions shared by the C ABI (host) and the kernels (device).
//
// Workspace layout, per call (offsets from the caller's 256-byte aligned base):
//   [table]     MatDesc[batch], then the phase prefix arrays int32[NPHASE][batch+1]
//   [inv]       float[batch]: 1 / (||U||_F + eps) per matrix
//   [partials]  float[prepare blocks]: per-block sums of squares (Frobenius norm)
//   per matrix  X ping, X pong: s_pad x l_pad;  A (Gram), B (polynomial): s_pad x s_pad
// X ping starts out holding U itself; the first Gram and product scale by the
// norm factor.
// Every matrix is held in its wide orientation (short side first): a matrix
// with more rows than columns is transposed on the way in and back on the way
// out.  s_pad and l_pad round the short and long sides up to the GEMM tile
// (256); the padding holds zeros, which the iteration keeps at zero, so the
// product kernels need no bounds checks.  X, A and B are stored in slabs of
// 256 x 32 elements (see slab_off in device_common.hpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace muon {

constexpr int kTile = 256;          // GEMM output tile (both sides) and padding granularity
constexpr int kTileW = 384;         // columns of X in a wide product tile (256 rows of B x 384)
constexpr int kEwTile = 64;         // tile side of the finish kernel
constexpr int kPrepTallS = 128;     // prepare's tall tiles: kPrepTallS (short side) x kPrepTallL
constexpr int kPrepTallL = 128;     //   (long side) of the iterate, the user's kPrepTallL x kPrepTallS
constexpr int kPrepWideRows = 32;   // prepare's wide tiles: kPrepWideRows x 256
constexpr int kWideTileCols = 256;  // long-side width of prepare's wide tiles
constexpr int kThreads = 256;       // threads per block, every kernel
constexpr int kAlign = 256;         // workspace sub-buffer alignment
constexpr int kXcd = 8;             // XCDs of the chip: workgroup b runs on XCD b % 8

enum Phase : int { PH_PREPARE = 0, PH_SYM = 1, PH_PROD = 2, PH_FINISH = 3, PH_PRODW = 4, NPHASE = 5 };
enum Mode : int { MODE_NS = 0, MODE_STEP = 1 };

struct MatDesc {
  const void* src;   // NS: x;   STEP: g
  void* mom;         // STEP: m (updated in place); NS: unused
  void* dst;         // NS: out; STEP: w (updated in place)
  void* x[2];        // ping-pong iterate, s_pad x l_pad, wide orientation
  void* gram;        // A = X X^T, s_pad x s_pad
  void* poly;        // B = b A + c A^2, s_pad x s_pad
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
struct XcdSplit {
  int32_t lo[kXcd + 1];  // XCD x takes tiles [lo[x], lo[x + 1]); lo[kXcd] = all tiles
  int32_t grid;          // kXcd * the longest range: workgroups of a one-tile-each launch
};

struct LaunchCtx {
  const MatDesc* desc;     // device copy of the descriptors
  const int32_t* prefix;   // device: NPHASE arrays of batch+1 block prefixes
  float* partials;         // device: per prepare-block sums of squares
  float* inv_norm;         // device: per matrix 1 / (||U||_F + eps)
  int32_t batch;
  int32_t max_blocks;      // matrix-core launches: most workgroups resident (0: one per tile)
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

// The allocation-free entry point (noalloc_scratch.hip).  noalloc_scratch:
// the device address of the library's scratch array on the current device
// (MUON_NOALLOC_MAX_WORKSPACE bytes, looked up once per device).
// launch_put_bytes: enqueues kernels on `s` that write the n host bytes at
// src to dst, carrying them as kernel arguments (no staging memory).
hipError_t noalloc_scratch(char** base);
hipError_t launch_put_bytes(const void* src, size_t n, void* dst, hipStream_t s);

}  // namespace muon

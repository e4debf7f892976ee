/*
 * muon_mi355x.h - C ABI of the batched Muon optimizer step for AMD MI355X (gfx950).
 *
 * The operation.  Muon is the optimizer used for almost all weight matrices of
 * the model described on "How PyTorch Scaled a Near-1T MoE on Europe's Public
 * Supercomputer" (§Three optimizations that changed the economics, FlexShard
 * bullet).  Its Newton-Schulz update works on whole matrices; placing whole
 * experts on one rank lets every rank orthogonalize its own matrices with no
 * communication, and running Newton-Schulz on the GPU instead of the host CPU
 * is what shortened the optimizer step there.  Muon keeps one optimizer state
 * per matrix ("Domyn is training a 1T-parameter MoE on Europe's Jupiter
 * supercomputer, and published the recipe", §What moved the number).
 *
 * For each matrix of a ragged batch, muon_step_batched computes
 *     M' = beta*M + G                          (momentum, the single state)
 *     U  = G + beta*M'  if nesterov, else M'
 *     X0 = U / (||U||_F + eps), transposed when rows > cols (short side)
 *     k times:  A = X X^T;  B = b*A + c*A*A;  X = a*X + B*X
 *     O  = X_k, transposed back to rows x cols
 *     W' = W - lr * sqrt(max(1, rows/cols)) * O
 * and muon_ns_batched computes O from U = x alone.  The pages fix no
 * polynomial, step count or epsilon; the usual quintic is
 * (a, b, c) = (3.4445, -4.7750, 2.0315) with k = 5, and (1.5, -0.5, 0) is the
 * cubic iteration that converges to the polar factor.
 *
 * Conventions shared by every entry point:
 *  - Matrices are dense, row-major, contiguous: element (i, j) of a rows x cols
 *    matrix is at ptr[i*cols + j].  One dtype covers every tensor of a call.
 *  - Device pointers (x, out, w, g, m, workspace) must be 16-byte aligned
 *    device memory of the current HIP device (m may be pinned host memory, see
 *    momentum_host).  Host arrays (rows, cols, the pointer arrays, the
 *    parameter structs) are read during the call only.
 *  - The buffers of different matrices of one call must not overlap (this is
 *    not checked); the aliasing allowed within one matrix is stated per entry
 *    point.
 *  - The caller owns every buffer, the workspace included.  The library
 *    allocates no device memory and keeps no pointer after it returns; it owns
 *    only a pool of small pinned host staging buffers for the descriptor
 *    upload, allocated on first use and kept until the process ends, and, once
 *    a step with momentum_host = 1 has run on a device, two copy streams and
 *    their events there.  A call takes a staging buffer whose upload has
 *    completed, or a new one when all are in flight (at most 256 per device).
 *  - Work is enqueued on `stream` (a hipStream_t; NULL is the default stream)
 *    and the call returns without waiting for the GPU, except with more than
 *    256 calls in flight on one device, when it waits for the oldest one's
 *    descriptor upload, and for a step with momentum_host = 1, which first
 *    waits for the previous such step on the device (see muon_step_params).  Buffers must stay alive and untouched until the
 *    stream has finished the work.  Two calls may run concurrently only with
 *    distinct workspaces.
 *  - Every argument is validated before anything is enqueued; on any error
 *    nothing is launched and the outputs are untouched.  batch == 0 is a no-op
 *    that returns MUON_OK.
 *  - NaN and Inf propagate; there is no check.  A zero input gives a zero
 *    output (eps keeps the normalization finite).
 *  - Results are deterministic: the kernels use no floating-point atomics.  The
 *    matrix-core launches hand out the last tiles of each XCD's share with
 *    integer atomics on counters in the workspace, to whichever XCD is free;
 *    which CU computes a tile never changes its value.
 *  - No C++ exception crosses this interface.
 *
 * Precision.  MUON_BF16: tensors are bf16; products accumulate in fp32 on the
 * matrix cores; every stored intermediate (X, A, B, M', W') is rounded to
 * nearest even.  MUON_FP32: tensors and all arithmetic are fp32.
 */
#ifndef MUON_MI355X_H
#define MUON_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of every tensor in a call. */
typedef enum { MUON_BF16 = 0, MUON_FP32 = 1 } muon_dtype;

/* Return codes. */
typedef enum {
  MUON_OK = 0,
  MUON_ERR_INVALID_ARG = 1, /* null pointer, dim <= 0, misaligned pointer, bad dtype, steps < 0,
                               aliasing that is not allowed, non-finite parameter */
  MUON_ERR_UNSUPPORTED = 2, /* a dimension beyond the supported maximum (MUON_MAX_DIM) */
  MUON_ERR_WORKSPACE = 3,   /* workspace null or smaller than muon_workspace_bytes() */
  MUON_ERR_HIP = 4          /* a HIP runtime call or launch failed; see muon_last_error_detail() */
} muon_status;

/* Largest supported rows or cols of one matrix. */
#define MUON_MAX_DIM 65536

/* Newton-Schulz settings: X <- a*X + (b*A + c*A^2)*X with A = X X^T, `steps` times,
 * after X0 = U / (||U||_F + eps).  steps == 0 returns X0.  c == 0 skips A^2. */
typedef struct {
  int32_t steps;
  float a, b, c;
  float eps;
  /* 0: the matrix-core launches fill the GPU.  N > 0: each of them (bf16) keeps
   * at most N workgroups resident, one per CU, each looping over tiles, so that
   * work on other streams keeps the remaining CUs; this is for orthogonalizing
   * the dense matrices while expert compute goes on ("How PyTorch Scaled a
   * Near-1T MoE on Europe's Public Supercomputer", §Three optimizations that
   * changed the economics, FlexShard bullet).  Results do not depend on it,
   * bit for bit: with N = 0 the products that store the iterate take tiles of
   * 256 x 384 where every matrix allows it (bf16, every long side padded to a
   * multiple of 384), with N > 0 tiles of 256 x 256, and both add up every
   * element the same way. */
  int32_t cu_budget;
  /* e4m3 operands in the first fp8_steps iterations (0: none; bf16 only,
   * 0 <= fp8_steps < steps, no cu_budget).  FP8 for expert matrix math is an
   * open question on "Domyn is training a 1T-parameter MoE on Europe's Jupiter
   * supercomputer, and published the recipe" (§What moved the number, closing
   * paragraph).  In those iterations the three products take e4m3 operands
   * with one power-of-two scale per 32 elements along the contracted side
   * (the block maximum at most 448), formed from the bf16 X, A and B; the
   * products accumulate in fp32, the a X and b A terms are added in fp32 from
   * the bf16 matrices, and every result is stored in bf16 as before.  With
   * fp8_steps = 2 of 5 the output is as close to the exact iteration as the
   * bf16 path's; more e4m3 steps are not (the polynomial amplifies their
   * noise once the singular values have grown).  Such a call needs
   * muon_workspace_bytes_ex(..., MUON_WS_FP8) bytes of workspace. */
  int32_t fp8_steps;
} muon_ns_params;

/*
 * Full step settings: learning rate, momentum coefficient, Nesterov flag (0/1),
 * and where the momentum lives.
 *
 * momentum_host = 1 keeps the optimizer state in host memory, as the pages do
 * when they move optimizer state off the accelerator ("Domyn is training a
 * 1T-parameter MoE on Europe's Jupiter supercomputer, and published the
 * recipe", §What moved the number, Offloading bullet).  Every m[i] must then be
 * pinned host memory (hipHostMalloc, or a pinned torch tensor), updated in
 * place.  The batch then runs in up to 16 chunks of about equal momentum bytes:
 * a chunk's momentum is copied to the device by DMA, updated there, and copied
 * back as soon as the momentum pass is done, on two library-owned streams of
 * default priority, so that the copies of neighbouring chunks overlap this
 * chunk's Newton-Schulz work.  The results are bit-identical to momentum in
 * device memory.  The workspace must hold
 * muon_workspace_bytes_ex(..., MUON_WS_MOMENTUM_HOST) bytes, and m[i] must not
 * be touched by the host until the stream has finished the work.  Such a call
 * may block the calling thread: it first waits until the previous such call on
 * this device has finished on the GPU (with the copies of two calls queued at
 * once, the copies slow down by a large and varying factor).  It cannot be
 * captured into a HIP graph.
 * Otherwise (0) m[i] are device memory.
 */
typedef struct {
  float lr;
  float beta;
  int32_t nesterov;
  muon_ns_params ns;
  int32_t momentum_host;
} muon_step_params;

/*
 * Bytes of device workspace a call over this batch needs (the same for
 * muon_ns_batched and muon_step_batched).  rows[i], cols[i]: shape of matrix i.
 * Returns SIZE_MAX on invalid arguments (detail in muon_last_error_detail()).
 * batch == 0 returns 0.  Host-only: launches nothing, needs no GPU.
 */
size_t muon_workspace_bytes(int32_t batch, const int64_t* rows, const int64_t* cols, int32_t dtype);

/*
 * Bytes of device workspace a call with the options in `flags` needs:
 *   MUON_WS_FP8            a bf16 call with fp8_steps > 0: two e4m3 copies of
 *                          each padded iterate more (s_pad * l_pad bytes each,
 *                          plus a scale byte per 32)
 *   MUON_WS_MOMENTUM_HOST  a step with momentum_host = 1: the batch runs in up
 *                          to 16 chunks, each with its own part, plus two
 *                          staging slots for a chunk's momentum
 * flags = 0 is muon_workspace_bytes().  Returns SIZE_MAX on invalid arguments
 * or unknown flags.  Host-only.
 */
#define MUON_WS_FP8 1u
#define MUON_WS_MOMENTUM_HOST 2u
size_t muon_workspace_bytes_ex(int32_t batch, const int64_t* rows, const int64_t* cols,
                               int32_t dtype, uint32_t flags);

/*
 * Orthogonalize a ragged batch: out[i] = NS_k(x[i]) (shape rows[i] x cols[i]).
 *   batch       number of matrices (>= 0)
 *   rows, cols  host arrays[batch] of shapes, each in [1, MUON_MAX_DIM]
 *   x           host array[batch] of device pointers to the inputs (read only)
 *   out         host array[batch] of device pointers to the outputs; out[i] may equal x[i]
 *               (in place) but must not overlap another matrix's buffers otherwise
 *   dtype       MUON_BF16 or MUON_FP32
 *   p           Newton-Schulz settings (host pointer)
 *   workspace   device buffer of at least muon_workspace_bytes() bytes, 256-byte aligned
 *   stream      hipStream_t to enqueue on
 */
int32_t muon_ns_batched(int32_t batch, const int64_t* rows, const int64_t* cols,
                        const void* const* x, void* const* out, int32_t dtype,
                        const muon_ns_params* p, void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * orthogonalization as muon_ns_batched (same kernels, bit-identical results),
 * with no workspace argument: the workspace is a library-owned array of
 * MUON_NOALLOC_MAX_WORKSPACE bytes in device memory (one per GPU the library
 * runs on, held until the process ends).  The call allocates no device or
 * pinned memory and creates no HIP objects; it enqueues only kernel launches
 * on `stream` (the descriptor table travels as kernel arguments) and takes no
 * part in per-kernel timing.
 *   Arguments as muon_ns_batched.  A batch whose muon_workspace_bytes() exceeds
 *   MUON_NOALLOC_MAX_WORKSPACE returns MUON_ERR_WORKSPACE and launches nothing.
 *   Every call on one GPU uses that GPU's one array: calls that overlap on a GPU
 *   (on different streams, or from different threads) race and give undefined
 *   results.  Calls in order on one stream are safe; the array keeps the last
 *   call's contents, and every call writes each part it reads before reading it.
 */
#define MUON_NOALLOC_MAX_WORKSPACE ((size_t)256 << 20)
int32_t muon_ns_batched_noalloc(int32_t batch, const int64_t* rows, const int64_t* cols,
                                const void* const* x, void* const* out, int32_t dtype,
                                const muon_ns_params* p, void* stream);

/*
 * One Muon step over a ragged batch, in place on w[i] and m[i].
 *   w           host array[batch] of device pointers to the weights (updated in place)
 *   g           host array[batch] of device pointers to the gradients (read only)
 *   m           host array[batch] of device pointers to the momentum buffers (updated in place)
 *   w[i], g[i], m[i] must be pairwise distinct.  Other arguments as muon_ns_batched.
 */
int32_t muon_step_batched(int32_t batch, const int64_t* rows, const int64_t* cols,
                          void* const* w, const void* const* g, void* const* m, int32_t dtype,
                          const muon_step_params* p, void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * AdamW for the parameters Muon does not cover.  The model runs Muon on about
 * 99.5% of its parameters and AdamW on the rest ("Domyn is training a
 * 1T-parameter MoE on Europe's Jupiter supercomputer, and published the
 * recipe", §The model and the machine, optimizer row).  The pages do not spell
 * AdamW out; this is Adam with decoupled weight decay in the form PyTorch's
 * AdamW takes, for step number t >= 1 (the step being taken):
 *     p <- p * (1 - lr * weight_decay)
 *     m <- beta1 * m + (1 - beta1) * g
 *     v <- beta2 * v + (1 - beta2) * g^2
 *     p <- p - lr / (1 - beta1^t) * m / (sqrt(v) / sqrt(1 - beta2^t) + eps)
 * The arithmetic is fp32; the bias corrections are formed on the host in double.
 */
typedef struct {
  float lr;
  float beta1, beta2;     /* each in [0, 1) */
  float eps;              /* >= 0 */
  float weight_decay;
  int32_t step;           /* t >= 1 */
} muon_adamw_params;

/*
 * Bytes of device workspace muon_adamw_batched needs for this batch (the
 * descriptor table).  numel[i] >= 0: element count of tensor i.  Returns
 * SIZE_MAX on invalid arguments.  Host-only.
 */
size_t muon_adamw_workspace_bytes(int32_t batch, const int64_t* numel);

/*
 * One AdamW step over a ragged batch of flat tensors, in place.
 *   numel[i]   element count of tensor i (0 allowed: nothing to do)
 *   p[i], g[i] parameters and gradients, `dtype` elements (MUON_BF16 or MUON_FP32);
 *              p is updated in place, g is read only
 *   m[i], v[i] first and second moments, always fp32, updated in place
 *   workspace  device buffer of at least muon_adamw_workspace_bytes() bytes,
 *              256-byte aligned
 * Device pointers must be 16-byte aligned device memory; p, g, m and v of one
 * tensor must be distinct.  Conventions (ownership, stream, validation before
 * any launch, status codes) are those listed at the top of this header.
 */
int32_t muon_adamw_batched(int32_t batch, const int64_t* numel, void* const* p,
                           const void* const* g, float* const* m, float* const* v, int32_t dtype,
                           const muon_adamw_params* params, void* workspace,
                           size_t workspace_bytes, void* stream);

/* Kernels of the step, and the momentum copies of a step with the momentum in
 * host memory, for per-kernel timing. */
typedef enum {
  MUON_K_PREPARE = 0,   /* momentum, U into the iterate (short side first), sums of squares */
  MUON_K_NORM = 1,      /* 1 / (||U||_F + eps) per matrix */
  MUON_K_GRAM = 2,      /* A = X X^T */
  MUON_K_POLY = 3,      /* B = b A + c A^2 */
  MUON_K_PROD = 4,      /* X <- a X + B X, except the first and (bf16) the last */
  MUON_K_FINISH = 5,    /* W update, or the output copy (fp32, or no Newton-Schulz steps) */
  MUON_K_ADAMW = 6,     /* muon_adamw_batched */
  MUON_K_PROD_FINISH = 7, /* bf16: the last X <- a X + B X, writing W (or the output) itself */
  MUON_K_PROD_FIRST = 8,  /* the first X <- a X + B X (its iterate is U, scaled as it is stored) */
  MUON_K_QUANT8 = 9,      /* e4m3 steps: the block-scaled e4m3 copies of X, A and B */
  MUON_K_GRAM8 = 10,      /* e4m3 steps: A = X X^T */
  MUON_K_POLY8 = 11,      /* e4m3 steps: B = b A + c A^2 */
  MUON_K_PROD8 = 12,      /* e4m3 steps: X <- a X + B X */
  MUON_K_MOM_IN = 13,     /* momentum_host: one chunk's momentum copied to the device (DMA) */
  MUON_K_MOM_OUT = 14,    /* momentum_host: one chunk's momentum copied back to the host (DMA) */
  MUON_K_COUNT = 15
} muon_kernel;

/*
 * Per-kernel timing, off by default.  While enabled (process-wide), every call
 * records a pair of HIP events on its stream around each kernel launch (and, with
 * the momentum in host memory, on the copy streams around each chunk's copies).
 * muon_timing_read waits for the recorded events, adds their elapsed times to
 * per-kernel totals, and returns the total milliseconds and the number of
 * launches of `kernel` since the last muon_timing_reset.  Returns MUON_OK,
 * MUON_ERR_INVALID_ARG (bad kernel id or null output) or MUON_ERR_HIP.
 */
int32_t muon_timing_enable(int32_t enable);
int32_t muon_timing_read(int32_t kernel, double* total_ms, int64_t* launches);
int32_t muon_timing_reset(void);

/*
 * Measurement aid: a plain HBM stream with the access pattern of the momentum
 * pass (16-byte vectors, lane-contiguous, every load of a block issued before
 * its first store), for the read + write ceiling that the bandwidth-bound
 * kernels are held against.  Output k receives input k % n_in, except that
 * with two inputs and one output it receives their bitwise XOR; `bytes` bytes
 * each, with the nontemporal hint when `nontemporal` is 1.
 *   n_in, n_out  1 or 2
 *   in, out      host arrays of 16-byte aligned device pointers
 *   bytes        a multiple of 16384 (0: no-op)
 * Returns MUON_OK, MUON_ERR_INVALID_ARG (nothing launched) or MUON_ERR_HIP
 * (launch failure; muon_last_error_detail() is not set by this call).
 */
int32_t muon_hbm_stream(int32_t n_in, const void* const* in, int32_t n_out, void* const* out,
                        size_t bytes, int32_t nontemporal, void* stream);

/* Static string naming a status code. */
const char* muon_status_string(int32_t status);

/* Detail of the last error returned on this thread ("" if none).  Valid until the
 * next call on this thread. */
const char* muon_last_error_detail(void);

#ifdef __cplusplus
}
#endif

#endif /* MUON_MI355X_H */

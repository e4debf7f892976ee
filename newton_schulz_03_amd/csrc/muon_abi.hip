// C ABI of the batched Muon step: argument validation, workspace planning, the
// descriptor upload and the launch sequence.  See include/muon_mi355x.h for the
// contract.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "gemm_common.hpp"
#include "muon_internal.hpp"
#include "muon_mi355x.h"

namespace muon {
namespace {

thread_local std::string g_detail;

int32_t fail(int32_t status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_detail = buf;
  return status;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }
int64_t cdiv(int64_t x, int64_t a) { return (x + a - 1) / a; }

struct Plan {
  int32_t batch = 0;
  bool bf16 = true;
  size_t esize = 2;
  std::vector<MatDesc> desc;        // workspace pointers filled in by bind()
  std::vector<size_t> mat_off;      // byte offset of matrix i's buffers
  std::vector<int32_t> prefix;      // NPHASE x (batch + 1)
  int32_t totals[NPHASE] = {};
  int32_t per[NPHASE] = {};         // blocks per matrix where every matrix has as many; else 0
  XcdSplit split_gram{}, split_poly{}, split_prod{};  // matrix-core launches over the XCDs
  // Wide product tiles (256 x kTileW): every matrix's padded long side is a
  // multiple of kTileW.  Then the products that store the iterate use them.
  bool wide_prod = false;
  XcdSplit split_prodw{};
  bool fp8 = false;                 // the workspace holds the e4m3 buffers (f8)
  std::vector<int32_t> order;       // the single claim queues of ragged launches, packed
  size_t order_off = 0;             // the order table, kOrderKinds * kOrderCap int32 reserved
  size_t table_bytes = 0;           // descriptors and prefixes (uploaded, with the used orders)
  size_t inv_off = 0;
  size_t sched_off = 0;             // two sets of kSchedInts claim counters
  size_t partials_off = 0;
  size_t total_bytes = 0;
};

// A matrix-core tile costs its 32-wide K slices (about 1350 cycles each) plus
// a fixed start and store of about 14k cycles, i.e. about 12 slices more.
constexpr int64_t kTileOverheadSlices = 12;

// Cut the tiles of one matrix-core launch into kXcd contiguous ranges of about
// equal work: XCD x starts at the first tile with at least x/8 of the launch's
// work before it.  Matrix i contributes cnt[i] tiles of slices[i] K slices.
// The last 1/16 of each range (at least 8 tiles, a multiple of 8) is claimed at
// run time, and the grid has as many extra workgroups per XCD: on one chip the
// XCDs' tile rates differed by up to 7%, and a fixed split waits for the
// slowest.  With `queue`, when the pool tiles differ in cost and number at
// most kOrderCap, they form one queue, appended to `order`: longest first
// (ties in tile order), so that the launch ends with its shortest tiles.  The
// Gram keeps per-XCD pools: its tiles stream the whole long side, and one
// taken by another XCD finds none of its operands in that XCD's L2 (a single
// queue made the Gram 0.2-1.6% slower on ragged batches, the other launches
// 0.5-2% faster).
int32_t make_split(const std::vector<int64_t>& cnt, const std::vector<int64_t>& slices,
                   XcdSplit& sp, std::vector<int32_t>& order, bool queue) {
  int64_t total = 0;
  for (size_t i = 0; i < cnt.size(); ++i) total += cnt[i] * (slices[i] + kTileOverheadSlices);
  int64_t tiles_before = 0, work_before = 0;
  int x = 1;
  sp.lo[0] = 0;
  for (size_t i = 0; i < cnt.size(); ++i) {
    const int64_t w = slices[i] + kTileOverheadSlices;
    while (x < kXcd) {
      // the first tile k of this matrix with 8 * (work_before + k * w) >= x * total
      const int64_t need = x * total - kXcd * work_before;
      const int64_t k = need <= 0 ? 0 : cdiv(need, kXcd * w);
      if (k >= cnt[i]) break;
      sp.lo[x++] = static_cast<int32_t>(tiles_before + k);
    }
    tiles_before += cnt[i];
    work_before += cnt[i] * w;
  }
  while (x <= kXcd) sp.lo[x++] = static_cast<int32_t>(tiles_before);
  int64_t longest = 0;
  for (x = 0; x < kXcd; ++x) longest = std::max<int64_t>(longest, sp.lo[x + 1] - sp.lo[x]);
  const int64_t pool = longest == 0 ? 0 : std::max<int64_t>(8, cdiv(cdiv(longest, 16), 8) * 8);
  if ((longest + pool) * kXcd > 0x7fffffffLL)
    return fail(MUON_ERR_UNSUPPORTED, "batch too large: more than 2^31 blocks in one launch");
  sp.pool = static_cast<int32_t>(pool);
  for (x = 0; x < kXcd; ++x)
    sp.dyn[x] = sp.lo[x + 1] - static_cast<int32_t>(std::min<int64_t>(pool, sp.lo[x + 1] - sp.lo[x]));
  sp.grid = static_cast<int32_t>((longest + pool) * kXcd);
  sp.norder = 0;
  sp.order_off = 0;
  // the pool tiles with their costs (tile t of the launch belongs to the matrix
  // whose tiles [first, first + cnt) hold it)
  std::vector<std::pair<int64_t, int32_t>> q;  // (-cost, tile)
  size_t i = 0;
  int64_t first = 0;
  for (x = 0; x < kXcd; ++x) {
    for (int32_t t = sp.dyn[x]; t < sp.lo[x + 1]; ++t) {
      while (t >= first + cnt[i]) first += cnt[i++];
      q.emplace_back(-(slices[i] + kTileOverheadSlices), t);
    }
  }
  bool ragged = false;
  for (const auto& e : q) ragged = ragged || e.first != q.front().first;
  if (queue && ragged && q.size() <= static_cast<size_t>(kOrderCap)) {
    std::sort(q.begin(), q.end());
    sp.norder = static_cast<int32_t>(q.size());
    sp.order_off = static_cast<int32_t>(order.size());
    for (const auto& e : q) order.push_back(e.second);
  }
  return MUON_OK;
}

// Shapes and counts only; no pointers.  fp8: the workspace also holds the
// e4m3 buffers of the e4m3 steps.  Returns MUON_OK or an error (with detail).
int32_t make_plan(int32_t batch, const int64_t* rows, const int64_t* cols, int32_t dtype, Plan& pl,
                  bool fp8 = false) {
  if (batch < 0) return fail(MUON_ERR_INVALID_ARG, "batch = %d is negative", batch);
  if (dtype != MUON_BF16 && dtype != MUON_FP32)
    return fail(MUON_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (batch > 0 && (rows == nullptr || cols == nullptr))
    return fail(MUON_ERR_INVALID_ARG, "rows/cols array is null");
  pl.batch = batch;
  pl.bf16 = dtype == MUON_BF16;
  pl.fp8 = fp8;
  pl.esize = pl.bf16 ? 2 : 4;
  const int64_t vec = 16 / static_cast<int64_t>(pl.esize);
  pl.desc.assign(batch, MatDesc{});
  pl.mat_off.assign(batch, 0);
  pl.prefix.assign(static_cast<size_t>(NPHASE) * (batch + 1), 0);
  int64_t tot[NPHASE] = {};
  // per matrix: symmetric and product tiles; K slices of the Gram (long side)
  // and of A^2 and the product (short side)
  std::vector<int64_t> sym_cnt(batch), prod_cnt(batch), prodw_cnt(batch), k_long(batch),
      k_short(batch);
  bool all_wide = batch > 0;
  for (int32_t i = 0; i < batch; ++i) {
    const int64_t r = rows[i], c = cols[i];
    if (r <= 0 || c <= 0)
      return fail(MUON_ERR_INVALID_ARG, "matrix %d has shape %lld x %lld", i, (long long)r,
                  (long long)c);
    if (r > MUON_MAX_DIM || c > MUON_MAX_DIM)
      return fail(MUON_ERR_UNSUPPORTED, "matrix %d has shape %lld x %lld; the maximum side is %d",
                  i, (long long)r, (long long)c, MUON_MAX_DIM);
    MatDesc& d = pl.desc[i];
    d.rows = r;
    d.cols = c;
    d.numel = r * c;
    d.tall = r > c ? 1 : 0;
    d.s = static_cast<int32_t>(d.tall ? c : r);
    d.l = static_cast<int32_t>(d.tall ? r : c);
    d.s_pad = static_cast<int32_t>(round_up(d.s, kTile));
    d.l_pad = static_cast<int32_t>(round_up(d.l, kTile));
    d.vec_ok = (c % vec) == 0 ? 1 : 0;
    d.scale = static_cast<float>(std::sqrt(std::max(1.0, static_cast<double>(r) / static_cast<double>(c))));
    const int64_t ts = d.s_pad / kTile, tl = d.l_pad / kTile;
    const int64_t cnt[NPHASE] = {
        d.tall ? static_cast<int64_t>(d.s_pad / kPrepTallS) * (d.l_pad / kPrepTallL)
               : static_cast<int64_t>(d.s_pad / kPrepWideRows) * (d.l_pad / kWideTileCols),  // PH_PREPARE
        ts * (ts + 1) / 2,                                                   // PH_SYM
        ts * tl,                                                             // PH_PROD
        cdiv(r, kEwTile) * cdiv(c, kEwTile),                                 // PH_FINISH
        d.l_pad % kTileW == 0 ? ts * (d.l_pad / kTileW) : 0,                 // PH_PRODW
        static_cast<int64_t>(d.s_pad / kQ8Tile) * (d.l_pad / kQ8Tile),       // PH_Q8X
        static_cast<int64_t>(d.s_pad / kQ8Tile) * (d.s_pad / kQ8Tile),       // PH_Q8S
    };
    sym_cnt[i] = cnt[PH_SYM];
    prod_cnt[i] = cnt[PH_PROD];
    prodw_cnt[i] = cnt[PH_PRODW];
    all_wide = all_wide && d.l_pad % kTileW == 0;
    k_long[i] = d.l_pad / 32;
    k_short[i] = d.s_pad / 32;
    for (int ph = 0; ph < NPHASE; ++ph) {
      pl.prefix[static_cast<size_t>(ph) * (batch + 1) + i] = static_cast<int32_t>(tot[ph]);
      tot[ph] += cnt[ph];
      if (tot[ph] > 0x7fffffffLL)
        return fail(MUON_ERR_UNSUPPORTED, "batch too large: more than 2^31 blocks in one launch");
    }
  }
  for (int ph = 0; ph < NPHASE; ++ph) {
    const int32_t* pre = pl.prefix.data() + static_cast<size_t>(ph) * (batch + 1);
    pl.prefix[static_cast<size_t>(ph) * (batch + 1) + batch] = static_cast<int32_t>(tot[ph]);
    pl.totals[ph] = static_cast<int32_t>(tot[ph]);
    // a uniform batch: the kernels find a block's matrix by one division
    const int32_t first = batch > 0 ? pre[1] - pre[0] : 0;
    bool same = first > 0;
    for (int32_t i = 1; same && i < batch; ++i) same = pre[i + 1] - pre[i] == first;
    pl.per[ph] = same ? first : 0;
  }
  int32_t st;
  pl.order.clear();
  if ((st = make_split(sym_cnt, k_long, pl.split_gram, pl.order, false)) != MUON_OK) return st;
  if ((st = make_split(sym_cnt, k_short, pl.split_poly, pl.order, true)) != MUON_OK) return st;
  if ((st = make_split(prod_cnt, k_short, pl.split_prod, pl.order, true)) != MUON_OK) return st;
  pl.wide_prod = all_wide && pl.bf16;
  if (pl.wide_prod &&
      (st = make_split(prodw_cnt, k_short, pl.split_prodw, pl.order, true)) != MUON_OK)
    return st;
  size_t off = 0;
  off += align_up(sizeof(MatDesc) * batch, kAlign);
  off += align_up(sizeof(int32_t) * pl.prefix.size(), kAlign);
  pl.table_bytes = off;
  pl.inv_off = off;
  off += align_up(sizeof(float) * static_cast<size_t>(batch), kAlign);
  pl.sched_off = off;
  off += align_up(sizeof(int32_t) * 2 * kSchedInts, kAlign);
  pl.partials_off = off;
  off += align_up(sizeof(float) * static_cast<size_t>(tot[PH_PREPARE]), kAlign);
  for (int32_t i = 0; i < batch; ++i) {
    const MatDesc& d = pl.desc[i];
    pl.mat_off[i] = off;
    const size_t xb = align_up(static_cast<size_t>(d.s_pad) * d.l_pad * pl.esize, kAlign);
    const size_t sb = align_up(static_cast<size_t>(d.s_pad) * d.s_pad * pl.esize, kAlign);
    off += 2 * xb + 2 * sb + (fp8 ? 2 * f8_buffer_bytes(d.s_pad, d.l_pad) : 0);
  }
  // the order table last: the matrices keep the offsets they have without it
  // (placed after the prefixes, it slowed the Gram by up to 2% on ragged
  // batches, with kernels unchanged)
  pl.order_off = off;
  off += align_up(sizeof(int32_t) * kOrderKinds * kOrderCap, kAlign);
  pl.total_bytes = batch == 0 ? 0 : off;
  return MUON_OK;
}

// Fill the workspace pointers of every descriptor.
void bind(Plan& pl, char* ws) {
  for (int32_t i = 0; i < pl.batch; ++i) {
    MatDesc& d = pl.desc[i];
    const size_t xb = align_up(static_cast<size_t>(d.s_pad) * d.l_pad * pl.esize, kAlign);
    const size_t sb = align_up(static_cast<size_t>(d.s_pad) * d.s_pad * pl.esize, kAlign);
    char* base = ws + pl.mat_off[i];
    d.x[0] = base;
    d.x[1] = base + xb;
    d.gram = base + 2 * xb;
    d.poly = base + 2 * xb + sb;  // the e4m3 buffers, if any, follow (f8_buffer)
  }
}

// Pinned host staging for the descriptor upload: a pool of slots per device,
// each guarded by an event recorded after its copy.  A call takes a slot whose
// copy has completed (asked without waiting) or, when every slot still has a
// copy in flight, a new one, so that the call does not wait for the GPU; only
// past kMaxSlots calls in flight on one device does it wait for the oldest.
struct Slot {
  void* host = nullptr;
  size_t cap = 0;
  hipEvent_t done = nullptr;
  bool pending = false;
};
constexpr size_t kMaxSlots = 256;
struct Pool {
  std::vector<Slot> slot;
  size_t oldest = 0;  // round-robin start of the search, and the slot waited for when full
};
std::mutex g_pool_mu;
std::map<int, Pool> g_pools;

int32_t hip_fail(hipError_t e, const char* what) {
  return fail(MUON_ERR_HIP, "%s: %s (%s)", what, hipGetErrorName(e), hipGetErrorString(e));
}

// A slot of `pool` whose previous copy (if any) has completed; index in *idx.
int32_t free_slot(Pool& pool, size_t* idx) {
  const size_t n = pool.slot.size();
  for (size_t k = 0; k < n; ++k) {
    const size_t i = (pool.oldest + k) % n;
    Slot& s = pool.slot[i];
    if (!s.pending) {
      *idx = i;
      return MUON_OK;
    }
    const hipError_t q = hipEventQuery(s.done);
    if (q == hipSuccess) {
      s.pending = false;
      *idx = i;
      return MUON_OK;
    }
    if (q != hipErrorNotReady) return hip_fail(q, "hipEventQuery (staging slot)");
  }
  if (n < kMaxSlots) {
    pool.slot.emplace_back();
    *idx = n;
    return MUON_OK;
  }
  Slot& s = pool.slot[pool.oldest % n];
  const hipError_t e = hipEventSynchronize(s.done);
  if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize (staging slot)");
  s.pending = false;
  *idx = pool.oldest % n;
  return MUON_OK;
}

// Copies `bytes` composed by `fill` into a pinned slot, then to `dst` on
// `stream`; with bytes2 > 0, the slot's bytes from align_up(bytes, kAlign) on
// (bytes2 of them, also composed by `fill`) go to dst2 from the same slot.
template <typename Fill>
int32_t stage_upload(size_t bytes, Fill fill, void* dst, hipStream_t stream, size_t bytes2 = 0,
                     void* dst2 = nullptr) {
  const size_t host_bytes = bytes2 > 0 ? align_up(bytes, kAlign) + bytes2 : bytes;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lock(g_pool_mu);
  Pool& pool = g_pools[dev];
  size_t idx = 0;
  int32_t st = free_slot(pool, &idx);
  if (st != MUON_OK) return st;
  Slot& s = pool.slot[idx];
  pool.oldest = (idx + 1) % pool.slot.size();
  if (s.done == nullptr) {
    e = hipEventCreateWithFlags(&s.done, hipEventDisableTiming);
    if (e != hipSuccess) return hip_fail(e, "hipEventCreateWithFlags");
  }
  if (s.cap < host_bytes) {
    if (s.host) (void)hipHostFree(s.host);
    s.host = nullptr;
    s.cap = 0;
    const size_t cap = std::max<size_t>(host_bytes, 64 * 1024);
    e = hipHostMalloc(&s.host, cap, hipHostMallocDefault);
    if (e != hipSuccess) return hip_fail(e, "hipHostMalloc (staging)");
    s.cap = cap;
  }
  char* h = static_cast<char*>(s.host);
  std::memset(h, 0, host_bytes);
  fill(h);
  e = hipMemcpyAsync(dst, h, bytes, hipMemcpyHostToDevice, stream);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync (descriptor table)");
  if (bytes2 > 0) {
    e = hipMemcpyAsync(dst2, h + align_up(bytes, kAlign), bytes2, hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync (descriptor table)");
  }
  e = hipEventRecord(s.done, stream);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  s.pending = true;
  return MUON_OK;
}

int32_t upload_table(const Plan& pl, void* ws, hipStream_t stream) {
  // the descriptors and prefixes at the workspace's start; the used part of the
  // order table, at its end, from the same staging slot
  const size_t order_bytes = sizeof(int32_t) * pl.order.size();
  return stage_upload(
      pl.table_bytes,
      [&](char* h) {
        std::memcpy(h, pl.desc.data(), sizeof(MatDesc) * pl.batch);
        std::memcpy(h + align_up(sizeof(MatDesc) * pl.batch, kAlign), pl.prefix.data(),
                    sizeof(int32_t) * pl.prefix.size());
        if (order_bytes > 0)
          std::memcpy(h + align_up(pl.table_bytes, kAlign), pl.order.data(), order_bytes);
      },
      ws, stream, order_bytes, static_cast<char*>(ws) + pl.order_off);
}

// The descriptor table as kernel arguments (no staging buffer, nothing but
// kernel launches on the stream): the allocation-free entry point, and the
// chunks of a step with the momentum in host memory, whose small copies would
// otherwise queue with the chunks' momentum copies.
int32_t put_table(const Plan& pl, char* ws, hipStream_t stream) {
  const size_t desc_bytes = sizeof(MatDesc) * pl.batch;
  hipError_t e = launch_put_bytes(pl.desc.data(), desc_bytes, ws, stream);
  if (e == hipSuccess)
    e = launch_put_bytes(pl.prefix.data(), sizeof(int32_t) * pl.prefix.size(),
                         ws + align_up(desc_bytes, kAlign), stream);
  if (e == hipSuccess && !pl.order.empty())
    e = launch_put_bytes(pl.order.data(), sizeof(int32_t) * pl.order.size(), ws + pl.order_off,
                         stream);
  return e == hipSuccess ? MUON_OK : hip_fail(e, "launch descriptor copy");
}

// AdamW: descriptors, then the block prefix array.
struct AdamPlan {
  int32_t batch = 0;
  bool bf16 = true;
  std::vector<AdamDesc> desc;
  std::vector<int32_t> prefix;
  size_t prefix_off = 0;
  size_t total_bytes = 0;
};

int32_t make_adam_plan(int32_t batch, const int64_t* numel, AdamPlan& pl) {
  if (batch < 0) return fail(MUON_ERR_INVALID_ARG, "batch = %d is negative", batch);
  if (batch > 0 && numel == nullptr) return fail(MUON_ERR_INVALID_ARG, "numel array is null");
  pl.batch = batch;
  pl.desc.assign(batch, AdamDesc{});
  pl.prefix.assign(batch + 1, 0);
  int64_t total = 0;
  for (int32_t i = 0; i < batch; ++i) {
    if (numel[i] < 0) return fail(MUON_ERR_INVALID_ARG, "tensor %d: numel %lld is negative", i,
                                  static_cast<long long>(numel[i]));
    pl.desc[i].numel = numel[i];
    total += adamw_blocks(numel[i]);
    if (total > INT32_MAX) return fail(MUON_ERR_UNSUPPORTED, "batch needs more than 2^31 blocks");
    pl.prefix[i + 1] = static_cast<int32_t>(total);
  }
  pl.prefix_off = align_up(sizeof(AdamDesc) * batch, kAlign);
  pl.total_bytes = batch == 0 ? 0 : pl.prefix_off + align_up(sizeof(int32_t) * (batch + 1), kAlign);
  return MUON_OK;
}

// Per-kernel timing: pairs of events recorded around each launch while enabled.
struct TimingRec {
  int kernel;
  hipEvent_t start, stop;
};
std::mutex g_timing_mu;
bool g_timing_on = false;
std::vector<hipEvent_t> g_event_pool;
std::vector<TimingRec> g_pending;
double g_total_ms[MUON_K_COUNT] = {};
int64_t g_launches[MUON_K_COUNT] = {};

hipEvent_t take_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Brackets one launch with timing events when timing is enabled (and allowed:
// the allocation-free entry point never creates events).
struct TimedLaunch {
  int kernel;
  hipStream_t stream;
  hipEvent_t start = nullptr, stop = nullptr;
  TimedLaunch(int k, hipStream_t s, bool allowed = true) : kernel(k), stream(s) {
    if (!allowed) return;
    std::lock_guard<std::mutex> lock(g_timing_mu);
    if (!g_timing_on) return;
    start = take_event();
    stop = take_event();
    if (start && stop) (void)hipEventRecord(start, stream);
  }
  void done() {
    if (!start || !stop) return;
    (void)hipEventRecord(stop, stream);
    std::lock_guard<std::mutex> lock(g_timing_mu);
    g_pending.push_back({kernel, start, stop});
  }
};

int32_t drain_timing() {
  for (const TimingRec& r : g_pending) {
    hipError_t e = hipEventSynchronize(r.stop);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize (timing)");
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, r.start, r.stop);
    if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
    g_total_ms[r.kernel] += ms;
    g_launches[r.kernel] += 1;
    g_event_pool.push_back(r.start);
    g_event_pool.push_back(r.stop);
  }
  g_pending.clear();
  return MUON_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int32_t check_ns_params(const muon_ns_params* p, int32_t dtype) {
  if (p == nullptr) return fail(MUON_ERR_INVALID_ARG, "params pointer is null");
  if (p->steps < 0) return fail(MUON_ERR_INVALID_ARG, "steps = %d is negative", p->steps);
  if (p->cu_budget < 0)
    return fail(MUON_ERR_INVALID_ARG, "cu_budget = %d is negative", p->cu_budget);
  if (p->fp8_steps < 0)
    return fail(MUON_ERR_INVALID_ARG, "fp8_steps = %d is negative", p->fp8_steps);
  if (p->fp8_steps > 0) {
    if (dtype != MUON_BF16)
      return fail(MUON_ERR_INVALID_ARG, "fp8_steps needs bf16 tensors");
    if (p->fp8_steps >= p->steps)
      return fail(MUON_ERR_INVALID_ARG, "fp8_steps = %d: the last of the %d steps is bf16",
                  p->fp8_steps, p->steps);
    if (p->cu_budget != 0)
      return fail(MUON_ERR_INVALID_ARG, "fp8_steps and cu_budget cannot be combined");
  }
  if (!std::isfinite(p->a) || !std::isfinite(p->b) || !std::isfinite(p->c) ||
      !std::isfinite(p->eps) || p->eps < 0.f)
    return fail(MUON_ERR_INVALID_ARG, "Newton-Schulz coefficients must be finite and eps >= 0");
  return MUON_OK;
}

int32_t check_ws(const Plan& pl, void* ws, size_t ws_bytes) {
  if (ws == nullptr || ws_bytes < pl.total_bytes)
    return fail(MUON_ERR_WORKSPACE, "workspace of %zu bytes at %p; %zu bytes needed", ws_bytes, ws,
                pl.total_bytes);
  if ((reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) != 0)
    return fail(MUON_ERR_INVALID_ARG, "workspace pointer %p is not 256-byte aligned", ws);
  return MUON_OK;
}

// Enqueue the whole step after the table is in place.
// after_prepare (optional): recorded on the stream once the prepare kernel,
// the last reader and writer of the momentum, is enqueued.
int32_t run(const Plan& pl, char* ws, hipStream_t stream, const ElemParams& ep,
            const muon_ns_params& ns, bool timed = true, hipEvent_t after_prepare = nullptr) {
  LaunchCtx c;
  c.desc = reinterpret_cast<const MatDesc*>(ws);
  c.prefix = reinterpret_cast<const int32_t*>(ws + align_up(sizeof(MatDesc) * pl.batch, kAlign));
  c.partials = reinterpret_cast<float*>(ws + pl.partials_off);
  c.inv_norm = reinterpret_cast<float*>(ws + pl.inv_off);
  c.orders = reinterpret_cast<const int32_t*>(ws + pl.order_off);
  // claim counters: the finalize kernel zeroes both sets; matrix-core launch i
  // uses set i % 2 and zeroes the other for launch i + 1
  int32_t* const sets = reinterpret_cast<int32_t*>(ws + pl.sched_off);
  c.sched = sets;
  c.sched_next = sets + kSchedInts;
  int gemm_launches = 0;
  auto gemm_ctx = [&]() -> const LaunchCtx& {
    c.sched = sets + kSchedInts * (gemm_launches & 1);
    c.sched_next = sets + kSchedInts * ((gemm_launches + 1) & 1);
    ++gemm_launches;
    return c;
  };
  c.batch = pl.batch;
  c.max_blocks = ns.cu_budget;
  for (int ph = 0; ph < NPHASE; ++ph) c.per[ph] = pl.per[ph];
  c.stream = stream;
  hipError_t e;
  {
    TimedLaunch t(MUON_K_PREPARE, stream, timed);
    if ((e = launch_prepare(c, pl.totals[PH_PREPARE], pl.bf16, ep)) != hipSuccess)
      return hip_fail(e, "launch momentum/iterate/sum-of-squares");
    t.done();
  }
  if (after_prepare != nullptr && (e = hipEventRecord(after_prepare, stream)) != hipSuccess)
    return hip_fail(e, "hipEventRecord (after the momentum pass)");
  {
    TimedLaunch t(MUON_K_NORM, stream, timed);
    if ((e = launch_finalize(c, ep)) != hipSuccess) return hip_fail(e, "launch norm finalize");
    t.done();
  }
  const bool use_poly = ns.c != 0.f;
  // bf16: the last product writes the user's matrix itself (no finish pass)
  const bool fused = pl.bf16 && ns.steps > 0;
  int32_t cur = 0;
  for (int k = 0; k < ns.steps; ++k) {
    if (k < ns.fp8_steps) {
      // e4m3 step: block-scaled e4m3 copies of X (and X^T), A, then B feed the
      // three products; every result is stored in bf16 as in a bf16 step
      {
        TimedLaunch t(MUON_K_QUANT8, stream, timed);
        if ((e = launch_quant8(c, pl.totals[PH_Q8X], Q8_X, cur)) != hipSuccess)
          return hip_fail(e, "launch e4m3 copies of X");
        t.done();
      }
      {
        TimedLaunch t(MUON_K_GRAM8, stream, timed);
        if ((e = launch_gram8(gemm_ctx(), pl.split_gram, use_poly ? 1.f : ns.b, k == 0)) != hipSuccess)
          return hip_fail(e, "launch Gram (e4m3)");
        t.done();
      }
      {
        TimedLaunch t(MUON_K_QUANT8, stream, timed);
        if ((e = launch_quant8(c, pl.totals[PH_Q8S], Q8_A, cur)) != hipSuccess)
          return hip_fail(e, "launch e4m3 copy of A");
        t.done();
      }
      if (use_poly) {
        {
          TimedLaunch t(MUON_K_POLY8, stream, timed);
          if ((e = launch_poly8(gemm_ctx(), pl.split_poly, ns.b, ns.c)) != hipSuccess)
            return hip_fail(e, "launch polynomial (e4m3)");
          t.done();
        }
        TimedLaunch t(MUON_K_QUANT8, stream, timed);
        if ((e = launch_quant8(c, pl.totals[PH_Q8S], Q8_B, cur)) != hipSuccess)
          return hip_fail(e, "launch e4m3 copy of B");
        t.done();
      }
      {
        TimedLaunch t(MUON_K_PROD8, stream, timed);
        if ((e = launch_prod8(gemm_ctx(), pl.split_prod, cur, ns.a, k == 0)) != hipSuccess)
          return hip_fail(e, "launch product (e4m3)");
        t.done();
      }
      cur ^= 1;
      continue;
    }
    {
      TimedLaunch t(MUON_K_GRAM, stream, timed);
      if ((e = launch_gram(gemm_ctx(), pl.split_gram, pl.bf16, cur, use_poly ? 1.f : ns.b, k == 0)) !=
          hipSuccess)
        return hip_fail(e, "launch Gram");
      t.done();
    }
    if (use_poly) {
      TimedLaunch t(MUON_K_POLY, stream, timed);
      if ((e = launch_poly(gemm_ctx(), pl.split_poly, pl.bf16, ns.b, ns.c)) != hipSuccess)
        return hip_fail(e, "launch polynomial");
      t.done();
    }
    const bool last = fused && k + 1 == ns.steps;
    {
      TimedLaunch t(last ? MUON_K_PROD_FINISH : k == 0 ? MUON_K_PROD_FIRST : MUON_K_PROD, stream,
                    timed);
      const int32_t fin = !last ? FIN_NONE : ep.mode == MODE_STEP ? FIN_STEP : FIN_NS;
      // wide tiles for the products that store the iterate, unless a CU budget
      // asks for the looping launches (256-wide tiles only)
      if (pl.wide_prod && fin == FIN_NONE && ns.cu_budget == 0) {
        if ((e = launch_prod_wide(gemm_ctx(), pl.split_prodw, cur, ns.a, use_poly, k == 0)) != hipSuccess)
          return hip_fail(e, "launch product (wide tiles)");
      } else if ((e = launch_prod(gemm_ctx(), pl.split_prod, pl.bf16, cur, ns.a, use_poly, k == 0, fin,
                                  ep.lr)) != hipSuccess) {
        return hip_fail(e, "launch product");
      }
      t.done();
    }
    cur ^= 1;
  }
  if (fused) return MUON_OK;
  ElemParams fp = ep;
  fp.cur = cur;
  fp.scale_x = ns.steps == 0 ? 1 : 0;  // no product took the norm factor
  {
    TimedLaunch t(MUON_K_FINISH, stream, timed);
    if ((e = launch_finish(c, pl.totals[PH_FINISH], pl.bf16, fp)) != hipSuccess)
      return hip_fail(e, "launch finish");
    t.done();
  }
  return MUON_OK;
}

// ---------------------------------------------------------------------------
// Momentum in pinned host memory.  The batch goes in up to kMaxChunks
// contiguous chunks of about equal momentum bytes, each a call of its own (its
// plan, table and part of the workspace).  Chunk k's momentum is copied to the
// device by DMA on an internal copy-in stream, into one of two staging slots
// that follow the chunks' parts of the workspace; the prepare kernel updates it
// there in place, and an internal copy-out stream copies it back as soon as
// that kernel is done.  So the host-link traffic of chunks k - 1 and k + 1
// overlaps chunk k's Newton-Schulz work.  Events order the three streams; the
// caller's stream waits for the last copy back, and the first copy in waits
// for the work enqueued on the caller's stream before the call.  Each chunk's
// matrices take the same kernels as in one call over the whole batch, so the
// results are the same bits.
constexpr int kMaxChunks = 16;

struct ChunkPlan {
  std::vector<int32_t> first;     // chunk k: matrices [first[k], first[k + 1])
  std::vector<Plan> plans;
  std::vector<size_t> ws_off;     // workspace offset of chunk k's part
  std::vector<size_t> stage_off;  // per matrix: offset of its momentum within its chunk's slot
  std::vector<size_t> bytes;      // per matrix: momentum bytes
  size_t staging_off = 0;         // the two slots, staging_bytes each
  size_t staging_bytes = 0;
  size_t total_bytes = 0;
};

// The shapes must have passed make_plan.
int32_t make_chunks(int32_t batch, const int64_t* rows, const int64_t* cols, int32_t dtype,
                    bool fp8, ChunkPlan& cp) {
  const size_t esize = dtype == MUON_BF16 ? 2 : 4;
  cp.stage_off.assign(batch, 0);
  cp.bytes.assign(batch, 0);
  size_t total = 0;
  for (int32_t i = 0; i < batch; ++i) {
    cp.bytes[i] = esize * static_cast<size_t>(rows[i]) * static_cast<size_t>(cols[i]);
    total += align_up(cp.bytes[i], kAlign);
  }
  const size_t target = (total + kMaxChunks - 1) / kMaxChunks;  // so at most kMaxChunks chunks
  cp.first.assign(1, 0);
  size_t acc = 0;
  for (int32_t i = 0; i < batch; ++i) {
    cp.stage_off[i] = acc;
    acc += align_up(cp.bytes[i], kAlign);
    if (acc >= target || i + 1 == batch) {
      cp.staging_bytes = std::max(cp.staging_bytes, acc);
      cp.first.push_back(i + 1);
      acc = 0;
    }
  }
  const int nchunks = static_cast<int>(cp.first.size()) - 1;
  cp.plans.assign(nchunks, Plan{});
  cp.ws_off.assign(nchunks, 0);
  size_t off = 0;
  for (int k = 0; k < nchunks; ++k) {
    const int32_t a = cp.first[k];
    const int32_t st = make_plan(cp.first[k + 1] - a, rows + a, cols + a, dtype, cp.plans[k], fp8);
    if (st != MUON_OK) return st;
    cp.ws_off[k] = off;
    off += align_up(cp.plans[k].total_bytes, kAlign);
  }
  cp.staging_off = off;
  cp.total_bytes = off + 2 * cp.staging_bytes;
  return MUON_OK;
}

// The internal streams (default priority) and events of the chunked calls on
// one device, created on first use and kept until the process ends.
struct CopyStreams {
  hipStream_t in = nullptr, out = nullptr;
  hipEvent_t start = nullptr;
  hipEvent_t in_done[kMaxChunks], prep_done[kMaxChunks], out_done[kMaxChunks];
  hipEvent_t in_end = nullptr, out_end = nullptr;  // the join of a call
  hipEvent_t done = nullptr;  // the end of the last call
  bool pending = false;       // done has been recorded
  std::mutex mu;  // one chunked call enqueues at a time on a device
};
std::mutex g_copy_mu;
std::map<int, CopyStreams*> g_copy;

int32_t copy_streams(CopyStreams** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lock(g_copy_mu);
  auto it = g_copy.find(dev);
  if (it != g_copy.end()) {
    *out = it->second;
    return MUON_OK;
  }
  CopyStreams* cs = new CopyStreams();
  if ((e = hipStreamCreateWithFlags(&cs->in, hipStreamNonBlocking)) != hipSuccess ||
      (e = hipStreamCreateWithFlags(&cs->out, hipStreamNonBlocking)) != hipSuccess ||
      (e = hipEventCreateWithFlags(&cs->start, hipEventDisableTiming)) != hipSuccess)
    return hip_fail(e, "creating the copy streams");
  if ((e = hipEventCreateWithFlags(&cs->done, hipEventDisableTiming | hipEventBlockingSync)) !=
          hipSuccess ||
      (e = hipEventCreateWithFlags(&cs->in_end, hipEventDisableTiming)) != hipSuccess ||
      (e = hipEventCreateWithFlags(&cs->out_end, hipEventDisableTiming)) != hipSuccess)
    return hip_fail(e, "creating the copy events");
  for (int k = 0; k < kMaxChunks; ++k) {
    if ((e = hipEventCreateWithFlags(&cs->in_done[k], hipEventDisableTiming)) != hipSuccess ||
        (e = hipEventCreateWithFlags(&cs->prep_done[k], hipEventDisableTiming)) != hipSuccess ||
        (e = hipEventCreateWithFlags(&cs->out_done[k], hipEventDisableTiming)) != hipSuccess)
      return hip_fail(e, "creating the copy events");
  }
  g_copy[dev] = cs;
  *out = cs;
  return MUON_OK;
}

// Enqueues the chunked step (see above).  m[i] are pinned host pointers.
int32_t run_chunked(ChunkPlan& cp, char* ws, hipStream_t user, const ElemParams& ep,
                    const muon_ns_params& ns, void* const* w, const void* const* g,
                    void* const* m) {
  CopyStreams* cs = nullptr;
  int32_t st = copy_streams(&cs);
  if (st != MUON_OK) return st;
  std::lock_guard<std::mutex> lock(cs->mu);
  hipError_t e;
  auto ok = [&](hipError_t r, const char* what) -> bool {
    e = r;
    if (r == hipSuccess) return true;
    st = hip_fail(r, what);
    return false;
  };
  // The previous call on this device must have finished before this one is
  // enqueued.  With the copies of two calls queued at once, the runtime has
  // been measured to move part of them onto shader copies that queue behind
  // the Newton-Schulz kernels, and calls then took two to four times as long.
  if (cs->pending && !ok(hipEventSynchronize(cs->done), "hipEventSynchronize")) return st;
  if (!ok(hipEventRecord(cs->start, user), "hipEventRecord") ||
      !ok(hipStreamWaitEvent(cs->in, cs->start, 0), "hipStreamWaitEvent") ||
      !ok(hipStreamWaitEvent(cs->out, cs->start, 0), "hipStreamWaitEvent"))
    return st;
  const int nchunks = static_cast<int>(cp.plans.size());
  auto chunks = [&]() -> int32_t {
    for (int k = 0; k < nchunks; ++k) {
      const int32_t a = cp.first[k], b = cp.first[k + 1];
      char* slot = ws + cp.staging_off + static_cast<size_t>(k & 1) * cp.staging_bytes;
      // copy in, once the slot's previous chunk has gone back to the host
      if (k >= 2 && !ok(hipStreamWaitEvent(cs->in, cs->out_done[k - 2], 0), "hipStreamWaitEvent"))
        return st;
      {
        TimedLaunch t(MUON_K_MOM_IN, cs->in);
        for (int32_t i = a; i < b; ++i)
          if (!ok(hipMemcpyAsync(slot + cp.stage_off[i], m[i], cp.bytes[i], hipMemcpyHostToDevice,
                                 cs->in), "hipMemcpyAsync (momentum to the device)"))
            return st;
        t.done();
      }
      if (!ok(hipEventRecord(cs->in_done[k], cs->in), "hipEventRecord")) return st;
      // the chunk's step, on the caller's stream
      Plan& pl = cp.plans[k];
      char* wsk = ws + cp.ws_off[k];
      bind(pl, wsk);
      for (int32_t i = a; i < b; ++i) {
        MatDesc& d = pl.desc[i - a];
        d.src = g[i];
        d.dst = w[i];
        d.mom = slot + cp.stage_off[i];
      }
      if (!ok(hipStreamWaitEvent(user, cs->in_done[k], 0), "hipStreamWaitEvent")) return st;
      if ((st = put_table(pl, wsk, user)) != MUON_OK) return st;
      if ((st = run(pl, wsk, user, ep, ns, true, cs->prep_done[k])) != MUON_OK) return st;
      // copy back, as soon as the momentum pass is done
      if (!ok(hipStreamWaitEvent(cs->out, cs->prep_done[k], 0), "hipStreamWaitEvent")) return st;
      {
        TimedLaunch t(MUON_K_MOM_OUT, cs->out);
        for (int32_t i = a; i < b; ++i)
          if (!ok(hipMemcpyAsync(m[i], slot + cp.stage_off[i], cp.bytes[i], hipMemcpyDeviceToHost,
                                 cs->out), "hipMemcpyAsync (momentum to the host)"))
            return st;
        t.done();
      }
      if (!ok(hipEventRecord(cs->out_done[k], cs->out), "hipEventRecord")) return st;
    }
    return MUON_OK;
  };
  const int32_t body = chunks();
  // The join, also after an error part-way (so that nothing this call enqueued
  // on the copy streams runs unordered with the caller's later work): the
  // caller's stream waits for the last work of both copy streams.
  const bool joined = ok(hipEventRecord(cs->in_end, cs->in), "hipEventRecord") &&
                      ok(hipEventRecord(cs->out_end, cs->out), "hipEventRecord") &&
                      ok(hipStreamWaitEvent(user, cs->in_end, 0), "hipStreamWaitEvent") &&
                      ok(hipStreamWaitEvent(user, cs->out_end, 0), "hipStreamWaitEvent") &&
                      ok(hipEventRecord(cs->done, user), "hipEventRecord");
  if (joined) cs->pending = true;
  if (body != MUON_OK) return body;
  return joined ? MUON_OK : st;
}

}  // namespace
}  // namespace muon

using namespace muon;

extern "C" size_t muon_workspace_bytes(int32_t batch, const int64_t* rows, const int64_t* cols,
                                       int32_t dtype) {
  Plan pl;
  if (make_plan(batch, rows, cols, dtype, pl) != MUON_OK) return SIZE_MAX;
  return pl.total_bytes;
}

extern "C" size_t muon_workspace_bytes_ex(int32_t batch, const int64_t* rows, const int64_t* cols,
                                          int32_t dtype, uint32_t flags) {
  g_detail.clear();
  if ((flags & ~(MUON_WS_FP8 | MUON_WS_MOMENTUM_HOST)) != 0) {
    fail(MUON_ERR_INVALID_ARG, "unknown workspace flags 0x%x", flags);
    return SIZE_MAX;
  }
  const bool fp8 = (flags & MUON_WS_FP8) != 0;
  if (fp8 && dtype != MUON_BF16) {
    fail(MUON_ERR_INVALID_ARG, "e4m3 steps need bf16 tensors");
    return SIZE_MAX;
  }
  Plan pl;
  if (make_plan(batch, rows, cols, dtype, pl, fp8) != MUON_OK) return SIZE_MAX;
  if ((flags & MUON_WS_MOMENTUM_HOST) == 0 || batch == 0) return pl.total_bytes;
  ChunkPlan cp;
  if (make_chunks(batch, rows, cols, dtype, fp8, cp) != MUON_OK) return SIZE_MAX;
  return cp.total_bytes;
}

namespace muon {
namespace {

// Validation of the orthogonalize-only call's pointer arguments.
int32_t check_ns_pointers(int32_t batch, const void* const* x, void* const* out) {
  if (x == nullptr || out == nullptr) return fail(MUON_ERR_INVALID_ARG, "x/out array is null");
  for (int32_t i = 0; i < batch; ++i) {
    if (x[i] == nullptr || out[i] == nullptr)
      return fail(MUON_ERR_INVALID_ARG, "matrix %d: null device pointer", i);
    if (!aligned16(x[i]) || !aligned16(out[i]))
      return fail(MUON_ERR_INVALID_ARG, "matrix %d: device pointer not 16-byte aligned", i);
  }
  return MUON_OK;
}

void bind_ns(Plan& pl, char* ws, const void* const* x, void* const* out) {
  bind(pl, ws);
  for (int32_t i = 0; i < pl.batch; ++i) {
    pl.desc[i].src = x[i];
    pl.desc[i].mom = nullptr;
    pl.desc[i].dst = out[i];
  }
}

}  // namespace
}  // namespace muon

extern "C" int32_t muon_ns_batched(int32_t batch, const int64_t* rows, const int64_t* cols,
                                   const void* const* x, void* const* out, int32_t dtype,
                                   const muon_ns_params* p, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  try {
    g_detail.clear();
    Plan pl;
    int32_t st = make_plan(batch, rows, cols, dtype, pl, p != nullptr && p->fp8_steps > 0);
    if (st != MUON_OK) return st;
    if ((st = check_ns_params(p, dtype)) != MUON_OK) return st;
    if (batch == 0) return MUON_OK;
    if ((st = check_ns_pointers(batch, x, out)) != MUON_OK) return st;
    if ((st = check_ws(pl, workspace, workspace_bytes)) != MUON_OK) return st;
    char* ws = static_cast<char*>(workspace);
    bind_ns(pl, ws, x, out);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if ((st = upload_table(pl, ws, s)) != MUON_OK) return st;
    ElemParams ep{};
    ep.mode = MODE_NS;
    ep.eps = p->eps;
    return run(pl, ws, s, ep, *p);
  } catch (...) {
    return fail(MUON_ERR_HIP, "unexpected host exception");
  }
}

extern "C" int32_t muon_ns_batched_noalloc(int32_t batch, const int64_t* rows, const int64_t* cols,
                                           const void* const* x, void* const* out, int32_t dtype,
                                           const muon_ns_params* p, void* stream) {
  try {
    g_detail.clear();
    Plan pl;
    int32_t st = make_plan(batch, rows, cols, dtype, pl, p != nullptr && p->fp8_steps > 0);
    if (st != MUON_OK) return st;
    if ((st = check_ns_params(p, dtype)) != MUON_OK) return st;
    if (batch == 0) return MUON_OK;
    if ((st = check_ns_pointers(batch, x, out)) != MUON_OK) return st;
    if (pl.total_bytes > MUON_NOALLOC_MAX_WORKSPACE)
      return fail(MUON_ERR_WORKSPACE,
                  "the batch needs %zu bytes of workspace; the allocation-free call has %zu",
                  pl.total_bytes, static_cast<size_t>(MUON_NOALLOC_MAX_WORKSPACE));
    char* ws = nullptr;
    const hipError_t e = noalloc_scratch(&ws);
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress (the scratch array)");
    bind_ns(pl, ws, x, out);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if ((st = put_table(pl, ws, s)) != MUON_OK) return st;
    ElemParams ep{};
    ep.mode = MODE_NS;
    ep.eps = p->eps;
    return run(pl, ws, s, ep, *p, /*timed=*/false);
  } catch (...) {
    return fail(MUON_ERR_HIP, "unexpected host exception");
  }
}

extern "C" int32_t muon_step_batched(int32_t batch, const int64_t* rows, const int64_t* cols,
                                     void* const* w, const void* const* g, void* const* m,
                                     int32_t dtype, const muon_step_params* p, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  try {
    g_detail.clear();
    Plan pl;
    int32_t st = make_plan(batch, rows, cols, dtype, pl, p != nullptr && p->ns.fp8_steps > 0);
    if (st != MUON_OK) return st;
    if (p == nullptr) return fail(MUON_ERR_INVALID_ARG, "params pointer is null");
    if ((st = check_ns_params(&p->ns, dtype)) != MUON_OK) return st;
    if (!std::isfinite(p->lr) || !std::isfinite(p->beta))
      return fail(MUON_ERR_INVALID_ARG, "lr and beta must be finite");
    if (p->nesterov != 0 && p->nesterov != 1)
      return fail(MUON_ERR_INVALID_ARG, "nesterov must be 0 or 1");
    if (p->momentum_host != 0 && p->momentum_host != 1)
      return fail(MUON_ERR_INVALID_ARG, "momentum_host must be 0 or 1");
    if (batch == 0) return MUON_OK;
    if (w == nullptr || g == nullptr || m == nullptr)
      return fail(MUON_ERR_INVALID_ARG, "w/g/m array is null");
    for (int32_t i = 0; i < batch; ++i) {
      if (w[i] == nullptr || g[i] == nullptr || m[i] == nullptr)
        return fail(MUON_ERR_INVALID_ARG, "matrix %d: null device pointer", i);
      if (!aligned16(w[i]) || !aligned16(g[i]) || !aligned16(m[i]))
        return fail(MUON_ERR_INVALID_ARG, "matrix %d: device pointer not 16-byte aligned", i);
      if (w[i] == g[i] || w[i] == m[i] || static_cast<const void*>(m[i]) == g[i])
        return fail(MUON_ERR_INVALID_ARG, "matrix %d: w, g and m must be distinct buffers", i);
    }
    ElemParams ep{};
    ep.mode = MODE_STEP;
    ep.nesterov = p->nesterov;
    ep.beta = p->beta;
    ep.eps = p->ns.eps;
    ep.lr = p->lr;
    char* ws = static_cast<char*>(workspace);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (p->momentum_host) {
      ChunkPlan cp;
      if ((st = make_chunks(batch, rows, cols, dtype, p->ns.fp8_steps > 0, cp)) != MUON_OK) return st;
      if (ws == nullptr || workspace_bytes < cp.total_bytes)
        return fail(MUON_ERR_WORKSPACE, "workspace of %zu bytes at %p; %zu bytes needed with the "
                    "momentum in host memory", workspace_bytes, workspace, cp.total_bytes);
      if ((reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) != 0)
        return fail(MUON_ERR_INVALID_ARG, "workspace pointer %p is not 256-byte aligned", ws);
      for (int32_t i = 0; i < batch; ++i) {
        hipPointerAttribute_t attr{};
        const hipError_t e = hipPointerGetAttributes(&attr, m[i]);
        if (e != hipSuccess || attr.type != hipMemoryTypeHost) {
          (void)hipGetLastError();
          return fail(MUON_ERR_INVALID_ARG,
                      "matrix %d: momentum_host is set but m is not pinned host memory", i);
        }
      }
      return run_chunked(cp, ws, s, ep, p->ns, w, g, m);
    }
    if ((st = check_ws(pl, workspace, workspace_bytes)) != MUON_OK) return st;
    bind(pl, ws);
    for (int32_t i = 0; i < batch; ++i) {
      pl.desc[i].src = g[i];
      pl.desc[i].dst = w[i];
      pl.desc[i].mom = m[i];
    }
    if ((st = upload_table(pl, ws, s)) != MUON_OK) return st;
    return run(pl, ws, s, ep, p->ns);
  } catch (...) {
    return fail(MUON_ERR_HIP, "unexpected host exception");
  }
}

extern "C" size_t muon_adamw_workspace_bytes(int32_t batch, const int64_t* numel) {
  g_detail.clear();
  AdamPlan pl;
  if (make_adam_plan(batch, numel, pl) != MUON_OK) return SIZE_MAX;
  return pl.total_bytes;
}

extern "C" int32_t muon_adamw_batched(int32_t batch, const int64_t* numel, void* const* p,
                                      const void* const* g, float* const* m, float* const* v,
                                      int32_t dtype, const muon_adamw_params* prm,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  try {
    g_detail.clear();
    AdamPlan pl;
    int32_t st = make_adam_plan(batch, numel, pl);
    if (st != MUON_OK) return st;
    if (dtype != MUON_BF16 && dtype != MUON_FP32)
      return fail(MUON_ERR_INVALID_ARG, "unknown dtype %d", dtype);
    pl.bf16 = dtype == MUON_BF16;
    if (prm == nullptr) return fail(MUON_ERR_INVALID_ARG, "params pointer is null");
    if (!std::isfinite(prm->lr) || !std::isfinite(prm->weight_decay) || !std::isfinite(prm->eps) ||
        prm->eps < 0.f)
      return fail(MUON_ERR_INVALID_ARG, "lr, weight_decay must be finite and eps finite and >= 0");
    if (!(prm->beta1 >= 0.f && prm->beta1 < 1.f) || !(prm->beta2 >= 0.f && prm->beta2 < 1.f))
      return fail(MUON_ERR_INVALID_ARG, "beta1 and beta2 must lie in [0, 1)");
    if (prm->step < 1) return fail(MUON_ERR_INVALID_ARG, "step = %d: must be >= 1", prm->step);
    if (batch == 0) return MUON_OK;
    if (p == nullptr || g == nullptr || m == nullptr || v == nullptr)
      return fail(MUON_ERR_INVALID_ARG, "p/g/m/v array is null");
    for (int32_t i = 0; i < batch; ++i) {
      if (numel[i] == 0) continue;
      const void* q[4] = {p[i], g[i], m[i], v[i]};
      for (int k = 0; k < 4; ++k) {
        if (q[k] == nullptr) return fail(MUON_ERR_INVALID_ARG, "tensor %d: null device pointer", i);
        if (!aligned16(q[k]))
          return fail(MUON_ERR_INVALID_ARG, "tensor %d: device pointer not 16-byte aligned", i);
        for (int l = 0; l < k; ++l)
          if (q[k] == q[l])
            return fail(MUON_ERR_INVALID_ARG, "tensor %d: p, g, m and v must be distinct", i);
      }
      pl.desc[i].p = p[i];
      pl.desc[i].g = g[i];
      pl.desc[i].m = m[i];
      pl.desc[i].v = v[i];
    }
    if (workspace == nullptr || workspace_bytes < pl.total_bytes)
      return fail(MUON_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes,
                  pl.total_bytes);
    if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0)
      return fail(MUON_ERR_INVALID_ARG, "workspace not %d-byte aligned", kAlign);
    char* ws = static_cast<char*>(workspace);
    hipStream_t s = static_cast<hipStream_t>(stream);
    st = stage_upload(
        pl.total_bytes,
        [&](char* h) {
          std::memcpy(h, pl.desc.data(), sizeof(AdamDesc) * pl.batch);
          std::memcpy(h + pl.prefix_off, pl.prefix.data(), sizeof(int32_t) * pl.prefix.size());
        },
        ws, s);
    if (st != MUON_OK) return st;
    const double t = static_cast<double>(prm->step);
    const double bc1 = 1.0 - std::pow(static_cast<double>(prm->beta1), t);
    const double bc2 = 1.0 - std::pow(static_cast<double>(prm->beta2), t);
    AdamParams a{};
    a.decay = static_cast<float>(1.0 - static_cast<double>(prm->lr) * prm->weight_decay);
    a.beta1 = prm->beta1;
    a.one_minus_beta1 = static_cast<float>(1.0 - prm->beta1);
    a.beta2 = prm->beta2;
    a.one_minus_beta2 = static_cast<float>(1.0 - prm->beta2);
    a.step_size = static_cast<float>(prm->lr / bc1);
    a.inv_bc2_sqrt = static_cast<float>(1.0 / std::sqrt(bc2));
    a.eps = prm->eps;
    AdamCtx c{};
    c.desc = reinterpret_cast<const AdamDesc*>(ws);
    c.prefix = reinterpret_cast<const int32_t*>(ws + pl.prefix_off);
    c.batch = pl.batch;
    c.stream = s;
    TimedLaunch tl(MUON_K_ADAMW, s);
    hipError_t e = launch_adamw(c, pl.prefix[pl.batch], pl.bf16, a);
    if (e != hipSuccess) return hip_fail(e, "launch adamw");
    tl.done();
    return MUON_OK;
  } catch (...) {
    return fail(MUON_ERR_HIP, "unexpected host exception");
  }
}

extern "C" const char* muon_status_string(int32_t status) {
  switch (status) {
    case MUON_OK: return "MUON_OK";
    case MUON_ERR_INVALID_ARG: return "MUON_ERR_INVALID_ARG";
    case MUON_ERR_UNSUPPORTED: return "MUON_ERR_UNSUPPORTED";
    case MUON_ERR_WORKSPACE: return "MUON_ERR_WORKSPACE";
    case MUON_ERR_HIP: return "MUON_ERR_HIP";
    default: return "MUON_UNKNOWN_STATUS";
  }
}

extern "C" const char* muon_last_error_detail(void) { return muon::g_detail.c_str(); }

extern "C" int32_t muon_timing_enable(int32_t enable) {
  std::lock_guard<std::mutex> lock(g_timing_mu);
  g_timing_on = enable != 0;
  return MUON_OK;
}

extern "C" int32_t muon_timing_read(int32_t kernel, double* total_ms, int64_t* launches) {
  g_detail.clear();
  if (kernel < 0 || kernel >= MUON_K_COUNT || total_ms == nullptr || launches == nullptr)
    return fail(MUON_ERR_INVALID_ARG, "bad kernel id %d or null output", kernel);
  std::lock_guard<std::mutex> lock(g_timing_mu);
  const int32_t st = drain_timing();
  if (st != MUON_OK) return st;
  *total_ms = g_total_ms[kernel];
  *launches = g_launches[kernel];
  return MUON_OK;
}

extern "C" int32_t muon_timing_reset(void) {
  g_detail.clear();
  std::lock_guard<std::mutex> lock(g_timing_mu);
  const int32_t st = drain_timing();
  for (int k = 0; k < MUON_K_COUNT; ++k) {
    g_total_ms[k] = 0.0;
    g_launches[k] = 0;
  }
  return st;
}

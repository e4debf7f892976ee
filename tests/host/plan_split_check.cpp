// Host-only check of how the matrix-core launches deal tiles to the XCDs.
//
// Built with `hipcc --offload-host-only` against the ABI source itself, with
// stub kernel launchers (no kernel is compiled or run).  For ragged batches of
// random shapes it checks, for the Gram, A^2 and product launches of the plan:
//   - the ranges start at 0, end at the launch's tile count and never shrink;
//   - the grid is 8 times the longest range plus the pool (the tiles at the end
//     of each range that workgroups claim at run time);
//   - split_tile (the static part of what the kernels call) maps the grid's
//     workgroups onto every tile outside the pools exactly once, the rest to -1;
//   - a model of the run-time claims (random interleavings of the claiming
//     workgroups' counter reads and increments) hands out every pool tile
//     exactly once;
//   - a ragged launch's single claim queue (not the Gram's) holds exactly its
//     pool tiles, longest first, and a uniform launch has none;
//   - every XCD's range holds at most 1/8 of the launch's work plus one tile.
//   - the tile orders (prod_tile, sym_tile) take every tile of a grid once, and
//     sym_tile takes the diagonal tiles of each band of kTileGroup rows in a row.
//   - the wide product tiles (256 x kTileW) are planned exactly when every
//     padded long side is a multiple of kTileW, in bf16, and split the same way.
//   - the chunks of a step with the momentum in host memory cover the batch
//     once, at most kMaxChunks of them, each inside its staging slot.
// Prints "OK <plans>" and exits 0, or names the first failure and exits 1.
#include "muon_abi.hip"

#include <random>

namespace muon {
hipError_t launch_prepare(const LaunchCtx&, int32_t, bool, const ElemParams&) { return hipSuccess; }
hipError_t launch_finalize(const LaunchCtx&, const ElemParams&) { return hipSuccess; }
hipError_t launch_finish(const LaunchCtx&, int32_t, bool, const ElemParams&) { return hipSuccess; }
hipError_t launch_gram(const LaunchCtx&, const XcdSplit&, bool, int32_t, float, bool) {
  return hipSuccess;
}
hipError_t launch_poly(const LaunchCtx&, const XcdSplit&, bool, float, float) {
  return hipSuccess;
}
hipError_t launch_prod(const LaunchCtx&, const XcdSplit&, bool, int32_t, float, bool, bool,
                       int32_t, float) {
  return hipSuccess;
}
hipError_t launch_prod_wide(const LaunchCtx&, const XcdSplit&, int32_t, float, bool, bool) {
  return hipSuccess;
}
hipError_t launch_adamw(const AdamCtx&, int32_t, bool, const AdamParams&) { return hipSuccess; }
hipError_t noalloc_scratch(char**) { return hipErrorInvalidSymbol; }
hipError_t launch_quant8(const LaunchCtx&, int32_t, int32_t, int32_t) { return hipSuccess; }
hipError_t launch_gram8(const LaunchCtx&, const XcdSplit&, float, bool) { return hipSuccess; }
hipError_t launch_poly8(const LaunchCtx&, const XcdSplit&, float, float) { return hipSuccess; }
hipError_t launch_prod8(const LaunchCtx&, const XcdSplit&, int32_t, float, bool) {
  return hipSuccess;
}
hipError_t launch_put_bytes(const void*, size_t, void*, hipStream_t) { return hipSuccess; }
int64_t adamw_blocks(int64_t n) { return n; }
}  // namespace muon

using namespace muon;

namespace {

int failures = 0;

void expect(bool ok, const char* what, int plan) {
  if (!ok && failures++ == 0) std::printf("FAIL plan %d: %s\n", plan, what);
}

// tiles: per-matrix tile counts; slices: K slices per tile of each matrix
void check_split(const XcdSplit& sp, const std::vector<int64_t>& tiles,
                 const std::vector<int64_t>& slices, const std::vector<int32_t>& order, bool queue,
                 int plan) {
  int64_t ntiles = 0;
  for (int64_t t : tiles) ntiles += t;
  expect(sp.lo[0] == 0 && sp.lo[kXcd] == ntiles, "ranges do not span the tiles", plan);
  int64_t longest = 0;
  for (int x = 0; x < kXcd; ++x) {
    expect(sp.lo[x + 1] >= sp.lo[x], "ranges shrink", plan);
    longest = std::max<int64_t>(longest, sp.lo[x + 1] - sp.lo[x]);
  }
  expect(sp.grid == kXcd * (longest + sp.pool), "grid is not 8 x (longest range + pool)", plan);
  expect(longest == 0 ? sp.pool == 0 : sp.pool >= 8 && sp.pool % 8 == 0 && 16 * sp.pool >= longest,
         "pool size", plan);
  for (int x = 0; x < kXcd; ++x)
    expect(sp.dyn[x] == sp.lo[x + 1] - std::min<int32_t>(sp.pool, sp.lo[x + 1] - sp.lo[x]),
           "pool start", plan);
  std::vector<int> seen(ntiles, 0);
  std::vector<int32_t> claimers;
  for (int32_t b = 0; b < sp.grid; ++b) {
    const int32_t t = split_tile(sp, b);
    if (t == -1) {
      claimers.push_back(b);
      continue;
    }
    expect(t >= 0 && t < ntiles, "split_tile out of range", plan);
    if (t >= 0 && t < ntiles) seen[t]++;
  }
  // a single queue exactly when the pool tiles differ in cost and fit the table
  std::vector<int64_t> tile_cost;
  for (size_t i = 0; i < tiles.size(); ++i)
    for (int64_t k = 0; k < tiles[i]; ++k) tile_cost.push_back(slices[i]);
  int32_t pooled = 0;
  int64_t pool_cost = -1;
  bool ragged = false;
  for (int x = 0; x < kXcd; ++x)
    for (int32_t t = sp.dyn[x]; t < sp.lo[x + 1]; ++t) {
      ++pooled;
      if (pool_cost < 0) pool_cost = tile_cost[t];
      ragged = ragged || tile_cost[t] != pool_cost;
    }
  expect((sp.norder > 0) == (queue && ragged && pooled <= kOrderCap), "single queue chosen wrongly",
         plan);
  if (sp.norder > 0) {
    // one queue: every pool tile once, costs not increasing; each claimer takes
    // the next entry (one increment), so entry k goes to the k-th claimer
    expect(claimers.size() >= static_cast<size_t>(sp.norder), "fewer claimers than queue entries",
           plan);
    expect(pooled == sp.norder && sp.norder <= kOrderCap, "queue length", plan);
    for (int32_t k = 0; k < sp.norder; ++k) {
      const int32_t t = order[sp.order_off + k];
      int x = 0;
      while (x < kXcd && !(t >= sp.dyn[x] && t < sp.lo[x + 1])) ++x;
      expect(x < kXcd, "queue entry outside the pools", plan);
      expect(k == 0 || tile_cost[t] <= tile_cost[order[sp.order_off + k - 1]],
             "queue not longest first", plan);
      if (t >= 0 && t < ntiles) seen[t]++;
    }
    for (int64_t t = 0; t < ntiles; ++t) expect(seen[t] == 1, "a tile is not taken exactly once", plan);
    return;
  }
  // the run-time claims, modelled step by step in a random interleaving: a
  // claimer increments its own XCD's counter; while it has no tile, it reads
  // every counter (one step) and increments the fullest pool's (the next)
  std::mt19937 rng(static_cast<uint32_t>(plan) * 7919u + 17u);
  int32_t cnt[kXcd] = {};
  struct Claimer { int32_t xcd, state = 0, pick = -1, rounds = 0; bool done = false; };
  std::vector<Claimer> cl;
  for (int32_t b : claimers) cl.push_back({b % kXcd});
  auto take = [&](Claimer&, int32_t y) {
    int32_t lo, dyn, hi;
    xcd_range(sp, y, lo, dyn, hi);
    if (dyn == hi) return false;
    const int32_t k = cnt[y]++;
    if (k >= hi - dyn) return false;
    seen[dyn + k]++;
    return true;
  };
  std::vector<size_t> live(cl.size());
  for (size_t i = 0; i < live.size(); ++i) live[i] = i;
  while (!live.empty()) {
    const size_t li = rng() % live.size();
    Claimer& c = cl[live[li]];
    if (c.state == 0) {
      c.done = take(c, c.xcd);
      c.state = 1;
    } else if (c.state == 1) {  // read the counters, pick the fullest pool
      int32_t best = -(1 << 30);
      for (int32_t y = 0; y < kXcd; ++y) {
        int32_t lo, dyn, hi;
        xcd_range(sp, y, lo, dyn, hi);
        best = std::max(best, (hi - dyn - cnt[y]) * kXcd + (kXcd - 1 - y));
      }
      if (best < kXcd || ++c.rounds > kXcd + 1) c.done = true;
      else { c.pick = kXcd - 1 - (best & (kXcd - 1)); c.state = 2; }
    } else {
      c.done = take(c, c.pick);
      c.state = 1;
    }
    if (c.done) { live[li] = live.back(); live.pop_back(); }
  }
  for (int64_t t = 0; t < ntiles; ++t) expect(seen[t] == 1, "a tile is not taken exactly once", plan);
  // work per XCD: every boundary sits at the first tile whose preceding work
  // reaches x/8 of the total, so no range exceeds 1/8 by a whole tile
  std::vector<int64_t> cost;
  int64_t total = 0, heaviest = 0;
  for (size_t i = 0; i < tiles.size(); ++i)
    for (int64_t k = 0; k < tiles[i]; ++k) {
      cost.push_back(slices[i] + kTileOverheadSlices);
      total += cost.back();
      heaviest = std::max(heaviest, cost.back());
    }
  for (int x = 0; x < kXcd; ++x) {
    int64_t w = 0;
    for (int32_t t = sp.lo[x]; t < sp.lo[x + 1]; ++t) w += cost[t];
    expect(kXcd * w < total + kXcd * heaviest, "an XCD gets more than 1/8 of the work + one tile",
           plan);
  }
}

}  // namespace

int main() {
  std::mt19937 rng(12345);
  const int64_t dims[] = {1, 7, 255, 256, 257, 512, 1000, 1024, 2048, 4095, 6144, 8192};
  int plans = 0;
  // long sides whose padding is a multiple of kTileW, for batches that take wide tiles
  const int64_t wide_dims[] = {700, 768, 1500, 1536, 2304, 3000, 6144, 6100};
  for (int trial = 0; trial < 900; ++trial) {
    const int batch = 1 + static_cast<int>(rng() % (trial < 500 ? 24 : 300));
    std::vector<int64_t> r(batch), c(batch);
    for (int i = 0; i < batch; ++i) {
      r[i] = dims[rng() % 12];
      c[i] = dims[rng() % 12];
      if (trial >= 600) {  // a wide-tile batch: long side from wide_dims, short side below it
        const int64_t l = wide_dims[rng() % 8], sh = 1 + static_cast<int64_t>(rng() % l);
        r[i] = (rng() & 1) ? l : sh;
        c[i] = r[i] == l ? sh : l;
      }
    }
    Plan pl;
    const int32_t dtype = (trial & 1) ? MUON_FP32 : MUON_BF16;
    if (make_plan(batch, r.data(), c.data(), dtype, pl) != MUON_OK) {
      expect(false, "make_plan failed", trial);
      continue;
    }
    std::vector<int64_t> sym(batch), prod(batch), prodw(batch), k_long(batch), k_short(batch);
    bool all_wide = true;
    for (int i = 0; i < batch; ++i) {
      const int64_t ts = pl.desc[i].s_pad / kTile, tl = pl.desc[i].l_pad / kTile;
      sym[i] = ts * (ts + 1) / 2;
      prod[i] = ts * tl;
      prodw[i] = ts * (pl.desc[i].l_pad / kTileW);
      all_wide = all_wide && pl.desc[i].l_pad % kTileW == 0;
      k_long[i] = pl.desc[i].l_pad / 32;
      k_short[i] = pl.desc[i].s_pad / 32;
    }
    // per[ph]: set exactly when every matrix has as many blocks, and then
    // block b lies in matrix b / per[ph] of the prefix table
    for (int ph = 0; ph < NPHASE; ++ph) {
      const int32_t* pre = pl.prefix.data() + static_cast<size_t>(ph) * (batch + 1);
      bool same = pre[1] - pre[0] > 0;
      for (int i = 1; i < batch; ++i) same = same && pre[i + 1] - pre[i] == pre[1] - pre[0];
      expect(pl.per[ph] == (same ? pre[1] - pre[0] : 0), "per-matrix block count wrong", trial);
      if (pl.per[ph] > 0)
        for (int i = 0; i <= batch; ++i)
          expect(pre[i] == i * pl.per[ph], "uniform prefix not a multiple", trial);
    }
    check_split(pl.split_gram, sym, k_long, pl.order, false, trial);
    check_split(pl.split_poly, sym, k_short, pl.order, true, trial);
    check_split(pl.split_prod, prod, k_short, pl.order, true, trial);
    expect(pl.wide_prod == (all_wide && dtype == MUON_BF16), "wide tiles planned wrongly", trial);
    expect(trial < 600 || dtype != MUON_BF16 || pl.wide_prod, "wide-tile batch not wide", trial);
    if (pl.wide_prod) check_split(pl.split_prodw, prodw, k_short, pl.order, true, trial);
    ++plans;
  }
  // the tile orders: every tile of a grid exactly once
  for (int32_t ts = 1; ts <= 40; ++ts) {
    for (int32_t tl = ts; tl <= ts + 9; ++tl) {
      std::vector<int> seen(static_cast<size_t>(ts) * tl, 0);
      for (int32_t t = 0; t < ts * tl; ++t) {
        int32_t ti = -1, tj = -1;
        prod_tile(t, ts, tl, ti, tj);
        const bool ok = ti >= 0 && ti < ts && tj >= 0 && tj < tl;
        expect(ok, "prod_tile out of the grid", ts);
        if (ok) seen[static_cast<size_t>(ti) * tl + tj]++;
      }
      for (int v : seen) expect(v == 1, "prod_tile does not take every tile once", ts);
    }
    std::vector<int> seen(static_cast<size_t>(ts) * ts, 0);
    for (int32_t t = 0; t < ts * (ts + 1) / 2; ++t) {
      int32_t ti = -1, tj = -1;
      sym_tile(t, ts, ti, tj);
      const bool ok = ti >= 0 && ti <= tj && tj < ts;
      expect(ok, "sym_tile outside the upper triangle", ts);
      if (ok) seen[static_cast<size_t>(ti) * ts + tj]++;
    }
    for (int32_t i = 0; i < ts; ++i)
      for (int32_t jj = i; jj < ts; ++jj)
        expect(seen[static_cast<size_t>(i) * ts + jj] == 1, "sym_tile does not take every tile once", ts);
    // the diagonal tiles of a band are consecutive, in row order
    for (int32_t a = 0; a < ts; a += kTileGroup) {
      int32_t first = -1;
      for (int32_t t = 0; t < ts * (ts + 1) / 2; ++t) {
        int32_t ti = -1, tj = -1;
        sym_tile(t, ts, ti, tj);
        if (ti == tj && ti >= a && ti < a + kTileGroup) {
          if (first < 0) first = t;
          expect(t == first + (ti - a), "sym_tile: the diagonal tiles of a band are not in a row", ts);
        }
      }
    }
  }
  // a uniform batch keeps equal ranges and one workgroup per tile
  {
    std::vector<int64_t> r(96, 2048), c(96, 6144);
    Plan pl;
    expect(make_plan(96, r.data(), c.data(), MUON_BF16, pl) == MUON_OK, "uniform plan", -1);
    // 2304 and 432 tiles per XCD; pools of 144 and 32 tiles
    expect(pl.split_prod.grid == 8 * (2304 + 144) && pl.split_gram.grid == 8 * (432 + 32),
           "uniform grid", -1);
    for (int x = 0; x <= kXcd; ++x) expect(pl.split_prod.lo[x] == 2304 * x, "uniform ranges", -1);
    expect(pl.wide_prod && pl.split_prodw.grid == 8 * (1536 + 96), "uniform wide grid", -1);
    for (int x = 0; x <= kXcd; ++x)
      expect(pl.split_prodw.lo[x] == 1536 * x, "uniform wide ranges", -1);
    // 8 x 24 product tiles, 36 upper tiles, 8 x 16 wide tiles per matrix
    expect(pl.per[PH_PROD] == 192 && pl.per[PH_SYM] == 36 && pl.per[PH_PRODW] == 128,
           "uniform per-matrix block counts", -1);
    // one matrix of another shape makes every count ragged
    r[40] = 1024;
    Plan pr;
    expect(make_plan(96, r.data(), c.data(), MUON_BF16, pr) == MUON_OK, "ragged plan", -1);
    expect(pr.per[PH_PROD] == 0 && pr.per[PH_SYM] == 0 && pr.per[PH_PRODW] == 0,
           "ragged per-matrix block counts", -1);
  }
  // the chunks of a step with the momentum in host memory: at most kMaxChunks
  // contiguous chunks covering every matrix once, each chunk's momentum inside
  // a staging slot, the chunks' workspace parts and the two slots disjoint
  for (int trial = 0; trial < 300; ++trial) {
    const int batch = 1 + static_cast<int>(rng() % (trial < 150 ? 40 : 400));
    std::vector<int64_t> r(batch), c(batch);
    for (int i = 0; i < batch; ++i) {
      r[i] = dims[rng() % 12];
      c[i] = dims[rng() % 12];
    }
    const int32_t dtype = (trial & 1) ? MUON_FP32 : MUON_BF16;
    const size_t esize = dtype == MUON_BF16 ? 2 : 4;
    ChunkPlan cp;
    if (make_chunks(batch, r.data(), c.data(), dtype, trial % 3 == 0 && dtype == MUON_BF16, cp) !=
        MUON_OK) {
      expect(false, "make_chunks failed", trial);
      continue;
    }
    const int nchunks = static_cast<int>(cp.plans.size());
    expect(nchunks >= 1 && nchunks <= kMaxChunks, "chunk count out of range", trial);
    expect(cp.first.size() == static_cast<size_t>(nchunks) + 1 && cp.first[0] == 0 &&
               cp.first[nchunks] == batch, "chunks do not span the batch", trial);
    size_t part_end = 0;
    for (int k = 0; k < nchunks; ++k) {
      expect(cp.first[k + 1] > cp.first[k], "an empty chunk", trial);
      expect(cp.plans[k].batch == cp.first[k + 1] - cp.first[k], "chunk plan size", trial);
      expect(cp.ws_off[k] == part_end && cp.ws_off[k] % kAlign == 0, "chunk parts not packed", trial);
      part_end = cp.ws_off[k] + align_up(cp.plans[k].total_bytes, kAlign);
      size_t slot_end = 0;
      for (int32_t i = cp.first[k]; i < cp.first[k + 1]; ++i) {
        expect(cp.bytes[i] == esize * static_cast<size_t>(r[i] * c[i]), "momentum bytes", trial);
        expect(cp.stage_off[i] == slot_end && cp.stage_off[i] % kAlign == 0,
               "momentum not packed in its slot", trial);
        slot_end = cp.stage_off[i] + align_up(cp.bytes[i], kAlign);
      }
      expect(slot_end <= cp.staging_bytes, "a chunk overflows its staging slot", trial);
    }
    expect(cp.staging_off == part_end, "slots do not follow the parts", trial);
    expect(cp.total_bytes == cp.staging_off + 2 * cp.staging_bytes, "total bytes", trial);
    ++plans;
  }
  // an empty batch launches nothing
  {
    Plan pl;
    expect(make_plan(0, nullptr, nullptr, MUON_BF16, pl) == MUON_OK, "empty plan", -1);
    expect(pl.split_gram.grid == 0 && pl.split_prod.grid == 0 && pl.split_prod.lo[kXcd] == 0,
           "empty batch grid", -1);
  }
  if (failures) return 1;
  std::printf("OK %d\n", plans);
  return 0;
}

// Host-side planning: validation, workspace layout and XCD-aware schedules.
#include "plan.hpp"

#include <algorithm>
#include <array>
#include <cmath>
#include <numeric>

namespace muon {

size_t elem_size(muon_dtype dt) { return dt == MUON_F32 ? 4 : 2; }

static int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

namespace {
struct Interval {
  uintptr_t lo, hi;  // [lo, hi)
  bool write;
  int32_t mat;
};
}  // namespace

muon_status validate_matrices(const muon_matrix* mats, int32_t n, muon_dtype dtype,
                              bool need_momentum) {
  if (dtype != MUON_F32 && dtype != MUON_BF16) return MUON_E_DTYPE;
  if (n < 0 || n > MUON_MAX_MATRICES) return MUON_E_SHAPE;
  if (n > 0 && mats == nullptr) return MUON_E_INVALID;
  const size_t es = elem_size(dtype);
  std::vector<Interval> iv;
  iv.reserve(3 * static_cast<size_t>(n));
  for (int32_t i = 0; i < n; ++i) {
    const muon_matrix& M = mats[i];
    if (M.rows < 0 || M.cols < 0 || M.rows > MUON_MAX_DIM || M.cols > MUON_MAX_DIM)
      return MUON_E_SHAPE;
    if (M.rows * M.cols > MUON_MAX_ELEMS) return MUON_E_SHAPE;
    if (M.rows == 0 || M.cols == 0) continue;  // empty: skipped
    if (M.ld < M.cols) return MUON_E_SHAPE;
    if (M.ld > (int64_t(1) << 40)) return MUON_E_SHAPE;
    if (M.grad == nullptr || M.out == nullptr) return MUON_E_INVALID;
    if (need_momentum && M.momentum == nullptr) return MUON_E_INVALID;
    auto misaligned = [es](const void* p) { return reinterpret_cast<uintptr_t>(p) % es != 0; };
    if (misaligned(M.grad) || misaligned(M.out) || (M.momentum && misaligned(M.momentum)))
      return MUON_E_ALIGN;
    const uintptr_t span = static_cast<uintptr_t>(((M.rows - 1) * M.ld + M.cols) * es);
    auto add = [&](const void* p, bool w) {
      uintptr_t lo = reinterpret_cast<uintptr_t>(p);
      iv.push_back({lo, lo + span, w, i});
    };
    add(M.out, true);
    if (M.momentum) add(M.momentum, true);
    if (M.grad != M.out) add(M.grad, false);
  }
  // Any overlap that involves a written buffer is an error (out may equal
  // its own grad exactly; that case is not recorded above).
  std::sort(iv.begin(), iv.end(), [](const Interval& x, const Interval& y) { return x.lo < y.lo; });
  // Sweep keeping the furthest-reaching interval seen so far, separately for
  // written and for any interval: a new interval overlaps an earlier written
  // one if it starts below the max end of the written ones, and a new written
  // interval overlaps anything that ends after its start.
  uintptr_t max_hi_any = 0, max_hi_w = 0;
  for (const Interval& x : iv) {
    if (x.lo < max_hi_w) return MUON_E_INVALID;
    if (x.write && x.lo < max_hi_any) return MUON_E_INVALID;
    max_hi_any = std::max(max_hi_any, x.hi);
    if (x.write) max_hi_w = std::max(max_hi_w, x.hi);
  }
  return MUON_OK;
}

namespace {
// bf16 sets keep X, A and B as fp16 matrix-core operands and X's low part
// as an e4m3 byte at the fixed scale 2^-18, which need every iterate's
// entries below 4 in magnitude (entries are bounded by the largest singular
// value). The iteration maps each singular value of X0, all in [0, 1], by
// p(x) = a x + b x^3 + c x^5: the check follows 4097 points of [0, 1]
// through the configured steps and requires them to stay in [-2, 2]; B =
// b A + c A A then has eigenvalues below |b| 4 + |c| 16 (A = X X^T below 4),
// which must stay far inside fp16's range. The last result is cached.
bool iteration_in_range(float a, float b, float c, int32_t steps) {
  if (std::fabs(a) + 4.0 * std::fabs(b) + 16.0 * std::fabs(c) > 4096.0) return false;
  static thread_local float la = 0.f, lb = 0.f, lc = 0.f;
  static thread_local int32_t ls = -1;
  static thread_local bool lok = false;
  if (ls == steps && la == a && lb == b && lc == c) return lok;
  bool ok = true;
  for (int i = 0; i <= 4096 && ok; ++i) {
    double x = i / 4096.0;
    for (int32_t t = 0; t < steps; ++t) {
      const double x2 = x * x;
      x = x * (double(a) + x2 * (double(b) + double(c) * x2));
      if (!(std::fabs(x) <= 2.0)) {
        ok = false;
        break;
      }
    }
  }
  la = a, lb = b, lc = c, ls = steps, lok = ok;
  return ok;
}
}  // namespace

muon_status validate_config(const muon_config* cfg, muon_dtype dtype) {
  if (cfg == nullptr) return MUON_E_INVALID;
  if (!std::isfinite(cfg->a) || !std::isfinite(cfg->b) || !std::isfinite(cfg->c) ||
      !std::isfinite(cfg->momentum) || !std::isfinite(cfg->eps))
    return MUON_E_INVALID;
  if (cfg->steps < 0 || cfg->steps > MUON_MAX_STEPS) return MUON_E_INVALID;
  if (cfg->momentum < 0.f || cfg->momentum >= 1.f) return MUON_E_INVALID;
  if (cfg->nesterov != 0 && cfg->nesterov != 1) return MUON_E_INVALID;
  if (cfg->eps < 0.f) return MUON_E_INVALID;
  if (cfg->precision != MUON_PRECISION_DEFAULT) return MUON_E_INVALID;
  if (dtype == MUON_BF16 && !iteration_in_range(cfg->a, cfg->b, cfg->c, cfg->steps))
    return MUON_E_INVALID;
  return MUON_OK;
}

namespace {
// True if any interval that is written overlaps another interval.
bool overlaps(std::vector<Interval>& iv) {
  std::sort(iv.begin(), iv.end(), [](const Interval& x, const Interval& y) { return x.lo < y.lo; });
  uintptr_t max_hi_any = 0, max_hi_w = 0;
  for (const Interval& x : iv) {
    if (x.lo < max_hi_w) return true;
    if (x.write && x.lo < max_hi_any) return true;
    max_hi_any = std::max(max_hi_any, x.hi);
    if (x.write) max_hi_w = std::max(max_hi_w, x.hi);
  }
  return false;
}
}  // namespace

muon_status validate_weights(const HostPlan& plan, const muon_weight* w, int32_t n) {
  if (n != static_cast<int32_t>(plan.mats.size())) return MUON_E_SHAPE;
  if (n > 0 && w == nullptr) return MUON_E_INVALID;
  const size_t es = elem_size(plan.dtype);
  std::vector<Interval> iv;
  for (int32_t i = 0; i < n; ++i) {
    const muon_matrix& M = plan.mats[i];
    if (M.rows == 0 || M.cols == 0) continue;
    const muon_weight& W = w[i];
    if (W.weight == nullptr) return MUON_E_INVALID;
    if (W.ld < M.cols || W.ld > (int64_t(1) << 40)) return MUON_E_SHAPE;
    if (reinterpret_cast<uintptr_t>(W.weight) % es != 0) return MUON_E_ALIGN;
    if (!std::isfinite(W.lr_mul) || !std::isfinite(W.wd_mul)) return MUON_E_INVALID;
    auto add = [&](const void* p, int64_t ld, bool wr) {
      const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
      iv.push_back({lo, lo + static_cast<uintptr_t>(((M.rows - 1) * ld + M.cols) * es), wr, i});
    };
    add(W.weight, W.ld, true);
    add(M.out, M.ld, true);
    if (M.momentum) add(M.momentum, M.ld, true);
    if (M.grad != M.out) add(M.grad, M.ld, false);
  }
  return overlaps(iv) ? MUON_E_INVALID : MUON_OK;
}

muon_status validate_apply(const muon_apply* ap) {
  if (ap == nullptr) return MUON_E_INVALID;
  if (!std::isfinite(ap->lr) || !std::isfinite(ap->wd)) return MUON_E_INVALID;
  return MUON_OK;
}

namespace {

// A run of consecutive work items of one matrix, with its summed cost.
struct Chunk {
  int32_t mat;
  std::vector<WorkItem> items;
  double cost;
};

// Distributes chunks over the XCDs (longest-processing-time first, ties by
// lower XCD), keeps each XCD's chunks in matrix order, and interleaves the
// per-XCD lists so that block b (dispatched to XCD b % 8) takes the
// (b / 8)-th item of its XCD's list. Work of one matrix thus stays on one
// XCD (one L2) while the eight XCDs get about equal cost.
Schedule assign_xcd(std::vector<Chunk> chunks) {
  std::vector<size_t> order(chunks.size());
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(),
                   [&](size_t x, size_t y) { return chunks[x].cost > chunks[y].cost; });
  std::vector<double> load(kNumXcd, 0.0);
  std::vector<std::vector<size_t>> bins(kNumXcd);
  for (size_t ci : order) {
    int best = 0;
    for (int x = 1; x < kNumXcd; ++x)
      if (load[x] < load[best]) best = x;
    load[best] += chunks[ci].cost;
    bins[best].push_back(ci);
  }
  std::vector<std::vector<WorkItem>> lists(kNumXcd);
  size_t longest = 0;
  for (int x = 0; x < kNumXcd; ++x) std::sort(bins[x].begin(), bins[x].end());
  for (int x = 0; x < kNumXcd; ++x) {
    // Longest items first (they would otherwise form the tail); items of
    // equal cost stay in matrix order, so one matrix's tiles run together.
    std::vector<std::pair<double, WorkItem>> its;
    for (size_t ci : bins[x]) {
      const double per = chunks[ci].cost / double(chunks[ci].items.size());
      for (const WorkItem& w : chunks[ci].items) its.push_back({per, w});
    }
    std::stable_sort(its.begin(), its.end(),
                     [](const auto& p, const auto& q) { return p.first > q.first; });
    for (const auto& p : its) lists[x].push_back(p.second);
    longest = std::max(longest, lists[x].size());
  }
  Schedule s;
  s.items.assign(longest * kNumXcd, WorkItem{-1, -1, -1, -1});
  for (int x = 0; x < kNumXcd; ++x)
    for (size_t p = 0; p < lists[x].size(); ++p) s.items[p * kNumXcd + x] = lists[x][p];
  return s;
}

// Splits each matrix's item list into chunks of at most `max_cost` (the
// parts of one split Gram tile stay in one chunk, so they share an XCD).
void add_matrix_chunks(std::vector<Chunk>& chunks, int32_t mat, const std::vector<WorkItem>& items,
                       const std::vector<double>& costs, double max_cost) {
  Chunk cur{mat, {}, 0.0};
  for (size_t i = 0; i < items.size(); ++i) {
    const bool tile_start = ((items[i].c >> 8) & 255) == 0;
    if (!cur.items.empty() && cur.cost + costs[i] > max_cost && tile_start) {
      chunks.push_back(std::move(cur));
      cur = Chunk{mat, {}, 0.0};
    }
    cur.items.push_back(items[i]);
    cur.cost += costs[i];
  }
  if (!cur.items.empty()) chunks.push_back(std::move(cur));
}

// Places each reduce item of a split Gram tile on the XCD that ran the
// tile's parts in `gram` (block b runs on XCD b % 8), so that the reduce
// pass reads the partial tiles from that XCD's L2.
Schedule place_reduce(const Schedule& gram, const std::vector<WorkItem>& reduce) {
  auto key = [](const WorkItem& w) { return (int64_t(w.mat) << 32) | (int64_t(w.a) << 16) | w.b; };
  std::vector<std::pair<int64_t, int>> xcd_of;
  for (size_t b = 0; b < gram.items.size(); ++b) {
    const WorkItem& w = gram.items[b];
    if (w.mat >= 0 && (w.c & 255) >= 2 && ((w.c >> 8) & 255) == 0)
      xcd_of.push_back({key(w), static_cast<int>(b % kNumXcd)});
  }
  std::sort(xcd_of.begin(), xcd_of.end());
  std::vector<std::vector<WorkItem>> lists(kNumXcd);
  size_t longest = 0;
  for (const WorkItem& r : reduce) {
    auto it = std::lower_bound(xcd_of.begin(), xcd_of.end(), std::make_pair(key(r), -1));
    const int x = (it != xcd_of.end() && it->first == key(r)) ? it->second : 0;
    lists[x].push_back(r);
    longest = std::max(longest, lists[x].size());
  }
  Schedule s;
  s.items.assign(longest * kNumXcd, WorkItem{-1, -1, -1, -1});
  for (int x = 0; x < kNumXcd; ++x)
    for (size_t p = 0; p < lists[x].size(); ++p) s.items[p * kNumXcd + x] = lists[x][p];
  return s;
}

// Chained schedule (plan.hpp). Item durations are rough estimates in
// microseconds at full load (one stage of 32 k values takes about 1 us, a
// diagonal tile's stage about 0.7 us, an epilogue about 5 us); they only
// order the lists. Returns false (no chain) when the matrices cannot be
// spread evenly over the XCDs.
bool build_chain(HostPlan& P, const std::vector<std::vector<std::vector<WorkItem>>>& per) {
  const int32_t n = static_cast<int32_t>(P.info.size());
  constexpr int kPhases = 3;
  const int kind_of[kPhases] = {MUON_K_GRAM, MUON_K_POLY, MUON_K_UPDATE};
  auto dur = [&](int ph, const WorkItem& w) {
    const MatInfo& I = P.info[w.mat];
    const bool diag = ph < 2 && w.a == w.b;
    const double st = (ph == 0 ? I.np : I.mp) / 32.0;
    return (diag ? 0.7 : 1.0) * st + 5.0;
  };
  std::vector<double> work(n, 0.0);
  std::vector<std::array<double, kPhases>> longest(n);
  int32_t nonempty = 0;
  for (int32_t i = 0; i < n; ++i) {
    longest[i].fill(0.0);
    if (P.info[i].m == 0) continue;
    ++nonempty;
    for (int ph = 0; ph < kPhases; ++ph)
      for (const WorkItem& w : per[kind_of[ph]][i]) {
        work[i] += dur(ph, w);
        longest[i][ph] = std::max(longest[i][ph], dur(ph, w));
      }
  }
  if (nonempty < kNumXcd) return false;
  // matrices onto XCDs, heaviest first onto the lightest XCD
  std::vector<int32_t> order;
  for (int32_t i = 0; i < n; ++i)
    if (P.info[i].m > 0) order.push_back(i);
  std::stable_sort(order.begin(), order.end(), [&](int32_t x, int32_t y) { return work[x] > work[y]; });
  std::vector<double> load(kNumXcd, 0.0);
  std::vector<std::vector<int32_t>> bins(kNumXcd);
  double total = 0.0;
  for (int32_t i : order) {
    int best = 0;
    for (int x = 1; x < kNumXcd; ++x)
      if (load[x] < load[best]) best = x;
    load[best] += work[i];
    bins[best].push_back(i);
    total += work[i];
  }
  if (*std::max_element(load.begin(), load.end()) > kChainMaxImbalance * total / kNumXcd) return false;

  P.chain.clear();
  for (int x = 0; x < kNumXcd; ++x) {
    P.chain_beg[x] = static_cast<int32_t>(P.chain.size());
    // List scheduling of one step on the XCD's CUs: the CU that frees first
    // takes the next item of the matrix with the longest remaining chain
    // among those whose current phase is available, else of the matrix
    // whose phase becomes available first. A phase is available once every
    // item of the previous one has ended.
    struct M {
      int32_t mat, ph = 0;
      size_t pos = 0;
      double avail = 0.0, end = 0.0;
      int32_t need = 0;
    };
    std::vector<M> ms;
    for (int32_t i : bins[x]) ms.push_back(M{i});
    auto rest = [&](const M& m) {
      double r = 0.0;
      for (int ph = m.ph; ph < kPhases; ++ph) r += longest[m.mat][ph];
      return r;
    };
    std::vector<double> cu(kChainCus, 0.0);
    for (;;) {
      const size_t c = static_cast<size_t>(std::min_element(cu.begin(), cu.end()) - cu.begin());
      const double now = cu[c];
      int pick = -1;
      for (size_t k = 0; k < ms.size(); ++k) {
        const M& m = ms[k];
        if (m.ph >= kPhases) continue;
        if (pick < 0) {
          pick = static_cast<int>(k);
          continue;
        }
        const M& b = ms[pick];
        const bool ra = m.avail <= now, rb = b.avail <= now;
        if (ra != rb) {
          if (ra) pick = static_cast<int>(k);
        } else if (ra ? rest(m) > rest(b) : m.avail < b.avail) {
          pick = static_cast<int>(k);
        }
      }
      if (pick < 0) break;
      M& m = ms[pick];
      const std::vector<WorkItem>& items = per[kind_of[m.ph]][m.mat];
      const WorkItem& w = items[m.pos++];
      const double t0 = std::max(now, m.avail), t1 = t0 + dur(m.ph, w);
      cu[c] = t1;
      m.end = std::max(m.end, t1);
      P.chain.push_back(ChainItem{m.mat, static_cast<int16_t>(w.a), static_cast<int16_t>(w.b), m.need, kind_of[m.ph]});
      if (m.pos == items.size()) {
        m.need += static_cast<int32_t>(items.size());
        m.pos = 0;
        m.avail = m.end;
        m.end = 0.0;
        ++m.ph;
        while (m.ph < kPhases && per[kind_of[m.ph]][m.mat].empty()) ++m.ph;
      }
    }
  }
  P.chain_beg[kNumXcd] = static_cast<int32_t>(P.chain.size());
  for (int32_t i = 0; i < n; ++i) {
    int32_t c = 0;
    for (int ph = 0; ph < kPhases; ++ph) c += static_cast<int32_t>(per[kind_of[ph]][i].size());
    P.info[i].chain_n = c;
  }
  // each item also carries its matrix's count (one load less before a wait)
  for (ChainItem& c : P.chain) c.kind_n |= P.info[c.mat].chain_n << 8;
  return true;
}

}  // namespace

muon_status build_plan(const muon_matrix* mats, int32_t n, muon_dtype dtype, HostPlan* out) {
  muon_status st = validate_matrices(mats, n, dtype, false);
  if (st != MUON_OK) return st;
  HostPlan P;
  P.dtype = dtype;
  P.mats.assign(mats, mats + n);
  P.info.resize(n);
  const size_t es = elem_size(dtype);
  const bool bf16 = dtype == MUON_BF16;

  // Per-matrix layout; the partials region comes first.
  int32_t nparts = 0;
  std::vector<std::vector<WorkItem>> items(MUON_K_COUNT);
  for (int32_t i = 0; i < n; ++i) {
    const muon_matrix& M = mats[i];
    MatInfo& I = P.info[i];
    I = MatInfo{};
    I.grad = M.grad;
    I.mom = M.momentum;
    I.out = M.out;
    I.ld = M.ld;
    I.rows = static_cast<int32_t>(M.rows);
    I.cols = static_cast<int32_t>(M.cols);
    I.xl_off = I.xo_off[0] = I.xo_off[1] = I.a_off = I.b_off = -1;
    if (M.rows == 0 || M.cols == 0) continue;
    I.tall = M.rows > M.cols;
    I.m = static_cast<int32_t>(std::min(M.rows, M.cols));
    I.n = static_cast<int32_t>(std::max(M.rows, M.cols));
    I.mp = static_cast<int32_t>(round_up(I.m, bf16 ? kTileM16 : kGemmTile));
    I.np = static_cast<int32_t>(round_up(I.n, bf16 ? kTileN16 : kGemmTile));
    auto aligned16 = [](const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; };
    I.vec_ok = aligned16(M.grad) && aligned16(M.out) && (!M.momentum || aligned16(M.momentum)) &&
               (M.ld * es) % 16 == 0 && (M.cols * es) % 16 == 0;
    const int32_t rows_per_item =
        static_cast<int32_t>(std::max<int64_t>(1, kMomentumElems / M.cols));
    I.part_off = nparts;
    I.part_cnt = static_cast<int32_t>((M.rows + rows_per_item - 1) / rows_per_item);
    nparts += I.part_cnt;
    if (bf16) {
      I.tile_off = P.total_tiles;
      I.tile_cnt = (I.mp / kNormTile) * (I.np / kNormTile);
      P.total_tiles += I.tile_cnt;
    }
  }
  P.total_partials = nparts;
  // partial sums of u^2, then their exponents
  size_t off = round_up(static_cast<int64_t>(nparts) * 8, kWsAlign);
  auto take = [&off](size_t bytes) {
    int64_t o = static_cast<int64_t>(off);
    off = round_up(static_cast<int64_t>(off + bytes), kWsAlign);
    return o;
  };
  if (bf16 && P.total_tiles > 0) {
    P.tsum_off = take(static_cast<size_t>(P.total_tiles) * 4);
    P.tmax_off = take(static_cast<size_t>(P.total_tiles) * 4);
    P.x0s_off = take(static_cast<size_t>(n) * 16);
  }
  for (int32_t i = 0; i < n; ++i) {
    MatInfo& I = P.info[i];
    if (I.m == 0) continue;
    const size_t xel = static_cast<size_t>(I.mp) * I.np;
    const size_t ael = static_cast<size_t>(I.mp) * I.mp;
    if (bf16) {
      I.xl_off = take(xel);
      I.xo_off[0] = take(xel * 2);
      I.xo_off[1] = take(xel * 2);
      I.a_off = take(ael * 2);
      I.b_off = take(ael * 2);
    } else {
      I.xo_off[0] = take(xel * 4);
      I.xo_off[1] = take(xel * 4);
      I.a_off = take(ael * 4);
      I.b_off = take(ael * 4);
    }
  }
  P.ws_bytes = n == 0 || off == 0 ? 0 : off;
  bool any = false;
  for (const MatInfo& I : P.info) any = any || I.m > 0;
  if (!any) P.ws_bytes = 0;

  // Work items and their costs, per kernel.
  std::vector<std::vector<std::vector<WorkItem>>> per(kKinds, std::vector<std::vector<WorkItem>>(n));
  std::vector<std::vector<std::vector<double>>> cost(kKinds, std::vector<std::vector<double>>(n));
  for (int32_t i = 0; i < n; ++i) {
    const MatInfo& I = P.info[i];
    if (I.m == 0) continue;
    const int32_t rows_per_item = static_cast<int32_t>(std::max<int64_t>(1, kMomentumElems / I.cols));
    for (int32_t p = 0; p < I.part_cnt; ++p) {
      int32_t r0 = p * rows_per_item;
      int32_t nr = std::min(rows_per_item, I.rows - r0);
      per[MUON_K_MOMENTUM][i].push_back({i, r0, nr, I.part_off + p});
      cost[MUON_K_MOMENTUM][i].push_back(double(nr) * I.cols);
    }
    const int32_t nti = I.mp / kNormTile, ntj = I.np / kNormTile;
    for (int32_t ti = 0; ti < nti; ++ti)
      for (int32_t tj = 0; tj < ntj; ++tj) {
        per[MUON_K_NORMALIZE][i].push_back({i, ti, tj, 0});
        cost[MUON_K_NORMALIZE][i].push_back(1.0);
      }
    // scale pass: one workgroup per matrix
    if (bf16) {
      per[kX0Scale][i].push_back({i, 0, 0, 0});
      cost[kX0Scale][i].push_back(double(I.tile_cnt));
    }
    // Tiles of tm x tn; gram/poly keep the tiles that reach the upper
    // triangle (first row <= last column: tj * tn + tn - 1 >= ti * tm).
    const int32_t tm = bf16 ? kTileM16 : kGemmTile, tn = bf16 ? kTileN16 : kGemmTile;
    const int32_t gt = I.mp / tm, gc = I.mp / tn, gn = I.np / tn;
    const double area = double(tm) * tn;
    for (int32_t ti = 0; ti < gt; ++ti)
      for (int32_t tj = 0; tj < gc; ++tj) {
        if (int64_t(tj) * tn + tn - 1 < int64_t(ti) * tm) continue;
        per[MUON_K_GRAM][i].push_back({i, ti, tj, 0});
        cost[MUON_K_GRAM][i].push_back(area * I.np);
        per[MUON_K_POLY][i].push_back({i, ti, tj, 0});
        cost[MUON_K_POLY][i].push_back(area * I.mp);
      }
    // update: column panels outer so neighbouring tiles share the X panel
    for (int32_t tj = 0; tj < gn; ++tj)
      for (int32_t ti = 0; ti < gt; ++ti) {
        per[MUON_K_UPDATE][i].push_back({i, ti, tj, 0});
        cost[MUON_K_UPDATE][i].push_back(area * I.mp);
      }
  }
  // Split Gram tiles (bf16 sets). A Gram launch takes about max(longest
  // tile, total work / CUs). When the longest tiles (the k loops of the
  // widest matrices) are at least twice the work per CU, each tile of k
  // loop longer than `target` stages is cut into S parts of at most
  // `target` stages (S dividing stages / 8, so each part keeps whole groups
  // of 8 stages); the parts write fp32 partial tiles, and a second pass sums
  // them in part order, one 128 x 128 quarter of a tile per workgroup, and
  // stores A (and its mirror) like an ordinary tile.
  if (bf16) {
    double work = 0;
    int32_t longest = 0;
    for (int32_t i = 0; i < n; ++i) {
      const int32_t st = P.info[i].np / 32;
      work += double(st) * per[MUON_K_GRAM][i].size();
      if (!per[MUON_K_GRAM][i].empty()) longest = std::max(longest, st);
    }
    const int32_t target = std::max<int32_t>(kSplitMinStages, static_cast<int32_t>(std::ceil(work / kNumCu)));
    int32_t parts = 0;
    std::vector<int32_t> split(n, 1);
    if (longest >= 2 * target) {
      for (int32_t i = 0; i < n; ++i) {
        const int32_t st = P.info[i].np / 32, g8 = st / 8;
        if (per[MUON_K_GRAM][i].empty() || st < 2 * target) continue;
        int32_t S = g8;
        for (int32_t d = 2; d <= g8; ++d)
          if (g8 % d == 0 && st / d <= target) {
            S = d;
            break;
          }
        if (S < 2 || S > 255) continue;
        const int64_t need = int64_t(S) * per[MUON_K_GRAM][i].size();
        if (parts + need > kSplitMaxParts) continue;
        split[i] = S;
        parts += static_cast<int32_t>(need);
      }
    }
    if (parts > 0) {
      int32_t pbase = 0;
      for (int32_t i = 0; i < n; ++i) {
        const int32_t S = split[i];
        if (S < 2) continue;
        std::vector<WorkItem> items;
        std::vector<double> costs;
        for (size_t t = 0; t < per[MUON_K_GRAM][i].size(); ++t) {
          const WorkItem w = per[MUON_K_GRAM][i][t];
          for (int32_t sp = 0; sp < S; ++sp) {
            items.push_back({w.mat, w.a, w.b, (pbase << 16) | (sp << 8) | S});
            costs.push_back(cost[MUON_K_GRAM][i][t] / S);
          }
          for (int32_t qd = 0; qd < 4; ++qd) {  // the reduce pass takes quarters of 128 x 128
            per[kGramReduce][i].push_back({w.mat, w.a, w.b, (pbase << 16) | (qd << 8) | S});
            cost[kGramReduce][i].push_back(1.0);
          }
          pbase += S;
        }
        per[MUON_K_GRAM][i] = std::move(items);
        cost[MUON_K_GRAM][i] = std::move(costs);
      }
      P.split_parts = parts;
      P.split_off = take(static_cast<size_t>(parts) * kTileM16 * kTileN16 * 4);
      P.ws_bytes = off;
    }
  }
  // Groups: matrices by update cost, longest first, onto the lighter group.
  int64_t upd_tiles = 0;
  for (int32_t i = 0; i < n; ++i) upd_tiles += static_cast<int64_t>(per[MUON_K_UPDATE][i].size());
  int32_t nonempty = 0;
  for (int32_t i = 0; i < n; ++i) nonempty += P.info[i].m > 0;
  // Concurrent groups fill the partial last wave of tiles and the launch
  // gaps of sets whose update launch is a few waves of tiles deep; on deep
  // launches they only contend for the caches (measured: GPT-2-124M, 5 waves,
  // best with three; GPT-2-350M, 18 waves, within 1 % for one to three;
  // 2048 x 8192 set, 64 waves, one group 4 % faster than two, 11 % than three).
  const int64_t waves = upd_tiles / kNumCu;
  P.ngroups = (upd_tiles < kGroupMinTiles || nonempty < 2) ? 1 : waves < 8 ? 3 : waves < 24 ? 2 : 1;
  P.ngroups = std::min<int32_t>(P.ngroups, std::min<int32_t>(nonempty, kMaxGroups));
  std::vector<int32_t> group(n, 0);
  if (P.ngroups > 1) {
    std::vector<int32_t> order(n);
    std::iota(order.begin(), order.end(), 0);
    auto work = [&](int32_t i) {
      double w = 0;
      for (int k = MUON_K_GRAM; k < MUON_K_COUNT; ++k)
        for (double c : cost[k][i]) w += c;
      return w;
    };
    std::vector<double> wi(n);
    for (int32_t i = 0; i < n; ++i) wi[i] = work(i);
    std::stable_sort(order.begin(), order.end(), [&](int32_t x, int32_t y) { return wi[x] > wi[y]; });
    std::vector<double> load(P.ngroups, 0.0);
    for (int32_t i : order) {
      int best = 0;
      for (int g = 1; g < P.ngroups; ++g)
        if (load[g] < load[best]) best = g;
      group[i] = best;
      load[best] += wi[i];
    }
  }
  // Schedules of the matrices with group[i] == g (g < 0: all of them).
  auto schedule_of = [&](int k, int g, double share) {
    double gtotal = 0;
    for (int32_t i = 0; i < n; ++i)
      if (g < 0 || group[i] == g)
        for (double c : cost[k][i]) gtotal += c;
    // chunks no larger than 1/32 of the set's total keep the XCD bins
    // balanced even for sets with a few large matrices
    const double max_cost = std::max(gtotal / share / (4.0 * kNumXcd), 1.0);
    std::vector<Chunk> chunks;
    for (int32_t i = 0; i < n; ++i)
      if ((g < 0 || group[i] == g) && !per[k][i].empty())
        add_matrix_chunks(chunks, i, per[k][i], cost[k][i], max_cost);
    return assign_xcd(std::move(chunks));
  };
  for (int k : {int(MUON_K_MOMENTUM), int(MUON_K_NORMALIZE), int(MUON_K_GRAM), int(MUON_K_POLY),
                int(MUON_K_UPDATE), kX0Scale}) {
    P.sched[k].items.clear();
    for (int g = 0; g < P.ngroups; ++g) {
      P.gbeg[g][k] = static_cast<int32_t>(P.sched[k].items.size());
      const Schedule s = schedule_of(k, g, 1.0 / P.ngroups);
      P.sched[k].items.insert(P.sched[k].items.end(), s.items.begin(), s.items.end());
    }
    P.gbeg[P.ngroups][k] = static_cast<int32_t>(P.sched[k].items.size());
    P.whole[k] = P.ngroups == 1 ? P.sched[k] : schedule_of(k, -1, 1.0);
  }
  // reduce items of split Gram tiles, on the XCDs of their parts
  {
    auto reduce_of = [&](int g) {
      std::vector<WorkItem> r;
      for (int32_t i = 0; i < n; ++i)
        if (g < 0 || group[i] == g) r.insert(r.end(), per[kGramReduce][i].begin(), per[kGramReduce][i].end());
      return r;
    };
    const int k = kGramReduce;
    P.sched[k].items.clear();
    for (int g = 0; g < P.ngroups; ++g) {
      P.gbeg[g][k] = static_cast<int32_t>(P.sched[k].items.size());
      Schedule gram_g;
      gram_g.items.assign(P.sched[MUON_K_GRAM].items.begin() + P.gbeg[g][MUON_K_GRAM],
                          P.sched[MUON_K_GRAM].items.begin() + P.gbeg[g + 1][MUON_K_GRAM]);
      const Schedule s = place_reduce(gram_g, reduce_of(g));
      P.sched[k].items.insert(P.sched[k].items.end(), s.items.begin(), s.items.end());
    }
    P.gbeg[P.ngroups][k] = static_cast<int32_t>(P.sched[k].items.size());
    P.whole[k] = P.ngroups == 1 ? P.sched[k] : place_reduce(P.whole[MUON_K_GRAM], reduce_of(-1));
  }
  // The chained schedule (bf16 sets; no split Gram tiles, whose partial
  // sums need a pass of their own)
  if (bf16 && P.split_parts == 0 && P.x0s_off >= 0 && upd_tiles < int64_t(kChainMaxWaves) * kNumCu &&
      build_chain(P, per)) {
    P.chained = true;
    P.chain_off = take(static_cast<size_t>(kNumXcd + n) * 4);
    P.ws_bytes = off;
  }
  *out = std::move(P);
  return MUON_OK;
}

}  // namespace muon

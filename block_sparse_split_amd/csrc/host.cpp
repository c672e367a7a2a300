// Host side of libsplitkv: argument checks, the chunk cost model, LPT
// placement, the in-GPU work schedule and the C entry points.
//
// Sources: arXiv abstract of "Split-KV: Efficient Context Parallelism for
// Training Diffusion Drafters" and the rit.work blog post on Split-KV,
// section "Split-KV moves queries, not keys and values" (chunk costs known
// in advance from the full query set; chunks ordered from most to least
// expensive, each placed on the least-loaded participant).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <mutex>
#include <new>
#include <queue>
#include <stdexcept>
#include <string>
#include <utility>
#include <initializer_list>
#include <vector>

#include "launch.h"
#include "schedule.h"
#include "splitkv.h"
#include "timing.h"

namespace {

thread_local std::string g_err;

struct Fail {
  skv_status code;
  std::string msg;
};

[[noreturn]] void fail(skv_status code, const std::string& msg) {
  throw Fail{code, msg};
}

void require(bool ok, const char* msg) {
  if (!ok) fail(SKV_ERR_INVALID_ARG, msg);
}

template <class F>
skv_status guarded(F&& f) {
  try {
    g_err.clear();
    f();
    return SKV_OK;
  } catch (const Fail& e) {
    g_err = e.msg;
    return e.code;
  } catch (const std::bad_alloc&) {
    g_err = "host allocation failed";
    return SKV_ERR_INVALID_ARG;
  } catch (const std::exception& e) {
    g_err = e.what();
    return SKV_ERR_INVALID_ARG;
  }
}

void check_hip(hipError_t e, const char* what) {
  if (e != hipSuccess)
    fail(SKV_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// Number of anchor blocks whose visible interval [lo_i, a_i) meets a key
// interval [t0, t1), t0 < t1.  For a non-empty interval that holds exactly
// when a_i > t0 and lo_i < t1, and every block with lo_i >= t1 also has
// a_i > t0; so the count is #{a_i > t0} - #{lo_i >= t1} over the non-empty
// intervals, two binary searches in their sorted bounds.
struct VisibleCounter {
  std::vector<int32_t> a, l;  // sorted anchors and starts of non-empty intervals
  VisibleCounter(const int32_t* anchors, const int32_t* lo, int32_t nb) {
    for (int32_t i = 0; i < nb; ++i)
      if (lo[i] < anchors[i]) {
        a.push_back(anchors[i]);
        l.push_back(lo[i]);
      }
    std::sort(a.begin(), a.end());
    std::sort(l.begin(), l.end());
  }
  int64_t operator()(int64_t t0, int64_t t1) const {
    const auto ga = std::upper_bound(a.begin(), a.end(), t0,
                                     [](int64_t x, int32_t y) { return x < y; });
    const auto gl = std::lower_bound(l.begin(), l.end(), t1,
                                     [](int32_t y, int64_t x) { return y < x; });
    return int64_t(a.end() - ga) - int64_t(l.end() - gl);
  }
};

void check_blocks(const int32_t* anchors, const int32_t* lo, int32_t nb) {
  require(nb >= 0, "nb must be >= 0");
  require(nb == 0 || (anchors && lo), "anchors/lo must not be NULL");
  for (int32_t i = 0; i < nb; ++i)
    require(lo[i] >= 0 && anchors[i] >= lo[i], "need 0 <= lo[i] <= anchors[i]");
}

void chunk_costs(const int32_t* anchors, const int32_t* lo, int32_t nb,
                 const int32_t* pos, const int32_t* len, int32_t n,
                 int32_t tile_k, int64_t* out) {
  check_blocks(anchors, lo, nb);
  require(n >= 0 && tile_k >= 1, "need n_chunks >= 0 and tile_k >= 1");
  require(n == 0 || (pos && len && out), "chunk arrays must not be NULL");
  const VisibleCounter visible(anchors, lo, nb);
  for (int32_t c = 0; c < n; ++c) {
    require(len[c] >= 1 && pos[c] >= 0, "chunk_len must be >= 1, pos >= 0");
    int64_t total = 0;
    const int64_t end = int64_t(pos[c]) + len[c];
    for (int64_t t0 = pos[c]; t0 < end; t0 += tile_k)
      total += visible(t0, std::min(t0 + tile_k, end));
    out[c] = total;
  }
}

// LPT with a binary heap keyed by (load, bin): jobs by decreasing cost
// (stable in job index), each to the least-loaded bin, lowest bin on ties.
std::vector<int32_t> lpt(const std::vector<int64_t>& cost, int32_t m,
                         std::vector<int64_t>* load_out,
                         std::vector<int32_t>* order_out = nullptr) {
  require(m >= 1, "n_bins must be >= 1");
  const int32_t n = int32_t(cost.size());
  std::vector<int32_t> order(n);
  for (int32_t i = 0; i < n; ++i) {
    require(cost[i] >= 0, "costs must be >= 0");
    order[i] = i;
  }
  std::stable_sort(order.begin(), order.end(),
                   [&](int32_t a, int32_t b) { return cost[a] > cost[b]; });
  using Entry = std::pair<int64_t, int32_t>;  // (load, bin)
  std::priority_queue<Entry, std::vector<Entry>, std::greater<Entry>> heap;
  for (int32_t b = 0; b < m; ++b) heap.push({0, b});
  std::vector<int32_t> bin(n);
  std::vector<int64_t> load(m, 0);
  for (int32_t j : order) {
    Entry e = heap.top();
    heap.pop();
    bin[j] = e.second;
    e.first += cost[j];
    load[e.second] = e.first;
    heap.push(e);
  }
  if (load_out) *load_out = std::move(load);
  if (order_out) *order_out = std::move(order);
  return bin;
}

// LPT with splitting, for work that is divisible into equal steps (the
// partials of the pieces of one unit merge exactly).  Unit u is steps[u]
// steps; a piece [k0, k1) of it costs item_cost + step_cost * (k1 - k0),
// plus extra[u] if it is the unit's first piece (k0 == 0).  Pieces are taken
// largest cost first (ties: lower unit, then lower k0), each to the
// least-loaded bin (ties: lower bin).  A piece that would lift that bin
// above the target load T is cut after the longest step prefix that fits,
// provided the piece has two or more steps and the bin has room for its
// fixed part and one step; the rest returns to the pending set and pays
// item_cost again.  Otherwise the bin takes the piece whole.  A cut leaves
// its bin within one step of T, so no bin is cut twice and there are at
// most n_units + m pieces.
struct Piece {
  int32_t unit, k0, k1, bin;
  int64_t cost;
};

struct SplitJob {
  std::vector<int64_t> extra;
  std::vector<int32_t> steps;
  int64_t item_cost = 0, step_cost = 0;
  int32_t m = 1;

  int64_t cost(int32_t u, int32_t k0) const {
    return item_cost + (k0 == 0 ? extra[u] : 0) + step_cost * (steps[u] - k0);
  }

  std::vector<Piece> pass(int64_t target, std::vector<int64_t>* load_out) const {
    struct Pending {
      int64_t cost;
      int32_t unit, k0;
      bool operator<(const Pending& o) const {  // priority_queue: top = largest
        if (cost != o.cost) return cost < o.cost;
        if (unit != o.unit) return unit > o.unit;
        return k0 > o.k0;
      }
    };
    std::priority_queue<Pending> pend;
    for (int32_t u = 0; u < int32_t(steps.size()); ++u) pend.push({cost(u, 0), u, 0});
    using Bin = std::pair<int64_t, int32_t>;  // (load, bin)
    std::priority_queue<Bin, std::vector<Bin>, std::greater<Bin>> bins;
    for (int32_t b = 0; b < m; ++b) bins.push({0, b});
    std::vector<Piece> out;
    std::vector<int64_t> load(m, 0);
    while (!pend.empty()) {
      const Pending pc = pend.top();
      pend.pop();
      Bin bin = bins.top();
      bins.pop();
      const int32_t n = steps[pc.unit];
      int32_t k_end = n;
      int64_t placed = pc.cost;
      const int64_t head = item_cost + (pc.k0 == 0 ? extra[pc.unit] : 0);
      if (bin.first + pc.cost > target && n - pc.k0 > 1 &&
          target - bin.first >= head + step_cost) {
        const int64_t room = target - bin.first;
        int64_t acc = head;
        int32_t k = pc.k0;
        while (k < n && acc + step_cost <= room) acc += step_cost, ++k;
        if (k < n) {
          k_end = k;
          placed = acc;
          pend.push({cost(pc.unit, k), pc.unit, k});
        }
      }
      out.push_back({pc.unit, pc.k0, k_end, bin.second, placed});
      bin.first += placed;
      load[bin.second] = bin.first;
      bins.push(bin);
    }
    if (load_out) *load_out = std::move(load);
    return out;
  }

  // T starts at ceil(total cost / m); cuts add fixed costs, so T is reset
  // to the mean load a pass produced plus half an item cost, until it
  // repeats (at most four passes).
  int64_t auto_target() const {
    int64_t total = 0;
    for (int32_t u = 0; u < int32_t(steps.size()); ++u) total += cost(u, 0);
    int64_t target = (total + m - 1) / m;
    for (int p = 0; p < 4; ++p) {
      int64_t placed = 0;
      for (const Piece& pc : pass(target, nullptr)) placed += pc.cost;
      const int64_t next = (placed + m - 1) / m + item_cost / 2;
      if (next == target) break;
      target = next;
    }
    return target;
  }
};

// The same placement over bins of unequal speed (work per unit time): bin
// b has speed speed[b] and its time is load / speed.  Pieces in the same
// order go to the bin of least time (ties: lower bin), with the cut rule
// above against a target time T (a bin's room is (T - time) * speed).
// With every speed equal this is the placement above.  With `scale`, unit
// u's costs (fixed part and steps alike) are multiplied by scale[u] and
// rounded: a measured correction of the cost model for that unit's work.
struct SpeedJob {
  std::vector<int64_t> extra;
  std::vector<int32_t> steps;
  std::vector<double> speed;
  std::vector<double> scale;  // per unit; empty: 1
  int64_t item_cost = 0, step_cost = 0;

  int64_t scaled(int32_t u, int64_t c) const {
    return scale.empty() ? c : int64_t(std::llround(scale[u] * double(c)));
  }
  int64_t cost(int32_t u, int32_t k0) const {
    return scaled(u, item_cost + (k0 == 0 ? extra[u] : 0) + step_cost * (steps[u] - k0));
  }

  std::vector<Piece> pass(double target, std::vector<int64_t>* load_out) const {
    struct Pending {
      int64_t cost;
      int32_t unit, k0;
      bool operator<(const Pending& o) const {
        if (cost != o.cost) return cost < o.cost;
        if (unit != o.unit) return unit > o.unit;
        return k0 > o.k0;
      }
    };
    std::priority_queue<Pending> pend;
    for (int32_t u = 0; u < int32_t(steps.size()); ++u) pend.push({cost(u, 0), u, 0});
    const int32_t m = int32_t(speed.size());
    std::vector<int64_t> load(m, 0);
    std::vector<double> time(m, 0.0);
    std::vector<Piece> out;
    while (!pend.empty()) {
      const Pending pc = pend.top();
      pend.pop();
      int32_t b = 0;
      for (int32_t j = 1; j < m; ++j)
        if (time[j] < time[b]) b = j;
      const int32_t n = steps[pc.unit];
      int32_t k_end = n;
      int64_t placed = pc.cost;
      const int64_t head = item_cost + (pc.k0 == 0 ? extra[pc.unit] : 0);
      const double room = (target - time[b]) * speed[b];
      if (time[b] + double(pc.cost) / speed[b] > target && n - pc.k0 > 1 &&
          room >= double(scaled(pc.unit, head + step_cost))) {
        int64_t acc = head;
        int32_t k = pc.k0;
        while (k < n && double(scaled(pc.unit, acc + step_cost)) <= room) acc += step_cost, ++k;
        if (k < n) {
          k_end = k;
          placed = scaled(pc.unit, acc);
          pend.push({cost(pc.unit, k), pc.unit, k});
        }
      }
      out.push_back({pc.unit, pc.k0, k_end, b, placed});
      load[b] += placed;
      time[b] = double(load[b]) / speed[b];
    }
    if (load_out) *load_out = std::move(load);
    return out;
  }

  // The target whose pass finishes its slowest bin first, among T0 (1 +
  // i / 400), i = 0 .. 16, with T0 = total cost / total speed, and the
  // automatic target below (ties: the earlier candidate).
  double best_target() const {
    double total = 0, sp = 0;
    for (int32_t u = 0; u < int32_t(steps.size()); ++u) total += double(cost(u, 0));
    for (double v : speed) sp += v;
    const double t0 = total / sp;
    double best = auto_target(), best_end = finish(best);
    for (int i = 0; i <= 16; ++i) {
      const double t = t0 * (1.0 + i / 400.0);
      const double e = finish(t);
      if (e < best_end) best = t, best_end = e;
    }
    return best;
  }

  // time of the slowest bin of a pass at target T
  double finish(double target) const {
    std::vector<int64_t> load;
    pass(target, &load);
    double e = 0;
    for (size_t b = 0; b < load.size(); ++b) e = std::max(e, double(load[b]) / speed[b]);
    return e;
  }

  // T starts at total cost / total speed and is reset to the time a pass
  // placed per unit of speed plus half an item on a bin of mean speed,
  // until it repeats (at most four passes).
  double auto_target() const {
    double total = 0, sp = 0;
    for (int32_t u = 0; u < int32_t(steps.size()); ++u) total += double(cost(u, 0));
    for (double v : speed) sp += v;
    const double half_item = 0.5 * double(item_cost) * double(speed.size()) / sp;
    double target = total / sp;
    for (int p = 0; p < 4; ++p) {
      double placed = 0;
      for (const Piece& pc : pass(target, nullptr)) placed += double(pc.cost);
      const double next = placed / sp + half_item;
      if (std::abs(next - target) <= 1e-9 * target) break;
      target = next;
    }
    return target;
  }
};

// Work shares of XCD classes of unequal total speed.  Class c (total bin
// speed S_c) should hold total * S_c / sum S.  Each class above its share
// by more than `tol` gives away units, largest first, each that still fits
// the excess (so the small ones stay to pack its own workgroups); then,
// with `steps`, the tail of its smallest remaining unit of two or more
// steps that brings the excess nearest to zero (the tail pays `tail_fixed`
// again).  Units given away go, largest first, to the class furthest below
// its share.  Returns the new class of every unit (units appended by cuts
// included) and fills *tails with (unit, steps kept) per cut.
std::vector<int32_t> share_classes(std::vector<int64_t> cost, const std::vector<int32_t>& home,
                                   const std::vector<double>& cls_speed,
                                   const std::vector<int32_t>* steps, int64_t step_cost,
                                   int64_t tail_fixed, double tol,
                                   std::vector<std::pair<int32_t, int32_t>>* tails,
                                   const std::vector<double>* unit_scale = nullptr) {
  const int32_t n_cls = int32_t(cls_speed.size());
  std::vector<int32_t> where = home;
  std::vector<double> have(n_cls, 0.0), want(n_cls, 0.0);
  double total = 0, sp = 0;
  for (size_t i = 0; i < cost.size(); ++i) have[home[i]] += double(cost[i]), total += double(cost[i]);
  for (double v : cls_speed) sp += v;
  for (int32_t c = 0; c < n_cls; ++c) want[c] = total * cls_speed[c] / sp;
  std::vector<int32_t> given;
  for (int32_t c = 0; c < n_cls; ++c) {
    double excess = have[c] - want[c];
    if (excess <= tol) continue;
    // the class's own units (tails cut for earlier classes, appended to
    // `cost`, are already given away)
    std::vector<int32_t> ids;
    for (size_t i = 0; i < home.size(); ++i)
      if (home[i] == c) ids.push_back(int32_t(i));
    std::stable_sort(ids.begin(), ids.end(), [&](int32_t a, int32_t b) { return cost[a] > cost[b]; });
    std::vector<int32_t> kept;
    for (int32_t i : ids) {
      if (double(cost[i]) <= excess) {
        given.push_back(i);
        excess -= double(cost[i]);
        have[c] -= double(cost[i]);
      } else {
        kept.push_back(i);
      }
    }
    if (steps && excess > tol) {
      for (auto it = kept.rbegin(); it != kept.rend(); ++it) {
        const int32_t u = *it, n = (*steps)[u];
        if (n < 2) continue;
        // tail of t steps: moves tail_fixed + t * step_cost, the head keeps
        // the rest (the unit's cost less t * step_cost); both scaled by the
        // unit's cost scale if there is one
        const double sc = unit_scale ? (*unit_scale)[u] : 1.0;
        const int64_t t = std::min<int64_t>(n - 1, std::max<int64_t>(
            1, std::llround((excess / sc - double(tail_fixed)) / double(step_cost))));
        const int64_t moved = std::llround(sc * double(tail_fixed + t * step_cost));
        const int64_t kept_less = std::llround(sc * double(t * step_cost));
        tails->push_back({u, int32_t(n - t)});
        cost[u] -= kept_less;
        cost.push_back(moved);
        where.push_back(c);
        given.push_back(int32_t(cost.size() - 1));
        have[c] -= double(kept_less);
        break;
      }
    }
  }
  std::stable_sort(given.begin(), given.end(), [&](int32_t a, int32_t b) { return cost[a] > cost[b]; });
  for (int32_t i : given) {
    int32_t best = -1;
    for (int32_t c = 0; c < n_cls; ++c)
      if (best < 0 || want[c] - have[c] > want[best] - have[best]) best = c;
    where[i] = best;
    have[best] += double(cost[i]);
  }
  return where;
}

// Largest load scaled to a bin of mean speed: with it, max / (total / m) - 1
// is the plan's imbalance in time.
int64_t max_time_load(const std::vector<int64_t>& load, const std::vector<double>& speed) {
  double sp = 0, worst = 0;
  for (double v : speed) sp += v;
  const double mean = sp / double(speed.size());
  for (size_t b = 0; b < load.size(); ++b) worst = std::max(worst, double(load[b]) * mean / speed[b]);
  return int64_t(std::llround(worst));
}

std::atomic<int32_t> g_cu_cache[64];

int32_t device_cu_count() {
  int dev = 0;
  check_hip(hipGetDevice(&dev), "hipGetDevice");
  if (dev >= 0 && dev < 64) {
    int32_t c = g_cu_cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  check_hip(hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev),
            "hipDeviceGetAttribute(CU count)");
  if (dev >= 0 && dev < 64) g_cu_cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

struct Tile {
  int32_t row, pos, len;
};

struct Geometry {
  int32_t nb, hq, hkv, d, G, nq, rows_per_head, qt_per_head, n_local;
};

Geometry check_problem(const skv_problem* p) {
  require(p != nullptr, "problem must not be NULL");
  require(p->nb >= 1, "nb must be >= 1");
  require(p->hq >= 1 && p->hkv >= 1 && p->hq % p->hkv == 0,
          "hq must be a positive multiple of hkv");
  const int32_t G = p->hq / p->hkv;
  if (!(G == 1 || G == 2 || G == 4 || G == 8 || G == 16))
    fail(SKV_ERR_UNSUPPORTED, "hq/hkv must be 1, 2, 4, 8 or 16");
  if (!(p->d == 64 || p->d == 128)) fail(SKV_ERR_UNSUPPORTED, "d must be 64 or 128");
  if (!(p->dtype == SKV_BF16 || p->dtype == SKV_F32))
    fail(SKV_ERR_UNSUPPORTED, "dtype must be SKV_BF16 or SKV_F32");
  require(std::isfinite(p->scale) && p->scale > 0.f, "scale must be finite and > 0");
  require(p->nb <= (1 << 22), "nb too large");
  check_blocks(p->anchors, p->lo, p->nb);
  require(p->n_chunks >= 0, "n_chunks must be >= 0");
  require(p->with_draft == 0 || p->with_draft == 1, "with_draft must be 0 or 1");
  Geometry g{};
  g.nb = p->nb;
  g.hq = p->hq;
  g.hkv = p->hkv;
  g.d = p->d;
  g.G = G;
  g.nq = p->nb * skv::kBlock;
  g.rows_per_head = g.nq * G;
  g.qt_per_head = (g.rows_per_head + skv::kQTile - 1) / skv::kQTile;
  g.n_local = 0;
  if (p->n_chunks > 0) {
    require(p->chunk_pos && p->chunk_off, "chunk_pos/chunk_off must not be NULL");
    require(p->chunk_off[0] == 0, "chunk_off[0] must be 0");
    for (int32_t c = 0; c < p->n_chunks; ++c) {
      require(p->chunk_off[c + 1] > p->chunk_off[c], "chunks must hold >= 1 key");
      require(p->chunk_pos[c] >= 0, "chunk_pos must be >= 0");
      // key positions are int32 in the schedule and the kernels
      require(int64_t(p->chunk_pos[c]) + (p->chunk_off[c + 1] - p->chunk_off[c]) <= INT32_MAX,
              "chunk_pos + chunk length must not exceed INT32_MAX");
    }
    g.n_local = p->chunk_off[p->n_chunks];
  }
  return g;
}

// Key tiles of the shard, sorted by absolute position; chunks must not
// overlap in absolute position.
std::vector<Tile> build_tiles(const skv_problem* p) {
  std::vector<Tile> tiles;
  for (int32_t c = 0; c < p->n_chunks; ++c) {
    const int32_t n = p->chunk_off[c + 1] - p->chunk_off[c];
    for (int32_t u = 0; u < n; u += skv::kTileK)
      tiles.push_back({p->chunk_off[c] + u, p->chunk_pos[c] + u,
                       std::min(skv::kTileK, n - u)});
  }
  std::stable_sort(tiles.begin(), tiles.end(),
                   [](const Tile& a, const Tile& b) { return a.pos < b.pos; });
  for (size_t t = 1; t < tiles.size(); ++t)
    require(int64_t(tiles[t - 1].pos) + tiles[t - 1].len <= tiles[t].pos,
            "chunks overlap in absolute key position");
  return tiles;
}

struct Item {
  int32_t head, qt, t0, t1, slot, flags;
  int64_t cost;
};

// Cost of GPU work items in time units, fitted to per-workgroup times
// measured on MI355X (least squares over the 256 workgroups of the 32K
// workload, 1 % rms).  A forward / dQ item pays a fixed part (loading the
// query tile, filling and draining the tile ring, writing the output) of
// about 5.5 key steps, and every key step costs the same whether one or all
// of the tile's anchor blocks see it.  A dK/dV item pays about 2.6 row
// tiles, then one unit per 64-row tile of its block range.
constexpr int64_t kStepCost = 8;
constexpr int64_t kItemCost = 44;
constexpr int64_t kKvRowCost = 5;
constexpr int64_t kKvItemCost = 13;

struct KvItem {
  int32_t head, t0, nt, dtok0, ndraft, b0, b1;
  int64_t cost;
  int32_t whole = 0;  // row tiles [w0, w1) every row of which sees all keys: w0 | w1 << 16
};

// XCD classes: workgroup w runs on XCD w % 8 (round-robin dispatch), so the
// work of kv head h is kept on workgroups w with w % n_cls == h % n_cls.
int32_t xcd_classes(int32_t hkv, int32_t n_wg) {
  int32_t c = 1;
  if (hkv % 8 == 0 || 8 % hkv == 0) c = std::min(hkv, 8);
  if (n_wg % c != 0 || n_wg < c) c = 1;
  return c;
}

// LPT per XCD class; returns per-workgroup queues in assignment order.
template <class CostOf, class HeadOf>
std::vector<std::vector<int32_t>> place(int32_t n_items, int32_t n_wg,
                                        int32_t n_cls, CostOf cost_of,
                                        HeadOf head_of, int64_t* max_bin) {
  std::vector<std::vector<int32_t>> queue(n_wg);
  *max_bin = 0;
  const int32_t per = n_wg / n_cls;
  for (int32_t c = 0; c < n_cls; ++c) {
    std::vector<int32_t> ids;
    std::vector<int64_t> costs;
    for (int32_t i = 0; i < n_items; ++i)
      if (head_of(i) % n_cls == c) {
        ids.push_back(i);
        costs.push_back(cost_of(i));
      }
    std::vector<int64_t> load;
    std::vector<int32_t> order;
    std::vector<int32_t> bin = lpt(costs, per, &load, &order);
    for (int32_t j : order) queue[c + bin[j] * n_cls].push_back(ids[j]);
    for (int64_t l : load) *max_bin = std::max(*max_bin, l);
  }
  return queue;
}

int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// xcd_speed: NULL, or [3][kXcds] relative speeds (work per unit time) of
// each XCD in the forward, dQ and dK/dV kernels; with it, queue v is
// planned at the speed of XCD v % kXcds and the kernels claim queues by the
// XCD they run on.
void build_schedule(const skv_problem* p, int32_t n_wg, const float* xcd_speed,
                    const float* cost_scale, int32_t* image, int64_t capacity,
                    skv_schedule_info* info) {
  require(info != nullptr, "info must not be NULL");
  const Geometry g = check_problem(p);
  if (n_wg == 0) n_wg = device_cu_count();
  require(n_wg >= 1 && n_wg <= 65536, "n_workgroups must be in [1, 65536]");
  const bool xcd = xcd_speed != nullptr;
  std::vector<double> spd[3];
  if (xcd) {
    require(n_wg % skv::kXcds == 0, "per-XCD speeds need n_workgroups divisible by 8");
    for (int k = 0; k < 3; ++k)
      for (int32_t x = 0; x < skv::kXcds; ++x) {
        const float v = xcd_speed[k * skv::kXcds + x];
        require(std::isfinite(v) && v > 0.f, "XCD speeds must be finite and > 0");
      }
    for (int k = 0; k < 3; ++k)
      for (int32_t b = 0; b < n_wg; ++b) spd[k].push_back(xcd_speed[k * skv::kXcds + b % skv::kXcds]);
  }
  // cost scales: [2][hkv][qt_per_head] (forward, dQ), only with speeds
  require(cost_scale == nullptr || xcd, "cost scales need per-XCD speeds");
  if (cost_scale) {
    const int64_t n_sc = 2 * int64_t(g.hkv) * g.qt_per_head;
    for (int64_t i = 0; i < n_sc; ++i)
      require(std::isfinite(cost_scale[i]) && cost_scale[i] > 0.f,
              "cost scales must be finite and > 0");
  }
  const std::vector<Tile> tiles = build_tiles(p);
  const int32_t nt = int32_t(tiles.size());
  const int32_t* A = p->anchors;
  const int32_t* L = p->lo;
  const int32_t tok_per_qt = skv::kQTile / g.G;

  // Tiles that each anchor block sees: tiles are sorted and disjoint, so
  // their ends increase too and block b's interval [lo_b, a_b) meets the
  // contiguous range [tr_lo[b], tr_hi[b]) found by two binary searches.
  std::vector<int32_t> tr_lo(g.nb, 0), tr_hi(g.nb, 0);
  for (int32_t b = 0; b < g.nb; ++b) {
    if (L[b] >= A[b]) continue;
    tr_lo[b] = int32_t(std::partition_point(tiles.begin(), tiles.end(), [&](const Tile& t) {
                         return int64_t(t.pos) + t.len <= L[b];
                       }) - tiles.begin());
    tr_hi[b] = int32_t(std::partition_point(tiles.begin(), tiles.end(), [&](const Tile& t) {
                         return t.pos < A[b];
                       }) - tiles.begin());
    tr_hi[b] = std::max(tr_hi[b], tr_lo[b]);
  }
  // Lowest and highest block that sees each tile (-1: none): blocks in
  // order, each claiming the still-unclaimed tiles of its range; a
  // next-unclaimed pointer forest makes the sweep near-linear.
  auto claim = [&](bool ascending) {
    std::vector<int32_t> who(nt, -1), next(nt + 1);
    for (int32_t t = 0; t <= nt; ++t) next[t] = t;
    auto find = [&](int32_t x) {
      while (next[x] != x) x = next[x] = next[next[x]];
      return x;
    };
    for (int32_t i = 0; i < g.nb; ++i) {
      const int32_t b = ascending ? i : g.nb - 1 - i;
      for (int32_t t = find(tr_lo[b]); t < tr_hi[b]; t = find(t)) {
        who[t] = b;
        next[t] = t + 1;
      }
    }
    return who;
  };
  const std::vector<int32_t> tile_bmin = claim(true), tile_bmax = claim(false);
  // Tiles that some anchor block of the query tile sees, per query tile:
  // the union of its blocks' ranges.
  std::vector<Item> items;
  std::vector<std::vector<int32_t>> qt_vis(g.qt_per_head);
  for (int32_t qt = 0; qt < g.qt_per_head; ++qt) {
    const int32_t b0 = qt * tok_per_qt / skv::kBlock;
    const int32_t b1 = std::min(g.nb, ((qt + 1) * tok_per_qt + skv::kBlock - 1) / skv::kBlock);
    std::vector<std::pair<int32_t, int32_t>> rng;
    for (int32_t b = b0; b < b1; ++b)
      if (tr_hi[b] > tr_lo[b]) rng.push_back({tr_lo[b], tr_hi[b]});
    std::sort(rng.begin(), rng.end());
    int32_t upto = 0;  // ranges sorted by start: emit each tile once, in order
    for (const auto& r : rng) {
      for (int32_t t = std::max(upto, r.first); t < r.second; ++t) qt_vis[qt].push_back(t);
      upto = std::max(upto, r.second);
    }
  }
  // Forward / dQ items.  Units are runs of consecutive visible tiles of one
  // (kv head, query tile); the first run of a query tile also carries its
  // draft keys.  Costs are in the time units above: kItemCost per piece plus
  // kStepCost per 64-key step (draft steps included).  Per XCD class the
  // units are placed by LPT with splitting (SplitJob) on the class's
  // workgroups; a cut falls on a tile boundary.
  struct Unit {
    int32_t head, qt, k0, k1;  // tiles qt_vis[qt][k0 .. k1-1]
    int64_t draft_cost;        // cost of the draft steps (first run only)
  };
  // units of one kv head (the same for every head)
  std::vector<Unit> head_units;
  for (int32_t qt = 0; qt < g.qt_per_head; ++qt) {
    const int32_t b0 = qt * tok_per_qt / skv::kBlock;
    const int32_t b1 = std::min(g.nb, ((qt + 1) * tok_per_qt + skv::kBlock - 1) / skv::kBlock);
    // draft keys: the query tile's anchor blocks, in steps of 64
    const int64_t dcost =
        p->with_draft
            ? kStepCost * ((int64_t(b1 - b0) * skv::kBlock + skv::kTileK - 1) / skv::kTileK)
            : 0;
    const auto& vis = qt_vis[qt];
    if (vis.empty()) {  // still one item: it writes O = 0, LSE = -inf (or the draft part)
      head_units.push_back({0, qt, 0, 0, dcost});
      continue;
    }
    bool first = true;
    for (size_t i = 0; i < vis.size();) {
      size_t j = i + 1;
      while (j < vis.size() && vis[j] == vis[j - 1] + 1) ++j;
      head_units.push_back({0, qt, int32_t(i), int32_t(j), first ? dcost : 0});
      first = false;
      i = j;
    }
  }
  std::vector<Unit> units;
  for (int32_t h = 0; h < g.hkv; ++h)
    for (Unit u : head_units) {
      u.head = h;
      units.push_back(u);
    }
  const int32_t n_cls_fwd = xcd_classes(g.hkv, n_wg);
  const int32_t per_cls = n_wg / n_cls_fwd;
  std::vector<std::vector<int32_t>> q(n_wg);
  std::vector<int64_t> wg_load(n_wg, 0);
  // Items of one plan: per-class SplitJob (the uniform plan), or with
  // per-XCD speeds the classes first get work shares by their total speed
  // (a class above its share passes units, and one unit's tail, to the
  // classes below theirs) and each class's units are placed on its
  // workgroups at their speeds.  With speeds both are built and the one
  // whose slowest workgroup finishes first (at those speeds) is kept.
  auto class_speed = [&](const std::vector<double>& speed) {
    std::vector<double> cs(n_cls_fwd, 0.0);
    for (int32_t b = 0; b < n_wg; ++b) cs[b % n_cls_fwd] += speed[b];
    return cs;
  };
  struct FwdPlan {
    std::vector<Item> items;
    std::vector<std::vector<int32_t>> q;
    std::vector<int64_t> load;
  };
  // pieces of `units` placed per class: where[u] is unit u's class, and
  // the class's workgroups run at `speed` (nullptr: uniform SplitJob)
  auto plan_fwd = [&](const std::vector<Unit>& us, const std::vector<int32_t>& where,
                      const std::vector<double>* speed, const std::vector<double>* uscale) {
    FwdPlan pl;
    pl.q.assign(n_wg, {});
    pl.load.assign(n_wg, 0);
    for (int32_t cls = 0; cls < n_cls_fwd; ++cls) {
      std::vector<int32_t> ids;
      std::vector<int64_t> extra;
      std::vector<int32_t> steps;
      for (int32_t ui = 0; ui < int32_t(us.size()); ++ui)
        if (where[ui] == cls) {
          ids.push_back(ui);
          extra.push_back(us[ui].draft_cost);
          steps.push_back(us[ui].k1 - us[ui].k0);
        }
      std::vector<int64_t> load;
      std::vector<Piece> pieces;
      if (speed || uscale) {
        SpeedJob job;
        job.item_cost = kItemCost;
        job.step_cost = kStepCost;
        job.extra = extra;
        job.steps = steps;
        for (int32_t b = cls; b < n_wg; b += n_cls_fwd)
          job.speed.push_back(speed ? (*speed)[b] : 1.0);
        if (uscale)
          for (int32_t ui : ids) job.scale.push_back((*uscale)[ui]);
        pieces = job.pass(job.best_target(), &load);
      } else {
        SplitJob job;
        job.item_cost = kItemCost;
        job.step_cost = kStepCost;
        job.m = per_cls;
        job.extra = extra;
        job.steps = steps;
        pieces = job.pass(job.auto_target(), &load);
      }
      for (const Piece& pc : pieces) {
        const Unit& u = us[ids[pc.unit]];
        const auto& vis = qt_vis[u.qt];
        Item it{u.head, u.qt, pc.k1 > pc.k0 ? vis[u.k0 + pc.k0] : 0,
                pc.k1 > pc.k0 ? vis[u.k0 + pc.k1 - 1] + 1 : 0, -1, 0, pc.cost};
        if (pc.k0 == 0 && p->with_draft && u.draft_cost > 0) it.flags |= skv::kItemDraft;
        pl.q[cls + pc.bin * n_cls_fwd].push_back(int32_t(pl.items.size()));
        pl.items.push_back(it);
      }
      for (int32_t j = 0; j < int32_t(load.size()); ++j) pl.load[cls + j * n_cls_fwd] = load[j];
    }
    return pl;
  };
  auto slowest = [&](const std::vector<int64_t>& load, const std::vector<double>& speed) {
    double t = 0;
    for (int32_t b = 0; b < n_wg; ++b) t = std::max(t, double(load[b]) / speed[b]);
    return t;
  };
  std::vector<int32_t> home_of(units.size());
  for (size_t ui = 0; ui < units.size(); ++ui) home_of[ui] = units[ui].head % n_cls_fwd;
  // the uniform plan, or with speeds the per-XCD plan if its slowest
  // workgroup finishes first at those speeds; with cost scales (kernel k's
  // slice of cost_scale) both plans place the scaled costs
  auto best_plan = [&](const std::vector<double>* speed, int k) {
    std::vector<double> usc;
    if (cost_scale)
      for (const Unit& u : units)
        usc.push_back(cost_scale[(int64_t(k) * g.hkv + u.head) * g.qt_per_head + u.qt]);
    FwdPlan chosen = plan_fwd(units, home_of, nullptr, cost_scale ? &usc : nullptr);
    if (speed == nullptr) return chosen;
    std::vector<int64_t> ucost;
    std::vector<int32_t> usteps;
    for (size_t ui = 0; ui < units.size(); ++ui) {
      const Unit& u = units[ui];
      const int64_t c = kItemCost + u.draft_cost + kStepCost * (u.k1 - u.k0);
      ucost.push_back(cost_scale ? std::llround(usc[ui] * double(c)) : c);
      usteps.push_back(u.k1 - u.k0);
    }
    std::vector<std::pair<int32_t, int32_t>> tails;
    const std::vector<int32_t> where =
        share_classes(ucost, home_of, class_speed(*speed), &usteps, kStepCost, kItemCost,
                      double(kItemCost), &tails, cost_scale ? &usc : nullptr);
    std::vector<Unit> us = units;
    for (const auto& [u, keep] : tails) {  // unit u keeps its first `keep` steps
      Unit tail = us[u];
      tail.k0 = us[u].k0 + keep;
      tail.draft_cost = 0;
      us[u].k1 = us[u].k0 + keep;
      us.push_back(tail);
      if (cost_scale) usc.push_back(usc[u]);
    }
    FwdPlan sp = plan_fwd(us, where, speed, cost_scale ? &usc : nullptr);
    if (slowest(sp.load, *speed) < slowest(chosen.load, *speed)) chosen = std::move(sp);
    return chosen;
  };
  // query tiles with several items write partial slots, merged afterwards:
  // one split record (S_WORDS) per such tile; returns the slot count
  auto assign_slots = [&](std::vector<Item>& its, std::vector<int32_t>& rec) {
    int32_t slots = 0;
    std::vector<std::vector<int32_t>> of(int64_t(g.hkv) * g.qt_per_head);
    for (int32_t i = 0; i < int32_t(its.size()); ++i)
      of[int64_t(its[i].head) * g.qt_per_head + its[i].qt].push_back(i);
    for (int64_t k = 0; k < int64_t(of.size()); ++k) {
      if (of[k].size() < 2) continue;
      rec.insert(rec.end(), {int32_t(k / g.qt_per_head), int32_t(k % g.qt_per_head), slots,
                             int32_t(of[k].size())});
      for (int32_t i : of[k]) its[i].slot = slots++;
    }
    return slots;
  };
  {
    FwdPlan chosen = best_plan(xcd ? &spd[0] : nullptr, 0);
    items = std::move(chosen.items);
    q = std::move(chosen.q);
    wg_load = std::move(chosen.load);
  }
  std::vector<int32_t> split_rec;
  const int32_t n_slots = assign_slots(items, split_rec);
  // dQ runs the forward's items from the forward's queues, except with
  // per-XCD speeds: the two kernels' XCD speeds differ, so dQ then gets a
  // plan of its own (its own cuts, queues, partial slots and split records)
  const bool dq_own = xcd;
  FwdPlan dq;
  std::vector<int32_t> dq_split_rec;
  int32_t dq_slots = n_slots;
  if (dq_own) {
    dq = best_plan(&spd[1], 1);
    dq_slots = assign_slots(dq.items, dq_split_rec);
  }
  // dK/dV items: two consecutive tiles per item (one if a lone tile is
  // left), plus draft groups of 128 draft tokens.  An item walks the 64-row
  // tiles of its anchor blocks [b0, b1).
  auto kv_cost = [&](int32_t b0, int32_t b1) {
    const int64_t rows = int64_t(std::max(0, b1 - b0)) * skv::kBlock * g.G;
    return kKvItemCost + kKvRowCost * ((rows + skv::kTileK - 1) / skv::kTileK);
  };
  // The context items of every kv head cover the same tile pairs: build
  // them once.
  std::vector<KvItem> pairs;
  for (int32_t t = 0; t < nt; t += 2) {
    const int32_t n2 = std::min(2, nt - t);
    int32_t bmin = g.nb, bmax = -1;
    for (int32_t u = t; u < t + n2; ++u)
      if (tile_bmin[u] >= 0) {
        bmin = std::min(bmin, tile_bmin[u]);
        bmax = std::max(bmax, tile_bmax[u]);
      }
    if (bmax < 0) {  // no block sees these keys: zero gradients
      bmin = 0;
      bmax = -1;
    }
    pairs.push_back({0, t, n2, 0, 0, bmin, bmax + 1, kv_cost(bmin, bmax + 1)});
    // row tiles inside [b0, b1) whose anchor blocks all see every key of
    // the item: they need neither the per-row intervals nor masks
    const int64_t kmin = tiles[t].pos;
    const int64_t kend = int64_t(tiles[t + n2 - 1].pos) + tiles[t + n2 - 1].len;
    const int64_t rpb = int64_t(skv::kBlock) * g.G;  // rows per anchor block
    const int64_t r_begin = int64_t(bmin) * rpb, r_end = int64_t(bmax + 1) * rpb;
    const int64_t n_rt = (std::max<int64_t>(0, r_end - r_begin) + skv::kTileK - 1) / skv::kTileK;
    auto whole = [&](int64_t rt) {
      const int64_t r0 = r_begin + rt * skv::kTileK;
      if (r0 + skv::kTileK > r_end) return false;
      for (int64_t b = r0 / rpb; b <= (r0 + skv::kTileK - 1) / rpb; ++b)
        if (!(L[b] <= kmin && A[b] >= kend)) return false;
      return true;
    };
    // the kernels decode the high half with a signed shift: 15 bits
    if (n_rt < (int64_t(1) << 15)) {
      int64_t w0 = 0;
      while (w0 < n_rt && !whole(w0)) ++w0;
      int64_t w1 = w0;
      while (w1 < n_rt && whole(w1)) ++w1;
      if (w1 > w0) pairs.back().whole = int32_t(w0 | (w1 << 16));
    }
  }
  std::vector<KvItem> kv;
  for (int32_t h = 0; h < g.hkv; ++h) {
    for (KvItem it : pairs) {
      it.head = h;
      kv.push_back(it);
    }
    if (p->with_draft) {
      for (int32_t tok = 0; tok < g.nq; tok += skv::kKvGroup) {
        const int32_t nd = std::min(skv::kKvGroup, g.nq - tok);
        const int32_t b0 = tok / skv::kBlock, b1 = (tok + nd) / skv::kBlock;
        kv.push_back({h, 0, 0, tok, nd, b0, b1, kv_cost(b0, b1)});
      }
    }
  }
  const int32_t n_cls = n_cls_fwd;
  int64_t max_bin = 0, kv_max_bin = 0;
  for (int64_t l : wg_load) max_bin = std::max(max_bin, l);
  std::vector<std::vector<int32_t>> kq;
  if (xcd) {
    max_bin = max_time_load(wg_load, spd[0]);
    std::vector<int64_t> cost, load(n_wg, 0);
    std::vector<int32_t> home;
    for (const KvItem& k : kv) {
      cost.push_back(k.cost);
      home.push_back(k.head % n_cls);
    }
    const std::vector<int32_t> where = share_classes(
        cost, home, class_speed(spd[2]), nullptr, 0, 0, double(kKvItemCost), nullptr);
    // LPT per class at the workgroups' speeds: largest first (stable), each
    // to the class's workgroup of least time (ties: lower workgroup)
    std::vector<std::vector<int32_t>> kq_sp(n_wg);
    std::vector<int32_t> order(kv.size());
    for (size_t i = 0; i < kv.size(); ++i) order[i] = int32_t(i);
    std::stable_sort(order.begin(), order.end(),
                     [&](int32_t a, int32_t b) { return cost[a] > cost[b]; });
    std::vector<double> time(n_wg, 0.0);
    for (int32_t i : order) {
      int32_t best = -1;
      for (int32_t b = where[i]; b < n_wg; b += n_cls)
        if (best < 0 || time[b] < time[best]) best = b;
      kq_sp[best].push_back(i);
      load[best] += cost[i];
      time[best] = double(load[best]) / spd[2][best];
    }
    // keep the plain per-class plan if it finishes first at these speeds
    std::vector<int64_t> load_u;
    int64_t unused = 0;
    kq = place(int32_t(kv.size()), n_wg, n_cls, [&](int32_t i) { return kv[i].cost; },
               [&](int32_t i) { return kv[i].head; }, &unused);
    load_u.assign(n_wg, 0);
    for (int32_t b = 0; b < n_wg; ++b)
      for (int32_t i : kq[b]) load_u[b] += kv[i].cost;
    if (slowest(load, spd[2]) < slowest(load_u, spd[2])) kq = std::move(kq_sp);
    else load = load_u;
    kv_max_bin = max_time_load(load, spd[2]);
  } else {
    kq = place(int32_t(kv.size()), n_wg, n_cls, [&](int32_t i) { return kv[i].cost; },
               [&](int32_t i) { return kv[i].head; }, &kv_max_bin);
  }
  int64_t kv_total = 0;
  for (const auto& k : kv) kv_total += k.cost;
  int64_t item_total = 0;
  for (const auto& it : items) item_total += it.cost;
  int64_t dq_total = item_total, dq_max_bin = max_bin;
  if (dq_own) {
    dq_total = 0;
    for (const auto& it : dq.items) dq_total += it.cost;
    dq_max_bin = max_time_load(dq.load, spd[1]);
  }

  // Steps of an item that every row of its query tile sees whole: the
  // first maximal run of full-length tiles inside [max lo, min anchor) of
  // the tile's anchor blocks.  Packed as s0 | s1 << 16 in item steps (the
  // draft steps come first and are never whole); empty if the item has
  // 2^15 steps or more (the kernels decode the high half with a signed
  // shift).
  auto whole_steps = [&](const Item& it) -> int32_t {
    const int32_t b0 = it.qt * tok_per_qt / skv::kBlock;
    const int32_t b1 = std::min(g.nb, ((it.qt + 1) * tok_per_qt + skv::kBlock - 1) / skv::kBlock);
    if (b1 <= b0) return 0;
    int64_t lo_max = INT64_MIN, a_min = INT64_MAX;
    for (int32_t b = b0; b < b1; ++b) {
      lo_max = std::max<int64_t>(lo_max, L[b]);
      a_min = std::min<int64_t>(a_min, A[b]);
    }
    const int32_t nd = (it.flags & skv::kItemDraft)
                           ? ((b1 - b0) * skv::kBlock + skv::kTileK - 1) / skv::kTileK
                           : 0;
    if (int64_t(nd) + (it.t1 - it.t0) >= (int64_t(1) << 15)) return 0;
    auto whole = [&](int32_t t) {
      return tiles[t].len == skv::kTileK && tiles[t].pos >= lo_max &&
             int64_t(tiles[t].pos) + skv::kTileK <= a_min;
    };
    int32_t t = it.t0;
    while (t < it.t1 && !whole(t)) ++t;
    int32_t e = t;
    while (e < it.t1 && whole(e)) ++e;
    if (e == t) return 0;
    return (nd + (t - it.t0)) | ((nd + (e - it.t0)) << 16);
  };

  // Image layout.
  using namespace skv;
  int64_t off = H_WORDS;
  const int64_t off_anchors = off; off += g.nb;
  const int64_t off_lo = off; off += g.nb;
  const int64_t off_tiles = off; off += int64_t(nt) * T_WORDS;
  const int64_t off_items = off; off += int64_t(items.size()) * I_WORDS;
  const int64_t off_qoff = off; off += n_wg + 1;
  const int64_t off_queue = off; off += int64_t(items.size());
  const int64_t off_split = off; off += int64_t(split_rec.size());
  const int64_t off_kv = off; off += int64_t(kv.size()) * K_WORDS;
  const int64_t off_kvqoff = off; off += n_wg + 1;
  const int64_t off_kvqueue = off; off += int64_t(kv.size());
  const int64_t off_kvsuf = off; off += int64_t(kv.size());
  // dQ sections: the forward's unless dQ has a plan of its own
  int64_t off_dq_items = off_items, off_dq_qoff = off_qoff, off_dq_queue = off_queue,
          off_dq_split = off_split;
  if (dq_own) {
    off_dq_items = off; off += int64_t(dq.items.size()) * I_WORDS;
    off_dq_qoff = off; off += n_wg + 1;
    off_dq_queue = off; off += int64_t(dq.items.size());
    off_dq_split = off; off += int64_t(dq_split_rec.size());
  }
  const int64_t words = off;
  require(words < (int64_t(1) << 31), "schedule image too large");

  const int64_t rows_slot = skv::kQTile;
  // XCD mode: the per-XCD queue counters sit in the last kXcdCounterBytes
  // (forward: 8 words; backward: 8 for dQ, then 8 for dK/dV)
  const int64_t fwd_ws = align_up(int64_t(n_slots) * rows_slot * g.d * 4, 256) +
                         align_up(int64_t(n_slots) * rows_slot * 4, 256) +
                         (xcd ? kXcdCounterBytes : 0);
  // per-row statistics: per kv head, its rows plus kStatPad padding rows;
  // then dQ's partial slots, the dK/dV claim counters (one per queue) and,
  // in XCD mode, the per-XCD counters
  const int64_t bwd_ws = 4 * align_up(int64_t(g.hkv) * (g.rows_per_head + skv::kStatPad) * 4, 256) +
                         align_up(int64_t(dq_slots) * rows_slot * g.d * 4, 256) +
                         align_up(int64_t(n_wg) * 4, 256) + (xcd ? kXcdCounterBytes : 0);
  std::memset(info, 0, sizeof(*info));
  info->words = words;
  info->n_workgroups = n_wg;
  info->n_tiles = nt;
  info->n_qtiles = g.qt_per_head * g.hkv;
  info->n_items = int32_t(items.size());
  info->n_split_qtiles = int32_t(split_rec.size() / S_WORDS);
  info->n_partial_slots = n_slots;
  info->n_kv_items = int32_t(kv.size());
  info->fwd_workspace_bytes = fwd_ws;
  info->bwd_workspace_bytes = bwd_ws;
  info->item_cost_total = item_total;
  info->item_cost_max_bin = max_bin;
  info->kv_cost_total = kv_total;
  info->kv_cost_max_bin = kv_max_bin;
  info->xcd_mode = xcd ? 1 : 0;
  info->n_dq_items = dq_own ? int32_t(dq.items.size()) : info->n_items;
  info->n_dq_split_qtiles = dq_own ? int32_t(dq_split_rec.size() / S_WORDS) : info->n_split_qtiles;
  info->n_dq_partial_slots = dq_slots;
  info->dq_cost_total = dq_total;
  info->dq_cost_max_bin = dq_max_bin;
  info->nb = g.nb;
  info->hq = g.hq;
  info->hkv = g.hkv;
  info->d = g.d;
  info->n_local = g.n_local;
  info->with_draft = p->with_draft;
  if (image == nullptr) return;
  if (capacity < words)
    fail(SKV_ERR_WORKSPACE, "schedule image too small: need " +
                                std::to_string(words) + " int32 words");
  std::memset(image, 0, size_t(words) * 4);
  int32_t* H = image;
  H[H_MAGIC] = kMagic;
  H[H_VERSION] = kVersion;
  H[H_NB] = g.nb;
  H[H_HQ] = g.hq;
  H[H_HKV] = g.hkv;
  H[H_D] = g.d;
  H[H_G] = g.G;
  H[H_NLOCAL] = g.n_local;
  H[H_DRAFT] = p->with_draft;
  H[H_NTILES] = nt;
  H[H_QT_PER_HEAD] = g.qt_per_head;
  H[H_NITEMS] = int32_t(items.size());
  H[H_NWG] = n_wg;
  H[H_NSPLIT] = info->n_split_qtiles;
  H[H_NSLOTS] = n_slots;
  H[H_NKV] = int32_t(kv.size());
  H[H_OFF_ANCHORS] = int32_t(off_anchors);
  H[H_OFF_LO] = int32_t(off_lo);
  H[H_OFF_TILES] = int32_t(off_tiles);
  H[H_OFF_ITEMS] = int32_t(off_items);
  H[H_OFF_QOFF] = int32_t(off_qoff);
  H[H_OFF_QUEUE] = int32_t(off_queue);
  H[H_OFF_SPLIT] = int32_t(off_split);
  H[H_OFF_KV] = int32_t(off_kv);
  H[H_OFF_KVQOFF] = int32_t(off_kvqoff);
  H[H_OFF_KVQUEUE] = int32_t(off_kvqueue);
  H[H_NCLASS] = n_cls;
  H[H_XCD] = xcd ? 1 : 0;
  H[H_OFF_DQ_ITEMS] = int32_t(off_dq_items);
  H[H_OFF_DQ_QOFF] = int32_t(off_dq_qoff);
  H[H_OFF_DQ_QUEUE] = int32_t(off_dq_queue);
  H[H_OFF_DQ_SPLIT] = int32_t(off_dq_split);
  H[H_OFF_KVSUF] = int32_t(off_kvsuf);
  std::memcpy(image + off_anchors, A, size_t(g.nb) * 4);
  std::memcpy(image + off_lo, L, size_t(g.nb) * 4);
  for (int32_t t = 0; t < nt; ++t) {
    int32_t* w = image + off_tiles + int64_t(t) * T_WORDS;
    w[T_ROW] = tiles[t].row;
    w[T_POS] = tiles[t].pos;
    w[T_LEN] = tiles[t].len;
  }
  auto write_plan = [&](const std::vector<Item>& its, const std::vector<std::vector<int32_t>>& qs,
                        const std::vector<int32_t>& rec, int64_t o_items, int64_t o_qoff,
                        int64_t o_queue, int64_t o_split) {
    for (size_t i = 0; i < its.size(); ++i) {
      int32_t* w = image + o_items + int64_t(i) * I_WORDS;
      w[I_HEAD] = its[i].head;
      w[I_QT] = its[i].qt;
      w[I_T0] = its[i].t0;
      w[I_T1] = its[i].t1;
      w[I_SLOT] = its[i].slot;
      w[I_FLAGS] = its[i].flags;
      w[I_COST] = int32_t(std::min<int64_t>(its[i].cost, INT32_MAX));
      w[I_WHOLE] = whole_steps(its[i]);
    }
    int32_t at = 0;
    for (int32_t w = 0; w < n_wg; ++w) {
      image[o_qoff + w] = at;
      for (int32_t it : qs[w]) image[o_queue + at++] = it;
    }
    image[o_qoff + n_wg] = at;
    std::copy(rec.begin(), rec.end(), image + o_split);
  };
  write_plan(items, q, split_rec, off_items, off_qoff, off_queue, off_split);
  if (dq_own)
    write_plan(dq.items, dq.q, dq_split_rec, off_dq_items, off_dq_qoff, off_dq_queue,
               off_dq_split);
  for (size_t i = 0; i < kv.size(); ++i) {
    int32_t* w = image + off_kv + int64_t(i) * K_WORDS;
    w[K_HEAD] = kv[i].head;
    w[K_T0] = kv[i].t0;
    w[K_NT] = kv[i].nt;
    w[K_DTOK0] = kv[i].dtok0;
    w[K_NDRAFT] = kv[i].ndraft;
    w[K_B0] = kv[i].b0;
    w[K_B1] = kv[i].b1;
    w[K_COST] = int32_t(std::min<int64_t>(kv[i].cost, INT32_MAX));
    w[K_WHOLE] = kv[i].whole;
  }
  int32_t pos = 0;
  for (int32_t w = 0; w < n_wg; ++w) {
    image[off_kvqoff + w] = pos;
    for (int32_t it : kq[w]) image[off_kvqueue + pos++] = it;
    // summed cost of each position and the rest of its queue
    int64_t rest = 0;
    for (int32_t j = pos - 1; j >= image[off_kvqoff + w]; --j) {
      rest += kv[image[off_kvqueue + j]].cost;
      image[off_kvsuf + j] = int32_t(std::min<int64_t>(rest, INT32_MAX));
    }
  }
  image[off_kvqoff + n_wg] = pos;
}

// Tensors are read and written with 16-byte vector accesses (and the
// workspace with float4 stores); LSE arrays with 4-byte ones.
void require_aligned(std::initializer_list<const void*> ptrs, uintptr_t align,
                     const char* what) {
  for (const void* q : ptrs)
    if (q != nullptr && (reinterpret_cast<uintptr_t>(q) & (align - 1)) != 0)
      fail(SKV_ERR_INVALID_ARG, std::string(what) + " must be " + std::to_string(align) +
                                    "-byte aligned");
}

void check_info(const skv_problem* p, const skv_schedule_info* info,
                const int32_t* schedule) {
  const Geometry g = check_problem(p);
  require(info != nullptr && schedule != nullptr, "info/schedule must not be NULL");
  require(info->nb == g.nb && info->hq == g.hq && info->hkv == g.hkv &&
              info->d == g.d && info->n_local == g.n_local &&
              info->with_draft == p->with_draft,
          "schedule was built for a different problem");
  require(info->n_workgroups >= 1, "schedule has no workgroups");
}

size_t elem_size(int32_t dt) { return dt == SKV_BF16 ? 2 : 4; }

}  // namespace

extern "C" {

const char* skv_last_error(void) { return g_err.c_str(); }

int32_t skv_abi_version(void) { return SKV_ABI_VERSION; }

skv_status skv_chunk_costs(const int32_t* anchors, const int32_t* lo, int32_t nb,
                           const int32_t* chunk_pos, const int32_t* chunk_len,
                           int32_t n_chunks, int32_t tile_k, int64_t* out_cost) {
  return guarded([&] {
    chunk_costs(anchors, lo, nb, chunk_pos, chunk_len, n_chunks, tile_k, out_cost);
  });
}

skv_status skv_plan_lpt_costs(const int64_t* cost, int32_t n, int32_t n_bins,
                              int32_t* out_bin, int64_t* out_load) {
  return guarded([&] {
    require(n >= 0, "n must be >= 0");
    require(n == 0 || (cost && out_bin), "cost/out_bin must not be NULL");
    require(n_bins >= 1, "n_bins must be >= 1");
    std::vector<int64_t> c(cost, cost + n);
    std::vector<int64_t> load;
    std::vector<int32_t> bin = lpt(c, n_bins, &load);
    if (n) std::memcpy(out_bin, bin.data(), size_t(n) * 4);
    if (out_load) std::memcpy(out_load, load.data(), size_t(n_bins) * 8);
  });
}

skv_status skv_plan_lpt(const int32_t* anchors, const int32_t* lo, int32_t nb,
                        const int32_t* chunk_pos, const int32_t* chunk_len,
                        int32_t n_chunks, int32_t tile_k, int32_t n_bins,
                        int32_t* out_bin, int64_t* out_cost, int64_t* out_load) {
  return guarded([&] {
    require(n_bins >= 1, "n_bins must be >= 1");
    require(n_chunks >= 0, "n_chunks must be >= 0");
    require(n_chunks == 0 || out_bin, "out_bin must not be NULL");
    std::vector<int64_t> c(size_t(std::max(n_chunks, 0)));
    chunk_costs(anchors, lo, nb, chunk_pos, chunk_len, n_chunks, tile_k, c.data());
    std::vector<int64_t> load;
    std::vector<int32_t> bin = lpt(c, n_bins, &load);
    if (n_chunks) std::memcpy(out_bin, bin.data(), size_t(n_chunks) * 4);
    if (out_cost && n_chunks) std::memcpy(out_cost, c.data(), size_t(n_chunks) * 8);
    if (out_load) std::memcpy(out_load, load.data(), size_t(n_bins) * 8);
  });
}

skv_status skv_plan_lpt_split(const int64_t* extra, const int32_t* steps, int32_t n_units,
                              int64_t item_cost, int64_t step_cost, int32_t n_bins,
                              int64_t target, int32_t capacity, int32_t* out_pieces,
                              int64_t* out_cost, int32_t* out_n, int64_t* out_target,
                              int64_t* out_load) {
  return guarded([&] {
    require(n_units >= 0, "n_units must be >= 0");
    require(n_units == 0 || (extra && steps), "extra/steps must not be NULL");
    require(n_bins >= 1, "n_bins must be >= 1");
    require(item_cost >= 0 && step_cost >= 0, "item_cost/step_cost must be >= 0");
    require(target >= 0, "target must be >= 0 (0 = automatic)");
    require(capacity >= 0 && out_n && (capacity == 0 || (out_pieces && out_cost)),
            "out_pieces/out_cost/out_n must not be NULL");
    SplitJob job;
    job.item_cost = item_cost;
    job.step_cost = step_cost;
    job.m = n_bins;
    __int128 total = 0;
    for (int32_t u = 0; u < n_units; ++u) {
      require(extra[u] >= 0 && steps[u] >= 0, "extra/steps must be >= 0");
      total += __int128(item_cost) + extra[u] + __int128(step_cost) * steps[u];
      require(total <= (__int128(1) << 60), "total cost must not exceed 2^60");
      job.extra.push_back(extra[u]);
      job.steps.push_back(steps[u]);
    }
    const int64_t t = target == 0 ? job.auto_target() : target;
    std::vector<int64_t> load;
    const std::vector<Piece> pieces = job.pass(t, &load);
    *out_n = int32_t(pieces.size());
    if (out_target) *out_target = t;
    if (out_load) std::memcpy(out_load, load.data(), size_t(n_bins) * 8);
    if (int64_t(pieces.size()) > capacity)
      fail(SKV_ERR_WORKSPACE, "capacity too small: need " + std::to_string(pieces.size()) +
                                  " pieces");
    for (size_t i = 0; i < pieces.size(); ++i) {
      int32_t* w = out_pieces + 4 * i;
      w[0] = pieces[i].unit;
      w[1] = pieces[i].k0;
      w[2] = pieces[i].k1;
      w[3] = pieces[i].bin;
      out_cost[i] = pieces[i].cost;
    }
  });
}

skv_status skv_schedule_build(const skv_problem* p, int32_t n_workgroups,
                              int32_t* image, int64_t capacity_words,
                              skv_schedule_info* info) {
  return guarded([&] {
    build_schedule(p, n_workgroups, nullptr, nullptr, image, capacity_words, info);
  });
}

skv_status skv_schedule_build_xcd(const skv_problem* p, int32_t n_workgroups,
                                  const float* xcd_speed, const float* cost_scale,
                                  int32_t* image, int64_t capacity_words,
                                  skv_schedule_info* info) {
  return guarded([&] {
    require(xcd_speed != nullptr, "xcd_speed must not be NULL");
    build_schedule(p, n_workgroups, xcd_speed, cost_scale, image, capacity_words, info);
  });
}

skv_status skv_attn_fwd_partial(const skv_problem* p, const skv_schedule_info* info,
                                const int32_t* schedule, const void* Q, const void* K,
                                const void* V, const void* Kd, const void* Vd, void* O,
                                int32_t o_dtype, float* LSE, void* workspace,
                                int64_t workspace_bytes, void* stream) {
  return guarded([&] {
    check_info(p, info, schedule);
    require(Q && O && LSE, "Q/O/LSE must not be NULL");
    require(info->n_local == 0 || (K && V), "K/V must not be NULL");
    require(!p->with_draft || (Kd && Vd), "Kd/Vd must not be NULL with with_draft");
    require_aligned({Q, K, V, Kd, Vd, O, workspace}, 16, "Q/K/V/Kd/Vd/O/workspace");
    require_aligned({LSE}, 4, "LSE");
    if (!(o_dtype == SKV_BF16 || o_dtype == SKV_F32))
      fail(SKV_ERR_UNSUPPORTED, "o_dtype must be SKV_BF16 or SKV_F32");
    if (info->fwd_workspace_bytes > 0) {
      if (workspace_bytes < info->fwd_workspace_bytes || !workspace)
        fail(SKV_ERR_WORKSPACE, "workspace too small: need " +
                                    std::to_string(info->fwd_workspace_bytes) + " bytes");
    }
    skv::FwdArgs a{};
    a.sched = schedule;
    a.Q = Q; a.K = K; a.V = V; a.Kd = Kd; a.Vd = Vd;
    a.O = O; a.LSE = LSE;
    a.o_bf16 = o_dtype == SKV_BF16;
    a.dtype_bf16 = p->dtype == SKV_BF16;
    a.hq = p->hq; a.hkv = p->hkv; a.d = p->d; a.nb = p->nb;
    a.n_local = info->n_local;
    a.scale = p->scale;
    a.n_wg = info->n_workgroups;
    a.n_split = info->n_split_qtiles;
    a.n_slots = info->n_partial_slots;
    a.ws_O = static_cast<float*>(workspace);
    a.ws_LSE = workspace ? reinterpret_cast<float*>(
                   static_cast<char*>(workspace) +
                   align_up(int64_t(info->n_partial_slots) * skv::kQTile * p->d * 4, 256))
                         : nullptr;
    if (info->xcd_mode) {
      require(info->n_workgroups % skv::kXcds == 0 &&
                  info->fwd_workspace_bytes >= skv::kXcdCounterBytes,
              "inconsistent schedule info (per-XCD queues)");
      a.xcd_count = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) +
                                                info->fwd_workspace_bytes -
                                                skv::kXcdCounterBytes);
    }
    bool fits = true;
    a.wg_clock = a.dtype_bf16 ? skv::wg_clock_region(skv::kClockFwd, a.n_wg, &fits) : nullptr;
    require(fits, "per-workgroup clock buffer too small for this schedule's workgroups");
    check_hip(skv::launch_fwd(a, static_cast<hipStream_t>(stream)), "forward launch");
  });
}

skv_status skv_attn_fwd_partial_noalloc(const skv_problem* p, const skv_schedule_info* info,
                                        const int32_t* schedule, const void* Q, const void* K,
                                        const void* V, const void* Kd, const void* Vd, void* O,
                                        int32_t o_dtype, float* LSE, void* stream) {
  void* scratch = nullptr;
  const skv_status st = guarded([&] {
    require(info != nullptr, "info must not be NULL");
    if (info->fwd_workspace_bytes > skv::kNoAllocScratchBytes)
      fail(SKV_ERR_WORKSPACE,
           "this schedule needs " + std::to_string(info->fwd_workspace_bytes) +
               " bytes of forward workspace; the allocation-free forward holds at most " +
               std::to_string(skv::kNoAllocScratchBytes) +
               " (use skv_attn_fwd_partial with a workspace)");
    check_hip(skv::noalloc_scratch(&scratch), "hipGetSymbolAddress(scratch)");
  });
  if (st != SKV_OK) return st;
  return skv_attn_fwd_partial(p, info, schedule, Q, K, V, Kd, Vd, O, o_dtype, LSE, scratch,
                              skv::kNoAllocScratchBytes, stream);
}

skv_status skv_merge_lse(int32_t n_parts, int64_t rows, int32_t d, const void* O_parts,
                         int32_t in_dtype, const float* LSE_parts, void* O_out,
                         int32_t out_dtype, float* LSE_out, void* stream) {
  return guarded([&] {
    require(n_parts >= 1 && rows >= 0, "need n_parts >= 1 and rows >= 0");
    if (!(d == 64 || d == 128)) fail(SKV_ERR_UNSUPPORTED, "d must be 64 or 128");
    if (!((in_dtype == SKV_BF16 || in_dtype == SKV_F32) &&
          (out_dtype == SKV_BF16 || out_dtype == SKV_F32)))
      fail(SKV_ERR_UNSUPPORTED, "dtypes must be SKV_BF16 or SKV_F32");
    if (rows == 0) return;
    require(O_parts && LSE_parts && O_out && LSE_out, "pointers must not be NULL");
    require_aligned({O_parts, O_out}, 16, "O_parts/O_out");
    require_aligned({LSE_parts, LSE_out}, 4, "LSE_parts/LSE_out");
    const char* ob = static_cast<const char*>(O_out);
    const char* ib = static_cast<const char*>(O_parts);
    const int64_t out_bytes = rows * d * int64_t(elem_size(out_dtype));
    const int64_t in_bytes = int64_t(n_parts) * rows * d * int64_t(elem_size(in_dtype));
    require(ob + out_bytes <= ib || ib + in_bytes <= ob, "O_out must not alias O_parts");
    check_hip(skv::launch_merge(n_parts, rows, d, O_parts, in_dtype == SKV_BF16, LSE_parts,
                                O_out, out_dtype == SKV_BF16, LSE_out,
                                static_cast<hipStream_t>(stream)),
              "merge launch");
  });
}

skv_status skv_dq_finalize(int32_t n_parts, int64_t elems, const float* parts,
                           int64_t part_stride, void* dq_out, int32_t out_dtype,
                           void* stream) {
  return guarded([&] {
    require(n_parts >= 1 && elems >= 0, "need n_parts >= 1 and elems >= 0");
    if (!(out_dtype == SKV_BF16 || out_dtype == SKV_F32))
      fail(SKV_ERR_UNSUPPORTED, "out_dtype must be SKV_BF16 or SKV_F32");
    require(n_parts == 1 || (part_stride >= elems && part_stride % 4 == 0),
            "part_stride must be >= elems and a multiple of 4");
    if (elems == 0) return;
    require(parts && dq_out, "pointers must not be NULL");
    require_aligned({parts, dq_out}, 16, "parts/dq_out");
    const int64_t span = (int64_t(n_parts) - 1) * (n_parts > 1 ? part_stride : 0) + elems;
    require(span <= INT64_MAX / 4, "shares too large");
    const char* ib = reinterpret_cast<const char*>(parts);
    const char* ob = static_cast<const char*>(dq_out);
    const int64_t out_bytes = elems * int64_t(elem_size(out_dtype));
    const bool disjoint = ob + out_bytes <= ib || ib + span * 4 <= ob;
    require(disjoint || (ob == ib && out_dtype == SKV_F32),
            "dq_out must not overlap the shares (an fp32 dq_out may be share 0 itself)");
    check_hip(skv::launch_dq_finalize(n_parts, elems, n_parts > 1 ? part_stride : 0, parts,
                                      dq_out, out_dtype == SKV_BF16,
                                      static_cast<hipStream_t>(stream)),
              "dq_finalize launch");
  });
}

skv_status skv_attn_bwd(const skv_problem* p, const skv_schedule_info* info,
                        const int32_t* schedule, const void* Q, const void* K,
                        const void* V, const void* Kd, const void* Vd, const void* O,
                        const void* dO, const float* LSE, float* dQ, void* dK, void* dV,
                        void* dKd, void* dVd, int32_t grad_dtype, void* workspace,
                        int64_t workspace_bytes, void* stream) {
  return guarded([&] {
    check_info(p, info, schedule);
    require(Q && O && dO && LSE && dQ, "Q/O/dO/LSE/dQ must not be NULL");
    require(info->n_local == 0 || (K && V && dK && dV), "K/V/dK/dV must not be NULL");
    require(!p->with_draft || (Kd && Vd && dKd && dVd),
            "Kd/Vd/dKd/dVd must not be NULL with with_draft");
    require_aligned({Q, K, V, Kd, Vd, O, dO, dQ, dK, dV, dKd, dVd, workspace}, 16,
                    "Q/K/V/Kd/Vd/O/dO/dQ/dK/dV/dKd/dVd/workspace");
    require_aligned({LSE}, 4, "LSE");
    if (!(grad_dtype == SKV_BF16 || grad_dtype == SKV_F32))
      fail(SKV_ERR_UNSUPPORTED, "grad_dtype must be SKV_BF16 or SKV_F32");
    if (p->dtype != SKV_BF16) fail(SKV_ERR_UNSUPPORTED, "the backward takes bf16 inputs only");
    if (workspace_bytes < info->bwd_workspace_bytes || !workspace)
      fail(SKV_ERR_WORKSPACE, "workspace too small: need " +
                                  std::to_string(info->bwd_workspace_bytes) + " bytes");
    skv::BwdArgs a{};
    a.sched = schedule;
    a.Q = Q; a.K = K; a.V = V; a.Kd = Kd; a.Vd = Vd; a.O = O; a.dO = dO; a.LSE = LSE;
    a.dQ = dQ; a.dK = dK; a.dV = dV; a.dKd = dKd; a.dVd = dVd;
    a.grad_bf16 = grad_dtype == SKV_BF16;
    a.dtype_bf16 = p->dtype == SKV_BF16;
    a.hq = p->hq; a.hkv = p->hkv; a.d = p->d; a.nb = p->nb;
    a.n_local = info->n_local;
    a.scale = p->scale;
    a.n_wg = info->n_workgroups;
    a.n_split = info->n_dq_split_qtiles;
    a.n_slots = info->n_dq_partial_slots;
    a.with_draft = p->with_draft;
    const int64_t stat_bytes = align_up(
        int64_t(p->hkv) * (int64_t(p->nb) * 16 * (p->hq / p->hkv) + skv::kStatPad) * 4, 256);
    a.ws_nD = static_cast<float*>(workspace);
    a.ws_L2 = reinterpret_cast<float*>(static_cast<char*>(workspace) + stat_bytes);
    a.ws_LO = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + 2 * stat_bytes);
    a.ws_HI = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + 3 * stat_bytes);
    a.ws_dQ = reinterpret_cast<float*>(static_cast<char*>(workspace) + 4 * stat_bytes);
    a.stat_words = stat_bytes / 4;
    const int64_t dq_bytes =
        align_up(int64_t(info->n_dq_partial_slots) * skv::kQTile * p->d * 4, 256);
    const int64_t front_bytes = align_up(int64_t(info->n_workgroups) * 4, 256);
    require(info->bwd_workspace_bytes >= 4 * stat_bytes + dq_bytes + front_bytes +
                                             (info->xcd_mode ? skv::kXcdCounterBytes : 0),
            "inconsistent schedule info (backward workspace)");
    a.kv_front = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + 4 * stat_bytes +
                                             dq_bytes);
    if (info->xcd_mode) {
      require(info->n_workgroups % skv::kXcds == 0 &&
                  info->bwd_workspace_bytes >= 4 * stat_bytes + skv::kXcdCounterBytes,
              "inconsistent schedule info (per-XCD queues)");
      a.xcd_count = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) +
                                                info->bwd_workspace_bytes -
                                                skv::kXcdCounterBytes);
    }
    bool fits = true;
    a.wg_clock_dq = skv::wg_clock_region(skv::kClockDq, a.n_wg, &fits);
    a.wg_clock_kv = skv::wg_clock_region(skv::kClockKv, a.n_wg, &fits);
    require(fits, "per-workgroup clock buffer too small for this schedule's workgroups");
    check_hip(skv::launch_bwd(a, static_cast<hipStream_t>(stream)), "backward launch");
  });
}

}  // extern "C"

// Host-side work plan of the forward kernel: which key-block range of which
// query tile each workgroup processes, so that concurrently resident
// workgroups finish together.
//
// A workgroup's cost is proportional to the key blocks it streams. Under the
// causal mask the tiles of late query rows stream up to N/BN blocks and early
// ones a few, and without it N/BM tiles of equal cost may fill the resident
// slots unevenly; either way the last workgroups can leave most of the chip
// idle. The planner splits the heaviest tiles into up to sixteen contiguous
// key ranges (up to 64 for a single query tile; the block merge of the online
// softmax, "Exercises" of the interactive explainer "The Flash Attention",
// combines their partial states exactly), orders all items longest first,
// and keeps the split threshold
// whose simulated schedule finishes earliest. The simulation follows each
// compute unit: it holds up to `occ` workgroups, its throughput depends on
// how many are resident (a lone workgroup keeps a compute unit well under
// full use), and a freed slot takes the next workgroup in dispatch order.
// Plans depend only on the tiles' block counts and the device's compute
// units and occupancy, and are cached (a bounded, least-recently-used cache).
#include "fa_internal.h"

#include <algorithm>
#include <cmath>
#include <functional>
#include <list>
#include <map>
#include <memory>
#include <mutex>
#include <queue>
#include <tuple>
#include <vector>

namespace fa {

int fwd_tile_blocks(int N, int Nk, int t, bool causal, int bn) {
  long long kend = Nk;
  if (causal) kend = std::min<long long>(Nk, (long long)(t + 1) * FWD_BM + (long long)Nk - N);
  if (kend <= 0) return 0;
  return (int)((kend + bn - 1) / bn);
}

bool head_sequential(long long items, int cus, int occ) {
  if (cus <= 0 || occ <= 0) return false;
  return items >= 16ll * cus * occ;
}

bool fwd_pair_tiles(int N, int Nk, int d, int BH, bool causal, int cus, int occ) {
  const long long ntiles = ((long long)N + FWD_BM - 1) / FWD_BM;
  if (!causal || ntiles < 2 || Nk <= 0 || d <= 0 || BH <= 0 || cus <= 0 || occ <= 0) return false;
  if (2ll * Nk * d * 2 < FWD_L2_BYTES) return false;
  return (long long)BH * ((ntiles + 1) / 2) >= (long long)cus * occ;
}

bool fwd_head_sequential(int N, int Nk, int d, int BH, bool causal, int cus, int occ) {
  if (N <= 0 || BH <= 0 || BH % 8 != 0) return false;
  if (fwd_pair_tiles(N, Nk, d, BH, causal, cus, occ)) return false;
  return head_sequential((long long)BH * ((N + FWD_BM - 1) / FWD_BM), cus, occ);
}

namespace {

// Costs in units of one streamed key block of a workgroup on a full compute
// unit (about 1.5 us), from per-workgroup timestamps of the kernel: every
// item pays its prologue (Q and the first K/V block in flight, about 3 us);
// a split part also stores its partial state (about 2.5 us), shares in the
// merge (5 to 9 us for the last arrival) and streams its blocks a little
// slower.
constexpr double kItemCost = 2.0;
constexpr double kSplitCost = 7.0;
// The last part of a split tile to arrive reads every part's partial state:
// kSplitCost covers up to FWD_MAX_PARTS parts, and each part beyond them adds
// about this much.
constexpr double kMergePerPart = 0.15;
// A split plan is used only if it shortens the simulated schedule this much.
// On grids of several waves of workgroups the simulation still promises
// 7-20% where the device gains nothing, so only a clearly under-filled grid
// (few heads, long rows) is split.
constexpr double kMinGain = 0.75;
// Throughput of a compute unit with k resident workgroups, relative to a
// full one (per-block times measured on the forward: about 1.25 us for a
// workgroup alone, 1.5 us each with three resident).
double cu_throughput(int k, int occ) {
  if (k >= occ) return 1.0;
  return std::min(1.0, 0.40 + 0.35 * (k - 1));
}
// With this many waves of workgroups the tail is already small.
constexpr int kMaxWaves = 8;

struct Item {
  int tile, part, nparts;
  double cost;
};

// Schedule of items x BH workgroups (dispatch order: item-major, heads
// inner) on `cus` compute units of `occ` slots; returns the makespan in
// block-times of a full compute unit's workgroup.
double simulate(const std::vector<Item>& items, int BH, int cus, int occ) {
  const long long total = (long long)items.size() * BH;
  long long next = 0;
  auto cost_of = [&](long long w) { return items[(size_t)(w / BH)].cost; };
  struct Unit {
    std::vector<double> rem;  // remaining work of resident workgroups
    double t = 0.0;           // time the remaining work refers to
  };
  std::vector<Unit> unit((size_t)cus);
  // Each resident workgroup advances at cu_throughput(k) * occ / k
  // block-times per unit time (1 each with the compute unit full).
  auto rate = [&](const Unit& u) {
    const int k = (int)u.rem.size();
    return k ? cu_throughput(k, occ) * occ / k : 0.0;
  };
  typedef std::pair<double, int> Ev;  // (time of the next completion, unit)
  std::priority_queue<Ev, std::vector<Ev>, std::greater<Ev>> ev;
  auto schedule = [&](int c) {
    Unit& u = unit[(size_t)c];
    if (u.rem.empty()) return;
    const double mn = *std::min_element(u.rem.begin(), u.rem.end());
    ev.push({u.t + mn / rate(u), c});
  };
  for (int s = 0; s < occ && next < total; ++s)
    for (int c = 0; c < cus && next < total; ++c) unit[(size_t)c].rem.push_back(cost_of(next++));
  for (int c = 0; c < cus; ++c) schedule(c);
  double end = 0.0;
  while (!ev.empty()) {
    const Ev e = ev.top();
    ev.pop();
    Unit& u = unit[(size_t)e.second];
    if (u.rem.empty()) continue;
    const double mn = *std::min_element(u.rem.begin(), u.rem.end());
    if (std::abs(u.t + mn / rate(u) - e.first) > 1e-9 * (1.0 + e.first)) continue;  // stale
    const double done = mn;  // every resident workgroup advanced by this much
    for (double& r : u.rem) r -= done;
    u.t = e.first;
    end = std::max(end, u.t);
    for (size_t i = 0; i < u.rem.size();)
      if (u.rem[i] <= 1e-12) {
        u.rem[i] = u.rem.back();
        u.rem.pop_back();
      } else {
        ++i;
      }
    while ((int)u.rem.size() < occ && next < total) u.rem.push_back(cost_of(next++));
    schedule(e.second);
  }
  return end;
}

int max_parts(int ntiles) { return ntiles == 1 ? FWD_MAX_PARTS_ONE_TILE : FWD_MAX_PARTS; }

// Items for split threshold T (blocks): tiles above T are cut into
// min(max_parts, ceil(nb / T)) parts. T <= 0 means no split.
std::vector<Item> make_items(int N, int Nk, bool causal, int bn, int T) {
  const int ntiles = (N + FWD_BM - 1) / FWD_BM;
  std::vector<Item> items;
  for (int t = 0; t < ntiles; ++t) {
    const int nb = fwd_tile_blocks(N, Nk, t, causal, bn);
    int np = 1;
    if (T > 0 && nb > T) np = std::min(max_parts(ntiles), (nb + T - 1) / T);
    for (int part = 0; part < np; ++part) {
      const int blocks = (part + 1) * nb / np - part * nb / np;
      items.push_back({t, part, np,
                       blocks + kItemCost +
                           (np > 1 ? kSplitCost + kMergePerPart * std::max(0, np - FWD_MAX_PARTS)
                                   : 0.0)});
    }
  }
  std::stable_sort(items.begin(), items.end(), [](const Item& a, const Item& b) {
    if (a.cost != b.cost) return a.cost > b.cost;
    if (a.tile != b.tile) return a.tile > b.tile;
    return a.part < b.part;
  });
  return items;
}

std::shared_ptr<FwdPlan> build_plan(int N, int Nk, int BH, bool causal, int bn, int cus, int occ) {
  auto plan = std::make_shared<FwdPlan>();
  plan->nitems = 0;
  plan->nslots = 0;
  const int ntiles = (N + FWD_BM - 1) / FWD_BM;
  const long long slots = (long long)cus * occ;
  if (cus <= 0 || occ <= 0 || ntiles > 0xfff || (long long)BH * ntiles >= kMaxWaves * slots ||
      (long long)BH * ntiles > FWD_COUNTERS)
    return plan;
  const int nbmax = fwd_tile_blocks(N, Nk, ntiles - 1, causal, bn);
  const double base = simulate(make_items(N, Nk, causal, bn, 0), BH, cus, occ);
  double best = base * kMinGain;
  int bestT = 0;
  static const double fracs[] = {0.875, 0.75, 0.625, 0.5, 0.4, 1.0 / 3.0, 0.25, 0.125, 0.0625,
                                 1.0 / 24, 1.0 / 32, 1.0 / 48, 1.0 / 64};
  for (double f : fracs) {
    if (ntiles > 1 && f < 0.0625) break;  // at most 16 parts when several tiles split
    const int T = std::max(4, (int)(nbmax * f + 0.999));
    if (T >= nbmax) continue;
    const std::vector<Item> items = make_items(N, Nk, causal, bn, T);
    if ((int)items.size() > FWD_PLAN_MAX) continue;
    const double ms = simulate(items, BH, cus, occ);
    if (ms < best) {
      best = ms;
      bestT = T;
    }
  }
  if (bestT == 0) return plan;
  const std::vector<Item> items = make_items(N, Nk, causal, bn, bestT);
  // Slot bases: consecutive per split tile, in tile order.
  std::vector<int> base_of(ntiles, 0);
  int nslots = 0;
  for (int t = 0; t < ntiles; ++t) {
    const int nb = fwd_tile_blocks(N, Nk, t, causal, bn);
    const int np = (nb > bestT) ? std::min(max_parts(ntiles), (nb + bestT - 1) / bestT) : 1;
    base_of[t] = nslots;
    if (np > 1) nslots += np;
  }
  if (nslots >= (1 << 11) || ntiles > (1 << 9)) return plan;
  for (size_t i = 0; i < items.size(); ++i) {
    const Item& it = items[i];
    const int sb = (it.nparts > 1) ? base_of[it.tile] : 0;
    plan->item[i] = (uint32_t)it.tile | ((uint32_t)it.part << 9) | ((uint32_t)(it.nparts - 1) << 15) |
                    ((uint32_t)sb << 21);
  }
  plan->nitems = (int)items.size();
  plan->nslots = nslots;
  return plan;
}

}  // namespace

namespace {

// Plan cache: keyed on what a plan depends on (the block count of every query
// tile, the heads, compute units and occupancy), least recently used first
// out once FWD_PLAN_CACHE_MAX plans are held.
typedef std::tuple<int, int, int, std::vector<int>> PlanKey;
struct PlanCache {
  std::mutex mu;
  std::list<PlanKey> order;  // most recently used first
  std::map<PlanKey, std::pair<std::shared_ptr<const FwdPlan>, std::list<PlanKey>::iterator>> map;
};
PlanCache& plan_cache() {
  static PlanCache c;
  return c;
}

}  // namespace

std::shared_ptr<const FwdPlan> fwd_plan(int N, int Nk, int BH, bool causal, int bn, int cus,
                                        int occ) {
  const int ntiles = (N + FWD_BM - 1) / FWD_BM;
  std::vector<int> nbs;
  if (ntiles <= 0xfff) {
    nbs.reserve((size_t)ntiles);
    for (int t = 0; t < ntiles; ++t) nbs.push_back(fwd_tile_blocks(N, Nk, t, causal, bn));
  } else {
    nbs.push_back(-ntiles);  // too many tiles to plan for: never split
  }
  PlanKey key(BH, cus, occ, std::move(nbs));
  PlanCache& c = plan_cache();
  {
    std::lock_guard<std::mutex> lock(c.mu);
    auto it = c.map.find(key);
    if (it != c.map.end()) {
      c.order.splice(c.order.begin(), c.order, it->second.second);
      return it->second.first;
    }
  }
  // Built outside the lock (a pure function of the key); a concurrent
  // builder of the same key keeps whichever entry landed first.
  std::shared_ptr<const FwdPlan> plan = build_plan(N, Nk, BH, causal, bn, cus, occ);
  std::lock_guard<std::mutex> lock(c.mu);
  auto it = c.map.find(key);
  if (it != c.map.end()) {
    c.order.splice(c.order.begin(), c.order, it->second.second);
    return it->second.first;
  }
  c.order.push_front(key);
  c.map.emplace(std::move(key), std::make_pair(plan, c.order.begin()));
  while (c.map.size() > FWD_PLAN_CACHE_MAX) {
    c.map.erase(c.order.back());
    c.order.pop_back();
  }
  return plan;
}

size_t fwd_plan_cache_size() {
  PlanCache& c = plan_cache();
  std::lock_guard<std::mutex> lock(c.mu);
  return c.map.size();
}

FwdWorkspace fwd_workspace_layout(const FwdPlan& plan, int BH, int N, int d) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  FwdWorkspace w{0, 0, 0, 0};
  if (plan.nitems == 0) return w;
  (void)N;
  const size_t slots = (size_t)BH * plan.nslots;
  w.counters = 0;
  w.part_ml = up(sizeof(int) * (size_t)FWD_COUNTERS);
  w.part_o = w.part_ml + up(sizeof(float) * slots * FWD_ML_FLOATS);
  w.total = w.part_o + up(sizeof(float) * slots * FWD_BM * (size_t)d);
  return w;
}

}  // namespace fa

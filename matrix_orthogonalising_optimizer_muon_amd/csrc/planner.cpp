// Owner assignment: which rank updates which matrix, from measured per-shape costs.
//
// DMuon summary (gist.science), section 2.3 "compute-aware load balancing": update costs
// differ widely between matrix shapes, so a naive (round-robin) assignment leaves
// stragglers; the system measures, at initialisation, the time of several batch sizes (and
// kernel schemes) for every distinct shape and assigns owners to minimise the predicted
// makespan (the largest load over the owner ranks) with a mixed-integer linear program,
// falling back to a greedy heuristic when the search space is too large. DMuon
// announcement (agentren.cn), improvement 3: matrices grouped by shape, one full update per
// shape measured, then the slowest owner's completion time minimised.
//
// Model (the pages give no formula): a rank that owns k matrices of shape s updates them
// as one batched launch sequence in c_s(k) milliseconds, c_s read off the measured points
// (batch sizes b_1 < ... < b_P with times t_1 .. t_P): c_s(0) = 0, linear from the origin
// to the first point, linear between points, and past the last point extended with the
// last segment's slope (the last point's mean rate when only one point is given). The
// load of a rank is the sum of c_s over the shapes it owns; the makespan is the largest
// load. Matrices of one shape are interchangeable, so a plan is a count x[s][r] per shape
// and rank with sum_r x[s][r] = n_s.
//
// Exact search: depth-first over shapes (largest total cost first) and, within a shape,
// over ranks, choosing x[s][r]; ranks holding the same counts of every earlier shape are
// interchangeable, so along a run of such ranks the counts are taken non-increasing. A branch is cut when its
// lower bound reaches the best makespan found: the largest load so far, or the average of
// (loads so far + the least total cost the remaining matrices can be split into over the
// ranks left for them), the latter from a per-shape table of minimum split costs. The
// greedy plan (below) is the first incumbent. The optimum found equals the MILP's; with
// more than max_nodes nodes the search stops and the best plan so far is returned, marked
// not proven optimal (the pages' greedy fallback, improved by what the search found).
//
// Greedy: shapes in decreasing per-matrix cost at full batch, each matrix to the rank
// whose load grows to the smallest value; then single matrices move off the most loaded
// rank while that lowers the makespan.
#include "../../include/muon.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <limits>
#include <numeric>
#include <vector>

namespace {

struct Shape {
  int n = 0;                  // matrices of this shape in the list
  std::vector<double> b, t;   // measured batch sizes and times
  double cost(int k) const {
    if (k <= 0) return 0.0;
    const size_t P = b.size();
    if (k <= b[0]) return t[0] * k / b[0];
    for (size_t i = 1; i < P; ++i)
      if (k <= b[i]) return t[i - 1] + (t[i] - t[i - 1]) * (k - b[i - 1]) / (b[i] - b[i - 1]);
    const double slope = P >= 2 ? (t[P - 1] - t[P - 2]) / (b[P - 1] - b[P - 2]) : t[0] / b[0];
    return t[P - 1] + slope * (k - b[P - 1]);
  }
};

constexpr double kInf = std::numeric_limits<double>::infinity();

struct Search {
  const std::vector<Shape>& sh;
  std::vector<int> order;                      // shapes, largest total cost first
  int R;
  int64_t max_nodes, nodes = 0;
  bool aborted = false;
  // minsplit[s][j][k]: least total cost of k matrices of shape s over at most j ranks
  std::vector<std::vector<std::vector<double>>> minsplit;
  std::vector<double> rest_min;                // least total cost of shapes order[t..]
  std::vector<double> load;
  std::vector<std::vector<int>> x;             // x[s][r]
  double best = kInf;
  std::vector<std::vector<int>> best_x;

  Search(const std::vector<Shape>& shapes, int ranks, int64_t limit) : sh(shapes), R(ranks), max_nodes(limit) {}

  void prepare() {
    const int S = static_cast<int>(sh.size());
    order.resize(S);
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(),
                     [&](int a, int b) { return sh[a].cost(sh[a].n) > sh[b].cost(sh[b].n); });
    minsplit.assign(S, {});
    for (int s = 0; s < S; ++s) {
      const int n = sh[s].n;
      const int J = std::min(R, std::max(n, 1));
      auto& m = minsplit[s];
      m.assign(R + 1, std::vector<double>(n + 1, kInf));
      for (int j = 0; j <= R; ++j) m[j][0] = 0.0;
      if (static_cast<double>(J) * n * n <= 2e7) {
        for (int j = 1; j <= R; ++j) {
          if (j > J) { m[j] = m[J]; continue; }
          for (int k = 1; k <= n; ++k) {
            double v = kInf;
            for (int q = 0; q <= k; ++q) v = std::min(v, sh[s].cost(q) + m[j - 1][k - q]);
            m[j][k] = v;
          }
        }
      } else {
        // too large for the exact table: k matrices cost at least k times the best
        // per-matrix rate of any batch size, however they are split
        double rate = kInf;
        for (int k = 1; k <= n; ++k) rate = std::min(rate, sh[s].cost(k) / k);
        for (int j = 1; j <= R; ++j)
          for (int k = 1; k <= n; ++k) m[j][k] = rate * k;
      }
    }
    rest_min.assign(S + 1, 0.0);
    for (int t = S - 1; t >= 0; --t) rest_min[t] = rest_min[t + 1] + minsplit[order[t]][R][sh[order[t]].n];
    load.assign(R, 0.0);
    x.assign(S, std::vector<int>(R, 0));
  }

  // Ranks r..R-1 still to receive matrices of the current shape (left of them); after it,
  // shapes order[t+1..].
  void dfs(int t, int r, int left) {
    if (aborted) return;
    if (++nodes > max_nodes) { aborted = true; return; }
    const int S = static_cast<int>(order.size());
    if (t == S) {
      const double mk = *std::max_element(load.begin(), load.end());
      if (mk < best) { best = mk; best_x = x; }
      return;
    }
    const int s = order[t];
    if (r == R) {
      if (left != 0) return;
      dfs(t + 1, 0, t + 1 < S ? sh[order[t + 1]].n : 0);
      return;
    }
    // lower bound
    double mx = 0.0, sum = 0.0;
    for (int q = 0; q < R; ++q) { mx = std::max(mx, load[q]); sum += load[q]; }
    const double lb = std::max(mx, (sum + minsplit[s][R - r][left] + rest_min[t + 1]) / R);
    if (lb >= best * (1.0 - 1e-12)) return;
    const bool same = r > 0 && interchangeable(t, r);
    if (r == R - 1) {   // the last rank takes what is left
      if (same && left > x[s][r - 1]) return;   // the swapped plan is searched instead
      x[s][r] = left;
      load[r] += sh[s].cost(left);
      dfs(t, R, 0);
      load[r] -= sh[s].cost(left);
      x[s][r] = 0;
      return;
    }
    // Symmetry: ranks r-1 and r holding the same counts of every earlier shape are
    // interchangeable, so their counts of this shape are taken non-increasing.
    int cap = left;
    if (same) cap = std::min(cap, x[s][r - 1]);
    for (int k = cap; k >= 0; --k) {
      x[s][r] = k;
      const double c = sh[s].cost(k);
      load[r] += c;
      dfs(t, r + 1, left - k);
      load[r] -= c;
      x[s][r] = 0;
      if (aborted) return;
    }
  }

  bool interchangeable(int t, int r) const {
    for (int u = 0; u < t; ++u)
      if (x[order[u]][r] != x[order[u]][r - 1]) return false;
    return true;
  }
};

double plan_loads(const std::vector<Shape>& sh, const std::vector<std::vector<int>>& x, int R,
                  std::vector<double>& load) {
  load.assign(R, 0.0);
  for (size_t s = 0; s < sh.size(); ++s)
    for (int r = 0; r < R; ++r) load[r] += sh[s].cost(x[s][r]);
  return R > 0 ? *std::max_element(load.begin(), load.end()) : 0.0;
}

std::vector<std::vector<int>> greedy(const std::vector<Shape>& sh, int R) {
  const int S = static_cast<int>(sh.size());
  std::vector<int> order(S);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) {
    const double ca = sh[a].n ? sh[a].cost(sh[a].n) / sh[a].n : 0.0;
    const double cb = sh[b].n ? sh[b].cost(sh[b].n) / sh[b].n : 0.0;
    return ca > cb;
  });
  std::vector<std::vector<int>> x(S, std::vector<int>(R, 0));
  std::vector<double> load(R, 0.0);
  for (int s : order) {
    for (int i = 0; i < sh[s].n; ++i) {
      int bestr = 0;
      double bestv = kInf;
      for (int r = 0; r < R; ++r) {
        const double v = load[r] - sh[s].cost(x[s][r]) + sh[s].cost(x[s][r] + 1);
        if (v < bestv) { bestv = v; bestr = r; }
      }
      load[bestr] = bestv;
      ++x[s][bestr];
    }
  }
  // single-matrix moves off the most loaded rank while the makespan drops
  for (int iter = 0; iter < 100000 && R > 1; ++iter) {
    std::vector<double> ld;
    const double mk = plan_loads(sh, x, R, ld);
    std::vector<int> idx(R);
    std::iota(idx.begin(), idx.end(), 0);
    std::partial_sort(idx.begin(), idx.begin() + std::min(R, 3), idx.end(),
                      [&](int a, int b) { return ld[a] > ld[b] || (ld[a] == ld[b] && a < b); });
    const int top = idx[0];
    double best_mk = mk;
    int bs = -1, br = -1;
    for (int s = 0; s < S; ++s) {
      if (x[s][top] == 0) continue;
      const double dtop = sh[s].cost(x[s][top] - 1) - sh[s].cost(x[s][top]);
      for (int r = 0; r < R; ++r) {
        if (r == top) continue;
        const double nr = ld[r] - sh[s].cost(x[s][r]) + sh[s].cost(x[s][r] + 1);
        // the largest load of the other ranks: the second largest overall unless it is r
        const double others = R < 3 ? 0.0 : ld[idx[1] != r ? idx[1] : idx[2]];
        const double m2 = std::max(std::max(ld[top] + dtop, nr), R >= 3 ? others : 0.0);
        if (m2 < best_mk * (1.0 - 1e-12)) { best_mk = m2; bs = s; br = r; }
      }
    }
    if (bs < 0) break;
    --x[bs][top];
    ++x[bs][br];
  }
  return x;
}

}  // namespace

extern "C" int muon_owner_plan(const int32_t* shape_of, int count, const muon_shape_cost* shapes, int n_shapes,
                               int ranks, uint32_t flags, int64_t max_nodes, int32_t* owner, double* rank_ms,
                               double* makespan_ms, int32_t* optimal) {
  try {
    if (count < 0 || n_shapes < 0 || (count > 0 && (!shape_of || !owner)) || (n_shapes > 0 && !shapes))
      return MUON_ERR_ARG;
    if (ranks < 1 || ranks > MUON_MAX_PLAN_RANKS || (flags & ~MUON_PLAN_GREEDY) != 0 || max_nodes < 0)
      return MUON_ERR_ARG;
    std::vector<Shape> sh(n_shapes);
    for (int s = 0; s < n_shapes; ++s) {
      const muon_shape_cost& c = shapes[s];
      if (c.n_points < 1 || c.n_points > MUON_MAX_COST_POINTS) return MUON_ERR_ARG;
      for (int i = 0; i < c.n_points; ++i) {
        if (c.batch[i] < 1 || !std::isfinite(c.ms[i]) || c.ms[i] < 0.0) return MUON_ERR_ARG;
        if (i > 0 && c.batch[i] <= c.batch[i - 1]) return MUON_ERR_ARG;
        sh[s].b.push_back(c.batch[i]);
        sh[s].t.push_back(c.ms[i]);
      }
    }
    for (int i = 0; i < count; ++i) {
      if (shape_of[i] < 0 || shape_of[i] >= n_shapes) return MUON_ERR_ARG;
      ++sh[shape_of[i]].n;
    }
    std::vector<std::vector<int>> x = greedy(sh, ranks);
    std::vector<double> load;
    double mk = plan_loads(sh, x, ranks, load);
    bool proven = false;
    if (!(flags & MUON_PLAN_GREEDY)) {
      Search se(sh, ranks, max_nodes == 0 ? MUON_PLAN_DEFAULT_NODES : max_nodes);
      se.prepare();
      se.best = mk * (1.0 + 1e-12);   // the greedy plan is the incumbent; only strictly better plans replace it
      se.dfs(0, 0, n_shapes > 0 ? sh[se.order[0]].n : 0);
      if (!se.best_x.empty()) {
        x = se.best_x;
        mk = plan_loads(sh, x, ranks, load);
      }
      proven = !se.aborted;
    }
    // Matrices of each shape are dealt to ranks in list order, each to the rank with the
    // largest share of its count still open (ties to the lower rank), which spreads a
    // rank's matrices of one shape over the list (e.g. over layers).
    std::vector<std::vector<int>> given(n_shapes, std::vector<int>(ranks, 0));
    for (int i = 0; i < count; ++i) {
      const int s = shape_of[i];
      int br = -1;
      double bv = -1.0;
      for (int r = 0; r < ranks; ++r) {
        if (given[s][r] >= x[s][r]) continue;
        const double v = static_cast<double>(x[s][r] - given[s][r]) / x[s][r];
        if (v > bv) { bv = v; br = r; }
      }
      owner[i] = br;
      ++given[s][br];
    }
    if (rank_ms)
      for (int r = 0; r < ranks; ++r) rank_ms[r] = load[r];
    if (makespan_ms) *makespan_ms = mk;
    if (optimal) *optimal = proven ? 1 : 0;
    return MUON_OK;
  } catch (...) {
    return MUON_ERR_HIP;
  }
}

// C-ABI front end of the Muon update library: argument validation, the shape-adaptive
// plan (same-shape groups, plain vs Gram NS, tile size) and the stage sequence each
// group enqueues on the caller's stream.
//
// Sources: MuonX article (Baidu Baige, damodev.csdn.net), section 3.2 (Gram NS: segments
// 2+2+1, Gram matrix rebuilt after rounds 2 and 4, transform restarted per segment; 10
// long + 5 square products become 6 long + 11 square); DMuon summary (gist.science),
// sections 2.2 (symmetric Gram product, batching of similar shapes) and 2.4 (per-shape
// kernel configuration, cached); DMuon announcement (agentren.cn), improvement 2 (the
// execution stack adapts the math form and kernels to each matrix shape).
#include "../../include/muon.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <string>
#include <tuple>
#include <vector>

#include "internal.hpp"

// Stage profiler: with MUON_FLAG_PROFILE every launch is bracketed by a pair of
// hipEvents on the launch stream; muon_profile_read aggregates them per stage and shape.
struct ProfRecord {
  hipEvent_t start, stop;
  int stage;           // index into kStageNames
  int64_t m, n;        // canonical shape of the group
  int count;           // matrices in the launch
  double flops, bytes; // algorithmic work of the launch
  int tile;            // GEMM tile configuration, -1 for other stages
};

struct muon_ctx {
  int device;
  uint32_t flags;
  int cu_count;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> event_pool;
  std::vector<ProfRecord> records;
  size_t next_event = 0;
  hipEvent_t tune_ev[2] = {nullptr, nullptr};  // events of the tile measurements
  // Extra streams on which independent shape groups run beside the caller's stream,
  // forked from it and joined back into it through events (created on first use).
  std::vector<hipStream_t> lanes;
  std::vector<hipEvent_t> lane_join;
  hipEvent_t lane_fork = nullptr;
};

namespace muon {
namespace {

constexpr int64_t kPad = 64;          // canonical dims are padded to multiples of 64
constexpr int64_t kMaxDim = 1 << 20;  // per-dimension limit
constexpr int kMaxRounds = 64;
// Longest Gram segment on the bf16 path. The fp16 recurrence mixes eigenvalues that the
// iteration drives apart (large directions settle near 1/sigma, small ones grow as a^k)
// in one fp16 matrix; from 4 rounds on the small directions are lost. Measured against
// the fp64 oracle: a 512 x 2048 rank-16 gradient gives errors 3e-3 to 4e-3 with
// [2,2,1], [2,3] and [3,2], but 2e3 with [4,1] and inf with [5]; a 2560 x 9728 one 4e-2
// with [5]. Three rounds is also the longest segment of the open-source fp16 default
// 2 + 3 (MuonX article, section 3.2).
constexpr int kMaxBf16Segment = 3;
constexpr int kMaxBatch = 65535;      // grid.y limit per launch
constexpr size_t kAlign = 256;

inline int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Group {
  int64_t m = 0, n = 0;        // canonical m' <= n'
  int64_t Mp = 0, Np = 0;      // padded
  int mode = MUON_NS_GRAM;
  int tile_sq = TILE_64, tile_ap = TILE_64;  // TileCfg of the symmetric / apply stages
  std::vector<int> members;    // indices into the caller's list
  int table_base = 0;          // first descriptor of this group in the table
  // workspace offsets (bytes) and per-matrix element strides
  // X: canonical m' x n' iterate (first X0 = xs s U); XT[2]: its transposed
  // copies (ping-pong); SQ: m' x m' buffers of the Gram-space recurrence.
  size_t off_partials = 0, off_s = 0, off_x = 0, off_xt[2] = {0, 0}, off_sq[4] = {0, 0, 0, 0};
  int64_t stride_x = 0, stride_sq = 0;
  int mom_tiles_m = 0, mom_tiles_n = 0;
  int norm_blocks = 0;         // norm-pass blocks of one stored matrix (one partial each)
  int norm_ub = 1;             // kNormBlock-element groups per norm-pass block (1 or 4)
  bool gm_cached = false;      // G and M small enough to stay in the caches between passes
  bool single_wg = false;      // whole update per matrix in one workgroup (small shapes)
  bool has_tall = false;       // some member is stored transposed (rows > cols)
  double work = 0.0;
  muon_hparams hs{};           // the call's hparams with this group's mode and schedule
};

struct Plan {
  std::vector<Group> groups;
  std::vector<int> group_of;   // per caller index
  size_t off_table = 0;
  size_t bytes = 0;
};

inline bool finite(float x) { return std::isfinite(x); }

int validate_hparams(const muon_hparams* hp) {
  if (!hp) return MUON_ERR_ARG;
  if (!finite(hp->lr) || !finite(hp->weight_decay) || !finite(hp->eps) || hp->eps < 0.0f) return MUON_ERR_ARG;
  if (!finite(hp->momentum) || hp->momentum < 0.0f || hp->momentum >= 1.0f) return MUON_ERR_ARG;
  if (hp->nesterov != 0 && hp->nesterov != 1) return MUON_ERR_ARG;
  if (!finite(hp->a) || !finite(hp->b) || !finite(hp->c)) return MUON_ERR_ARG;
  if (hp->n_segments < 1 || hp->n_segments > MUON_MAX_SEGMENTS) return MUON_ERR_ARG;
  int rounds = 0;
  for (int i = 0; i < hp->n_segments; ++i) {
    if (hp->segments[i] < 1 || hp->segments[i] > kMaxRounds) return MUON_ERR_ARG;
    rounds += hp->segments[i];
  }
  if (rounds > kMaxRounds) return MUON_ERR_ARG;
  if (hp->mode != MUON_NS_AUTO && hp->mode != MUON_NS_PLAIN && hp->mode != MUON_NS_GRAM &&
      hp->mode != MUON_NS_AUTO_SCHEDULE)
    return MUON_ERR_ARG;
  for (int dt : {hp->w_dtype, hp->g_dtype, hp->m_dtype, hp->ns_dtype})
    if (dt != MUON_F32 && dt != MUON_BF16) return MUON_ERR_ARG;
  if (hp->ns_dtype == MUON_BF16 && hp->mode != MUON_NS_PLAIN && hp->mode != MUON_NS_AUTO_SCHEDULE) {
    for (int i = 0; i < hp->n_segments; ++i)
      if (hp->segments[i] > kMaxBf16Segment) return MUON_ERR_UNSUPPORTED;
  }
  return MUON_OK;
}

int validate_matrix(const muon_matrix& mt, bool need_ptrs) {
  if (mt.rows < 1 || mt.cols < 1 || mt.rows > kMaxDim || mt.cols > kMaxDim) return MUON_ERR_ARG;
  if (need_ptrs && (!mt.W || !mt.G || !mt.M)) return MUON_ERR_ARG;
  return MUON_OK;
}

int total_rounds(const muon_hparams& hp) {
  int r = 0;
  for (int i = 0; i < hp.n_segments; ++i) r += hp.segments[i];
  return r;
}

// Matmul FLOPs as the MuonX article counts them: long = 2 m'^2 n', square = 2 m'^3.
double dense_flops(int64_t m, int64_t n, int mode, const muon_hparams& hp) {
  const double L = 2.0 * m * m * n, S = 2.0 * m * m * m;
  if (mode == MUON_NS_PLAIN) {
    const int r = total_rounds(hp);
    return r * (2.0 * L + S);
  }
  double f = 0.0;
  for (int i = 0; i < hp.n_segments; ++i) f += 2.0 * L + (4.0 * hp.segments[i] - 3.0) * S;
  return f;
}

// FLOPs the kernels perform: symmetric outputs (X X^T and every m' x m' product, all of
// which are symmetric in exact arithmetic) compute one triangle.
double kernel_flops(int64_t m, int64_t n, int mode, const muon_hparams& hp) {
  const double syrk = 1.0 * m * m * n, apply = 2.0 * m * m * n, sq = 1.0 * m * m * m;
  if (mode == MUON_NS_PLAIN) return total_rounds(hp) * (syrk + sq + apply);
  double f = 0.0;
  for (int i = 0; i < hp.n_segments; ++i) f += syrk + apply + (4.0 * hp.segments[i] - 3.0) * sq;
  return f;
}

// Per-product costs of a group's shape: the measured times of its Gram product, m' x m'
// product and apply once a step has measured their tiles (and the context measures),
// else the FLOPs the kernels perform (m'^2 n', m'^3 and 2 m'^2 n'). Returns true when the
// costs are measured.
bool product_costs(const muon_ctx* ctx, const Group& g, bool f32, double& ts, double& tq, double& ta);

// Shape-adaptive choice of the NS form for MUON_NS_AUTO: Gram NS with the caller's
// segments pays when the long products it saves cost more than the square ones it adds
// (MuonX section 3.2: the benefit depends on the shape). The costs are the shape's
// measured stage times once its tiles are measured, before that the dense FLOP counts
// the article uses (plain r (2L + S) against Gram sum_j (2L + (4 s_j - 3) S)).
int choose_mode(const muon_ctx* ctx, const Group& g, const muon_hparams& hp, bool f32) {
  if (hp.mode != MUON_NS_AUTO) return hp.mode;  // AUTO_SCHEDULE is resolved per group later
  double ts, tq, ta;
  if (product_costs(ctx, g, f32, ts, tq, ta)) {
    const int R = total_rounds(hp);
    double gram = 0.0;
    for (int i = 0; i < hp.n_segments; ++i) gram += ts + ta + (4.0 * hp.segments[i] - 3.0) * tq;
    return gram < R * (ts + tq + ta) ? MUON_NS_GRAM : MUON_NS_PLAIN;
  }
  return dense_flops(g.m, g.n, MUON_NS_GRAM, hp) < dense_flops(g.m, g.n, MUON_NS_PLAIN, hp) ? MUON_NS_GRAM
                                                                                          : MUON_NS_PLAIN;
}

// Static tile choice (MUON_FLAG_MODEL_ONLY, and the default before a measurement):
// symmetric stages use 128 x 128 once a launch has at least half as many of them as the
// GPU has CUs, else 64 x 64; the apply uses 256 x 256 once there is one per CU.
int heuristic_sym(int64_t Mp, int64_t count, int cu) {
  const int64_t nt = (Mp + 127) / 128;
  return (2 * (nt * (nt + 1) / 2) * count >= cu) ? TILE_128 : TILE_64;
}
int heuristic_apply(int64_t Mp, int64_t Np, int64_t count, int cu, bool f32) {
  const int64_t t256 = ((Mp + 255) / 256) * ((Np + 255) / 256);
  if (!f32 && Mp >= 256 && t256 * count >= cu) return TILE_256_DMA;
  const int64_t t128 = ((Mp + 127) / 128) * ((Np + 127) / 128);
  return (2 * t128 * count >= cu) ? TILE_128 : TILE_64;
}

void choose_schedule(const muon_ctx* ctx, Group& g, const muon_hparams& hp, bool f32);

// Small shapes on the bf16 path can run their whole update in one workgroup per matrix
// (small.hip): padded m' <= 128 and m' n' <= 64 Ki elements, so U fits in one workgroup's
// LDS. One launch then replaces the ~20 of the staged path, which wins when the list holds
// only such shapes. Beside larger groups the staged launches of the small groups fill the
// gaps of the larger groups' launches on their own streams, while single-workgroup
// kernels (one workgroup per CU for their whole duration) delay them; measured on the
// 832-matrix list: 0.72 ms staged, 0.77-0.80 ms with single-workgroup small groups. So a
// list uses the kernel only when every group qualifies.
bool single_wg_shape(int64_t Mp, int64_t Np) { return Mp <= 128 && Mp * Np <= kSmallMaxElems; }

// The second momentum pass reads G and M again. When a group's G and M fit well inside the
// 256 MB Infinity Cache, the first pass loads them normally so the second finds them there
// (2560 x 9728: second pass 50-51 -> 42 us, first pass +1 us). Larger groups stream them past
// the caches (cached loads made their first pass 3% slower, the second no faster) and put
// more loads in flight per thread: four groups of 8 elements per thread in the first pass,
// two tiles per workgroup in the second.
void set_norm_blocking(Group& g, const muon_hparams& hp, size_t cnt) {
  const double gm_bytes = static_cast<double>(cnt) * g.m * g.n *
                          ((hp.g_dtype == MUON_BF16 ? 2 : 4) + (hp.m_dtype == MUON_BF16 ? 2 : 4));
  g.gm_cached = gm_bytes <= 128.0 * 1024 * 1024;
  g.norm_ub = g.gm_cached ? 1 : 4;
  const int64_t nb_elems = static_cast<int64_t>(kNormBlock) * g.norm_ub;
  g.norm_blocks = static_cast<int>((g.m * g.n + nb_elems - 1) / nb_elems);
}

int build_plan(const muon_ctx* ctx, const muon_matrix* mats, int count, const muon_hparams& hp,
               bool need_ptrs, Plan& plan) {
  plan = Plan{};
  plan.group_of.assign(count, -1);
  std::map<std::tuple<int64_t, int64_t>, std::vector<int>> keyed;
  for (int i = 0; i < count; ++i) {
    const int rc = validate_matrix(mats[i], need_ptrs);
    if (rc != MUON_OK) return rc;
    const int64_t m = std::min(mats[i].rows, mats[i].cols), n = std::max(mats[i].rows, mats[i].cols);
    keyed[{m, n}].push_back(i);
  }
  const bool f32 = hp.ns_dtype == MUON_F32;
  const size_t ex = f32 ? 4 : 2, esq = f32 ? 4 : 2;
  for (auto& kv : keyed) {
    const int64_t m = std::get<0>(kv.first), n = std::get<1>(kv.first);
    const std::vector<int>& all = kv.second;
    for (size_t b = 0; b < all.size(); b += kMaxBatch) {
      Group g;
      g.m = m; g.n = n;
      g.Mp = round_up(m, kPad); g.Np = round_up(n, kPad);
      g.members.assign(all.begin() + b, all.begin() + std::min(all.size(), b + kMaxBatch));
      for (int i : g.members) g.has_tall = g.has_tall || mats[i].rows > mats[i].cols;
      const int64_t cnt = static_cast<int64_t>(g.members.size());
      g.hs = hp;
      if (hp.mode == MUON_NS_AUTO_SCHEDULE) choose_schedule(ctx, g, hp, f32);
      else g.mode = choose_mode(ctx, g, hp, f32);
      g.hs.mode = g.mode;
      g.tile_sq = heuristic_sym(g.Mp, cnt, ctx->cu_count);
      g.tile_ap = heuristic_apply(g.Mp, g.Np, cnt, ctx->cu_count, f32);
      if (!dma_addressable(g.Mp, g.Np, g.Mp, g.Np, static_cast<int64_t>(ex))) {
        g.tile_sq = staged_tile(g.tile_sq);
        g.tile_ap = staged_tile(g.tile_ap);
      }
      g.work = kernel_flops(m, n, g.mode, g.hs) * cnt;
      plan.groups.push_back(std::move(g));
    }
  }
  bool all_small = !f32 && !(ctx->flags & MUON_FLAG_STAGED_ONLY);
  for (const Group& g : plan.groups) all_small = all_small && single_wg_shape(g.Mp, g.Np);
  if (all_small) {
    for (Group& g : plan.groups) {
      g.single_wg = true;
      g.tile_sq = g.tile_ap = -1;
      g.work = dense_flops(g.m, g.n, g.mode, g.hs) * static_cast<double>(g.members.size());
    }
  }
  // Largest work first: the big launches start while the host still enqueues the rest.
  std::stable_sort(plan.groups.begin(), plan.groups.end(),
                   [](const Group& a, const Group& b) { return a.work > b.work; });
  size_t off = 0;
  plan.off_table = off;
  off = align_up(off + sizeof(MatDesc) * static_cast<size_t>(count));
  int tb = 0;
  for (size_t gi = 0; gi < plan.groups.size(); ++gi) {
    Group& g = plan.groups[gi];
    const size_t cnt = g.members.size();
    g.table_base = tb;
    tb += static_cast<int>(cnt);
    for (int i : g.members) plan.group_of[i] = static_cast<int>(gi);
    g.mom_tiles_m = static_cast<int>(g.Mp / 64);
    g.mom_tiles_n = static_cast<int>(g.Np / 64);
    g.off_partials = off;
    set_norm_blocking(g, hp, cnt);
    off = align_up(off + sizeof(float) * cnt * g.norm_blocks);
    g.off_s = off;
    off = align_up(off + sizeof(float) * cnt);
    g.stride_x = g.Mp * g.Np;
    g.off_x = off;
    off = align_up(off + ex * static_cast<size_t>(g.stride_x) * cnt);
    for (int k = 0; k < 2; ++k) {
      g.off_xt[k] = off;
      off = align_up(off + ex * static_cast<size_t>(g.stride_x) * cnt);
    }
    g.stride_sq = g.Mp * g.Mp;
    // The automatic choices may pick plain NS before a shape's tiles are measured and
    // Gram NS after, so they always reserve the Gram path's four m' x m' buffers: the
    // workspace size does not change between steps.
    const int nsq = (g.mode == MUON_NS_GRAM || hp.mode == MUON_NS_AUTO || hp.mode == MUON_NS_AUTO_SCHEDULE) ? 4 : 2;
    for (int k = 0; k < nsq; ++k) {
      g.off_sq[k] = off;
      off = align_up(off + esq * static_cast<size_t>(g.stride_sq) * cnt);
    }
  }
  plan.bytes = off;
  return MUON_OK;
}

// ---- stage helpers ----
struct StepEnv {
  char* ws;
  hipStream_t st;
  bool f32;
  const muon_hparams* hp;
  muon_ctx* ctx;
  // muon_step_static: no tile measurement (cached choices or the static ones), no
  // profiler events, one stream; nothing is created or allocated.
  bool no_alloc = false;
  // muon_prepare: the momentum stages are replaced by a seeded stand-in iterate (launch_dry_x)
  // and the last product writes the workspace instead of W, so W, G, M are not touched.
  bool dry = false;
};

// One stage name per kernel: "momentum_norm" the first pass over G and M (partial sums of
// U^2), "momentum" the second (M' and the normalised iterate in both layouts).
constexpr const char* kStageNames[] = {"table", "momentum", "norm_finalize", "momentum_norm", "syrk",
                                       "square", "apply", "apply_update", "single_wg"};
enum Stage { ST_TABLE, ST_MOMENTUM, ST_FINALIZE, ST_MOMENTUM_NORM, ST_SYRK, ST_SQUARE, ST_APPLY, ST_UPDATE,
             ST_SINGLE_WG };
constexpr size_t kMaxRecords = 1 << 16;

inline muon_ctx* timer_ctx(const StepEnv& env) { return env.no_alloc ? nullptr : env.ctx; }

// Brackets one launch with events when profiling is on (no effect otherwise).
struct StageTimer {
  muon_ctx* ctx = nullptr;
  hipStream_t st = nullptr;
  ProfRecord rec{};
  bool on = false;
  StageTimer(muon_ctx* c, hipStream_t s, int stage, int64_t m, int64_t n, int count, double flops,
             double bytes) {
    if (!c || !(c->flags & MUON_FLAG_PROFILE) || c->records.size() >= kMaxRecords) return;
    if (c->next_event == c->event_pool.size()) {
      // Timing-only events: without the system-scope fence an event record does not write
      // back and invalidate the caches, which otherwise adds about 2 us to every timed launch
      // (2560 squares 27.7 -> 25.9 us event-timed, closer to the kernel trace).
      hipEvent_t a, b;
      if (hipEventCreateWithFlags(&a, hipEventDisableSystemFence) != hipSuccess) return;
      if (hipEventCreateWithFlags(&b, hipEventDisableSystemFence) != hipSuccess) {
        (void)hipEventDestroy(a);
        return;
      }
      c->event_pool.emplace_back(a, b);
    }
    const auto ev = c->event_pool[c->next_event];
    if (hipEventRecord(ev.first, s) != hipSuccess) return;
    ctx = c; st = s; on = true;
    rec = ProfRecord{ev.first, ev.second, stage, m, n, count, flops, bytes, -1};
  }
  void done() {
    if (!on) return;
    if (hipEventRecord(rec.stop, st) == hipSuccess) {
      ctx->records.push_back(rec);
      ++ctx->next_event;
    }
    on = false;
  }
};

inline float pow2_near(double x, int lo, int hi) {
  int e = static_cast<int>(std::lround(std::log2(std::max(x, 1.0))));
  e = std::max(lo, std::min(hi, e));
  return std::ldexp(1.0f, e);
}

GemmParams base_params(const Group& g, const StepEnv& env) {
  GemmParams p;
  std::memset(&p, 0, sizeof(p));
  p.count = static_cast<int32_t>(g.members.size());
  p.s = reinterpret_cast<const float*>(env.ws + g.off_s);
  p.alpha = 1.0f;
  p.Mvalid = static_cast<int32_t>(g.m);
  p.Nvalid = static_cast<int32_t>(g.n);
  return p;
}

void set_sym_tiles(GemmParams& p, int64_t Mp, int cfg) {
  const int tile = tile_bm(cfg);
  const int nt = static_cast<int>((Mp + tile - 1) / tile);
  p.tiles_m = p.tiles_n = nt;
  p.tiles = nt * (nt + 1) / 2;
}

// Launch a GEMM stage with the tile configuration measured for it. On the first launch
// of a (stage, path, shape, batch) the candidates are timed on the stage's own buffers
// (one warm-up and four timed launches each; the stream is synchronised for it) and the
// fastest is cached process-wide; MUON_FLAG_MODEL_ONLY keeps the static choice. A
// stage that updates W is timed through its apply twin, which writes only workspace.
// Measured tile configurations, shared by every context of the process:
// (device, stage, path, padded m', padded n' or m', batch) -> TileCfg.
using TuneKey = std::tuple<int, int, int, int64_t, int64_t, int>;
std::mutex g_tune_mu;
std::map<TuneKey, int> g_tuned;
std::map<TuneKey, float> g_tuned_ms;   // measured time of the chosen configuration

// MUON_NS_AUTO_SCHEDULE: plain NS or Gram NS with k balanced segments, whichever costs
// least for the group's shape. Costs per product kind are the measured times of the
// shape's Gram product, m' x m' product and apply when a step has measured their tiles,
// else the FLOPs the kernels perform (m'^2 n', m'^3 and 2 m'^2 n'). Ties keep plain NS,
// then the larger k.
bool product_costs(const muon_ctx* ctx, const Group& g, bool f32, double& ts, double& tq, double& ta) {
  ts = 1.0 * g.m * g.m * g.n; ta = 2.0 * g.m * g.m * g.n; tq = 1.0 * g.m * g.m * g.m;
  if (ctx->flags & MUON_FLAG_MODEL_ONLY) return false;
  const int cnt = static_cast<int>(g.members.size());
  std::lock_guard<std::mutex> lk(g_tune_mu);
  auto s = g_tuned_ms.find(std::make_tuple(ctx->device, static_cast<int>(OP_SYRK), f32 ? 1 : 0, g.Mp, g.Mp, cnt));
  auto q = g_tuned_ms.find(std::make_tuple(ctx->device, static_cast<int>(OP_SYM), f32 ? 1 : 0, g.Mp, g.Mp, cnt));
  auto a = g_tuned_ms.find(std::make_tuple(ctx->device, static_cast<int>(OP_APPLY), f32 ? 1 : 0, g.Mp, g.Np, cnt));
  if (s == g_tuned_ms.end() || q == g_tuned_ms.end() || a == g_tuned_ms.end()) return false;
  ts = s->second; tq = q->second; ta = a->second;
  return true;
}

void choose_schedule(const muon_ctx* ctx, Group& g, const muon_hparams& hp, bool f32) {
  const int R = total_rounds(hp);
  const int cap = f32 ? kMaxRounds : kMaxBf16Segment;
  double ts, tq, ta;
  product_costs(ctx, g, f32, ts, tq, ta);
  double best = R * (ts + tq + ta);
  int best_k = 0;  // plain
  const int kmin = (R + cap - 1) / cap, kmax = std::min(R, MUON_MAX_SEGMENTS);
  for (int k = kmax; k >= kmin; --k) {
    const double cost = k * (ts + ta) + (4.0 * R - 3.0 * k) * tq;
    if (cost < best * (1.0 - 1e-9)) { best = cost; best_k = k; }
  }
  if (best_k == 0) {
    g.mode = MUON_NS_PLAIN;
    return;
  }
  g.mode = MUON_NS_GRAM;
  g.hs.n_segments = best_k;
  for (int i = 0; i < MUON_MAX_SEGMENTS; ++i) g.hs.segments[i] = 0;
  for (int i = 0; i < best_k; ++i) g.hs.segments[i] = R / best_k + (i < R % best_k ? 1 : 0);
}

template <class Build>
hipError_t run_stage(const StepEnv& env, const Group& g, GemmOp op, int heuristic, bool sym,
                     Build build, int* used) {
  muon_ctx* ctx = env.ctx;
  // every operand of the group's stages is at most Mp x Np elements
  const bool dma_ok = dma_addressable(g.Mp, g.Np, g.Mp, g.Np, env.f32 ? 4 : 2);
  auto usable = [&](int c) { return dma_ok ? c : staged_tile(c); };
  int cfg = heuristic;
  if (!(ctx->flags & MUON_FLAG_MODEL_ONLY)) {
    const int key_op = (op == OP_UPDATE) ? OP_APPLY : op;
    const TuneKey key = std::make_tuple(ctx->device, key_op, env.f32 ? 1 : 0, g.Mp, sym ? g.Mp : g.Np,
                                        static_cast<int>(g.members.size()));
    bool found = false;
    {
      std::lock_guard<std::mutex> lk(g_tune_mu);
      auto it = g_tuned.find(key);
      if (it != g_tuned.end()) { cfg = it->second; found = true; }
    }
    if (!found && !env.no_alloc) {
      // Each candidate: one warm-up and four timed launches, its time the fastest of them.
      // The timed launches run in four passes over the candidates, alternately in forward
      // and in reverse order: back-to-back MFMA work lowers the clock under the power limit
      // within milliseconds, so passes in one fixed order would favour the first
      // candidates, and single launches vary by several percent. The first candidate (in
      // the order below) within 2% of the fastest wins, so that near-ties resolve the same
      // way from run to run.
      std::vector<int> cands;
      if (env.f32) {
        cands = {TILE_64, TILE_128, TILE_64_DMA, TILE_128_DMA, TILE_128_DMA_K2};
      } else if (sym) {
        cands = {TILE_64, TILE_128, TILE_128_DMA, TILE_128_DMA_K2};
        if (g.Mp >= 512) cands.push_back(TILE_256_DMA);
      } else {
        // General products: larger tiles first, so that a near-tie goes to the tile that
        // moves fewer operand bytes per FLOP. (On 2560 x 9728 the 256x192 tile is 6-7%
        // faster than 256x128 inside a step but within 1-5% of it when timed alone.)
        if (g.Mp >= 256) cands = {TILE_256_DMA, TILE_256x192_DMA, TILE_256x128_DMA};
        for (int c : {TILE_128_DMA_K2, TILE_128, TILE_64}) cands.push_back(c);
      }
      for (int& c : cands) c = usable(c);
      for (int i = 0; i < 2; ++i)
        if (!ctx->tune_ev[i] && hipEventCreate(&ctx->tune_ev[i]) != hipSuccess) return hipErrorUnknown;
      const GemmOp top = (op == OP_UPDATE) ? OP_APPLY : op;
      std::vector<float> times(cands.size(), 1e30f);
      std::vector<char> ok(cands.size(), 0);
      for (size_t ci = 0; ci < cands.size(); ++ci)  // warm-up; a configuration that fails to launch is skipped
        ok[ci] = launch_gemm(top, env.f32, cands[ci], build(cands[ci]), env.st) == hipSuccess;
      for (int pass = 0; pass < 4; ++pass) {
        for (size_t k = 0; k < cands.size(); ++k) {
          const size_t ci = pass % 2 == 0 ? k : cands.size() - 1 - k;
          if (!ok[ci]) continue;
          const int c = cands[ci];
          const GemmParams p = build(c);
          if (hipEventRecord(ctx->tune_ev[0], env.st) != hipSuccess) return hipErrorUnknown;
          if (launch_gemm(top, env.f32, c, p, env.st) != hipSuccess) return hipErrorUnknown;
          if (hipEventRecord(ctx->tune_ev[1], env.st) != hipSuccess) return hipErrorUnknown;
          if (hipEventSynchronize(ctx->tune_ev[1]) != hipSuccess) return hipErrorUnknown;
          float ms = 0.0f;
          if (hipEventElapsedTime(&ms, ctx->tune_ev[0], ctx->tune_ev[1]) != hipSuccess) return hipErrorUnknown;
          times[ci] = std::min(times[ci], ms);
        }
      }
      const float best = *std::min_element(times.begin(), times.end());
      float chosen = best;
      for (size_t ci = 0; ci < cands.size(); ++ci)
        if (times[ci] <= best * 1.02f) { cfg = cands[ci]; chosen = times[ci]; break; }
      std::lock_guard<std::mutex> lk(g_tune_mu);
      g_tuned[key] = cfg;
      g_tuned_ms[key] = chosen;
    }
  }
  cfg = usable(cfg);
  const GemmParams p = build(cfg);
  *used = cfg;
  return launch_gemm(op, env.f32, cfg, p, env.st);
}

// R = alpha * X X^T (symmetric), X the fp16 / fp32 iterate.
hipError_t syrk(const Group& g, const StepEnv& env, const void* X, void* R, float alpha) {
  auto build = [&](int cfg) {
    GemmParams p = base_params(g, env);
    p.A = X; p.B = X; p.C = R;
    p.lda = p.ldb = g.Np; p.ldc = g.Mp;
    p.sA = p.sB = g.stride_x; p.sC = g.stride_sq;
    p.M = p.N = static_cast<int32_t>(g.Mp); p.K = static_cast<int32_t>(g.Np);
    p.alpha = alpha;
    set_sym_tiles(p, g.Mp, cfg);
    return p;
  };
  const double cnt = static_cast<double>(g.members.size());
  StageTimer tm(timer_ctx(env), env.st, ST_SYRK, g.m, g.n, static_cast<int>(cnt), cnt * g.m * g.m * g.n, 0.0);
  const hipError_t e = run_stage(env, g, OP_SYRK, g.tile_sq, true, build, &tm.rec.tile);
  tm.done();
  return e;
}

// C = alpha * A B^T + beta * E + gamma * I, every operand m' x m' and symmetric.
hipError_t square(const Group& g, const StepEnv& env, const void* A, const void* B, const void* E,
                  void* C, float alpha, float beta, float gamma) {
  auto build = [&](int cfg) {
    GemmParams p = base_params(g, env);
    p.A = A; p.B = B; p.C = C; p.E = E;
    p.lda = p.ldb = p.ldc = p.lde = g.Mp;
    p.sA = p.sB = p.sC = p.sE = g.stride_sq;
    p.M = p.N = p.K = static_cast<int32_t>(g.Mp);
    p.alpha = alpha; p.beta = beta; p.gamma = gamma;
    p.e_from_a = (E != nullptr && E == A) ? 1 : 0;
    set_sym_tiles(p, g.Mp, cfg);
    return p;
  };
  const double cnt = static_cast<double>(g.members.size());
  StageTimer tm(timer_ctx(env), env.st, ST_SQUARE, g.m, g.n, static_cast<int>(cnt), cnt * g.m * g.m * g.m, 0.0);
  const hipError_t e = run_stage(env, g, OP_SYM, g.tile_sq, true, build, &tm.rec.tile);
  tm.done();
  return e;
}

// v = alpha * Q (XT)^T + beta * XT^T: writes X = oscale * v and XTout = oscale * v^T, or
// (update) the weight update with O = v.
hipError_t apply(const Group& g, const StepEnv& env, const void* Q, const void* XT, void* X,
                 void* XTout, float alpha, float beta, float oscale, bool use_e, bool update,
                 const MatDesc* table) {
  auto build = [&](int cfg) {
    GemmParams p = base_params(g, env);
    p.A = Q; p.B = XT; p.C = X; p.C2 = XTout; p.E = use_e ? XT : nullptr;
    p.e_trans = 1;
    p.lda = g.Mp; p.ldb = g.Mp; p.ldc = g.Np; p.ldc2 = g.Mp; p.lde = g.Mp;
    p.sA = g.stride_sq; p.sB = g.stride_x; p.sC = g.stride_x; p.sC2 = g.stride_x; p.sE = g.stride_x;
    p.M = static_cast<int32_t>(g.Mp); p.N = static_cast<int32_t>(g.Np); p.K = static_cast<int32_t>(g.Mp);
    p.alpha = alpha; p.beta = beta; p.oscale = oscale;
    p.tiles_m = static_cast<int32_t>((g.Mp + tile_bm(cfg) - 1) / tile_bm(cfg));
    p.tiles_n = static_cast<int32_t>((g.Np + tile_bn(cfg) - 1) / tile_bn(cfg));
    p.tiles = p.tiles_m * p.tiles_n;
    if (update) {
      p.table = table;
      p.lr = env.hp->lr;
      p.wd = env.hp->weight_decay;
      p.w_bf16 = env.hp->w_dtype == MUON_BF16;
    }
    return p;
  };
  const double cnt = static_cast<double>(g.members.size());
  const double wbytes = update ? cnt * g.m * g.n * 2.0 * (env.hp->w_dtype == MUON_BF16 ? 2.0 : 4.0) : 0.0;
  StageTimer tm(timer_ctx(env), env.st, update ? ST_UPDATE : ST_APPLY, g.m, g.n, static_cast<int>(cnt),
                cnt * 2.0 * g.m * g.m * g.n, wbytes);
  const hipError_t e = run_stage(env, g, update ? OP_UPDATE : OP_APPLY, g.tile_ap, false, build, &tm.rec.tile);
  tm.done();
  return e;
}

#define MUON_HIP(call)                       \
  do {                                       \
    if ((call) != hipSuccess) return MUON_ERR_HIP; \
  } while (0)

// True when every GEMM stage the group will launch already has a measured tile (or the
// context does not measure): such a group makes no host synchronisation and may run on
// a stream of its own next to other groups.
bool group_tuned(const muon_ctx* ctx, const Group& g, const muon_hparams& hp, bool f32) {
  if ((ctx->flags & MUON_FLAG_MODEL_ONLY) || g.single_wg) return true;
  (void)hp;
  const int cnt = static_cast<int>(g.members.size());
  std::vector<TuneKey> keys = {
      std::make_tuple(ctx->device, static_cast<int>(OP_SYRK), f32 ? 1 : 0, g.Mp, g.Mp, cnt),
      std::make_tuple(ctx->device, static_cast<int>(OP_SYM), f32 ? 1 : 0, g.Mp, g.Mp, cnt),
      std::make_tuple(ctx->device, static_cast<int>(OP_APPLY), f32 ? 1 : 0, g.Mp, g.Np, cnt)};
  std::lock_guard<std::mutex> lk(g_tune_mu);
  for (const TuneKey& k : keys)
    if (g_tuned.find(k) == g_tuned.end()) return false;
  return true;
}

constexpr int kMaxLanes = 4;  // streams per step, the caller's included

// A group whose update is at least 1e11 FLOPs (about 0.1 ms of MFMA work) keeps the whole GPU
// busy with its own launches; running another such group beside it only makes them compete
// for the CUs and the caches.
bool fills_gpu(const Group& g) { return g.work >= 1e11; }

// Creates the context's extra streams and events (default priority) up to `n` lanes.
bool ensure_lanes(muon_ctx* ctx, int n) {
  if (!ctx->lane_fork && hipEventCreateWithFlags(&ctx->lane_fork, hipEventDisableTiming) != hipSuccess) {
    ctx->lane_fork = nullptr;
    return false;
  }
  while (static_cast<int>(ctx->lanes.size()) < n - 1) {
    hipStream_t st = nullptr;
    hipEvent_t ev = nullptr;
    if (hipStreamCreateWithFlags(&st, hipStreamNonBlocking) != hipSuccess) return false;
    if (hipEventCreateWithFlags(&ev, hipEventDisableTiming) != hipSuccess) {
      (void)hipStreamDestroy(st);
      return false;
    }
    ctx->lanes.push_back(st);
    ctx->lane_join.push_back(ev);
  }
  return true;
}

// Groups whose descriptors travel in the momentum kernel's arguments (which then writes
// them to the table): staged groups of at most kTableChunk matrices.
bool inline_descs(const Group& g) {
  return !g.single_wg && g.members.size() <= static_cast<size_t>(kTableChunk);
}

int run_group(const Group& g, const StepEnv& env, MatDesc* table, const MatDesc* host_desc) {
  const muon_hparams& hp = g.hs;   // the group's mode and schedule
  const bool f32 = env.f32;
  void* X = env.ws + g.off_x;
  void* XT[2] = {env.ws + g.off_xt[0], env.ws + g.off_xt[1]};
  const int count = static_cast<int32_t>(g.members.size());
  float* s = reinterpret_cast<float*>(env.ws + g.off_s);

  if (g.single_wg) {
    SmallParams sp;
    std::memset(&sp, 0, sizeof(sp));
    sp.table = table;
    sp.count = count;
    sp.m = static_cast<int32_t>(g.m); sp.n = static_cast<int32_t>(g.n);
    sp.Mp = static_cast<int32_t>(g.Mp); sp.Np = static_cast<int32_t>(g.Np);
    sp.X = X; sp.XT[0] = XT[0]; sp.XT[1] = XT[1];
    const int nsq = (g.mode == MUON_NS_GRAM) ? 4 : 2;
    for (int k = 0; k < nsq; ++k) sp.S[k] = env.ws + g.off_sq[k];
    sp.sX = g.stride_x; sp.sXT = g.stride_x; sp.sS = g.stride_sq;
    sp.mu = hp.momentum; sp.eps = hp.eps; sp.lr = hp.lr; sp.wd = hp.weight_decay;
    sp.a = hp.a; sp.b = hp.b; sp.c = hp.c;
    sp.xs = pow2_near(std::sqrt(static_cast<double>(g.m) * g.n), 0, 14);
    sp.e = pow2_near(static_cast<double>(g.m), 0, 14);
    sp.nesterov = hp.nesterov;
    sp.plain = g.mode == MUON_NS_PLAIN;
    sp.rounds = total_rounds(hp);
    sp.n_segments = hp.n_segments;
    for (int k = 0; k < hp.n_segments; ++k) sp.segments[k] = hp.segments[k];
    sp.g_bf16 = hp.g_dtype == MUON_BF16; sp.m_bf16 = hp.m_dtype == MUON_BF16; sp.w_bf16 = hp.w_dtype == MUON_BF16;
    sp.dry = env.dry ? 1 : 0;
    const double gb = hp.g_dtype == MUON_BF16 ? 2.0 : 4.0, mb = hp.m_dtype == MUON_BF16 ? 2.0 : 4.0;
    const double wb = hp.w_dtype == MUON_BF16 ? 2.0 : 4.0;
    StageTimer tm(timer_ctx(env), env.st, ST_SINGLE_WG, g.m, g.n, count, dense_flops(g.m, g.n, g.mode, hp) * count,
                  static_cast<double>(count) * g.m * g.n * (gb + 2.0 * mb + 2.0 * wb));
    MUON_HIP(launch_small_ns(sp, env.st));
    tm.done();
    return MUON_OK;
  }

  // Scales of the bf16 path (powers of two, so exact): the iterate X and its transposed
  // copies are stored in fp16 multiplied by xs ~ sqrt(m' n') (entries ~ 1); the Gram-like
  // matrices (R, Q R, A) are stored multiplied by e ~ m' so their entries sit in fp16's
  // normal range; the polynomial coefficients absorb e.
  const float e = f32 ? 1.0f : pow2_near(static_cast<double>(g.m), 0, 14);
  const float xs = f32 ? 1.0f : pow2_near(std::sqrt(static_cast<double>(g.m) * g.n), 0, 14);
  const float a = hp.a, b1 = hp.b / e, c1 = hp.c / (e * e);
  const float ixs = 1.0f / xs;

  // Momentum in two passes over G and M: partial sums of U^2, the norm, then M' and the
  // normalised iterate X0 = xs * s * U in both layouts (X and XT[0]).
  MomentumParams mp;
  std::memset(&mp, 0, sizeof(mp));
  mp.table = table;
  mp.X = X; mp.XT = XT[0];
  mp.sX = g.stride_x;
  mp.m = static_cast<int32_t>(g.m); mp.n = static_cast<int32_t>(g.n);
  mp.Mp = static_cast<int32_t>(g.Mp); mp.Np = static_cast<int32_t>(g.Np);
  mp.tiles_m = g.mom_tiles_m; mp.tiles_n = g.mom_tiles_n;
  mp.norm_blocks = g.norm_blocks;
  mp.count = count;
  mp.mu = hp.momentum; mp.nesterov = hp.nesterov;
  mp.g_bf16 = hp.g_dtype == MUON_BF16; mp.m_bf16 = hp.m_dtype == MUON_BF16; mp.x_f16 = !f32;
  mp.keep_gm = g.gm_cached;
  mp.norm_ub = g.norm_ub;
  mp.xscale = xs;
  mp.s = s;
  mp.partials = reinterpret_cast<float*>(env.ws + g.off_partials);
  if (inline_descs(g)) {
    mp.inl.n = count;
    for (int i = 0; i < count; ++i) mp.inl.d[i] = host_desc[i];
    mp.table_out = table;
  }
  const double gb = hp.g_dtype == MUON_BF16 ? 2.0 : 4.0, mb = hp.m_dtype == MUON_BF16 ? 2.0 : 4.0;
  const double xb = f32 ? 4.0 : 2.0;
  const double elems = static_cast<double>(count) * g.m * g.n;
  if (env.dry) {
    MUON_HIP(launch_dry_x(mp, env.st));
  } else {
    {
      // algorithmic bytes: G and M read
      StageTimer tm(timer_ctx(env), env.st, ST_MOMENTUM_NORM, g.m, g.n, count, 0.0, elems * (gb + mb));
      MUON_HIP(launch_momentum_norm(mp, env.st));
      tm.done();
    }
    {
      StageTimer tm(timer_ctx(env), env.st, ST_FINALIZE, g.m, g.n, count, 0.0, 4.0 * count * g.norm_blocks);
      MUON_HIP(launch_norm_finalize(mp.partials, g.norm_blocks, count, hp.eps, s, env.st));
      tm.done();
    }
    {
      // algorithmic bytes: G and M read, M' written, X0 written in two layouts
      StageTimer tm(timer_ctx(env), env.st, ST_MOMENTUM, g.m, g.n, count, 0.0, elems * (gb + 2.0 * mb + 2.0 * xb));
      MUON_HIP(launch_momentum_x(mp, env.st));
      tm.done();
    }
  }

  int cur = 0;
  if (g.mode == MUON_NS_PLAIN) {
    void* A = env.ws + g.off_sq[0];
    void* B = env.ws + g.off_sq[1];
    const int rounds = total_rounds(hp);
    for (int r = 0; r < rounds; ++r) {
      const bool last = r == rounds - 1;
      // A' = e X X^T
      MUON_HIP(syrk(g, env, X, A, e * ixs * ixs));
      MUON_HIP(square(g, env, A, A, A, B, c1, b1, 0.0f));           // B = b A + c A^2
      // X' = a X + B X  (X taken from its transposed copy, which carries xs)
      MUON_HIP(apply(g, env, B, XT[cur], X, XT[cur ^ 1], ixs, a * ixs, xs, true, last && !env.dry, table));
      cur ^= 1;
    }
  } else {
    void* R = env.ws + g.off_sq[0];
    void* Q = env.ws + g.off_sq[1];
    void* T1 = env.ws + g.off_sq[2];
    void* T2 = env.ws + g.off_sq[3];
    for (int sgi = 0; sgi < hp.n_segments; ++sgi) {
      const bool last = sgi == hp.n_segments - 1;
      MUON_HIP(syrk(g, env, X, R, e * ixs * ixs));
      MUON_HIP(square(g, env, R, R, R, Q, c1, b1, a));            // Q = P(R)
      for (int k = 1; k < hp.segments[sgi]; ++k) {
        MUON_HIP(square(g, env, Q, R, nullptr, T1, 1.0f, 0.0f, 0.0f));   // T = Q R
        MUON_HIP(square(g, env, T1, Q, nullptr, T2, 1.0f, 0.0f, 0.0f));  // A = T Q^T
        MUON_HIP(square(g, env, T2, T2, T2, T1, c1, b1, a));             // P = aI + bA + cA^2
        MUON_HIP(square(g, env, T1, Q, nullptr, T2, 1.0f, 0.0f, 0.0f));  // Q <- P Q
        std::swap(Q, T2);
      }
      MUON_HIP(apply(g, env, Q, XT[cur], X, XT[cur ^ 1], ixs, 0.0f, xs, false, last && !env.dry, table));
      cur ^= 1;
    }
  }
  return MUON_OK;
}

struct DeviceGuard {
  int prev = -1;
  bool ok = false;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) == hipSuccess && hipSetDevice(dev) == hipSuccess) ok = true;
  }
  ~DeviceGuard() {
    if (prev >= 0) (void)hipSetDevice(prev);
  }
};


// File-scope scratch for muon_step_static (callers that cannot allocate device memory).
// Each device holds its own copy; host code uses only the per-device address that
// hipGetSymbolAddress returned for it (the array's name is not a device address on the
// host).
constexpr size_t kStaticScratchBytes = MUON_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
hipError_t g_scratch_err[kMaxDevices] = {};

// Called by muon_init once per device, with that device current.
void init_scratch(int device) {
  if (device < 0 || device >= kMaxDevices) return;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[device]) return;
  void* ptr = nullptr;
  const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e == hipSuccess && ptr) g_scratch_ptr[device] = ptr;
  else g_scratch_err[device] = e == hipSuccess ? hipErrorInvalidSymbol : e;
}

void* scratch_ptr(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  return g_scratch_ptr[device];
}

int step_impl(muon_ctx* ctx, const muon_matrix* mats, int count, const muon_hparams* hp, void* workspace,
              size_t workspace_bytes, void* stream, bool no_alloc, bool dry = false) {
  {
    if (!ctx || count < 0 || (count > 0 && !mats)) return MUON_ERR_ARG;
    const int rc = validate_hparams(hp);
    if (rc != MUON_OK) return rc;
    if (count == 0) return MUON_OK;
    Plan plan;
    const int pc = build_plan(ctx, mats, count, *hp, !dry, plan);
    if (pc != MUON_OK) return pc;
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0 ||
        workspace_bytes < plan.bytes)
      return MUON_ERR_WORKSPACE;
    if (ctx->device < 0) return MUON_ERR_DEVICE;
    DeviceGuard dg(ctx->device);
    if (!dg.ok) return MUON_ERR_HIP;
    StepEnv env{static_cast<char*>(workspace), static_cast<hipStream_t>(stream),
                hp->ns_dtype == MUON_F32, hp, ctx, no_alloc, dry};
    MatDesc* table = reinterpret_cast<MatDesc*>(env.ws + plan.off_table);
    // Descriptor table, ordered by group, written by small kernels (no host sync).
    std::vector<MatDesc> descs(count);
    for (const Group& g : plan.groups) {
      for (size_t i = 0; i < g.members.size(); ++i) {
        const muon_matrix& mt = mats[g.members[i]];
        MatDesc d{};
        d.W = mt.W; d.G = mt.G; d.M = mt.M;
        d.rows = mt.rows; d.cols = mt.cols;
        d.transposed = mt.rows > mt.cols ? 1 : 0;
        descs[g.table_base + i] = d;
      }
    }
    // Groups with inline descriptors get their entries from their momentum kernel.
    for (const Group& g : plan.groups) {
      if (inline_descs(g)) continue;
      const int base = g.table_base, n = static_cast<int>(g.members.size());
      for (int b = 0; b < n; b += kTableChunk) {
        TableChunk c;
        std::memset(&c, 0, sizeof(c));
        c.n = std::min(kTableChunk, n - b);
        for (int i = 0; i < c.n; ++i) c.d[i] = descs[base + b + i];
        StageTimer tm(timer_ctx(env), env.st, ST_TABLE, 0, 0, c.n, 0.0, sizeof(MatDesc) * c.n);
        MUON_HIP(launch_write_table(c, table + base + b, env.st));
        tm.done();
      }
    }
    // Independent shape groups whose launches do not fill the GPU run on up to
    // kMaxLanes - 1 extra streams beside the caller's (largest work first, each to the least
    // loaded lane), when none of them still has tiles to measure and the context does not
    // profile; groups that fill the GPU run in order on the caller's stream. (Measured on the
    // 7B list, whose three groups all fill the GPU: 314 ms on one stream, 324 ms with the
    // groups on four streams; on the 832-matrix list, none of whose groups does: 0.69 ms on
    // four streams, 0.75 ms on one.)
    int small = 0;
    for (const Group& g : plan.groups) small += fills_gpu(g) ? 0 : 1;
    int nl = std::min<int>(kMaxLanes, small + (small < static_cast<int>(plan.groups.size()) ? 1 : 0));
    if ((ctx->flags & (MUON_FLAG_PROFILE | MUON_FLAG_ONE_STREAM)) || no_alloc || small == 0) nl = 1;
    for (size_t i = 0; nl > 1 && i < plan.groups.size(); ++i)
      if (!group_tuned(ctx, plan.groups[i], *hp, env.f32)) nl = 1;
    if (nl > 1 && !ensure_lanes(ctx, nl)) nl = 1;
    if (nl == 1) {
      for (const Group& g : plan.groups) {
        const int r = run_group(g, env, table + g.table_base, descs.data() + g.table_base);
        if (r != MUON_OK) return r;
      }
      return MUON_OK;
    }
    MUON_HIP(hipEventRecord(ctx->lane_fork, env.st));
    for (int l = 0; l < nl - 1; ++l) MUON_HIP(hipStreamWaitEvent(ctx->lanes[l], ctx->lane_fork, 0));
    std::vector<double> load(nl, 0.0);
    int r = MUON_OK;
    for (const Group& g : plan.groups) {
      // groups that fill the GPU stay on the caller's stream (lane 0)
      const int l = fills_gpu(g) ? 0 : static_cast<int>(std::min_element(load.begin(), load.end()) - load.begin());
      load[l] += g.work;
      StepEnv le = env;
      if (l > 0) le.st = ctx->lanes[l - 1];
      r = run_group(g, le, table + g.table_base, descs.data() + g.table_base);
      if (r != MUON_OK) break;
    }
    // The caller's stream waits for every lane, also after a failed launch, so nothing
    // the step enqueued outlives the caller's view of the stream.
    for (int l = 0; l < nl - 1; ++l) {
      if (hipEventRecord(ctx->lane_join[l], ctx->lanes[l]) != hipSuccess ||
          hipStreamWaitEvent(env.st, ctx->lane_join[l], 0) != hipSuccess)
        r = MUON_ERR_HIP;
    }
    return r;
  }
}


}  // namespace
}  // namespace muon

using namespace muon;

extern "C" {

void muon_hparams_default(muon_hparams* hp) {
  if (!hp) return;
  std::memset(hp, 0, sizeof(*hp));
  hp->lr = 0.02f;
  hp->momentum = 0.95f;
  hp->weight_decay = 0.0f;
  hp->eps = 1e-7f;
  hp->nesterov = 1;
  hp->a = 3.4445f;
  hp->b = -4.7750f;
  hp->c = 2.0315f;
  hp->n_segments = 3;
  hp->segments[0] = 2;
  hp->segments[1] = 2;
  hp->segments[2] = 1;
  hp->mode = MUON_NS_AUTO;
  hp->w_dtype = MUON_F32;
  hp->g_dtype = MUON_BF16;
  hp->m_dtype = MUON_BF16;
  hp->ns_dtype = MUON_BF16;
}

int muon_init(muon_ctx** out, int device, uint32_t flags) {
  try {
    if (!out) return MUON_ERR_ARG;
    *out = nullptr;
    if ((flags & ~(MUON_FLAG_MODEL_ONLY | MUON_FLAG_PROFILE | MUON_FLAG_STAGED_ONLY | MUON_FLAG_ONE_STREAM)) != 0)
      return MUON_ERR_ARG;
    if (device == -1) {  // host-only context: planning and validation, no launches
      muon_ctx* c = new (std::nothrow) muon_ctx;
      if (!c) return MUON_ERR_HIP;
      c->device = -1;
      c->flags = flags;
      c->cu_count = 256;
      *out = c;
      return MUON_OK;
    }
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess) return MUON_ERR_DEVICE;
    if (device < 0 || device >= n) return MUON_ERR_DEVICE;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) != hipSuccess) return MUON_ERR_DEVICE;
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return MUON_ERR_DEVICE;
    {
      DeviceGuard dg(device);
      if (!dg.ok) return MUON_ERR_HIP;
      init_scratch(device);
    }
    muon_ctx* c = new (std::nothrow) muon_ctx;
    if (!c) return MUON_ERR_HIP;
    c->device = device;
    c->flags = flags;
    c->cu_count = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 256;
    *out = c;
    return MUON_OK;
  } catch (...) {
    return MUON_ERR_HIP;
  }
}

int muon_workspace_size(muon_ctx* ctx, const muon_matrix* mats, int count, const muon_hparams* hp,
                        size_t* bytes) {
  try {
    if (!ctx || !bytes || count < 0 || (count > 0 && !mats)) return MUON_ERR_ARG;
    const int rc = validate_hparams(hp);
    if (rc != MUON_OK) return rc;
    Plan plan;
    const int pc = build_plan(ctx, mats, count, *hp, false, plan);
    if (pc != MUON_OK) return pc;
    *bytes = count == 0 ? 0 : plan.bytes;
    return MUON_OK;
  } catch (...) {
    return MUON_ERR_HIP;
  }
}

int muon_step(muon_ctx* ctx, const muon_matrix* mats, int count, const muon_hparams* hp,
              void* workspace, size_t workspace_bytes, void* stream) {
  try {
    return step_impl(ctx, mats, count, hp, workspace, workspace_bytes, stream, false);
  } catch (...) {
    return MUON_ERR_HIP;
  }
}

int muon_prepare(muon_ctx* ctx, const muon_matrix* mats, int count, const muon_hparams* hp, void* workspace,
                 size_t workspace_bytes, void* stream, double* ms) {
  try {
    if (ms) *ms = 0.0;
    if (!ctx || count < 0 || (count > 0 && !mats)) return MUON_ERR_ARG;
    const int rc = validate_hparams(hp);
    if (rc != MUON_OK) return rc;
    if (count == 0) return MUON_OK;
    {
      Plan plan;
      const int pc = build_plan(ctx, mats, count, *hp, false, plan);
      if (pc != MUON_OK) return pc;
      if (!workspace || (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0 || workspace_bytes < plan.bytes)
        return MUON_ERR_WORKSPACE;
    }
    if (ctx->device < 0) return MUON_ERR_DEVICE;
    DeviceGuard dg(ctx->device);
    if (!dg.ok) return MUON_ERR_HIP;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    // First dry run: every stage whose tiles are not cached measures them (the plan may then
    // change, e.g. MUON_NS_AUTO's plain / Gram choice, so a second run measures the rest).
    for (int pass = 0; pass < 2; ++pass) {
      const int r = step_impl(ctx, mats, count, hp, workspace, workspace_bytes, stream, false, true);
      if (r != MUON_OK) return r;
    }
    for (int i = 0; i < 2; ++i)
      if (!ctx->tune_ev[i] && hipEventCreate(&ctx->tune_ev[i]) != hipSuccess) return MUON_ERR_HIP;
    MUON_HIP(hipEventRecord(ctx->tune_ev[0], st));
    const int r = step_impl(ctx, mats, count, hp, workspace, workspace_bytes, stream, false, true);
    if (r != MUON_OK) return r;
    MUON_HIP(hipEventRecord(ctx->tune_ev[1], st));
    MUON_HIP(hipEventSynchronize(ctx->tune_ev[1]));
    float t = 0.0f;
    MUON_HIP(hipEventElapsedTime(&t, ctx->tune_ev[0], ctx->tune_ev[1]));
    if (ms) *ms = t;
    return MUON_OK;
  } catch (...) {
    return MUON_ERR_HIP;
  }
}

int muon_step_static(muon_ctx* ctx, const muon_matrix* mats, int count, const muon_hparams* hp,
                     void* stream) {
  try {
    if (!ctx || count < 0 || (count > 0 && !mats)) return MUON_ERR_ARG;
    const int rc = validate_hparams(hp);
    if (rc != MUON_OK) return rc;
    if (count == 0) return MUON_OK;
    Plan plan;
    const int pc = build_plan(ctx, mats, count, *hp, true, plan);
    if (pc != MUON_OK) return pc;
    if (plan.bytes > kStaticScratchBytes) return MUON_ERR_WORKSPACE;
    if (ctx->device < 0) return MUON_ERR_DEVICE;
    void* ptr = scratch_ptr(ctx->device);
    if (!ptr) return MUON_ERR_HIP;
    return step_impl(ctx, mats, count, hp, ptr, kStaticScratchBytes, stream, true);
  } catch (...) {
    return MUON_ERR_HIP;
  }
}

int muon_tune_save(muon_ctx* ctx, const char* path) {
  try {
    if (!ctx || !path) return MUON_ERR_ARG;
    std::vector<std::tuple<TuneKey, int, float>> rows;
    {
      std::lock_guard<std::mutex> lk(g_tune_mu);
      for (const auto& kv : g_tuned)
        if (std::get<0>(kv.first) == ctx->device) {
          auto t = g_tuned_ms.find(kv.first);
          rows.emplace_back(kv.first, kv.second, t == g_tuned_ms.end() ? -1.0f : t->second);
        }
    }
    FILE* f = std::fopen(path, "w");
    if (!f) return MUON_ERR_ARG;
    bool ok = true;
    for (const auto& row : rows) {
      const TuneKey& k = std::get<0>(row);
      ok = ok && std::fprintf(f, "%d %d %lld %lld %d %d %.9g\n", std::get<1>(k), std::get<2>(k),
                              static_cast<long long>(std::get<3>(k)), static_cast<long long>(std::get<4>(k)),
                              std::get<5>(k), std::get<1>(row), static_cast<double>(std::get<2>(row))) > 0;
    }
    ok = (std::fclose(f) == 0) && ok;
    return ok ? MUON_OK : MUON_ERR_ARG;
  } catch (...) {
    return MUON_ERR_HIP;
  }
}

int muon_tune_load(muon_ctx* ctx, const char* path, int* n_loaded) {
  try {
    if (n_loaded) *n_loaded = 0;
    if (!ctx || !path) return MUON_ERR_ARG;
    FILE* f = std::fopen(path, "r");
    if (!f) return MUON_ERR_ARG;
    std::vector<std::tuple<TuneKey, int, float>> rows;
    bool ok = true;
    char line[256];
    while (ok && std::fgets(line, sizeof(line), f)) {
      int op = 0, f32 = 0, cnt = 0, tile = 0, used = 0;
      long long mp = 0, np = 0;
      float ms = -1.0f;
      bool blank = true;
      for (const char* c = line; *c; ++c)
        if (*c != ' ' && *c != '\t' && *c != '\n' && *c != '\r') blank = false;
      if (blank) continue;
      // six integers, then optionally the measured time in ms (negative: none)
      const int got = std::sscanf(line, "%d %d %lld %lld %d %d %n", &op, &f32, &mp, &np, &cnt, &tile, &used);
      if (got != 6) {
        ok = false;
        break;
      }
      if (line[used] != '\0') {
        int used2 = 0;
        if (std::sscanf(line + used, "%f %n", &ms, &used2) != 1 || line[used + used2] != '\0' ||
            !std::isfinite(ms)) {
          ok = false;
          break;
        }
      }
      const bool sym = op == OP_SYRK_IN || op == OP_SYM || op == OP_SYRK;
      ok = (sym || op == OP_APPLY) && (f32 == 0 || f32 == 1) && mp >= kPad && np >= kPad &&
           mp % kPad == 0 && np % kPad == 0 && mp <= kMaxDim && np <= kMaxDim && cnt >= 1 &&
           cnt <= kMaxBatch && tile >= 0 && tile < TILE_COUNT && (!sym || mp == np) &&
           tile_available(sym, f32 == 1, tile);
      if (ok) rows.emplace_back(std::make_tuple(ctx->device, op, f32, static_cast<int64_t>(mp),
                                                static_cast<int64_t>(np), cnt), tile, ms);
    }
    ok = ok && !std::ferror(f);
    std::fclose(f);
    if (!ok) return MUON_ERR_ARG;
    std::lock_guard<std::mutex> lk(g_tune_mu);
    for (const auto& row : rows) {
      g_tuned[std::get<0>(row)] = std::get<1>(row);
      if (std::get<2>(row) >= 0.0f) g_tuned_ms[std::get<0>(row)] = std::get<2>(row);
      else g_tuned_ms.erase(std::get<0>(row));
    }
    if (n_loaded) *n_loaded = static_cast<int>(rows.size());
    return MUON_OK;
  } catch (...) {
    return MUON_ERR_HIP;
  }
}

int muon_plan_info(muon_ctx* ctx, const muon_matrix* mats, int count, const muon_hparams* hp,
                   int index, muon_plan_entry* out) {
  try {
    if (!ctx || !out || !mats || count <= 0 || index < 0 || index >= count) return MUON_ERR_ARG;
    const int rc = validate_hparams(hp);
    if (rc != MUON_OK) return rc;
    Plan plan;
    const int pc = build_plan(ctx, mats, count, *hp, false, plan);
    if (pc != MUON_OK) return pc;
    const Group& g = plan.groups[plan.group_of[index]];
    out->mode = g.mode;
    out->transposed = mats[index].rows > mats[index].cols ? 1 : 0;
    out->m = g.m;
    out->n = g.n;
    out->group = plan.group_of[index];
    out->tile_sym = g.tile_sq;
    out->tile_apply = g.tile_ap;
    out->single_wg = g.single_wg ? 1 : 0;
    if (!g.single_wg && !(ctx->flags & MUON_FLAG_MODEL_ONLY)) {
      const int f32 = hp->ns_dtype == MUON_F32 ? 1 : 0;
      const int cnt = static_cast<int>(g.members.size());
      std::lock_guard<std::mutex> lk(g_tune_mu);
      auto a = g_tuned.find(std::make_tuple(ctx->device, static_cast<int>(OP_SYM), f32, g.Mp, g.Mp, cnt));
      if (a != g_tuned.end()) out->tile_sym = a->second;
      auto b = g_tuned.find(std::make_tuple(ctx->device, static_cast<int>(OP_APPLY), f32, g.Mp, g.Np, cnt));
      if (b != g_tuned.end()) out->tile_apply = b->second;
    }
    if (!g.single_wg && !dma_addressable(g.Mp, g.Np, g.Mp, g.Np, hp->ns_dtype == MUON_F32 ? 4 : 2)) {
      out->tile_sym = staged_tile(out->tile_sym);
      out->tile_apply = staged_tile(out->tile_apply);
    }
    out->dense_flops = dense_flops(g.m, g.n, g.mode, g.hs);
    out->kernel_flops = g.single_wg ? out->dense_flops : kernel_flops(g.m, g.n, g.mode, g.hs);
    std::memset(out->segments, 0, sizeof(out->segments));
    if (g.mode == MUON_NS_PLAIN) {
      out->n_segments = 1;
      out->segments[0] = total_rounds(g.hs);
    } else {
      out->n_segments = g.hs.n_segments;
      for (int k = 0; k < g.hs.n_segments; ++k) out->segments[k] = g.hs.segments[k];
    }
    return MUON_OK;
  } catch (...) {
    return MUON_ERR_HIP;
  }
}

int muon_debug_stage(muon_ctx* ctx, int stage, const muon_matrix* mat, const muon_hparams* hp, const void* in,
                     void* out, void* out2, float* scale, void* workspace, size_t workspace_bytes, void* stream) {
  try {
    if (!ctx || !mat || stage < MUON_STAGE_NORM || stage > MUON_STAGE_UPDATE) return MUON_ERR_ARG;
    const int rc = validate_hparams(hp);
    if (rc != MUON_OK) return rc;
    const int vm = validate_matrix(*mat, false);
    if (vm != MUON_OK) return vm;
    const bool need_gm = stage != MUON_STAGE_UPDATE, need_w = stage == MUON_STAGE_UPDATE;
    if ((need_gm && (!mat->G || !mat->M)) || (need_w && (!mat->W || !in)) || !out || (stage != MUON_STAGE_NORM && !out2))
      return MUON_ERR_ARG;
    Group g;
    g.m = std::min(mat->rows, mat->cols); g.n = std::max(mat->rows, mat->cols);
    g.Mp = round_up(g.m, kPad); g.Np = round_up(g.n, kPad);
    g.members = {0};
    g.has_tall = mat->rows > mat->cols;
    g.mom_tiles_m = static_cast<int>(g.Mp / 64); g.mom_tiles_n = static_cast<int>(g.Np / 64);
    set_norm_blocking(g, *hp, 1);   // the kernels muon_step runs for this matrix alone
    g.stride_x = g.Mp * g.Np; g.stride_sq = g.Mp * g.Mp;
    const bool f32 = hp->ns_dtype == MUON_F32;
    g.tile_ap = heuristic_apply(g.Mp, g.Np, 1, ctx->cu_count, f32);
    g.hs = *hp;
    // workspace: descriptor, partials, s
    const size_t off_part = kAlign, off_s = align_up(off_part + sizeof(float) * g.norm_blocks);
    const size_t need = off_s + kAlign;
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0 || workspace_bytes < need)
      return MUON_ERR_WORKSPACE;
    if (ctx->device < 0) return MUON_ERR_DEVICE;
    DeviceGuard dg(ctx->device);
    if (!dg.ok) return MUON_ERR_HIP;
    char* ws = static_cast<char*>(workspace);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    MatDesc* table = reinterpret_cast<MatDesc*>(ws);
    TableChunk c;
    std::memset(&c, 0, sizeof(c));
    c.n = 1;
    c.d[0].W = mat->W; c.d[0].G = mat->G; c.d[0].M = mat->M;
    c.d[0].rows = mat->rows; c.d[0].cols = mat->cols; c.d[0].transposed = mat->rows > mat->cols ? 1 : 0;
    MUON_HIP(launch_write_table(c, table, st));
    const float xs = f32 ? 1.0f : pow2_near(std::sqrt(static_cast<double>(g.m) * g.n), 0, 14);
    if (scale) *scale = xs;
    if (stage == MUON_STAGE_UPDATE) {
      StepEnv env{ws, st, f32, hp, ctx, true, false};
      g.off_s = off_s;
      // O = Q X / xs from Q (in, Mp x Mp) and xs X^T (out2, Np x Mp); W updated through the
      // orientation map (out is unused but must be non-null).
      MUON_HIP(apply(g, env, in, out2, out, nullptr, 1.0f / xs, 0.0f, xs, false, true, table));
      return MUON_OK;
    }
    MomentumParams mp;
    std::memset(&mp, 0, sizeof(mp));
    mp.table = table;
    mp.X = out; mp.XT = out2;
    mp.sX = g.stride_x;
    mp.m = static_cast<int32_t>(g.m); mp.n = static_cast<int32_t>(g.n);
    mp.Mp = static_cast<int32_t>(g.Mp); mp.Np = static_cast<int32_t>(g.Np);
    mp.tiles_m = g.mom_tiles_m; mp.tiles_n = g.mom_tiles_n;
    mp.norm_blocks = g.norm_blocks;
    mp.norm_ub = g.norm_ub;
    mp.keep_gm = g.gm_cached;
    mp.count = 1;
    mp.mu = hp->momentum; mp.nesterov = hp->nesterov;
    mp.g_bf16 = hp->g_dtype == MUON_BF16; mp.m_bf16 = hp->m_dtype == MUON_BF16; mp.x_f16 = !f32;
    mp.xscale = xs;
    float* s = stage == MUON_STAGE_NORM ? static_cast<float*>(out) : reinterpret_cast<float*>(ws + off_s);
    mp.s = s;
    mp.partials = reinterpret_cast<float*>(ws + off_part);
    MUON_HIP(launch_momentum_norm(mp, st));
    MUON_HIP(launch_norm_finalize(mp.partials, g.norm_blocks, 1, hp->eps, s, st));
    if (stage == MUON_STAGE_ITERATE) MUON_HIP(launch_momentum_x(mp, st));
    return MUON_OK;
  } catch (...) {
    return MUON_ERR_HIP;
  }
}

int muon_debug_gemm(muon_ctx* ctx, int kind, int ns_dtype, int tile, int64_t M, int64_t N, int64_t K,
                    const void* A, const void* B, const void* E, void* C, void* C2, float alpha,
                    float beta, float gamma, float oscale, void* stream) {
  try {
    if (kind == 0 && !B) B = A;  // X X^T: the second operand is X itself
    if (!ctx || !A || !B || !C) return MUON_ERR_ARG;
    if (kind < 0 || kind > 2 || (ns_dtype != MUON_F32 && ns_dtype != MUON_BF16)) return MUON_ERR_ARG;
    if (tile < 0 || tile >= TILE_COUNT) return MUON_ERR_ARG;
    if (M < 64 || N < 64 || K < 64 || M % 64 || N % 64 || K % 64 || M > kMaxDim || N > kMaxDim ||
        K > kMaxDim)
      return MUON_ERR_ARG;
    if ((kind == 0 || kind == 1) && (M != N || tile_bm(tile) != tile_bn(tile))) return MUON_ERR_ARG;
    if (!dma_addressable(M, K, N, K, ns_dtype == MUON_F32 ? 4 : 2)) tile = staged_tile(tile);
    if (ctx->device < 0) return MUON_ERR_DEVICE;
    DeviceGuard dg(ctx->device);
    if (!dg.ok) return MUON_ERR_HIP;
    GemmParams p;
    std::memset(&p, 0, sizeof(p));
    p.count = 1;
    p.A = A; p.B = B; p.C = C; p.E = E;
    p.M = static_cast<int32_t>(M); p.N = static_cast<int32_t>(N); p.K = static_cast<int32_t>(K);
    p.Mvalid = p.M; p.Nvalid = p.N;
    p.alpha = alpha; p.beta = beta; p.gamma = gamma; p.oscale = oscale;
    p.lda = K; p.ldb = K;
    GemmOp op;
    if (kind == 2) {
      op = OP_APPLY;
      p.C2 = C2;
      p.ldc = N; p.ldc2 = M; p.lde = M; p.e_trans = 1;
      p.tiles_m = static_cast<int32_t>((M + tile_bm(tile) - 1) / tile_bm(tile));
      p.tiles_n = static_cast<int32_t>((N + tile_bn(tile) - 1) / tile_bn(tile));
      p.tiles = p.tiles_m * p.tiles_n;
    } else {
      op = kind == 0 ? OP_SYRK_IN : OP_SYM;
      p.ldc = N; p.lde = N;
      p.e_from_a = (kind == 1 && E != nullptr && E == A && K == N) ? 1 : 0;
      const int nt = static_cast<int>((M + tile_bm(tile) - 1) / tile_bm(tile));
      p.tiles_m = p.tiles_n = nt;
      p.tiles = nt * (nt + 1) / 2;
    }
    const hipError_t le = launch_gemm(op, ns_dtype == MUON_F32, tile, p, static_cast<hipStream_t>(stream));
    if (le == hipErrorInvalidValue) return MUON_ERR_UNSUPPORTED;
    if (le != hipSuccess) return MUON_ERR_HIP;
    return MUON_OK;
  } catch (...) {
    return MUON_ERR_HIP;
  }
}

int muon_profile_read(muon_ctx* ctx, muon_profile_entry* out, int capacity, int* n_out) {
  try {
    if (!ctx || !n_out || capacity < 0 || (capacity > 0 && !out)) return MUON_ERR_ARG;
    *n_out = 0;
    if (!(ctx->flags & MUON_FLAG_PROFILE)) return MUON_ERR_ARG;
    if (ctx->records.empty()) return MUON_OK;
    DeviceGuard dg(ctx->device);
    if (!dg.ok) return MUON_ERR_HIP;
    if (hipEventSynchronize(ctx->records.back().stop) != hipSuccess) return MUON_ERR_HIP;
    std::map<std::tuple<int, int64_t, int64_t, int, int>, muon_profile_entry> agg;
    std::vector<std::tuple<int, int64_t, int64_t, int, int>> order;
    for (const ProfRecord& r : ctx->records) {
      float ms = 0.0f;
      if (hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) return MUON_ERR_HIP;
      const auto key = std::make_tuple(r.stage, r.m, r.n, r.count, r.tile);
      auto it = agg.find(key);
      if (it == agg.end()) {
        muon_profile_entry e;
        std::memset(&e, 0, sizeof(e));
        std::strncpy(e.stage, kStageNames[r.stage], sizeof(e.stage) - 1);
        e.m = r.m; e.n = r.n; e.count = r.count; e.tile = r.tile;
        it = agg.emplace(key, e).first;
        order.push_back(key);
      }
      it->second.launches += 1;
      it->second.total_ms += ms;
      it->second.flops += r.flops;
      it->second.bytes += r.bytes;
    }
    ctx->records.clear();
    ctx->next_event = 0;
    int n = 0;
    for (const auto& k : order) {
      if (n < capacity) out[n] = agg[k];
      ++n;
    }
    *n_out = n;
    return n > capacity ? MUON_ERR_ARG : MUON_OK;
  } catch (...) {
    return MUON_ERR_HIP;
  }
}

void muon_adamw_hparams_default(muon_adamw_hparams* hp) {
  if (!hp) return;
  hp->lr = 1e-3f;
  hp->beta1 = 0.9f;
  hp->beta2 = 0.999f;
  hp->eps = 1e-8f;
  hp->weight_decay = 0.01f;
  hp->step = 1;
  hp->w_dtype = MUON_F32;
  hp->g_dtype = MUON_BF16;
}

int muon_adamw_step(muon_ctx* ctx, const muon_adamw_tensor* tensors, int count, const muon_adamw_hparams* hp,
                    void* stream) {
  try {
    if (!ctx || !hp || count < 0 || (count > 0 && !tensors)) return MUON_ERR_ARG;
    if (!finite(hp->lr) || !finite(hp->weight_decay) || !finite(hp->eps) || hp->eps < 0.0f) return MUON_ERR_ARG;
    if (!finite(hp->beta1) || !finite(hp->beta2) || hp->beta1 < 0.0f || hp->beta1 >= 1.0f ||
        hp->beta2 < 0.0f || hp->beta2 >= 1.0f || hp->step < 1)
      return MUON_ERR_ARG;
    if ((hp->w_dtype != MUON_F32 && hp->w_dtype != MUON_BF16) || (hp->g_dtype != MUON_F32 && hp->g_dtype != MUON_BF16))
      return MUON_ERR_ARG;
    for (int i = 0; i < count; ++i) {
      const muon_adamw_tensor& t = tensors[i];
      if (t.numel < 0) return MUON_ERR_ARG;
      if (t.numel > 0 && (!t.W || !t.G || !t.m || !t.v)) return MUON_ERR_ARG;
    }
    if (count == 0) return MUON_OK;
    if (ctx->device < 0) return MUON_ERR_DEVICE;
    DeviceGuard dg(ctx->device);
    if (!dg.ok) return MUON_ERR_HIP;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    // bias corrections in double, then fp32 (as the kernel computes)
    const double bc1 = 1.0 - std::pow(static_cast<double>(hp->beta1), hp->step);
    const double bc2 = 1.0 - std::pow(static_cast<double>(hp->beta2), hp->step);
    AdamChunk c;
    std::memset(&c, 0, sizeof(c));
    c.w_bf16 = hp->w_dtype == MUON_BF16; c.g_bf16 = hp->g_dtype == MUON_BF16;
    c.lr = hp->lr; c.wd = hp->weight_decay; c.b1 = hp->beta1; c.b2 = hp->beta2; c.eps = hp->eps;
    c.bc1 = static_cast<float>(bc1);
    c.bc2s = static_cast<float>(std::sqrt(bc2));
    int64_t blocks = 0;
    auto flush = [&]() -> hipError_t {
      const hipError_t e = launch_adamw(c, blocks, st);
      c.n = 0;
      blocks = 0;
      return e;
    };
    for (int i = 0; i < count; ++i) {
      const muon_adamw_tensor& t = tensors[i];
      if (t.numel == 0) continue;
      const int64_t nb = adam_blocks(t.numel);
      if (c.n == kAdamChunk || blocks + nb > (int64_t{1} << 31) - 1) MUON_HIP(flush());
      AdamTensor& a = c.t[c.n++];
      a.W = t.W; a.G = t.G; a.m = t.m; a.v = t.v;
      a.numel = t.numel;
      a.block0 = blocks;
      auto al16 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) % 16) == 0; };
      a.vec = al16(t.W) && al16(t.G) && al16(t.m) && al16(t.v);
      blocks += nb;
    }
    MUON_HIP(flush());
    return MUON_OK;
  } catch (...) {
    return MUON_ERR_HIP;
  }
}

int muon_destroy(muon_ctx* ctx) {
  if (!ctx) return MUON_OK;
  if (ctx->device >= 0) {
    DeviceGuard dg(ctx->device);
    for (auto& ev : ctx->event_pool) {
      (void)hipEventDestroy(ev.first);
      (void)hipEventDestroy(ev.second);
    }
    for (hipEvent_t ev : ctx->tune_ev)
      if (ev) (void)hipEventDestroy(ev);
    for (hipStream_t st : ctx->lanes) {
      (void)hipStreamSynchronize(st);
      (void)hipStreamDestroy(st);
    }
    for (hipEvent_t ev : ctx->lane_join) (void)hipEventDestroy(ev);
    if (ctx->lane_fork) (void)hipEventDestroy(ctx->lane_fork);
  }
  delete ctx;
  return MUON_OK;
}

const char* muon_status_str(int status) {
  switch (status) {
    case MUON_OK: return "MUON_OK: success";
    case MUON_ERR_ARG: return "MUON_ERR_ARG: invalid argument";
    case MUON_ERR_WORKSPACE: return "MUON_ERR_WORKSPACE: workspace null, misaligned or too small";
    case MUON_ERR_DEVICE: return "MUON_ERR_DEVICE: invalid device or not gfx950";
    case MUON_ERR_HIP: return "MUON_ERR_HIP: HIP runtime or launch failure";
    case MUON_ERR_UNSUPPORTED: return "MUON_ERR_UNSUPPORTED: request not implemented";
    default: return "unknown muon status";
  }
}

}  // extern "C"

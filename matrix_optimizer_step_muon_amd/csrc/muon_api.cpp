// C ABI of the whole-tensor Muon step (include/muon.h): validation, the
// static plan (orientation, padding, LPT tile tables, workspace layout) and
// the per-step launch sequence.
//
// The plan is computed once and reused every step, as the pages' planners are
// (Canzona analysis page, section 3.3, "Output and offline nature"). Each
// GEMM phase's tile list is sorted by cost, longest first. This is the pages'
// LPT rule (section 3.4, "Why LPT ordering matters"), with the cost of a tile
// taken as its exact multiply-add count. The pages also weigh a FLOPs-based cost
// against numel (section 5, Figure 16).

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <string>
#include <utility>
#include <vector>

#include "muon.h"
#include "muon_internal.h"

namespace {

thread_local std::string g_last_error;

muon_status fail(muon_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

muon_status hip_fail(hipError_t e, const char* what) {
  return fail(MUON_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Largest rows or cols. GEMM tile coordinates are packed in 16 bits each
// (Tile::ij), so a dimension may span at most 65536 tiles: 2^24 elements with
// the bf16 engine's 256-wide tiles, 2^23 with the fp32 engine's 128-wide ones.
constexpr int64_t kMaxDim = int64_t(1) << 24;
constexpr int64_t kMaxDimF32 = int64_t(65536) * muon::kTileF32;
constexpr int32_t kMaxNsSteps = 1000;

}  // namespace

// The error path of the other translation units (muon_partition.cpp); not
// exported from the library.
__attribute__((visibility("hidden"))) muon_status muon_fail_message(muon_status st, const char* msg) {
  return fail(st, msg);
}

struct muon_plan_s {
  muon_hparams hp{};
  int dtype = 1;       // muon_dtype: the storage types of w, g, m, delta
  int gemm_dtype = 1;  // the Newton-Schulz engine: 1 bf16, 0 fp32
  int elem = 2;        // workspace element size (X, A, B)
  int n = 0;
  int device = 0;
  int tile = muon::kTileBF16;
  int variant = muon::kGemm4W;

  std::vector<muon::MatDev> mats;  // host copy (device pointers inside)
  void* ws = nullptr;
  size_t ws_bytes = 0;
  bool ws_owned = false;  // allocated by the plan (muon_plan), not the static scratch

  muon::MatDev* d_mats = nullptr;
  int32_t* d_prefix = nullptr;
  float* d_partials = nullptr;
  float* d_scale = nullptr;
  int32_t* d_counters = nullptr;
  int32_t n_counters = 0;
  // Matrices are stored chain by chain: chain c owns the plan's matrices
  // [chain_first[c], chain_first[c + 1]). d_cprefix holds, at chain_first[c] + c,
  // that chain's own elementwise-tile prefix (starting at 0).
  std::vector<int32_t> chain_first;
  std::vector<int32_t> chain_ew_blocks;
  int32_t* d_cprefix = nullptr;
  // With several chains, the chains fork at the start of a step and each runs
  // the momentum and norm kernels over its own matrices. MUON_SPLIT_PROLOGUE=0
  // (a tuning knob) runs one momentum and one norm kernel over all matrices
  // before the fork instead.
  bool split_prologue = true;
  // GEMM phases run as `chains` independent chains of launches over disjoint
  // groups of matrices, chain 0 on the caller's stream and chain c on aux[c-1].
  // A chain's persistent kernel takes CUs only as the other chain's kernel
  // retires workgroups, i.e. in its tail, so the chains fill each other's
  // tails. Per chain: one tile table per phase.
  struct Chain {
    muon::Tile* d_tiles[3] = {nullptr, nullptr, nullptr};
    int32_t* d_qoff = nullptr;  // 3 x (kQueues + 1) queue offsets
    int32_t n_tiles[3] = {0, 0, 0};
    int32_t grid[3] = {0, 0, 0};
    int update_variant = muon::kGemm4W;  // engine of this chain's update launches
    muon::Tile* d_red = nullptr;         // this chain's split Gram tiles (reduce list)
    int32_t n_red = 0;
  };
  float* d_kpart = nullptr;  // split-K partial sums of the Gram pieces
  int32_t split_slots = 0;
  std::vector<Chain> chains;
  std::vector<hipStream_t> aux;
  hipEvent_t ev_fork = nullptr;
  std::vector<hipEvent_t> ev_join;
  int32_t ew_blocks = 0;

  bool timing = false;
  struct Rec { int kind; hipEvent_t start, end; };
  std::vector<Rec> pending;
  std::vector<hipEvent_t> pool;
  double total_ms[MUON_K_COUNT] = {};
  int64_t launches[MUON_K_COUNT] = {};
};

extern "C" {

const char* muon_last_error(void) { return g_last_error.c_str(); }

muon_status muon_hparams_default(muon_hparams* hp) {
  if (!hp) return fail(MUON_ERR_INVALID_ARG, "hp is NULL");
  hp->lr = 0.02f;
  hp->beta = 0.95f;
  hp->eps = 1e-7f;
  hp->a = 3.4445f;
  hp->b = -4.7750f;
  hp->c = 2.0315f;
  hp->ns_steps = 5;
  hp->nesterov = 1;
  hp->dtype = MUON_BF16;
  return MUON_OK;
}

}  // extern "C"

namespace {

muon_status validate(const muon_matrix* mats, int32_t n, const muon_hparams* hp) {
  if (!mats) return fail(MUON_ERR_INVALID_ARG, "mats is NULL");
  if (n < 1) return fail(MUON_ERR_INVALID_ARG, "n must be >= 1");
  if (!hp) return fail(MUON_ERR_INVALID_ARG, "hp is NULL");
  const float fs[6] = {hp->lr, hp->beta, hp->eps, hp->a, hp->b, hp->c};
  const char* names[6] = {"lr", "beta", "eps", "a", "b", "c"};
  for (int i = 0; i < 6; ++i)
    if (!std::isfinite(fs[i])) return fail(MUON_ERR_INVALID_ARG, std::string(names[i]) + " is not finite");
  if (!(hp->beta >= 0.f && hp->beta < 1.f)) return fail(MUON_ERR_INVALID_ARG, "beta must be in [0, 1)");
  if (hp->eps < 0.f) return fail(MUON_ERR_INVALID_ARG, "eps must be >= 0");
  if (hp->ns_steps < 0 || hp->ns_steps > kMaxNsSteps)
    return fail(MUON_ERR_INVALID_ARG, "ns_steps must be in [0, 1000]");
  if (hp->nesterov != 0 && hp->nesterov != 1) return fail(MUON_ERR_INVALID_ARG, "nesterov must be 0 or 1");
  if (hp->dtype != MUON_F32 && hp->dtype != MUON_BF16 && hp->dtype != MUON_BF16_F32_MASTER)
    return fail(MUON_ERR_UNSUPPORTED, "dtype must be MUON_F32, MUON_BF16 or MUON_BF16_F32_MASTER");
  // Element sizes of w, g, m and delta.
  const size_t es[4] = {hp->dtype == MUON_BF16 ? 2u : 4u, hp->dtype == MUON_F32 ? 4u : 2u,
                        hp->dtype == MUON_BF16 ? 2u : 4u, hp->dtype == MUON_BF16 ? 2u : 4u};

  struct Range { uintptr_t lo, hi; int mat; const char* what; };
  std::vector<Range> ranges;
  ranges.reserve(size_t(n) * 4);
  for (int32_t i = 0; i < n; ++i) {
    const muon_matrix& d = mats[i];
    const std::string at = "matrix " + std::to_string(i) + ": ";
    if (d.rows < 1 || d.cols < 1) return fail(MUON_ERR_INVALID_ARG, at + "rows and cols must be >= 1");
    if (d.rows > kMaxDim || d.cols > kMaxDim)
      return fail(MUON_ERR_INVALID_ARG, at + "rows and cols must be <= 2^24");
    if (hp->dtype == MUON_F32 && (d.rows > kMaxDimF32 || d.cols > kMaxDimF32))
      return fail(MUON_ERR_INVALID_ARG, at + "rows and cols must be <= 2^23 for MUON_F32");
    if (!d.g) return fail(MUON_ERR_INVALID_ARG, at + "g is NULL");
    if (!d.m) return fail(MUON_ERR_INVALID_ARG, at + "m is NULL");
    if (!d.w && !d.delta) return fail(MUON_ERR_INVALID_ARG, at + "w and delta are both NULL");
    const void* ptrs[4] = {d.w, d.g, d.m, d.delta};
    const char* what[4] = {"w", "g", "m", "delta"};
    for (int k = 0; k < 4; ++k) {
      if (!ptrs[k]) continue;
      const uintptr_t p = reinterpret_cast<uintptr_t>(ptrs[k]);
      if (p % 16 != 0) return fail(MUON_ERR_ALIGN, at + what[k] + " is not 16-byte aligned");
      ranges.push_back({p, p + uintptr_t(d.rows) * uintptr_t(d.cols) * es[k], i, what[k]});
    }
  }
  std::sort(ranges.begin(), ranges.end(), [](const Range& x, const Range& y) { return x.lo < y.lo; });
  for (size_t k = 1; k < ranges.size(); ++k)
    if (ranges[k].lo < ranges[k - 1].hi)
      return fail(MUON_ERR_ALIAS, "matrix " + std::to_string(ranges[k - 1].mat) + " " + ranges[k - 1].what +
                                      " overlaps matrix " + std::to_string(ranges[k].mat) + " " +
                                      ranges[k].what);
  return MUON_OK;
}

void free_plan(muon_plan_s* p) {
  if (!p) return;
  for (auto st : p->aux) (void)hipStreamDestroy(st);
  for (auto e : p->ev_join) (void)hipEventDestroy(e);
  if (p->ev_fork) (void)hipEventDestroy(p->ev_fork);
  if (p->ws && p->ws_owned) (void)hipFree(p->ws);
  for (auto& r : p->pending) { (void)hipEventDestroy(r.start); (void)hipEventDestroy(r.end); }
  for (auto e : p->pool) (void)hipEventDestroy(e);
  delete p;
}

// Host-side tables of a plan and their places in the workspace (byte
// offsets from its base). The plan's own fields hold the rest of the layout.
struct PlanTables {
  std::vector<size_t> off;  // per matrix: X ping, X pong, A, B
  size_t o_mats = 0, o_prefix = 0, o_cprefix = 0, o_parts = 0, o_scale = 0, o_ctr = 0;
  size_t o_qoff[8] = {};
  size_t o_tiles[8][3] = {};
  size_t o_red[8] = {};
  size_t o_kpart = 0;
  std::vector<int32_t> prefix, cprefix;
  std::vector<int32_t> qoff[8];
  std::vector<muon::Tile> tiles[8][3];
  std::vector<muon::Tile> red[8];
};

// One host -> device copy of a table into the workspace.
struct Upload { void* dst; const void* src; size_t bytes; };

// The host half of a plan: orientation, padding, chains, LPT tile tables and
// the workspace layout (p->ws_bytes). No HIP call. one_chain: a single chain
// whatever the tuning knobs say (the no-allocation step has no second
// stream). Arguments are validated by the caller.
// Split-K pieces of each matrix's Gram tiles (1: whole tiles).
//
// A Gram launch whose tiles are too few, or too unequal, to keep every CU
// busy lasts as long as its longest tile: one 1024 x 8192 matrix has 10 Gram
// tiles of K = 8192 for 256 CUs. Cutting the longest tiles along K into
// pieces that run on separate CUs, and adding the pieces' partial sums
// afterwards in a reduce launch, balances the launch. The choice is the
// pages' LPT reasoning applied to pieces of work (Canzona analysis page,
// section 3.4, "Why LPT ordering matters"): the planner estimates the
// launch's makespan with longest-first list scheduling over the CUs, in
// units of one 64-deep K step, for a few piece counts, and keeps the best if
// it saves at least 20% (the estimate is rough, and a split that gains
// little can lose: see below). Only tiles longer than an even share of the work are
// cut, into pieces of at least 4 K chunks of 256. The costs, measured on
// MI355X: a whole tile carries its epilogue (about 6 steps); a piece the
// store of its 256 KB of fp32 partial sums, which all CUs issue at about the
// same time (about 14 steps); a split the reduce launch (4 steps of launch
// gap, and its traffic, each piece read and each tile written once, at about
// 3.5 TB/s). With these, one 1024 x 8192 matrix goes from 1.16 to 0.70 ms per
// step and two 1024 x 5120 ones from 0.91 to 0.69 ms, while the Qwen3-1.7B
// layer (where the three MLP matrices' tiles are three times as long as the
// others, but there are 200 of them) and a 4096 x 16384 matrix (136 tiles of
// K = 16384) are faster whole, and stay whole. The pieces depend only on the
// batch's shapes and the CU count, not on the chains or block shapes, so
// those still change no result. MUON_SPLIT_K=S (a test and tuning knob) cuts
// every Gram tile into min(S, chunks / 2) pieces instead; S = 1 turns
// splitting off.
std::vector<int> gram_pieces(const std::vector<muon::MatDev>& mats, int64_t T, int n_cu) {
  const int n = int(mats.size());
  std::vector<int> one(n, 1);
  std::vector<int64_t> chunks(n), tiles(n);
  for (int i = 0; i < n; ++i) {
    chunks[i] = mats[i].np / 256;
    const int64_t tm = mats[i].mp / T;
    tiles[i] = tm * (tm + 1) / 2;
  }
  if (const char* v = std::getenv("MUON_SPLIT_K")) {
    const int S = std::max(1, std::min(muon::kMaxSplit, std::atoi(v)));
    std::vector<int> forced(n);
    for (int i = 0; i < n; ++i) forced[i] = int(std::max<int64_t>(1, std::min<int64_t>(S, chunks[i] / 2)));
    return forced;
  }
  // Costs in 64-deep K steps (about 1.6 us each on MI355X at its power limit).
  constexpr double kWhole = 6.0, kPiece = 14.0, kGap = 4.0;
  constexpr double kReduceBytesPerStep = 3.5e12 * 1.6e-6;
  constexpr double kPartBytes = 4.0 * muon::kPartFloats;
  double work = 0.0, longest = 0.0;
  for (int i = 0; i < n; ++i) {
    work += double(tiles[i]) * double(chunks[i] * 4);
    longest = std::max(longest, double(chunks[i] * 4));
  }
  if (n_cu < 1) return one;
  const double share = work / n_cu;
  if (longest <= share) return one;
  auto makespan = [&](const std::vector<int>& S) {
    std::vector<double> items;
    double reduce_bytes = 0.0;
    for (int i = 0; i < n; ++i) {
      for (int p = 0; p < S[i]; ++p) {
        const int64_t len = (p + 1) * chunks[i] / S[i] - p * chunks[i] / S[i];
        items.insert(items.end(), size_t(tiles[i]), double(len * 4) + (S[i] > 1 ? kPiece : kWhole));
      }
      if (S[i] > 1) reduce_bytes += double(tiles[i]) * (S[i] + 1) * kPartBytes;
    }
    std::sort(items.begin(), items.end(), std::greater<double>());
    std::vector<double> load(size_t(n_cu), 0.0);  // a min-heap of CU loads
    for (double x : items) {
      std::pop_heap(load.begin(), load.end(), std::greater<double>());
      load.back() += x;
      std::push_heap(load.begin(), load.end(), std::greater<double>());
    }
    double span = *std::max_element(load.begin(), load.end());
    if (reduce_bytes > 0.0) span += kGap + reduce_bytes / kReduceBytesPerStep;
    return span;
  };
  std::vector<int> best = one;
  const double base = makespan(one);
  double best_span = base;
  for (int S : {2, 3, 4, 6, 8, 12, 16}) {
    std::vector<int> cand(n, 1);
    for (int i = 0; i < n; ++i)
      if (double(chunks[i] * 4) > share) cand[i] = int(std::max<int64_t>(1, std::min<int64_t>(S, chunks[i] / 4)));
    const double span = makespan(cand);
    if (span < best_span) { best_span = span; best = cand; }
  }
  return best_span < 0.8 * base ? best : one;
}

muon_status plan_host(const muon_matrix* mats, int32_t n, const muon_hparams* hp, bool one_chain, int n_cu,
                      muon_plan_s* p, PlanTables& t) {
  std::vector<size_t>& off = t.off;
  std::vector<int32_t>& prefix = t.prefix;
  std::vector<int32_t>& cprefix = t.cprefix;
  size_t &o_mats = t.o_mats, &o_prefix = t.o_prefix, &o_cprefix = t.o_cprefix, &o_parts = t.o_parts,
         &o_scale = t.o_scale, &o_ctr = t.o_ctr;
  auto& o_qoff = t.o_qoff;
  auto& o_tiles = t.o_tiles;
  auto& qoff = t.qoff;
  auto& tiles = t.tiles;
  p->hp = *hp;
  p->dtype = hp->dtype;
  // Newton-Schulz runs in bf16 for MUON_BF16 and MUON_BF16_F32_MASTER.
  p->gemm_dtype = hp->dtype == MUON_F32 ? 0 : 1;
  p->elem = p->gemm_dtype == 1 ? 2 : 4;
  p->n = n;
  p->tile = p->gemm_dtype == 1 ? muon::kTileBF16 : muon::kTileF32;
  const int64_t T = p->tile;

  // MUON_GEMM_VARIANT=0|1|2|3 picks the bf16 engine pipeline (a tuning knob;
  // the default is the four-wave engine, 2).
  bool variant_forced = false;
  if (const char* v = std::getenv("MUON_GEMM_VARIANT")) {
    const int k = std::atoi(v);
    p->variant = k == 0 ? muon::kGemmBK64 : k == 1 ? muon::kGemmBK32 : k == 3 ? muon::kGemm4WDeep : muon::kGemm4W;
    variant_forced = true;
  }
  // Chains: two for the bf16 four-wave engines (MUON_CHAINS=C overrides, C in
  // [1, 8]), one otherwise; never more than there are matrices. Matrices go
  // largest first (multiply-adds of one iteration) to the lightest chain.
  const bool four_wave = p->variant == muon::kGemm4W || p->variant == muon::kGemm4WDeep;
  if (p->dtype == MUON_BF16_F32_MASTER && !four_wave)
    return fail(MUON_ERR_UNSUPPORTED, "MUON_BF16_F32_MASTER needs the four-wave GEMM engine (MUON_GEMM_VARIANT 2 or 3)");
  int C = (p->gemm_dtype == 1 && four_wave) ? 2 : 1;
  if (const char* v = std::getenv("MUON_CHAINS")) C = std::max(1, std::min(8, std::atoi(v)));
  C = std::min<int>(C, n);
  if (one_chain) C = 1;
  std::vector<std::vector<int32_t>> members(C);
  {
    std::vector<std::pair<int64_t, int32_t>> wts(n);
    for (int32_t i = 0; i < n; ++i) {
      const int64_t mp = int64_t(round_up(size_t(std::min(mats[i].rows, mats[i].cols)), size_t(T)));
      const int64_t np = int64_t(round_up(size_t(std::max(mats[i].rows, mats[i].cols)), size_t(T)));
      const int64_t tm = mp / T, tn = np / T, sym = tm * (tm + 1) / 2;
      wts[i] = {sym * np + sym * mp + tm * tn * mp, i};
    }
    std::stable_sort(wts.begin(), wts.end(), [](const auto& x, const auto& y) { return x.first > y.first; });
    std::vector<int64_t> load(C, 0);
    for (const auto& w : wts) {
      int best = 0;
      for (int c = 1; c < C; ++c)
        if (load[c] < load[best]) best = c;
      load[best] += w.first;
      members[best].push_back(w.second);
    }
    for (auto& g : members) std::sort(g.begin(), g.end());
  }
  // The plan stores each chain's matrices contiguously, chain 0 first, in
  // descriptor order within a chain: order[k] is the descriptor of slot k.
  std::vector<int32_t> order;
  p->chain_first.assign(C + 1, 0);
  for (int c = 0; c < C; ++c) {
    p->chain_first[c] = int32_t(order.size());
    order.insert(order.end(), members[c].begin(), members[c].end());
  }
  p->chain_first[C] = n;
  if (const char* v = std::getenv("MUON_SPLIT_PROLOGUE")) p->split_prologue = std::atoi(v) != 0;

  // Orientation, padding and workspace offsets.
  p->mats.resize(n);
  off.assign(size_t(n) * 4, 0);
  size_t cursor = 0;
  auto take = [&](size_t bytes) { size_t o = cursor; cursor = round_up(cursor + bytes, 256); return o; };
  prefix.assign(n + 1, 0);
  int32_t parts = 0;
  for (int32_t i = 0; i < n; ++i) {
    const muon_matrix& s = mats[order[i]];
    muon::MatDev& d = p->mats[i];
    std::memset(&d, 0, sizeof(d));
    d.rows = int32_t(s.rows);
    d.cols = int32_t(s.cols);
    d.tall = s.rows > s.cols;
    d.m = int32_t(std::min(s.rows, s.cols));
    d.n = int32_t(std::max(s.rows, s.cols));
    d.mp = int32_t(round_up(d.m, T));
    d.np = int32_t(round_up(d.n, T));
    d.ew_tiles_c = int32_t((s.cols + muon::kEwTile - 1) / muon::kEwTile);
    const int32_t tr = int32_t((s.rows + muon::kEwTile - 1) / muon::kEwTile);
    d.n_parts = tr * d.ew_tiles_c;
    d.part_off = parts;
    parts += d.n_parts;
    prefix[i + 1] = prefix[i] + d.n_parts;
    d.lr_scale = float(double(hp->lr) * std::sqrt(std::max(1.0, double(s.rows) / double(s.cols))));
    d.w = s.w;
    d.delta = s.delta;
    d.g = s.g;
    d.mom = s.m;
    // Row strides are one 128-byte line longer than the padded width. All
    // padded widths are multiples of 16 lines, and without the skew the rows
    // of a tile would fall on the same L2 channel.
    const int32_t skew = int32_t(128 / p->elem);
    d.ldx = d.np + skew;
    d.lda = d.mp + skew;
    const size_t xbytes = size_t(d.mp) * d.ldx * p->elem;
    const size_t abytes = size_t(d.mp) * d.lda * p->elem;
    off[i * 4 + 0] = take(xbytes);
    off[i * 4 + 1] = take(xbytes);
    off[i * 4 + 2] = take(abytes);
    off[i * 4 + 3] = take(abytes);
  }
  p->ew_blocks = prefix[n];
  cprefix.assign(n + C, 0);
  p->chain_ew_blocks.assign(C, 0);
  for (int c = 0; c < C; ++c) {
    const int32_t f = p->chain_first[c], base = f + c;
    for (int32_t i = f; i < p->chain_first[c + 1]; ++i) cprefix[base + (i - f) + 1] = cprefix[base + (i - f)] + (prefix[i + 1] - prefix[i]);
    p->chain_ew_blocks[c] = prefix[p->chain_first[c + 1]] - prefix[f];
  }
  o_mats = take(sizeof(muon::MatDev) * n);
  o_prefix = take(sizeof(int32_t) * (n + 1));
  o_cprefix = take(sizeof(int32_t) * (n + C));
  o_parts = take(sizeof(float) * std::max(parts, 1));
  o_scale = take(sizeof(float) * n);
  p->chains.resize(C);
  p->n_counters = std::max(C * 3 * hp->ns_steps * muon::kQueues, 1);
  o_ctr = take(sizeof(int32_t) * p->n_counters);

  // Tile tables. Each phase's tiles are cut into blocks of kBlockRows x
  // kBlockCols tiles of one matrix. Blocks are dealt longest first to the
  // least-loaded of the kQueues per-XCD queues: the LPT rule, with a block's
  // cost = its multiply-adds = tiles x tile area x K. All tiles of a phase have
  // the same area, so the cost is tiles x K. Ties keep (matrix, block) order,
  // and a block's tiles stay in row-major order.
  struct Block { int64_t cost; std::vector<muon::Tile> tiles; };
  std::vector<Block> blocks[8][3];
  // Blocks are walked column-major: consecutive blocks, dealt to different
  // XCDs, share the column operand's panels in the Infinity Cache. Tuning
  // knobs: MUON_BLOCK=RxC sets the block shape in tiles, and
  // MUON_BLOCK_ORDER=0 walks blocks row-major instead.
  // 4 x 4 blocks: 1.2% less step time than 4 x 8 on the Qwen3-32B layer with
  // two chains, 0.9% with one (same GPU; 2 x 8, 4 x 2, 2 x 4, 3 x 4, 4 x 3,
  // 4 x 6, 6 x 4 and 8 x 4 are all slower than 4 x 4).
  // bf16 matrices of at most kSmallTileRows tile rows take kSmallBlock x
  // kSmallBlock blocks (small_blocks); MUON_BLOCK or MUON_BLOCK_PHASES set one
  // shape for every matrix instead.
  int brows_ph[3], bcols_ph[3], border = 1;
  bool small_blocks = p->gemm_dtype == 1;
  for (int ph = 0; ph < 3; ++ph) { brows_ph[ph] = muon::kBlockRows; bcols_ph[ph] = muon::kBlockCols; }
  if (const char* v = std::getenv("MUON_BLOCK")) {
    int r = 0, c = 0;
    if (std::sscanf(v, "%dx%d", &r, &c) == 2 && r > 0 && c > 0 && r * c <= 1024) {
      for (int ph = 0; ph < 3; ++ph) { brows_ph[ph] = r; bcols_ph[ph] = c; }
      small_blocks = false;
    }
  }
  // MUON_BLOCK_PHASES=RxC,RxC,RxC: one shape per phase (gram, square, update).
  if (const char* v = std::getenv("MUON_BLOCK_PHASES")) {
    int r[3] = {0, 0, 0}, c[3] = {0, 0, 0};
    if (std::sscanf(v, "%dx%d,%dx%d,%dx%d", &r[0], &c[0], &r[1], &c[1], &r[2], &c[2]) == 6)
      for (int ph = 0; ph < 3; ++ph)
        if (r[ph] > 0 && c[ph] > 0 && r[ph] * c[ph] <= 1024) {
          brows_ph[ph] = r[ph];
          bcols_ph[ph] = c[ph];
          small_blocks = false;
        }
  }
  if (const char* v = std::getenv("MUON_BLOCK_ORDER")) border = std::atoi(v) != 0;
  // Split-K pieces of the Gram tiles (bf16 four-wave engines), their
  // partial-sum slots (consecutive per tile) and each chain's reduce list.
  std::vector<int> pieces(n, 1);
  if (p->gemm_dtype == 1 && four_wave) pieces = gram_pieces(p->mats, T, n_cu);
  std::vector<int32_t> slot_base(n, 0);
  int32_t slots = 0;
  for (int c = 0; c < C; ++c)
    for (int32_t i = p->chain_first[c]; i < p->chain_first[c + 1]; ++i) {
      slot_base[i] = slots;
      if (pieces[i] < 2) continue;
      const int32_t tm = int32_t(p->mats[i].mp / T);
      for (int32_t a = 0; a < tm; ++a)
        for (int32_t cc = a; cc < tm; ++cc) {
          t.red[c].push_back({i, (a << 16) | cc, pieces[i], slots});
          slots += pieces[i];
        }
    }
  p->split_slots = slots;
  // Update work (tiles x K) per chain, all of it and that of matrices with at
  // most kSmallTileRows tile rows: see update_variant below.
  int64_t upd_all[8] = {}, upd_small[8] = {};
  for (int c = 0; c < C; ++c)
  for (int32_t i = p->chain_first[c]; i < p->chain_first[c + 1]; ++i) {
    const muon::MatDev& d = p->mats[i];
    const int32_t tm = int32_t(d.mp / T), tn = int32_t(d.np / T);
    const bool small = small_blocks && tm <= muon::kSmallTileRows;
    for (int ph = 0; ph < 3; ++ph) {
      const int brows = small ? muon::kSmallBlock : brows_ph[ph], bcols = small ? muon::kSmallBlock : bcols_ph[ph];
      const int32_t cols = ph == muon::kUpdate ? tn : tm;
      const int64_t K = ph == muon::kGram ? d.np : d.mp;
      const int32_t nbr = (tm + brows - 1) / brows, nbc = (cols + bcols - 1) / bcols;
      // A split matrix's Gram blocks are formed piece by piece: the tiles of a
      // block then read the same K range of their panels.
      const int npc = ph == muon::kGram ? pieces[i] : 1;
      const int32_t chunks = int32_t(d.np / 256);
      for (int pc = 0; pc < npc; ++pc)
      for (int32_t bi = 0; bi < nbr * nbc; ++bi) {
        const int32_t r0 = (border ? bi % nbr : bi / nbc) * brows;
        const int32_t c0 = (border ? bi / nbr : bi % nbc) * bcols;
        const int32_t k0 = pc * chunks / npc, k1 = (pc + 1) * chunks / npc;
        Block b{0, {}};
        for (int32_t a = r0; a < std::min(tm, r0 + brows); ++a)
          for (int32_t c = c0; c < std::min(cols, c0 + bcols); ++c) {
            if (!(ph == muon::kUpdate || c >= a)) continue;
            if (npc == 1) {
              b.tiles.push_back({i, (a << 16) | c, 0, -1});
            } else {
              // Slot of this tile's piece: tiles are numbered row by row over
              // the upper triangle (the reduce list's order).
              const int32_t u = a * tm - a * (a - 1) / 2 + (c - a);
              b.tiles.push_back({i, (a << 16) | c, (k0 << 16) | (k1 - k0), slot_base[i] + u * npc + pc});
            }
          }
        if (b.tiles.empty()) continue;
        b.cost = int64_t(b.tiles.size()) * (npc == 1 ? K : int64_t(k1 - k0) * 256);
        if (ph == muon::kUpdate) {
          upd_all[c] += b.cost;
          if (tm <= muon::kSmallTileRows) upd_small[c] += b.cost;
        }
        blocks[c][ph].push_back(std::move(b));
      }
    }
  }
  for (int c = 0; c < C; ++c) {
  o_qoff[c] = take(sizeof(int32_t) * 3 * (muon::kQueues + 1));
  qoff[c].assign(3 * (muon::kQueues + 1), 0);
  for (int ph = 0; ph < 3; ++ph) {
    std::stable_sort(blocks[c][ph].begin(), blocks[c][ph].end(),
                     [](const Block& x, const Block& y) { return x.cost > y.cost; });
    std::vector<std::vector<muon::Tile>> q(muon::kQueues);
    int64_t load[muon::kQueues] = {};
    for (const Block& b : blocks[c][ph]) {
      int best = 0;
      for (int k = 1; k < muon::kQueues; ++k)
        if (load[k] < load[best]) best = k;
      load[best] += b.cost;
      q[best].insert(q[best].end(), b.tiles.begin(), b.tiles.end());
    }
    int32_t* qo = &qoff[c][ph * (muon::kQueues + 1)];
    for (int k = 0; k < muon::kQueues; ++k) {
      qo[k] = int32_t(tiles[c][ph].size());
      tiles[c][ph].insert(tiles[c][ph].end(), q[k].begin(), q[k].end());
    }
    qo[muon::kQueues] = int32_t(tiles[c][ph].size());
    p->chains[c].n_tiles[ph] = int32_t(tiles[c][ph].size());
    // A chain whose update work is mostly on matrices with m <= 4096 (K = m
    // <= 4096) runs its update launches on the four-wave engine with the
    // 4-stage ring of K step 32, which keeps three steps in flight: 4% faster
    // on such launches, 1% slower at K = 5120 (gram and square stay on the
    // default, which is faster for them at every size). Both engines sum each
    // tile's 16-deep K chunks in the same order, so the results are the same
    // bit for bit. MUON_GEMM_VARIANT sets one engine for everything.
    if (ph == muon::kUpdate)
      p->chains[c].update_variant = !variant_forced && p->gemm_dtype == 1 && p->variant == muon::kGemm4W &&
                                            2 * upd_small[c] > upd_all[c]
                                        ? muon::kGemm4WDeep
                                        : p->variant;
    o_tiles[c][ph] = take(sizeof(muon::Tile) * std::max<size_t>(tiles[c][ph].size(), 1));
  }
  p->chains[c].n_red = int32_t(t.red[c].size());
  t.o_red[c] = take(sizeof(muon::Tile) * std::max<size_t>(t.red[c].size(), 1));
  }
  t.o_kpart = take(sizeof(float) * size_t(muon::kPartFloats) * size_t(std::max(slots, 1)));
  p->ws_bytes = cursor;
  return MUON_OK;
}

// The engine choice that MUON_GEMM_VARIANT makes, checked against the dtype
// before any HIP call: fp32 master weights need a four-wave engine.
muon_status engine_check(const muon_hparams* hp) {
  if (hp->dtype != MUON_BF16_F32_MASTER) return MUON_OK;
  if (const char* v = std::getenv("MUON_GEMM_VARIANT")) {
    const int k = std::atoi(v);
    if (k == 0 || k == 1)
      return fail(MUON_ERR_UNSUPPORTED,
                  "MUON_BF16_F32_MASTER needs the four-wave GEMM engine (MUON_GEMM_VARIANT 2 or 3)");
  }
  return MUON_OK;
}

// Compute units of the current device.
muon_status device_cus(int* n_cu) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  e = hipDeviceGetAttribute(n_cu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
  return MUON_OK;
}

// Device facts of a plan on the current device: the device and the
// persistent grid of every GEMM launch (one workgroup per resident slot).
muon_status plan_device(muon_plan_s* p) {
  hipError_t e = hipGetDevice(&p->device);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  int n_cu = 0;
  e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, p->device);
  if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
  const int32_t resident = n_cu * muon::gemm_blocks_per_cu(p->gemm_dtype, p->variant);
  for (auto& ch : p->chains)
    for (int ph = 0; ph < 3; ++ph) ch.grid[ph] = std::max(1, std::min(ch.n_tiles[ph], resident));
  return MUON_OK;
}

// Points the plan at a workspace at `base` (ws_bytes long) and lists the
// table copies that fill it. The host tables must outlive the copies.
std::vector<Upload> plan_bind(muon_plan_s* p, const PlanTables& t, char* base) {
  p->ws = base;
  const int32_t n = p->n, C = int32_t(p->chains.size());
  for (int32_t i = 0; i < n; ++i) {
    muon::MatDev& d = p->mats[i];
    d.x[0] = base + t.off[i * 4 + 0];
    d.x[1] = base + t.off[i * 4 + 1];
    d.a = base + t.off[i * 4 + 2];
    d.b = base + t.off[i * 4 + 3];
  }
  p->d_mats = reinterpret_cast<muon::MatDev*>(base + t.o_mats);
  p->d_prefix = reinterpret_cast<int32_t*>(base + t.o_prefix);
  p->d_cprefix = reinterpret_cast<int32_t*>(base + t.o_cprefix);
  p->d_partials = reinterpret_cast<float*>(base + t.o_parts);
  p->d_scale = reinterpret_cast<float*>(base + t.o_scale);
  p->d_counters = reinterpret_cast<int32_t*>(base + t.o_ctr);
  std::vector<Upload> ups = {
      {p->d_mats, p->mats.data(), sizeof(muon::MatDev) * n},
      {p->d_prefix, t.prefix.data(), sizeof(int32_t) * (n + 1)},
      {p->d_cprefix, t.cprefix.data(), sizeof(int32_t) * t.cprefix.size()},
  };
  p->d_kpart = reinterpret_cast<float*>(base + t.o_kpart);
  for (int c = 0; c < C; ++c) {
    muon_plan_s::Chain& ch = p->chains[c];
    ch.d_red = reinterpret_cast<muon::Tile*>(base + t.o_red[c]);
    ups.push_back({ch.d_red, t.red[c].data(), sizeof(muon::Tile) * t.red[c].size()});
    ch.d_qoff = reinterpret_cast<int32_t*>(base + t.o_qoff[c]);
    ups.push_back({ch.d_qoff, t.qoff[c].data(), sizeof(int32_t) * t.qoff[c].size()});
    for (int ph = 0; ph < 3; ++ph) {
      ch.d_tiles[ph] = reinterpret_cast<muon::Tile*>(base + t.o_tiles[c][ph]);
      ups.push_back({ch.d_tiles[ph], t.tiles[c][ph].data(), sizeof(muon::Tile) * t.tiles[c][ph].size()});
    }
  }
  return ups;
}

}  // namespace

extern "C" {

muon_status muon_plan(const muon_matrix* mats, int32_t n, const muon_hparams* hp, muon_plan_t* out) {
  if (!out) return fail(MUON_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  muon_status st = validate(mats, n, hp);
  if (st != MUON_OK) return st;

  st = engine_check(hp);
  if (st != MUON_OK) return st;
  int n_cu = 0;
  st = device_cus(&n_cu);
  if (st != MUON_OK) return st;
  auto* p = new muon_plan_s();
  PlanTables t;
  st = plan_host(mats, n, hp, false, n_cu, p, t);
  if (st == MUON_OK) st = plan_device(p);
  if (st != MUON_OK) { free_plan(p); return st; }
  const int C = int(p->chains.size());
  hipError_t e = hipSuccess;
  // Auxiliary streams (default priority, not synchronising with the null
  // stream) and the fork / join events of the chains.
  for (int c = 1; c < C; ++c) {
    hipStream_t st = nullptr;
    e = hipStreamCreateWithFlags(&st, hipStreamNonBlocking);
    if (e != hipSuccess) { free_plan(p); return hip_fail(e, "hipStreamCreateWithFlags"); }
    p->aux.push_back(st);
    hipEvent_t ev = nullptr;
    e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
    if (e != hipSuccess) { free_plan(p); return hip_fail(e, "hipEventCreateWithFlags"); }
    p->ev_join.push_back(ev);
  }
  if (C > 1) {
    e = hipEventCreateWithFlags(&p->ev_fork, hipEventDisableTiming);
    if (e != hipSuccess) { free_plan(p); return hip_fail(e, "hipEventCreateWithFlags"); }
  }

  void* ws = nullptr;
  e = hipMalloc(&ws, p->ws_bytes);
  if (e != hipSuccess) {
    free_plan(p);
    (void)hipGetLastError();
    return fail(MUON_ERR_OOM, "hipMalloc of " + std::to_string(p->ws_bytes) + " workspace bytes failed");
  }
  p->ws = ws;
  p->ws_owned = true;
  e = hipMemset(p->ws, 0, p->ws_bytes);
  if (e != hipSuccess) { free_plan(p); return hip_fail(e, "hipMemset"); }
  const std::vector<Upload> ups = plan_bind(p, t, static_cast<char*>(ws));
  for (const Upload& u : ups) {
    if (u.bytes == 0) continue;
    e = hipMemcpy(u.dst, u.src, u.bytes, hipMemcpyHostToDevice);
    if (e != hipSuccess) { free_plan(p); return hip_fail(e, "hipMemcpy"); }
  }
  e = hipDeviceSynchronize();
  if (e != hipSuccess) { free_plan(p); return hip_fail(e, "hipDeviceSynchronize"); }
  *out = p;
  return MUON_OK;
}

muon_status muon_plan_workspace_bytes(muon_plan_t p, size_t* bytes) {
  if (!p || !bytes) return fail(MUON_ERR_INVALID_ARG, "NULL argument");
  *bytes = p->ws_bytes;
  return MUON_OK;
}

muon_status muon_plan_info(muon_plan_t p, int64_t* n_tiles, int64_t* grid) {
  if (!p) return fail(MUON_ERR_INVALID_ARG, "plan is NULL");
  for (int k = 0; k < MUON_K_COUNT; ++k) {
    int64_t t = 0, g = 0;
    if (k == MUON_K_MOMENTUM || k == MUON_K_APPLY) { t = p->ew_blocks; g = p->ew_blocks; }
    else if (k == MUON_K_NORM) { t = p->n; g = p->n; }
    else if (k == MUON_K_GRAM_REDUCE) {
      for (const auto& ch : p->chains) { t += ch.n_red; g = std::max<int64_t>(g, ch.n_red); }
    }
    else {
      for (const auto& ch : p->chains) {
        t += ch.n_tiles[k - MUON_K_GRAM];
        g = std::max<int64_t>(g, ch.grid[k - MUON_K_GRAM]);
      }
    }
    if (n_tiles) n_tiles[k] = t;
    if (grid) grid[k] = g;
  }
  return MUON_OK;
}

muon_status muon_plan_set_timing(muon_plan_t p, int32_t enable) {
  if (!p) return fail(MUON_ERR_INVALID_ARG, "plan is NULL");
  p->timing = enable != 0;
  return MUON_OK;
}

muon_status muon_plan_reset_timing(muon_plan_t p) {
  if (!p) return fail(MUON_ERR_INVALID_ARG, "plan is NULL");
  muon_status st = muon_plan_kernel_times(p, nullptr, nullptr);
  for (int k = 0; k < MUON_K_COUNT; ++k) { p->total_ms[k] = 0; p->launches[k] = 0; }
  return st;
}

muon_status muon_plan_kernel_times(muon_plan_t p, double* total_ms, int64_t* launches) {
  if (!p) return fail(MUON_ERR_INVALID_ARG, "plan is NULL");
  muon_status st = MUON_OK;
  for (auto& r : p->pending) {
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(r.end);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.start, r.end);
    if (e != hipSuccess && st == MUON_OK) st = hip_fail(e, "hipEventElapsedTime");
    p->total_ms[r.kind] += ms;
    p->launches[r.kind] += 1;
    p->pool.push_back(r.start);
    p->pool.push_back(r.end);
  }
  p->pending.clear();
  for (int k = 0; k < MUON_K_COUNT; ++k) {
    if (total_ms) total_ms[k] = p->total_ms[k];
    if (launches) launches[k] = p->launches[k];
  }
  return st;
}

muon_status muon_step(muon_plan_t p, void* stream) {
  if (!p) return fail(MUON_ERR_INVALID_ARG, "plan is NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (cur != p->device) {
    e = hipSetDevice(p->device);
    if (e != hipSuccess) return hip_fail(e, "hipSetDevice");
  }

  auto ev = [&](hipEvent_t* out) -> hipError_t {
    if (!p->pool.empty()) { *out = p->pool.back(); p->pool.pop_back(); return hipSuccess; }
    return hipEventCreate(out);
  };
  muon_status st = MUON_OK;
  auto run_on = [&](hipStream_t q, int kind, auto&& launch) {
    if (st != MUON_OK) return;
    hipEvent_t a = nullptr, b = nullptr;
    if (p->timing) {
      hipError_t r = ev(&a);
      if (r == hipSuccess) r = ev(&b);
      if (r == hipSuccess) r = hipEventRecord(a, q);
      if (r != hipSuccess) { st = hip_fail(r, "timing event"); return; }
    }
    hipError_t r = launch();
    if (r != hipSuccess) { st = hip_fail(r, "kernel launch"); return; }
    if (p->timing) {
      r = hipEventRecord(b, q);
      if (r != hipSuccess) { st = hip_fail(r, "hipEventRecord"); return; }
      p->pending.push_back({kind, a, b});
    }
  };
  auto run = [&](int kind, auto&& launch) { run_on(s, kind, launch); };
  auto sync = [&](hipError_t r, const char* what) {
    if (st == MUON_OK && r != hipSuccess) st = hip_fail(r, what);
  };

  muon::StepCoeffs co{p->hp.a, p->hp.b, p->hp.c, p->hp.beta, p->hp.eps, p->hp.nesterov};
  const int T = p->hp.ns_steps;
  const int C = int(p->chains.size());
  auto fork = [&] {
    sync(hipEventRecord(p->ev_fork, s), "hipEventRecord");
    for (auto q : p->aux) sync(hipStreamWaitEvent(q, p->ev_fork, 0), "hipStreamWaitEvent");
  };
  if (T == 0 || C == 1 || !p->split_prologue) {
    muon::EwArgs ew{p->d_mats, p->d_prefix, p->n, p->d_partials, p->d_counters, p->n_counters, p->d_scale, co};
    run(MUON_K_MOMENTUM, [&] { return muon::launch_momentum(p->dtype, ew, p->ew_blocks, s); });
    run(MUON_K_NORM, [&] { return muon::launch_norm(p->d_mats, p->d_partials, p->d_scale, p->n, p->hp.eps, s); });
    if (T == 0) run(MUON_K_APPLY, [&] { return muon::launch_apply(p->dtype, ew, p->ew_blocks, s); });
    if (T > 0 && C > 1) fork();
  } else {
    // Each chain's momentum and norm kernels cover its own matrices and clear
    // its own queue counters. The chains start together, and a chain whose
    // momentum ends first starts its GEMMs while the other's momentum (bound by
    // HBM) still runs: 0.3 ms less per step on the Qwen3-32B layer than one
    // momentum and norm kernel before the fork.
    fork();
    const int32_t per_chain = 3 * T * muon::kQueues;
    for (int c = 0; c < C; ++c) {
      hipStream_t q = c == 0 ? s : p->aux[c - 1];
      const int32_t f = p->chain_first[c], nc = p->chain_first[c + 1] - f;
      muon::EwArgs ew{p->d_mats + f, p->d_cprefix + f + c, nc, p->d_partials, p->d_counters + c * per_chain,
                      per_chain, p->d_scale + f, co};
      run_on(q, MUON_K_MOMENTUM, [&] { return muon::launch_momentum(p->dtype, ew, p->chain_ew_blocks[c], q); });
      run_on(q, MUON_K_NORM,
             [&] { return muon::launch_norm(p->d_mats + f, p->d_partials, p->d_scale + f, nc, p->hp.eps, q); });
    }
  }
  for (int it = 0; it < T; ++it) {
    for (int ph = 0; ph < 3; ++ph) {
      for (int c = 0; c < C; ++c) {
        const muon_plan_s::Chain& ch = p->chains[c];
        if (ch.n_tiles[ph] == 0) continue;
        hipStream_t q = c == 0 ? s : p->aux[c - 1];
        muon::PhaseArgs a{p->d_mats, ch.d_tiles[ph], ch.d_qoff + ph * (muon::kQueues + 1),
                          p->d_counters + ((c * T + it) * 3 + ph) * muon::kQueues, p->d_scale, it & 1, it == 0,
                          it == T - 1, p->dtype == MUON_BF16_F32_MASTER ? 1 : 0, co,
                          ph == muon::kGram && ch.n_red > 0 ? p->d_kpart : nullptr};
        run_on(q, MUON_K_GRAM + ph,
               [&] {
                 const int v = ph == muon::kUpdate ? ch.update_variant : p->variant;
                 return muon::launch_phase(p->gemm_dtype, v, muon::Phase(ph), a, ch.grid[ph], q);
               });
        if (ph == muon::kGram && ch.n_red > 0)
          run_on(q, MUON_K_GRAM_REDUCE, [&] { return muon::launch_gram_reduce(a, ch.d_red, ch.n_red, q); });
      }
    }
  }
  if (T > 0 && C > 1) {
    for (int c = 1; c < C; ++c) {
      sync(hipEventRecord(p->ev_join[c - 1], p->aux[c - 1]), "hipEventRecord");
      sync(hipStreamWaitEvent(s, p->ev_join[c - 1], 0), "hipStreamWaitEvent");
    }
  }
  if (cur != p->device) (void)hipSetDevice(cur);
  return st;
}

muon_status muon_step_noalloc(const muon_matrix* mats, int32_t n, const muon_hparams* hp, void* stream) {
  muon_status st = validate(mats, n, hp);
  if (st == MUON_OK) st = engine_check(hp);
  if (st != MUON_OK) return st;
  auto too_big = [](size_t bytes) {
    return fail(MUON_ERR_INVALID_ARG, "the batch needs " + std::to_string(bytes) + " workspace bytes, more than the " +
                                          std::to_string(muon::kScratchBytes) + " bytes of static scratch; use muon_plan");
  };
  {
    // Before any HIP call: the workspace without split-K pieces, a lower
    // bound of the one planned below.
    muon_plan_s probe;
    PlanTables t0;
    st = plan_host(mats, n, hp, true, 0, &probe, t0);
    if (st == MUON_OK && probe.ws_bytes > muon::kScratchBytes) st = too_big(probe.ws_bytes);
    if (st != MUON_OK) return st;
  }
  int n_cu = 0;
  st = device_cus(&n_cu);
  if (st != MUON_OK) return st;
  auto* p = new muon_plan_s();
  PlanTables t;
  st = plan_host(mats, n, hp, true, n_cu, p, t);
  if (st == MUON_OK && p->ws_bytes > muon::kScratchBytes) st = too_big(p->ws_bytes);
  if (st == MUON_OK) st = plan_device(p);
  void* base = nullptr;
  if (st == MUON_OK) {
    const hipError_t e = muon::scratch_address(&base);
    if (e != hipSuccess) st = hip_fail(e, "hipGetSymbolAddress");
  }
  if (st != MUON_OK) { free_plan(p); return st; }
  // The previous call's contents are still in the array: clear the
  // workspace (the X buffers' padding must read as zero), copy the tables
  // in, and run the step, all on `stream`.
  hipStream_t s = static_cast<hipStream_t>(stream);
  const std::vector<Upload> ups = plan_bind(p, t, static_cast<char*>(base));
  hipError_t e = muon::launch_zero(base, p->ws_bytes, s);
  for (size_t k = 0; e == hipSuccess && k < ups.size(); ++k)
    e = muon::launch_upload(ups[k].dst, ups[k].src, ups[k].bytes, s);
  if (e != hipSuccess) st = hip_fail(e, "kernel launch");
  if (st == MUON_OK) st = muon_step(p, stream);
  free_plan(p);  // host tables only: the workspace is the static array
  return st;
}

muon_status muon_plan_destroy(muon_plan_t p) {
  if (!p) return MUON_OK;
  hipError_t e = hipDeviceSynchronize();
  free_plan(p);
  if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize");
  return MUON_OK;
}

}  // extern "C"

// ---------------------------------------------------------------- TP shard apply

struct muon_apply_plan_s {
  int dtype = 1;
  int n = 0;
  int device = 0;
  void* ws = nullptr;
  muon::ShardDev* d_shards = nullptr;
  int32_t* d_prefix = nullptr;
  int32_t blocks = 0;
};

namespace {

// A strided view: element (i, j), i < rows, j < cols, at base + (i*ld + j)*elem.
struct View { uintptr_t base; int64_t rows, cols, ld; int shard; const char* what; };

uintptr_t view_end(const View& v, size_t elem) {
  return v.base + uintptr_t(((v.rows - 1) * v.ld + v.cols) * int64_t(elem));
}

// Whether two views share an element. Views with the same row stride (and an
// offset that is a whole number of elements) are compared by their row and
// column ranges; other views whose address ranges overlap count as sharing.
bool views_share(const View& a, const View& b, size_t elem) {
  if (view_end(a, elem) <= b.base || view_end(b, elem) <= a.base) return false;
  if (a.ld != b.ld) return true;
  const View& lo = a.base <= b.base ? a : b;
  const View& hi = a.base <= b.base ? b : a;
  const uintptr_t off = hi.base - lo.base;
  if (off % elem != 0) return true;
  const int64_t e = int64_t(off / elem), dr = e / lo.ld, dc = e % lo.ld;
  if (dc + hi.cols > lo.ld) return true;  // hi's rows wrap into lo's next row
  const bool rows_meet = dr < lo.rows;    // hi starts dr rows below lo
  const bool cols_meet = dc < lo.cols;    // and dc columns to the right
  return rows_meet && cols_meet;
}

muon_status validate_shards(const muon_shard* sh, int32_t n, int32_t dtype) {
  if (!sh) return fail(MUON_ERR_INVALID_ARG, "shards is NULL");
  if (n < 1) return fail(MUON_ERR_INVALID_ARG, "n must be >= 1");
  if (dtype != MUON_F32 && dtype != MUON_BF16) return fail(MUON_ERR_UNSUPPORTED, "dtype must be MUON_F32 or MUON_BF16");
  const size_t elem = dtype == MUON_BF16 ? 2 : 4;
  std::vector<View> ps, ds;
  int64_t tiles = 0;
  for (int32_t i = 0; i < n; ++i) {
    const muon_shard& s = sh[i];
    const std::string at = "shard " + std::to_string(i) + ": ";
    if (!s.p || !s.d) return fail(MUON_ERR_INVALID_ARG, at + "p or d is NULL");
    if (s.rows < 1 || s.cols < 1) return fail(MUON_ERR_INVALID_ARG, at + "rows and cols must be >= 1");
    if (s.rows > kMaxDim || s.cols > kMaxDim) return fail(MUON_ERR_INVALID_ARG, at + "rows and cols must be <= 2^24");
    if (s.ldp < s.cols || s.ldd < s.cols) return fail(MUON_ERR_INVALID_ARG, at + "ldp and ldd must be >= cols");
    if (s.ldp > (int64_t(1) << 40) || s.ldd > (int64_t(1) << 40)) return fail(MUON_ERR_INVALID_ARG, at + "row stride too large");
    if (reinterpret_cast<uintptr_t>(s.p) % elem || reinterpret_cast<uintptr_t>(s.d) % elem)
      return fail(MUON_ERR_ALIGN, at + "p or d is not aligned to the element size");
    const int64_t tcols = muon::kApplyRowBytes / int64_t(elem);
    tiles += ((s.rows + muon::kApplyRows - 1) / muon::kApplyRows) * ((s.cols + tcols - 1) / tcols);
    if (tiles > INT32_MAX) return fail(MUON_ERR_INVALID_ARG, "more than 2^31 - 1 tiles");
    ps.push_back({reinterpret_cast<uintptr_t>(s.p), s.rows, s.cols, s.ldp, i, "p"});
    ds.push_back({reinterpret_cast<uintptr_t>(s.d), s.rows, s.cols, s.ldd, i, "d"});
  }
  // Written views against written and read views: sort everything by start,
  // and compare each written view with the views that start before it ends.
  std::vector<View> all(ps);
  all.insert(all.end(), ds.begin(), ds.end());
  std::sort(all.begin(), all.end(), [](const View& x, const View& y) { return x.base < y.base; });
  for (size_t a = 0; a < all.size(); ++a) {
    const uintptr_t end = view_end(all[a], elem);
    for (size_t b = a + 1; b < all.size() && all[b].base < end; ++b) {
      const bool written = all[a].what[0] == 'p' || all[b].what[0] == 'p';
      if (!written) continue;
      if (views_share(all[a], all[b], elem))
        return fail(MUON_ERR_ALIAS, "shard " + std::to_string(all[a].shard) + " " + all[a].what + " overlaps shard " +
                                        std::to_string(all[b].shard) + " " + all[b].what);
    }
  }
  return MUON_OK;
}

void free_apply_plan(muon_apply_plan_s* p) {
  if (!p) return;
  if (p->ws) (void)hipFree(p->ws);
  delete p;
}

}  // namespace

extern "C" {

muon_status muon_apply_plan(const muon_shard* shards, int32_t n, int32_t dtype, muon_apply_plan_t* out) {
  if (!out) return fail(MUON_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  muon_status st = validate_shards(shards, n, dtype);
  if (st != MUON_OK) return st;
  const size_t elem = dtype == MUON_BF16 ? 2 : 4;
  std::vector<muon::ShardDev> h(n);
  std::vector<int32_t> prefix(n + 1, 0);
  for (int32_t i = 0; i < n; ++i) {
    const muon_shard& s = shards[i];
    muon::ShardDev& d = h[i];
    d.p = s.p;
    d.d = s.d;
    d.ldp = s.ldp;
    d.ldd = s.ldd;
    d.rows = int32_t(s.rows);
    d.cols = int32_t(s.cols);
    const int64_t tcols = muon::kApplyRowBytes / int64_t(elem), ve = 16 / int64_t(elem);
    d.tiles_c = int32_t((s.cols + tcols - 1) / tcols);
    d.vec = s.cols % ve == 0 && s.ldp % ve == 0 && s.ldd % ve == 0 && reinterpret_cast<uintptr_t>(s.p) % 16 == 0 &&
            reinterpret_cast<uintptr_t>(s.d) % 16 == 0;
    const int32_t tr = int32_t((s.rows + muon::kApplyRows - 1) / muon::kApplyRows);
    prefix[i + 1] = prefix[i] + tr * d.tiles_c;
  }
  auto* p = new muon_apply_plan_s();
  p->dtype = dtype;
  p->n = n;
  p->blocks = prefix[n];
  hipError_t e = hipGetDevice(&p->device);
  if (e != hipSuccess) { free_apply_plan(p); return hip_fail(e, "hipGetDevice"); }
  const size_t o_prefix = round_up(sizeof(muon::ShardDev) * n, 256);
  const size_t bytes = o_prefix + sizeof(int32_t) * (n + 1);
  e = hipMalloc(&p->ws, bytes);
  if (e != hipSuccess) {
    p->ws = nullptr;
    free_apply_plan(p);
    (void)hipGetLastError();
    return fail(MUON_ERR_OOM, "hipMalloc of " + std::to_string(bytes) + " bytes failed");
  }
  p->d_shards = static_cast<muon::ShardDev*>(p->ws);
  p->d_prefix = reinterpret_cast<int32_t*>(static_cast<char*>(p->ws) + o_prefix);
  e = hipMemcpy(p->d_shards, h.data(), sizeof(muon::ShardDev) * n, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(p->d_prefix, prefix.data(), sizeof(int32_t) * (n + 1), hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) { free_apply_plan(p); return hip_fail(e, "hipMemcpy"); }
  *out = p;
  return MUON_OK;
}

muon_status muon_apply(muon_apply_plan_t p, void* stream) {
  if (!p) return fail(MUON_ERR_INVALID_ARG, "plan is NULL");
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (cur != p->device && (e = hipSetDevice(p->device)) != hipSuccess) return hip_fail(e, "hipSetDevice");
  e = muon::launch_shard_apply(p->dtype, p->d_shards, p->d_prefix, p->n, p->blocks, static_cast<hipStream_t>(stream));
  if (cur != p->device) (void)hipSetDevice(cur);
  return e == hipSuccess ? MUON_OK : hip_fail(e, "kernel launch");
}

muon_status muon_mfma_probe(float* out, int32_t blocks, int32_t iters, void* stream) {
  if (!out) return fail(MUON_ERR_INVALID_ARG, "out is NULL");
  if (blocks < 1 || blocks > (1 << 20)) return fail(MUON_ERR_INVALID_ARG, "blocks must be in [1, 2^20]");
  if (iters < 1) return fail(MUON_ERR_INVALID_ARG, "iters must be >= 1");
  const hipError_t e = muon::launch_mfma_probe(out, blocks, iters, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MUON_OK : hip_fail(e, "kernel launch");
}

muon_status muon_apply_plan_destroy(muon_apply_plan_t p) {
  if (!p) return MUON_OK;
  hipError_t e = hipDeviceSynchronize();
  free_apply_plan(p);
  return e == hipSuccess ? MUON_OK : hip_fail(e, "hipDeviceSynchronize");
}

}  // extern "C"

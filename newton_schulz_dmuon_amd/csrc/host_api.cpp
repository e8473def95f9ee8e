// C ABI of the owner-side Muon step: argument validation, the per-call plan
// (orientation, padding, workspace layout, grouped launch tables) and the
// launch sequence.  Every check runs before the first HIP call, so a
// rejected call has no effect on any buffer.

#include <algorithm>
#include <array>
#include <cstdarg>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <numeric>
#include <string>
#include <tuple>
#include <vector>

#include "../../include/dmuon.h"
#include "internal.h"

namespace dmuon {
namespace {

thread_local std::string g_last_error;

int fail(int status, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int hip_fail(hipError_t e, const char *what) {
  return fail(DMUON_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

int64_t elem_size(int32_t dt) { return dt == DMUON_F32 ? 4 : 2; }

bool dtype_ok(int32_t dt) { return dt == DMUON_BF16 || dt == DMUON_F32; }

constexpr int64_t kMaxDim = int64_t(1) << 31;
constexpr int64_t kMaxNumel = int64_t(1) << 40;
// The step's kernels address an operand row block with 32-bit offsets
// (256 rows x 4 bytes x 2^22 < 2^32) and tiles with 16-bit indices.
constexpr int64_t kMaxStepDim = int64_t(1) << 22;

// ---------------------------------------------------------------- aliasing --
struct Interval {
  uintptr_t lo, hi;  // [lo, hi)
  bool written;
  const char *what;
  int32_t index;
};

// Fails if a written interval overlaps any other interval.
int check_aliasing(std::vector<Interval> &iv) {
  std::sort(iv.begin(), iv.end(), [](const Interval &x, const Interval &y) {
    return x.lo != y.lo ? x.lo < y.lo : x.hi < y.hi;
  });
  uintptr_t max_any = 0, max_written = 0;
  const Interval *any_at = nullptr, *wr_at = nullptr;
  for (const Interval &x : iv) {
    if (x.hi <= x.lo) continue;
    if (x.written && any_at && x.lo < max_any)
      return fail(DMUON_ERR_ALIAS, "%s of matrix %d overlaps %s of matrix %d", x.what, x.index,
                  any_at->what, any_at->index);
    if (!x.written && wr_at && x.lo < max_written)
      return fail(DMUON_ERR_ALIAS, "%s of matrix %d overlaps %s of matrix %d", x.what, x.index,
                  wr_at->what, wr_at->index);
    if (x.hi > max_any) { max_any = x.hi; any_at = &x; }
    if (x.written && x.hi > max_written) { max_written = x.hi; wr_at = &x; }
  }
  return DMUON_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ------------------------------------------------------------- validation --
int validate_config(const dmuon_step_config *cfg) {
  if (!cfg) return fail(DMUON_ERR_INVALID_ARG, "cfg is NULL");
  if (cfg->ns_steps < 0 || cfg->ns_steps > 64)
    return fail(DMUON_ERR_INVALID_ARG, "ns_steps %d outside [0, 64]", cfg->ns_steps);
  const float vals[] = {cfg->a, cfg->b, cfg->c, cfg->lr, cfg->momentum, cfg->eps};
  for (float v : vals)
    if (!std::isfinite(v)) return fail(DMUON_ERR_INVALID_ARG, "non-finite step coefficient");
  if (cfg->eps < 0.f) return fail(DMUON_ERR_INVALID_ARG, "eps < 0");
  const uint32_t known = DMUON_FLAG_NS_FP32 | DMUON_FLAG_NESTEROV | DMUON_FLAG_GRAM_NS | DMUON_FLAG_CHECK_FINITE |
                         DMUON_FLAG_CHAIN_LAUNCH;
  if (cfg->flags & ~known) return fail(DMUON_ERR_INVALID_ARG, "unknown flag bits 0x%x", cfg->flags & ~known);
  return DMUON_OK;
}

int validate_step_shapes(const dmuon_matrix *mats, int32_t n) {
  for (int32_t i = 0; i < n; ++i)
    if (mats[i].rows > kMaxStepDim || mats[i].cols > kMaxStepDim)
      return fail(DMUON_ERR_INVALID_ARG, "matrix %d: %lld x %lld exceeds the step's limit of %lld per side", i,
                  (long long)mats[i].rows, (long long)mats[i].cols, (long long)kMaxStepDim);
  return DMUON_OK;
}

int validate_shapes(const dmuon_matrix *mats, int32_t n) {
  if (n < 0) return fail(DMUON_ERR_INVALID_ARG, "n < 0");
  if (n > 0 && !mats) return fail(DMUON_ERR_INVALID_ARG, "mats is NULL");
  for (int32_t i = 0; i < n; ++i) {
    const dmuon_matrix &d = mats[i];
    if (d.rows < 1 || d.cols < 1 || d.rows >= kMaxDim || d.cols >= kMaxDim ||
        d.rows * d.cols > kMaxNumel)
      return fail(DMUON_ERR_INVALID_ARG, "matrix %d: bad shape %lld x %lld", i,
                  (long long)d.rows, (long long)d.cols);
    if (!dtype_ok(d.param_dtype) || !dtype_ok(d.grad_dtype))
      return fail(DMUON_ERR_UNSUPPORTED_DTYPE, "matrix %d: dtype codes %d/%d", i, d.param_dtype,
                  d.grad_dtype);
    if (d.reserved != 0) return fail(DMUON_ERR_INVALID_ARG, "matrix %d: reserved != 0", i);
    if (!std::isfinite(d.scale)) return fail(DMUON_ERR_INVALID_ARG, "matrix %d: scale not finite", i);
  }
  return DMUON_OK;
}

// ------------------------------------------------------------------- plan --
// Launch kinds, in the order of the DMUON_LAUNCH_* codes of the C ABI.
enum LaunchKind : int32_t {
  kLkMomentumSumsq = DMUON_LAUNCH_MOMENTUM_SUMSQ,
  kLkMomentumOrient = DMUON_LAUNCH_MOMENTUM_ORIENT,
  kLkNorm = DMUON_LAUNCH_NORM,
  kLkUpdateDirect = DMUON_LAUNCH_UPDATE_DIRECT,
  kLkGram = DMUON_LAUNCH_GRAM,
  kLkSquare = DMUON_LAUNCH_SQUARE,
  kLkApply = DMUON_LAUNCH_APPLY,
  kLkFinal = DMUON_LAUNCH_FINAL,
  kLkGramSquare = DMUON_LAUNCH_GRAM_SQUARE,  // parts of kinds Gram and Square
  kLkChain = DMUON_LAUNCH_CHAIN              // every bf16 part of the step
};

// Workspace buffers a GEMM launch can name per matrix: the direct chain uses
// A and B; the Gram-space chain also A', T, Q0, Q1 (m_p x m_p each).  With
// hi + lo pairs (split_pairs), B_lo holds the low half of B (direct chain)
// or of a later iteration's P (Gram-space chain), Q0_lo that of the first P,
// T_lo that of T = P P.
enum Buf : int32_t {
  kBufNone = -1, kBufA = 0, kBufB, kBufA1, kBufT, kBufQ0, kBufQ1, kBufBlo, kBufQ0lo, kBufTlo, kBufCount
};

// One part of a grouped GEMM launch: a group of matrices (0 direct chain, 1
// Gram-space chain, 2 direct chain in fp32 for small matrices of a bf16
// step) and, for every matrix of it, which buffer each MatDev
// pointer names (a: Gram output, Square L; b: Square output, Apply L; r:
// Square R; l_lo, r_lo: low halves of L and R; o_lo: low half of a Square
// output), which X^T buffer is read (cur; the other one is written), and
// the stage's coefficients.
struct Part {
  int32_t group, a, b, r, cur, first;
  float ca, cb, cc, cdiag;
  int32_t l_lo = kBufNone, r_lo = kBufNone, o_lo = kBufNone;
  int32_t kind = 0;  // the stage this part runs (kLkGram ... kLkFinal)
  auto key() const {
    return std::make_tuple(group, a, b, r, cur, first, ca, cb, cc, cdiag, l_lo, r_lo, o_lo, kind);
  }
  bool operator<(const Part &o) const { return key() < o.key(); }
  // passes of the K loop (each a full product): 1 + one per low half read;
  // a Square without its own R reads L twice
  int32_t passes() const {
    const bool r_split = r_lo != kBufNone || (kind == DMUON_LAUNCH_SQUARE && r == kBufNone && l_lo != kBufNone);
    return 1 + (l_lo != kBufNone) + (kind == DMUON_LAUNCH_SQUARE && r_split);
  }
  // tile-list stage: 0 Gram, 1 Square, 2 Apply / Final
  int32_t stage() const { return kind == kLkGram ? 0 : kind == kLkSquare ? 1 : 2; }
};

struct Launch {
  int32_t kind;
  bool fp32 = false;        // fp32 operands (kernel instance); parts share it
  std::vector<Part> parts;  // GEMM launches: all of this kind, or (kLkGramSquare)
                            // of kinds Gram and Square
  int32_t table = 0;        // MatDev table: the parts' matrices, in order
  int32_t list = 0;         // tile list over that table
  int32_t role = 0;         // 0 whole tiles, 1 pieces of split tiles, 2 their reduce
  int32_t tile = 256;       // tile size: 256, or 128 (bf16 Square, whole tiles)
  double flops = 0;         // algorithmic flops (symmetric products: upper triangle)
};

struct Plan {
  std::vector<MatDev> mats;                   // every matrix: table 0
  // per matrix, the buffers beyond A and B (index buf - kBufA1; nullptr in
  // the sizing pass) and a bit mask of the ones it has
  std::vector<std::array<void *, kBufCount - kBufA1>> extra;
  std::vector<uint32_t> have;
  // matrix indices: direct chain, Gram-space chain, fp32 direct chain of
  // the small matrices of a bf16 step
  std::vector<int32_t> groups[3];
  std::vector<std::vector<Part>> tables;      // tables 1..: the parts of a launch
  std::vector<std::vector<TileEntry>> lists;
  std::vector<StageXcd> list_xcd;
  std::vector<Launch> prog;
  int64_t ew_total = 0, tr_total = 0;
  // workspace layout (byte offsets)
  std::vector<int64_t> off_table, off_list;
  int64_t off_partials = 0, off_inv = 0, off_flags = -1;
  int64_t off_splitk = -1, splitk_slots = 0;  // partial slots of split tiles
  int64_t off_chain = -1, chain_counters = 0;  // chained mode: tickets, timeout, counters
  int64_t table_bytes = 0;  // [0, table_bytes) is uploaded
  int64_t total_bytes = 0;
};

// Tile lists of one grouped GEMM launch, one per XCD; every matrix has its
// stage (0 Gram, 1 Square, 2 Apply; a launch can hold Gram and Square
// matrices).  Tiles are grouped into 4 x 8 blocks that share operand panels
// (the upper triangle's part of them for the symmetric products, which read
// panels ti and tj of one matrix; B panel ti and X^T panel tj for Apply).
// Blocks go, in order, to the XCD with the least work so far; each XCD's
// list keeps that order, so the tiles running together on one XCD read few
// distinct panels through its L2.  The order: a full stage's blocks
// costliest first (tiles x K depth; ties in matrix order, each matrix's
// blocks column by column, so that the XCDs starting together share the
// X^T panels); a symmetric stage's blocks matrix by matrix, costliest matrix
// first, each matrix's blocks together (its diagonal blocks, which hold
// fewer tiles, would otherwise run after every matrix's full blocks, far
// from the fetch of the panels they share).
void build_stage_tiles(const std::vector<MatDev> &mats, const std::vector<int32_t> &passes,
                       const std::vector<int32_t> &stages, int32_t tile, std::vector<TileEntry> &out,
                       StageXcd &xcd) {
  struct Block {
    int64_t cost;
    int32_t mat, ti0, tj0;
  };
  std::vector<Block> blocks;
  for (int32_t i = 0; i < static_cast<int32_t>(mats.size()); ++i) {
    const MatDev &d = mats[i];
    const int32_t st = stages[i];
    const bool sym = st < 2;
    const int bm = 4, bn = 8;
    const int64_t depth = (st == 0 ? d.np : d.mp) * passes[i];
    const int32_t rows = static_cast<int32_t>(d.mp / tile), cols = static_cast<int32_t>((sym ? d.mp : d.np) / tile);
    auto add = [&](int32_t bi, int32_t bj) {
      int64_t nt = 0;
      for (int32_t ti = bi; ti < std::min(bi + bm, rows); ++ti)
        for (int32_t tj = bj; tj < std::min(bj + bn, cols); ++tj) nt += (!sym || tj >= ti);
      if (nt) blocks.push_back(Block{nt * depth, i, bi, bj});
    };
    if (sym) {
      for (int32_t bi = 0; bi < rows; bi += bm)
        for (int32_t bj = bi; bj < cols; bj += bn) add(bi, bj);
    } else {
      // column of blocks by column of blocks: the XCDs that start together
      // take blocks of one column, which share its R panels
      for (int32_t bj = 0; bj < cols; bj += bn)
        for (int32_t bi = 0; bi < rows; bi += bm) add(bi, bj);
    }
  }
  // costliest first; a symmetric stage by its matrices' whole cost (above)
  std::vector<int64_t> mat_cost(mats.size(), 0);
  for (const Block &b : blocks) mat_cost[b.mat] += b.cost;
  std::stable_sort(blocks.begin(), blocks.end(), [&](const Block &x, const Block &y) {
    const bool sx = stages[x.mat] < 2, sy = stages[y.mat] < 2;
    const int64_t cx = sx ? mat_cost[x.mat] : x.cost, cy = sy ? mat_cost[y.mat] : y.cost;
    return cx > cy;
  });
  std::vector<TileEntry> lists[kXcds];
  int64_t load[kXcds] = {0};
  for (const Block &b : blocks) {
    int x = 0;
    for (int y = 1; y < kXcds; ++y)
      if (load[y] < load[x]) x = y;
    load[x] += b.cost;
    const MatDev &d = mats[b.mat];
    const bool sym = stages[b.mat] < 2;
    const int bm = 4, bn = 8;
    const int32_t rows = static_cast<int32_t>(d.mp / tile), cols = static_cast<int32_t>((sym ? d.mp : d.np) / tile);
    for (int32_t ti = b.ti0; ti < std::min(b.ti0 + bm, rows); ++ti)
      for (int32_t tj = b.tj0; tj < std::min(b.tj0 + bn, cols); ++tj)
        if (!sym || tj >= ti)
          lists[x].push_back(TileEntry{b.mat, static_cast<uint16_t>(ti), static_cast<uint16_t>(tj)});
  }
  out.clear();
  for (int x = 0; x < kXcds; ++x) {
    xcd.first[x] = static_cast<int32_t>(out.size());
    xcd.count[x] = static_cast<int32_t>(lists[x].size());
    out.insert(out.end(), lists[x].begin(), lists[x].end());
  }
}

// The tile lists depend only on the stage and the matrices' padded shapes
// and dimensions, and a training run calls the step with the same shapes
// every time: keep the last lists built (a small cache, cleared when full).
std::mutex g_tiles_mu;
std::map<std::vector<int64_t>, std::pair<std::vector<TileEntry>, StageXcd>> g_tiles_cache;
constexpr size_t kTilesCacheMax = 64;

void cached_stage_tiles(const std::vector<MatDev> &mats, const std::vector<int32_t> &passes,
                        const std::vector<int32_t> &stages, int32_t tile, std::vector<TileEntry> &out,
                        StageXcd &xcd) {
  std::vector<int64_t> key;
  key.reserve(1 + 6 * mats.size());
  key.push_back(tile);
  for (size_t i = 0; i < mats.size(); ++i) {
    const MatDev &d = mats[i];
    key.push_back(stages[i]);
    key.push_back(d.mp);
    key.push_back(d.np);
    key.push_back(d.tm);
    key.push_back(d.tn);
    key.push_back(passes[i]);
  }
  {
    std::lock_guard<std::mutex> lock(g_tiles_mu);
    auto it = g_tiles_cache.find(key);
    if (it != g_tiles_cache.end()) {
      out = it->second.first;
      xcd = it->second.second;
      return;
    }
  }
  build_stage_tiles(mats, passes, stages, tile, out, xcd);
  std::lock_guard<std::mutex> lock(g_tiles_mu);
  if (g_tiles_cache.size() >= kTilesCacheMax) g_tiles_cache.clear();
  g_tiles_cache.emplace(std::move(key), std::make_pair(out, xcd));
}

// Work-groups of the momentum / orientation pass for one matrix, 8192
// elements each: a tall matrix (its own X^T) in contiguous 8192-element
// runs, otherwise 64 x 128 blocks of X.  One sum-of-squares partial each.
int64_t orient_groups(const MatDev &d) { return (d.mp / kTrTile) * (d.np / kTrTile) / 2; }

// A matrix takes the Gram-space chain when asked for, with at least five
// iterations, n >= 2m and m >= kFp32BelowM (below that a bf16 step runs the
// matrix's chain in fp32): the m x m chain then costs fewer flops than the
// direct iterations, and the iterate's singular values stay within a factor
// (sqrt(n)+sqrt(m))/(sqrt(n)-sqrt(m)) < 6 of each other for Gaussian-like
// inputs.  Below five iterations the rounding of the first phase's Q is not
// damped by later iterations: on ill-conditioned inputs (rank one plus
// noise) two iterations come out about 18x, three to four 2-4x less
// accurate than the direct chain in a bf16 emulation, so those keep it.
bool uses_gram(const MatDev &d, const dmuon_step_config &cfg) {
  return (cfg.flags & DMUON_FLAG_GRAM_NS) && cfg.ns_steps >= 5 && d.n >= 2 * d.m && d.m >= kFp32BelowM;
}

// From six iterations on, the bf16 chain keeps B (direct chain), and every
// P and T = P P (Gram-space chain), as hi + lo pairs.  The default quintic
// amplifies rounding errors on part of its band, and the rounding of B (or
// P) is the largest contributor: in a bf16 emulation on Gaussian inputs of
// the Qwen2.5-7B and Qwen2.5-1.5B shapes, pairs take the error at 8
// iterations from 1.5-2.7e-2 to 0.7-1.4e-2, where keeping X or A in fp32
// instead changes it by 1-10%.  In the Gram-space chain T comes next (P
// alone leaves 1.9e-2 on a 17 x 100 input at 6 iterations, P and T 1.0e-2).
// Up to five iterations bf16 storage stays below about 1.4e-2 on those
// inputs, so the pairs' extra passes are not paid.
constexpr int kSplitFromSteps = 6;
bool split_pairs(const dmuon_step_config &cfg) {
  return !(cfg.flags & DMUON_FLAG_NS_FP32) && cfg.ns_steps >= kSplitFromSteps;
}

// Phases of the Gram-space chain: two iterations each, the last one a
// single iteration when K is odd (5 -> 2 + 2 + 1, 8 -> 2 + 2 + 2 + 2).  Each
// phase starts from an explicit X (a fresh A = X X^T) and ends with
// X <- Q X.  Over a phase Q's eigenvalues reach a^L on the directions of
// small singular values, and its bf16 rounding is relative to that: phases
// of three lose accuracy on ill-conditioned inputs (rank one plus noise:
// 4-5x the direct chain's error), phases of two stay at 0.5-1.05x of it
// there and on Gaussian inputs.  With singular values spread over one or
// two decades the chain is 2-3x less accurate than the direct one whatever
// the split: that loss is in the bf16 storage of P, T and Q themselves.
std::vector<int> gram_phases(int K) {
  std::vector<int> L(K / 2, 2);
  if (K % 2) L.push_back(1);
  return L;
}

// Builds the plan; with ws == nullptr only sizes are computed.
// ---- split K for launches that leave CUs idle ----
// A launch with fewer tiles than the chip has CUs runs as long as its
// longest tile while most CUs idle (a single Qwen2.5-1.5B layer: about a
// hundred Gram tiles of 140 K steps for 256 CUs).  Such a launch can run
// its tiles in pieces over K instead: a launch of pieces, each writing its
// fp32 accumulators to a partial slot, then a launch of reduce entries that
// sum each tile's slots in a fixed order and run the tile's epilogue.  The
// host picks the piece count per tile (at most kMaxPieces, pieces of at
// least kMinPieceSteps steps) whose estimated time is least: the list
// schedule of the pieces over the CUs, plus kSplitLaunchSteps for the reduce
// launch, plus kSplitStepsPerPiece for each piece's partial slot (256 KB
// written, then read back by the reduce, all pieces sharing the HBM: about
// 0.07 of a K step each); no split when that does not beat the whole tiles.
// Times are in K steps of one 256 x 256 tile (about 1.9 us).
constexpr int kCUs = 256;
constexpr int kMaxPieces = 16;
constexpr int64_t kMinPieceSteps = 16;
constexpr double kSplitLaunchSteps = 8.0;
constexpr double kSplitStepsPerPiece = 0.07;

// Greedy list schedule of item lengths (longest first) on `machines`
// machines: the finishing time of the last one.
int64_t list_makespan(std::vector<int64_t> len, int machines) {
  std::sort(len.begin(), len.end(), std::greater<int64_t>());
  std::vector<int64_t> heap(machines, 0);  // min-heap of machine loads
  for (int64_t l : len) {
    std::pop_heap(heap.begin(), heap.end(), std::greater<int64_t>());
    heap.back() += l;
    std::push_heap(heap.begin(), heap.end(), std::greater<int64_t>());
  }
  return *std::max_element(heap.begin(), heap.end());
}

// Pieces per tile for a launch whose tiles need steps[t] K steps; all ones
// when splitting does not pay.
std::vector<int32_t> choose_pieces(const std::vector<int64_t> &steps) {
  std::vector<int32_t> best(steps.size(), 1);
  if (steps.empty() || static_cast<int64_t>(steps.size()) >= kCUs) return best;
  double best_t = static_cast<double>(list_makespan(steps, kCUs));
  for (int smax = 2; smax <= kMaxPieces; ++smax) {
    std::vector<int32_t> pieces(steps.size());
    std::vector<int64_t> len;
    bool any = false;
    for (size_t t = 0; t < steps.size(); ++t) {
      pieces[t] = static_cast<int32_t>(std::max<int64_t>(1, std::min<int64_t>(smax, steps[t] / kMinPieceSteps)));
      any |= pieces[t] > 1;
      for (int32_t q = 0; q < pieces[t]; ++q)
        len.push_back((steps[t] * (q + 1)) / pieces[t] - (steps[t] * q) / pieces[t]);
    }
    if (!any) break;
    const double t_split = static_cast<double>(list_makespan(len, kCUs)) + kSplitLaunchSteps +
                           kSplitStepsPerPiece * static_cast<double>(len.size());
    if (t_split < best_t) {
      best_t = t_split;
      best = pieces;
    }
  }
  return best;
}

// A Square launch can run 128 x 128 tiles instead (bf16, whole tiles): four
// times the tiles, each a quarter of the work, two work-groups per CU.  The
// estimate: a 128-tile K step costs kSmallStepCost of a 256-tile step on
// one of 2 x kCUs slots; the 128-tiles are taken when their list schedule
// beats the 256-tiles' by kSmallMargin.
constexpr double kSmallStepCost = 0.5;
constexpr double kSmallMargin = 0.8;
bool small_tiles_pay(const std::vector<int64_t> &steps256, const std::vector<int64_t> &steps128) {
  if (steps256.empty() || static_cast<int64_t>(steps256.size()) >= kCUs) return false;
  const double t256 = static_cast<double>(list_makespan(steps256, kCUs));
  const double t128 = kSmallStepCost * static_cast<double>(list_makespan(steps128, 2 * kCUs));
  return t128 < kSmallMargin * t256;
}

// Per-XCD lists of entries with costs: costliest first, each to the XCD
// with the least work so far (as build_stage_tiles does for blocks).
void assign_xcds(const std::vector<std::pair<int64_t, TileEntry>> &items, std::vector<TileEntry> &out,
                 StageXcd &xcd) {
  std::vector<size_t> order(items.size());
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(),
                   [&](size_t a, size_t b) { return items[a].first > items[b].first; });
  std::vector<TileEntry> lists[kXcds];
  int64_t load[kXcds] = {0};
  for (size_t o : order) {
    int x = 0;
    for (int y = 1; y < kXcds; ++y)
      if (load[y] < load[x]) x = y;
    load[x] += items[o].first;
    lists[x].push_back(items[o].second);
  }
  out.clear();
  for (int x = 0; x < kXcds; ++x) {
    xcd.first[x] = static_cast<int32_t>(out.size());
    xcd.count[x] = static_cast<int32_t>(lists[x].size());
    out.insert(out.end(), lists[x].begin(), lists[x].end());
  }
}

// K-loop steps of every row of a launch's table (its parts' matrices).
std::vector<int64_t> row_steps(const Plan &p, const Launch &l) {
  std::vector<int64_t> out;
  const int64_t kstep = l.fp32 ? 32 : 64;  // elements per 128-byte K step
  for (const Part &pt : l.parts)
    for (int32_t i : p.groups[pt.group]) {
      const MatDev &d = p.mats[i];
      out.push_back(pt.passes() * ((pt.kind == kLkGram ? d.np : d.mp) / kstep));
    }
  return out;
}

// In a bf16 step, a matrix with m = min(r, c) < kFp32BelowM runs its chain
// in fp32 (its own launches, group 2).  Such a matrix's singular values
// start near 1/sqrt(m), reach the quintic's band within one or two
// iterations and stay there, where rounding errors grow: in a bf16
// emulation on Gaussian inputs, bf16 storage gives up to 2.0-2.3e-2 at five
// iterations for m = 17-32 and 2.1-2.8e-2 at eight even with B as a pair,
// against at most 1.2e-2 at m >= 128.  Its products are at most one
// 256-tile wide, so fp32 costs next to nothing.
bool small_fp32(const MatDev &d, const dmuon_step_config &cfg) {
  return !(cfg.flags & DMUON_FLAG_NS_FP32) && d.m < kFp32BelowM;
}

// The chained mode (DMUON_FLAG_CHAIN_LAUNCH): the bf16 launches of the
// merged program become one launch.  Its table is the launches' tables one
// after the other, so row r is one matrix at one stage.  Each matrix goes,
// with all its stages, to one XCD (largest total work first, to the XCD with
// the least so far); an XCD's queue holds its matrices' tiles in program
// order (launch by launch; a stage's tiles in the blocks of
// build_stage_tiles).  Entry fields: k0 = the counter of the matrix's
// previous launch (-1 for its first), k1 = that launch's tile count for the
// matrix, slot = the counter of this launch for the matrix.  All of a
// matrix's rows in one launch (Square launches can hold two parts of it)
// signal one counter.
void chain_launch(Plan &p, const std::vector<Launch> &in_chain) {
  Launch c;
  c.kind = kLkChain;
  for (const Launch &l : in_chain) {
    c.parts.insert(c.parts.end(), l.parts.begin(), l.parts.end());
    c.flops += l.flops;
  }
  p.tables.push_back(c.parts);
  c.table = static_cast<int32_t>(p.tables.size());
  const std::vector<int64_t> rs = row_steps(p, c);
  struct Row {
    int32_t row, mat, launch;
    bool sym;
  };
  std::vector<Row> rows;
  for (size_t j = 0; j < in_chain.size(); ++j)
    for (const Part &pt : in_chain[j].parts)
      for (int32_t i : p.groups[pt.group])
        rows.push_back(Row{static_cast<int32_t>(rows.size()), i, static_cast<int32_t>(j),
                           pt.kind == kLkGram || pt.kind == kLkSquare});
  auto tiles_of = [&](const Row &r) {
    const MatDev &d = p.mats[r.mat];
    return r.sym ? static_cast<int64_t>(d.tm) * (d.tm + 1) / 2 : static_cast<int64_t>(d.tm) * d.tn;
  };
  // owner XCD of every matrix, by total work
  const int32_t n = static_cast<int32_t>(p.mats.size());
  std::vector<int64_t> work(n, 0);
  for (const Row &r : rows) work[r.mat] += tiles_of(r) * rs[r.row];
  std::vector<int32_t> order;
  for (int32_t i = 0; i < n; ++i)
    if (work[i] > 0) order.push_back(i);
  std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) { return work[a] > work[b]; });
  std::vector<int32_t> owner(n, -1);
  int64_t load[kXcds] = {0};
  for (int32_t i : order) {
    int x = 0;
    for (int y = 1; y < kXcds; ++y)
      if (load[y] < load[x]) x = y;
    load[x] += work[i];
    owner[i] = x;
  }
  // counters: one per (matrix, launch); each row waits on its matrix's
  // previous launch
  // (matrix, launch) -> its counter and the counter it waits on
  std::map<std::pair<int32_t, int32_t>, std::pair<int32_t, int32_t>> counter;
  std::vector<int64_t> tiles_in;      // counter -> tiles that signal it
  std::vector<int32_t> last(n, -1);   // the matrix's latest counter so far
  std::vector<int32_t> wait_on(rows.size(), -1), sig(rows.size(), -1);
  for (const Row &r : rows) {
    auto key = std::make_pair(r.mat, r.launch);
    auto it = counter.find(key);
    if (it == counter.end()) {
      // a second row of the matrix in the same launch finds this entry and
      // waits as the first did
      it = counter.emplace(key, std::make_pair(static_cast<int32_t>(tiles_in.size()), last[r.mat])).first;
      tiles_in.push_back(0);
      last[r.mat] = it->second.first;
    }
    sig[r.row] = it->second.first;
    wait_on[r.row] = it->second.second;
    tiles_in[it->second.first] += tiles_of(r);
  }
  p.chain_counters = static_cast<int64_t>(tiles_in.size());
  std::vector<TileEntry> lists[kXcds];
  for (const Row &r : rows) {
    const MatDev &d = p.mats[r.mat];
    const int32_t bm = 4, bn = r.sym ? 4 : 8;
    const int32_t rows_t = d.tm, cols_t = r.sym ? d.tm : d.tn;
    const int32_t w = wait_on[r.row];
    const int32_t need = w >= 0 ? static_cast<int32_t>(tiles_in[w]) : 0;
    for (int32_t bi = 0; bi < rows_t; bi += bm)
      for (int32_t bj = r.sym ? bi : 0; bj < cols_t; bj += bn)
        for (int32_t ti = bi; ti < std::min(bi + bm, rows_t); ++ti)
          for (int32_t tj = bj; tj < std::min(bj + bn, cols_t); ++tj)
            if (!r.sym || tj >= ti) {
              TileEntry e{r.row, static_cast<uint16_t>(ti), static_cast<uint16_t>(tj)};
              e.k0 = w;
              e.k1 = need;
              e.slot = sig[r.row];
              lists[owner[r.mat]].push_back(e);
            }
  }
  p.lists.emplace_back();
  p.list_xcd.emplace_back();
  std::vector<TileEntry> &out = p.lists.back();
  StageXcd &xcd = p.list_xcd.back();
  for (int x = 0; x < kXcds; ++x) {
    xcd.first[x] = static_cast<int32_t>(out.size());
    xcd.count[x] = static_cast<int32_t>(lists[x].size());
    out.insert(out.end(), lists[x].begin(), lists[x].end());
  }
  c.list = static_cast<int32_t>(p.lists.size()) - 1;
  p.prog.push_back(std::move(c));
}

void build_plan(const dmuon_matrix *in, int32_t n, const dmuon_step_config &cfg, char *ws,
                Plan &p) {
  const bool fp32 = cfg.flags & DMUON_FLAG_NS_FP32;
  const int K = cfg.ns_steps;
  const bool split = split_pairs(cfg);
  p.mats.resize(n);
  p.extra.assign(n, {});
  p.have.assign(n, 0);
  for (auto &g : p.groups) g.clear();
  int64_t ew = 0, tr = 0;
  for (int32_t i = 0; i < n; ++i) {
    const dmuon_matrix &s = in[i];
    MatDev &d = p.mats[i];
    std::memset(&d, 0, sizeof d);
    d.param = s.param;
    d.grad = s.grad;
    d.mom = s.momentum;
    d.orth = s.orth_out;
    d.rows = s.rows;
    d.cols = s.cols;
    d.transposed = s.rows > s.cols;
    d.m = std::min(s.rows, s.cols);
    d.n = std::max(s.rows, s.cols);
    d.mp = round_up(d.m, kPad);
    d.np = round_up(d.n, kPad);
    d.tm = static_cast<int32_t>(d.mp / kGemmTile);
    d.tn = static_cast<int32_t>(d.np / kGemmTile);
    d.param_dt = s.param_dtype;
    d.grad_dt = s.grad_dtype;
    d.scale = s.scale;
    d.ew_first = ew;
    d.ew_count = static_cast<int32_t>((s.rows * s.cols + kEwChunk - 1) / kEwChunk);
    ew += d.ew_count;
    d.tr_first = tr;
    tr += orient_groups(d);
    d.ws_f32 = fp32 || small_fp32(d, cfg);
    if (K > 0) p.groups[uses_gram(d, cfg) ? 1 : small_fp32(d, cfg) ? 2 : 0].push_back(i);
  }
  p.ew_total = ew;
  p.tr_total = K > 0 ? tr : 0;

  // ---- the launch program ----
  p.tables.clear();
  p.lists.clear();
  p.list_xcd.clear();
  p.prog.clear();
  p.splitk_slots = 0;
  // algorithmic flops of one stage over a group
  auto flops = [&](int g, int32_t kind) {
    double f = 0;
    for (int32_t i : p.groups[g]) {
      const double m = static_cast<double>(p.mats[i].m), nn = static_cast<double>(p.mats[i].n);
      f += kind == kLkGram ? m * (m + 1) * nn : kind == kLkSquare ? m * m * (m + 1) : 2 * m * m * nn;
    }
    return f;
  };
  auto gemm = [&](std::vector<Launch> &chain, int32_t kind, std::vector<Part> parts) {
    Launch l;
    l.kind = kind;
    l.parts = std::move(parts);
    for (Part &pt : l.parts) pt.kind = kind;
    // executed flops: every pass of the K loop is a full product
    for (const Part &pt : l.parts) l.flops += flops(pt.group, kind) * pt.passes();
    chain.push_back(std::move(l));
  };
  std::vector<Launch> chain[3];
  // direct chain: K x (A = X X^T; B = b A + c A A; X <- a X + B X); with
  // pairs (bf16 only), Square also stores B's low half and Apply reads it,
  // from the third iteration on: the first two iterations' rounding of B
  // does not show in the result (bf16 emulation: the same error as pairs
  // in every iteration, m >= 128, 6 and 8 iterations)
  auto direct_chain = [&](int32_t g, bool pairs, bool chain_fp32) {
    for (int k = 0; k < K; ++k) {
      const int32_t cur = k & 1, first = k == 0;
      const Part pt{g, kBufA, kBufB, kBufNone, cur, first, cfg.a, cfg.b, cfg.c, 0.f};
      Part sq = pt, ap = pt;
      if (pairs && k >= 2) {
        sq.o_lo = kBufBlo;
        ap.l_lo = kBufBlo;
      }
      gemm(chain[g], kLkGram, {pt});
      gemm(chain[g], kLkSquare, {sq});
      gemm(chain[g], k + 1 == K ? kLkFinal : kLkApply, {ap});
    }
    for (Launch &l : chain[g]) l.fp32 = chain_fp32;
  };
  if (K > 0 && !p.groups[0].empty()) direct_chain(0, split, fp32);
  if (K > 0 && !p.groups[2].empty()) direct_chain(2, false, true);
  if (K > 0 && !p.groups[1].empty()) {
    // Gram-space chain, per phase of L iterations from X:
    //   A = X X^T; Q = I
    //   L times: P = a I + b A + c A A;  A <- A P P (not after the last);  Q <- Q P
    //   X <- Q X   (the step's last phase: the update instead)
    // A, P, Q are polynomials in the phase's first A, so every product is of
    // commuting symmetric matrices: upper tiles + mirror.  P of the first
    // iteration is written to Q0 and is Q.  T = P P and Q P both read only
    // P: one launch.
    // With pairs, every P is stored as hi + lo (the first in Q0 / Q0_lo,
    // later ones in B / B_lo) and read as such by P P, Q P and, when Q is
    // still the first P (a phase of one iteration), by X <- Q X; T = P P is
    // stored as T / T_lo and read as such by A T.
    const std::vector<int> phases = gram_phases(K);
    auto lo_of = [&](int32_t buf) { return !split ? kBufNone : buf == kBufQ0 ? kBufQ0lo : kBufBlo; };
    int32_t cur = 0;
    for (size_t ph = 0; ph < phases.size(); ++ph) {
      const int32_t first = ph == 0, last_phase = ph + 1 == phases.size();
      auto part = [&](int32_t a_, int32_t b_, int32_t r_, float cb, float cc, float cdiag) {
        return Part{1, a_, b_, r_, cur, 0, 0.f, cb, cc, cdiag};
      };
      gemm(chain[1], kLkGram, {Part{1, kBufA, kBufB, kBufNone, cur, first, 0.f, 0.f, 0.f, 0.f}});
      int32_t acur = kBufA, anext = kBufA1, qcur = kBufQ0;
      bool q_is_p0 = true;  // Q still holds the phase's first P (a pair)
      for (int i = 0; i < phases[ph]; ++i) {
        const int32_t pbuf = i == 0 ? kBufQ0 : kBufB;
        Part pp = part(acur, pbuf, kBufNone, cfg.b, cfg.c, cfg.a);  // P
        pp.o_lo = lo_of(pbuf);
        gemm(chain[1], kLkSquare, {pp});
        std::vector<Part> next;
        if (i + 1 < phases[ph]) {
          Part t = part(pbuf, kBufT, kBufNone, 0.f, 1.f, 0.f);  // T = P P
          t.l_lo = lo_of(pbuf);
          t.o_lo = split ? kBufTlo : kBufNone;
          next.push_back(t);
        }
        if (i > 0) {
          const int32_t qnext = qcur == kBufQ0 ? kBufQ1 : kBufQ0;
          Part qp = part(qcur, qnext, pbuf, 0.f, 1.f, 0.f);  // Q P
          qp.l_lo = q_is_p0 ? lo_of(qcur) : kBufNone;
          qp.r_lo = lo_of(pbuf);
          next.push_back(qp);
          qcur = qnext;
          q_is_p0 = false;
        }
        if (!next.empty()) gemm(chain[1], kLkSquare, next);
        if (i + 1 < phases[ph]) {
          Part at = part(acur, anext, kBufT, 0.f, 1.f, 0.f);  // A T
          at.r_lo = split ? kBufTlo : kBufNone;
          gemm(chain[1], kLkSquare, {at});
          std::swap(acur, anext);
        }
      }
      Part ap{1, kBufA, qcur, kBufNone, cur, first, 0.f, 0.f, 0.f, 0.f};
      ap.l_lo = q_is_p0 ? lo_of(qcur) : kBufNone;
      gemm(chain[1], last_phase ? kLkFinal : kLkApply, {ap});
      cur ^= 1;
    }
    for (Launch &l : chain[1]) l.fp32 = fp32;
  }
  // The two chains touch disjoint matrices: merge them into one sequence
  // that keeps each chain's order and runs a launch of each chain as one
  // grouped launch where it can, which fills the chip better than either
  // launch alone.  Launches of the same kind merge (score 2); a Gram launch
  // of one chain merges with a Square launch of the other (score 1: one
  // kernel instance dispatches each tile to its stage's code).  The merge
  // maximises the total score by dynamic programming over the two chains; a
  // list-schedule simulation of workload 4 (Llama-3.1-8B share) puts this
  // weighting at the best merge of any weighting (19 launches instead of 21).
  auto mixable = [](int32_t x, int32_t y) {
    return (x == kLkGram && y == kLkSquare) || (x == kLkSquare && y == kLkGram);
  };
  std::vector<Launch> merged;
  {
    const size_t n0 = chain[0].size(), n1 = chain[1].size();
    std::vector<std::vector<int32_t>> best(n0 + 1, std::vector<int32_t>(n1 + 1, 0));
    auto pair_score = [&](size_t i, size_t j) {
      const int32_t x = chain[0][i].kind, y = chain[1][j].kind;
      return x == y ? 2 : mixable(x, y) ? 1 : 0;
    };
    for (size_t i = n0 + 1; i-- > 0;)
      for (size_t j = n1 + 1; j-- > 0;) {
        if (i == n0 && j == n1) continue;
        int32_t b = 0;
        if (i < n0) b = std::max(b, best[i + 1][j]);
        if (j < n1) b = std::max(b, best[i][j + 1]);
        if (i < n0 && j < n1 && pair_score(i, j) > 0) b = std::max(b, best[i + 1][j + 1] + pair_score(i, j));
        best[i][j] = b;
      }
    size_t i = 0, j = 0;
    while (i < n0 || j < n1) {
      if (i < n0 && j < n1 && pair_score(i, j) > 0 && best[i][j] == best[i + 1][j + 1] + pair_score(i, j)) {
        Launch l = chain[0][i];
        if (l.kind != chain[1][j].kind) l.kind = kLkGramSquare;
        l.parts.insert(l.parts.end(), chain[1][j].parts.begin(), chain[1][j].parts.end());
        l.flops += chain[1][j].flops;
        merged.push_back(std::move(l));
        ++i, ++j;
      } else if (j >= n1 || (i < n0 && best[i + 1][j] >= best[i][j + 1])) {
        merged.push_back(chain[0][i++]);
      } else {
        merged.push_back(chain[1][j++]);
      }
    }
  }
  // the small matrices' fp32 launches share no launch with the bf16 ones
  // (another kernel instance): they run after them
  merged.insert(merged.end(), chain[2].begin(), chain[2].end());
  if (K == 0) {
    p.prog.push_back(Launch{kLkMomentumSumsq});
    p.prog.push_back(Launch{kLkNorm});
    p.prog.push_back(Launch{kLkUpdateDirect});
  } else {
    p.prog.push_back(Launch{kLkMomentumOrient});
    p.prog.push_back(Launch{kLkNorm});
  }
  p.chain_counters = 0;
  if ((cfg.flags & DMUON_FLAG_CHAIN_LAUNCH) && K > 0) {
    std::vector<Launch> rest, in_chain;
    for (Launch &l : merged) (l.fp32 ? rest : in_chain).push_back(std::move(l));
    if (!in_chain.empty()) chain_launch(p, in_chain);
    merged = std::move(rest);
  }
  // tables and tile lists, shared by launches with equal parts / groups
  std::map<std::vector<Part>, int32_t> table_of;
  std::map<std::vector<int32_t>, int32_t> list_of;
  for (Launch &l : merged) {
    auto t = table_of.find(l.parts);
    if (t == table_of.end()) {
      t = table_of.emplace(l.parts, 1 + static_cast<int32_t>(p.tables.size())).first;
      p.tables.push_back(l.parts);
    }
    l.table = t->second;
    std::vector<int32_t> key;  // (group, passes, stage) of every part
    for (const Part &pt : l.parts) {
      key.push_back(pt.group);
      key.push_back(pt.passes());
      key.push_back(pt.stage());
    }
    auto li = list_of.find(key);
    if (li == list_of.end()) {
      std::vector<MatDev> shapes;
      std::vector<int32_t> passes, stages;
      for (size_t q = 0; q < key.size(); q += 3)
        for (int32_t i : p.groups[key[q]]) {
          shapes.push_back(p.mats[i]);
          passes.push_back(key[q + 1]);
          stages.push_back(key[q + 2]);
        }
      p.lists.emplace_back();
      p.list_xcd.emplace_back();
      cached_stage_tiles(shapes, passes, stages, 256, p.lists.back(), p.list_xcd.back());
      li = list_of.emplace(key, static_cast<int32_t>(p.lists.size()) - 1).first;
    }
    l.list = li->second;
    const std::vector<int64_t> rs = row_steps(p, l);
    std::vector<int64_t> steps;
    for (const TileEntry &e : p.lists[l.list]) steps.push_back(rs[e.mat]);
    // a bf16 Square launch with too few 256-tiles for the CUs runs 128-tiles
    // where the list-schedule estimate says they finish sooner (a 128-tile
    // list enters the plan, and the workspace, only when taken)
    if (l.kind == kLkSquare && !l.fp32 && static_cast<int64_t>(steps.size()) < kCUs) {
      std::vector<int32_t> key128 = key;
      key128.push_back(128);
      auto l128 = list_of.find(key128);
      if (l128 == list_of.end()) {
        std::vector<MatDev> shapes;
        std::vector<int32_t> passes, stages;
        for (size_t q = 0; q < key.size(); q += 3)
          for (int32_t i : p.groups[key[q]]) {
            shapes.push_back(p.mats[i]);
            passes.push_back(key[q + 1]);
            stages.push_back(key[q + 2]);
          }
        std::vector<TileEntry> t128;
        StageXcd x128;
        cached_stage_tiles(shapes, passes, stages, 128, t128, x128);
        std::vector<int64_t> steps128;
        for (const TileEntry &e : t128) steps128.push_back(rs[e.mat]);
        if (small_tiles_pay(steps, steps128)) {
          p.lists.push_back(std::move(t128));
          p.list_xcd.push_back(x128);
          l128 = list_of.emplace(key128, static_cast<int32_t>(p.lists.size()) - 1).first;
        }
      }
      if (l128 != list_of.end()) {
        l.tile = 128;
        l.list = l128->second;
        p.prog.push_back(std::move(l));
        continue;
      }
    }
    // split K where the launch leaves CUs idle
    const std::vector<TileEntry> &tl = p.lists[l.list];
    const std::vector<int32_t> pieces = choose_pieces(steps);
    if (*std::max_element(pieces.begin(), pieces.end()) > 1) {
      std::vector<std::pair<int64_t, TileEntry>> pc, rd;
      int32_t slot = 0;
      for (size_t t = 0; t < tl.size(); ++t) {
        TileEntry r = tl[t];
        r.k0 = pieces[t];
        r.k1 = 0;
        r.slot = slot;
        rd.emplace_back(1, r);
        for (int32_t q = 0; q < pieces[t]; ++q) {
          TileEntry e = tl[t];
          e.k0 = static_cast<int32_t>((steps[t] * q) / pieces[t]);
          e.k1 = static_cast<int32_t>((steps[t] * (q + 1)) / pieces[t]);
          e.slot = slot++;
          pc.emplace_back(e.k1 - e.k0, e);
        }
      }
      p.splitk_slots = std::max<int64_t>(p.splitk_slots, slot);
      Launch lp = l, lr = l;
      lp.role = 1;
      lr.role = 2;
      lr.flops = 0;
      p.lists.emplace_back();
      p.list_xcd.emplace_back();
      assign_xcds(pc, p.lists.back(), p.list_xcd.back());
      lp.list = static_cast<int32_t>(p.lists.size()) - 1;
      p.lists.emplace_back();
      p.list_xcd.emplace_back();
      assign_xcds(rd, p.lists.back(), p.list_xcd.back());
      lr.list = static_cast<int32_t>(p.lists.size()) - 1;
      p.prog.push_back(std::move(lp));
      p.prog.push_back(std::move(lr));
      continue;
    }
    p.prog.push_back(std::move(l));
  }

  // ---- workspace layout ----
  int64_t off = 0;
  const size_t ntab = 1 + p.tables.size();
  p.off_table.assign(ntab, 0);
  for (size_t t = 0; t < ntab; ++t) {
    p.off_table[t] = off;
    int64_t cnt = t == 0 ? n : 0;
    if (t > 0)
      for (const Part &pt : p.tables[t - 1]) cnt += static_cast<int64_t>(p.groups[pt.group].size());
    off = round_up(off + int64_t(sizeof(MatDev)) * cnt, 256);
  }
  p.off_list.assign(p.lists.size(), 0);
  for (size_t l = 0; l < p.lists.size(); ++l) {
    p.off_list[l] = off;
    off = round_up(off + int64_t(sizeof(TileEntry)) * static_cast<int64_t>(p.lists[l].size()), 256);
  }
  p.table_bytes = off;
  p.off_splitk = -1;
  if (p.splitk_slots > 0) {
    p.off_splitk = off;
    off = round_up(off + 4 * kPartialSlotFloats * p.splitk_slots, 256);
  }
  p.off_partials = off;
  off = round_up(off + 8 * (K > 0 ? tr : ew), 256);
  p.off_inv = off;
  off = round_up(off + 256 * int64_t(n), 256);  // one 256-byte slot per matrix
  p.off_flags = -1;
  if (cfg.flags & DMUON_FLAG_CHECK_FINITE) {  // one int32 per matrix
    p.off_flags = off;
    off = round_up(off + 4 * int64_t(n), 256);
  }
  p.off_chain = -1;
  if (p.chain_counters > 0) {  // tickets, timeout word, counters
    p.off_chain = off;
    off = round_up(off + 4 * (kChainCounters + p.chain_counters), 256);
  }
  for (int32_t i = 0; i < n; ++i) {
    MatDev &d = p.mats[i];
    // sum-of-squares partials: one per orientation tile, or per flat chunk
    // when there is no Newton-Schulz iteration
    d.partials = ws ? reinterpret_cast<double *>(ws + p.off_partials) +
                          (K > 0 ? d.tr_first : d.ew_first)
                    : nullptr;
    d.part_count = K > 0 ? static_cast<int32_t>(orient_groups(d)) : d.ew_count;
    d.inv_norm = ws ? reinterpret_cast<float *>(ws + p.off_inv + 256 * int64_t(i)) : nullptr;
    d.nonfinite = ws && p.off_flags >= 0 ? reinterpret_cast<int32_t *>(ws + p.off_flags) + i : nullptr;
    if (K == 0) continue;
    const int64_t es = d.ws_f32 ? 4 : 2;
    const int64_t xb = d.mp * d.np * es, ab = d.mp * d.mp * es;
    const int nbuf = K >= 2 ? 2 : 1;
    for (int b = 0; b < nbuf; ++b) {
      d.xt[b] = ws ? ws + off : nullptr;
      off = round_up(off + xb, 256);
    }
    d.a = ws ? ws + off : nullptr;
    off = round_up(off + ab, 256);
    d.b = ws ? ws + off : nullptr;
    off = round_up(off + ab, 256);
    auto add = [&](int32_t buf) {
      p.extra[i][buf - kBufA1] = ws ? ws + off : nullptr;
      p.have[i] |= 1u << buf;
      off = round_up(off + ab, 256);
    };
    p.have[i] |= (1u << kBufA) | (1u << kBufB);
    if (uses_gram(d, cfg))
      for (int32_t b : {kBufA1, kBufT, kBufQ0, kBufQ1}) add(b);
    if (split && !d.ws_f32) {
      add(kBufBlo);
      if (uses_gram(d, cfg)) {
        add(kBufQ0lo);
        add(kBufTlo);
      }
    }
  }
  p.total_bytes = off;
}

// The chained launch's waits: every entry waits (k0 >= 0) only for a
// counter whose k1 signalling entries all sit earlier in the same XCD's
// queue, so that the work-groups holding them took their tickets first and
// are running; counters are signalled only by entries of one XCD.
bool chain_consistent(const Plan &p, const Launch &l) {
  if (l.role != 0 || l.tile != 256 || l.fp32 || p.off_chain < 0) return false;
  const std::vector<TileEntry> &tl = p.lists[l.list];
  const StageXcd &xcd = p.list_xcd[l.list];
  const int64_t nc = p.chain_counters;
  std::vector<int64_t> total(nc, 0);
  std::vector<int32_t> xcd_of(nc, -1);
  for (int x = 0; x < kXcds; ++x)
    for (int32_t q = xcd.first[x]; q < xcd.first[x] + xcd.count[x]; ++q) {
      const TileEntry &e = tl[q];
      if (e.slot < 0 || e.slot >= nc) return false;
      if (xcd_of[e.slot] >= 0 && xcd_of[e.slot] != x) return false;
      xcd_of[e.slot] = x;
      ++total[e.slot];
    }
  for (int x = 0; x < kXcds; ++x) {
    std::vector<int64_t> seen(nc, 0);
    for (int32_t q = xcd.first[x]; q < xcd.first[x] + xcd.count[x]; ++q) {
      const TileEntry &e = tl[q];
      if (e.k0 >= 0) {
        if (e.k0 >= nc || xcd_of[e.k0] != x || e.k1 != total[e.k0] || seen[e.k0] != total[e.k0]) return false;
        if (e.k0 == e.slot) return false;
      } else if (e.k0 != -1) {
        return false;
      }
      ++seen[e.slot];
    }
  }
  return true;
}

// Internal consistency of a plan, checked on the host before any launch:
// every tile of every GEMM launch names a matrix of that launch's table and
// a tile inside it (upper triangle for the symmetric stages), and each
// table's X^T buffers exist where the launch reads or writes them.
bool plan_consistent(const Plan &p) {
  for (const Launch &l : p.prog) {
    if (l.kind < kLkGram) continue;
    if (l.table < 1 || l.table > static_cast<int32_t>(p.tables.size())) return false;
    if (l.list < 0 || l.list >= static_cast<int32_t>(p.lists.size())) return false;
    std::vector<const MatDev *> rows;
    std::vector<bool> row_sym;
    for (const Part &pt : p.tables[l.table - 1]) {
      if (pt.group < 0 || pt.group > 2) return false;
      // a part runs its launch's stage; a mixed launch holds Gram and
      // Square parts only
      if (l.kind == kLkChain ? pt.kind < kLkGram || pt.kind > kLkFinal
          : l.kind == kLkGramSquare ? pt.kind != kLkGram && pt.kind != kLkSquare
                                    : pt.kind != l.kind)
        return false;
      // a capturing Square (b A from its R tile) must not read a pair: the
      // capture is taken in the first pass only
      if (pt.kind == kLkSquare && pt.cb != 0.f && (pt.l_lo != kBufNone || pt.r_lo != kBufNone)) return false;
      if (pt.kind != kLkSquare && (pt.r_lo != kBufNone || pt.o_lo != kBufNone)) return false;
      if (pt.kind == kLkGram && pt.l_lo != kBufNone) return false;
      for (int32_t i : p.groups[pt.group]) {
        rows.push_back(&p.mats[i]);
        row_sym.push_back(pt.kind == kLkGram || pt.kind == kLkSquare);
        for (int32_t b : {pt.a, pt.b, pt.r, pt.l_lo, pt.r_lo, pt.o_lo})
          if (b != kBufNone && !(p.have[i] >> b & 1u)) return false;
        // the second X^T buffer is read (cur = 1) or written (Apply); the
        // sizing pass has no addresses yet
        const bool needs_xt1 = pt.cur || pt.kind == kLkApply;
        if (needs_xt1 && p.mats[i].xt[0] && !p.mats[i].xt[1]) return false;
      }
    }
    const int32_t n = static_cast<int32_t>(rows.size());
    // 128-tiles: bf16 Square launches of whole tiles only
    if (l.tile != 256 && (l.tile != 128 || l.kind != kLkSquare || l.fp32 || l.role != 0)) return false;
    const std::vector<int64_t> rs = row_steps(p, l);
    for (const TileEntry &e : p.lists[l.list]) {
      if (e.mat < 0 || e.mat >= n) return false;
      const MatDev &d = *rows[e.mat];
      const bool sym = row_sym[e.mat];
      const int64_t rows = d.mp / l.tile, cols = (sym ? d.mp : d.np) / l.tile;
      if (e.ti >= rows || e.tj >= cols || (sym && e.tj < e.ti)) return false;
      // pieces: a step range inside the tile's K loop and a slot; reduce
      // entries: at least one slot, all inside the partial region
      if (l.role == 1 && (e.k0 < 0 || e.k1 <= e.k0 || e.k1 > rs[e.mat] || e.slot < 0 || e.slot >= p.splitk_slots))
        return false;
      if (l.role == 2 && (e.k1 != 0 || e.k0 < 1 || e.slot < 0 || e.slot + e.k0 > p.splitk_slots)) return false;
    }
    if (l.kind == kLkChain && !chain_consistent(p, l)) return false;
  }
  return true;
}

// Every GEMM launch computes each output tile of each of its table rows
// exactly once: whole, chained and reduce entries once per tile (the upper
// triangle for the symmetric products), and a split launch's pieces of a
// tile cover its K steps without gap or overlap.  Checked by
// dmuon_step_launches (the host tests), not on every step.
bool plan_covers(const Plan &p) {
  for (const Launch &l : p.prog) {
    if (l.kind < kLkGram) continue;
    std::vector<const MatDev *> rows;
    std::vector<bool> row_sym;
    for (const Part &pt : p.tables[l.table - 1])
      for (int32_t i : p.groups[pt.group]) {
        rows.push_back(&p.mats[i]);
        row_sym.push_back(pt.kind == kLkGram || pt.kind == kLkSquare);
      }
    const std::vector<int64_t> rs = row_steps(p, l);
    std::vector<int64_t> first(rows.size() + 1, 0);
    for (size_t r = 0; r < rows.size(); ++r) {
      const MatDev &d = *rows[r];
      first[r + 1] = first[r] + (d.mp / l.tile) * ((row_sym[r] ? d.mp : d.np) / l.tile);
    }
    std::vector<int32_t> seen(static_cast<size_t>(first.back()), 0);
    std::vector<std::vector<std::pair<int32_t, int32_t>>> pieces(l.role == 1 ? seen.size() : 0);
    for (const TileEntry &e : p.lists[l.list]) {
      const MatDev &d = *rows[e.mat];
      const int64_t cols = (row_sym[e.mat] ? d.mp : d.np) / l.tile;
      const int64_t at = first[e.mat] + e.ti * cols + e.tj;
      if (l.role == 1)
        pieces[at].emplace_back(e.k0, e.k1);
      else if (seen[at]++)
        return false;
    }
    for (size_t r = 0; r < rows.size(); ++r) {
      const MatDev &d = *rows[r];
      const int64_t nr = d.mp / l.tile, nc = (row_sym[r] ? d.mp : d.np) / l.tile;
      for (int64_t ti = 0; ti < nr; ++ti)
        for (int64_t tj = row_sym[r] ? ti : 0; tj < nc; ++tj) {
          const int64_t at = first[r] + ti * nc + tj;
          if (l.role != 1) {
            if (seen[at] != 1) return false;
            continue;
          }
          std::vector<std::pair<int32_t, int32_t>> &pc = pieces[at];
          std::sort(pc.begin(), pc.end());
          int64_t k = 0;
          for (const auto &q : pc) {
            if (q.first != k) return false;
            k = q.second;
          }
          if (k != rs[r]) return false;
        }
    }
  }
  return true;
}

// The MatDev array of table t (0: every matrix; else, for each part of the
// launch in turn, its group's matrices with the part's buffers, X^T order
// and coefficients).
std::vector<MatDev> table_contents(const Plan &p, size_t t) {
  if (t == 0) return p.mats;
  std::vector<MatDev> out;
  for (const Part &pt : p.tables[t - 1]) {
    for (int32_t i : p.groups[pt.group]) {
      MatDev d = p.mats[i];
      auto buf = [&](int32_t b) -> void * {
        if (b == kBufNone) return nullptr;
        if (b == kBufA) return p.mats[i].a;
        if (b == kBufB) return p.mats[i].b;
        return p.extra[i][b - kBufA1];
      };
      d.a = buf(pt.a);
      d.b = buf(pt.b);
      d.sq_r = buf(pt.r);
      d.l_lo = buf(pt.l_lo);
      d.r_lo = buf(pt.r_lo);
      d.out_lo = buf(pt.o_lo);
      if (pt.cur) std::swap(d.xt[0], d.xt[1]);
      d.ca = pt.ca;
      d.cb = pt.cb;
      d.cc = pt.cc;
      d.cdiag = pt.cdiag;
      d.first_it = pt.first;
      d.gemm_kind = pt.kind == kLkGram     ? kModeGram
                    : pt.kind == kLkSquare ? kModeSquare
                    : pt.kind == kLkApply  ? kModeApply
                                           : kModeFinal;
      out.push_back(d);
    }
  }
  return out;
}

// ------------------------------------------------- pinned staging uploads --
struct Slot {
  void *host = nullptr;
  size_t cap = 0;
  hipEvent_t ev = nullptr;
  bool pending = false;
};
struct Ring {
  Slot slots[4];
  int next = 0;
};
std::mutex g_ring_mu;
std::map<int, Ring> g_rings;

// Copies `bytes` of host data to device memory `dst` on `st`, through a
// pinned staging slot that is reused only after its previous copy finished.
int upload(void *dst, const std::vector<char> &src, hipStream_t st) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lock(g_ring_mu);
  Ring &ring = g_rings[dev];
  Slot &s = ring.slots[ring.next];
  ring.next = (ring.next + 1) % 4;
  if (s.pending) {
    e = hipEventSynchronize(s.ev);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    s.pending = false;
  }
  if (!s.ev) {
    e = hipEventCreateWithFlags(&s.ev, hipEventDisableTiming);
    if (e != hipSuccess) return hip_fail(e, "hipEventCreateWithFlags");
  }
  if (s.cap < src.size()) {
    if (s.host) (void)hipHostFree(s.host);
    s.host = nullptr;
    s.cap = 0;
    const size_t cap = std::max<size_t>(65536, src.size() * 2);
    e = hipHostMalloc(&s.host, cap, hipHostMallocDefault);
    if (e != hipSuccess) return hip_fail(e, "hipHostMalloc");
    s.cap = cap;
  }
  std::memcpy(s.host, src.data(), src.size());
  e = hipMemcpyAsync(dst, s.host, src.size(), hipMemcpyHostToDevice, st);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync");
  e = hipEventRecord(s.ev, st);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  s.pending = true;
  return DMUON_OK;
}

// The no-allocation path's table upload: a static (pageable) host buffer,
// reused only after the copy from it has completed (an event per device,
// created on first use; events are not memory allocations).
constexpr size_t kNoAllocTableBytes = size_t(4) << 20;
std::mutex g_static_mu;
char g_static_host[kNoAllocTableBytes];
hipEvent_t g_static_ev[64] = {};
hipEvent_t g_static_last = nullptr;

int upload_static(void *dst, const std::vector<char> &src, hipStream_t st) {
  if (src.size() > kNoAllocTableBytes)
    return fail(DMUON_ERR_WORKSPACE_TOO_SMALL, "launch tables need %zu bytes, the static staging holds %zu",
                src.size(), kNoAllocTableBytes);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(DMUON_ERR_INVALID_ARG, "device %d beyond the static path's 64", dev);
  std::lock_guard<std::mutex> lock(g_static_mu);
  if (g_static_last) {
    e = hipEventSynchronize(g_static_last);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    g_static_last = nullptr;
  }
  if (!g_static_ev[dev]) {
    e = hipEventCreateWithFlags(&g_static_ev[dev], hipEventDisableTiming);
    if (e != hipSuccess) return hip_fail(e, "hipEventCreateWithFlags");
  }
  std::memcpy(g_static_host, src.data(), src.size());
  e = hipMemcpyAsync(dst, g_static_host, src.size(), hipMemcpyHostToDevice, st);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync");
  e = hipEventRecord(g_static_ev[dev], st);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  g_static_last = g_static_ev[dev];
  return DMUON_OK;
}

int check_launch(hipError_t e, const char *what) {
  return e == hipSuccess ? DMUON_OK : hip_fail(e, what);
}

}  // namespace
}  // namespace dmuon

using namespace dmuon;

extern "C" {

int dmuon_abi_version(void) { return DMUON_ABI_VERSION; }

const char *dmuon_error_string(int status) {
  switch (status) {
    case DMUON_OK: return "ok";
    case DMUON_ERR_INVALID_ARG: return "invalid argument";
    case DMUON_ERR_UNSUPPORTED_DTYPE: return "unsupported dtype";
    case DMUON_ERR_ALIAS: return "overlapping buffers";
    case DMUON_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case DMUON_ERR_MISALIGNED: return "misaligned pointer";
    case DMUON_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char *dmuon_last_error(void) { return g_last_error.c_str(); }

int dmuon_partition_lpt(const int64_t *numel, int32_t n, int32_t n_owners, int32_t *owner_out,
                        int64_t *load_out) {
  g_last_error.clear();
  if (n < 0) return fail(DMUON_ERR_INVALID_ARG, "n < 0");
  if (n_owners < 1) return fail(DMUON_ERR_INVALID_ARG, "n_owners < 1");
  if (n > 0 && (!numel || !owner_out)) return fail(DMUON_ERR_INVALID_ARG, "NULL array");
  for (int32_t i = 0; i < n; ++i)
    if (numel[i] < 0) return fail(DMUON_ERR_INVALID_ARG, "numel[%d] < 0", i);
  std::vector<int32_t> order(n);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(),
                   [&](int32_t x, int32_t y) { return numel[x] > numel[y]; });
  // owners keyed by (load, id): the smallest key takes the next matrix
  std::vector<std::pair<int64_t, int32_t>> heap;
  heap.reserve(n_owners);
  for (int32_t r = 0; r < n_owners; ++r) heap.emplace_back(0, r);
  auto cmp = [](const std::pair<int64_t, int32_t> &x, const std::pair<int64_t, int32_t> &y) {
    return x > y;  // min-heap
  };
  std::make_heap(heap.begin(), heap.end(), cmp);
  std::vector<int64_t> load(n_owners, 0);
  for (int32_t i : order) {
    std::pop_heap(heap.begin(), heap.end(), cmp);
    auto [l, r] = heap.back();
    owner_out[i] = r;
    load[r] = l + numel[i];
    heap.back() = {load[r], r};
    std::push_heap(heap.begin(), heap.end(), cmp);
  }
  if (load_out) std::copy(load.begin(), load.end(), load_out);
  return DMUON_OK;
}

int dmuon_pack_offsets(const int64_t *numel, int32_t n, int64_t align, int64_t *offset_out,
                       int64_t *total_out) {
  g_last_error.clear();
  if (n < 0 || align < 1) return fail(DMUON_ERR_INVALID_ARG, "n < 0 or align < 1");
  if (!total_out || (n > 0 && (!numel || !offset_out)))
    return fail(DMUON_ERR_INVALID_ARG, "NULL array");
  int64_t end = 0;
  for (int32_t i = 0; i < n; ++i) {
    if (numel[i] < 0) return fail(DMUON_ERR_INVALID_ARG, "numel[%d] < 0", i);
    const int64_t start = round_up(end, align);
    offset_out[i] = start;
    end = start + numel[i];
  }
  *total_out = round_up(end, align);
  return DMUON_OK;
}

int dmuon_nonfinite_flags_offset(const dmuon_matrix *mats, int32_t n, const dmuon_step_config *cfg,
                                 size_t *offset_out) {
  g_last_error.clear();
  if (!offset_out) return fail(DMUON_ERR_INVALID_ARG, "offset_out is NULL");
  int rc = validate_config(cfg);
  if (rc) return rc;
  if (!(cfg->flags & DMUON_FLAG_CHECK_FINITE))
    return fail(DMUON_ERR_INVALID_ARG, "DMUON_FLAG_CHECK_FINITE is not set");
  rc = validate_shapes(mats, n);
  if (rc) return rc;
  rc = validate_step_shapes(mats, n);
  if (rc) return rc;
  Plan p;
  build_plan(mats, n, *cfg, nullptr, p);
  *offset_out = static_cast<size_t>(p.off_flags);
  return DMUON_OK;
}

int dmuon_chain_status_offset(const dmuon_matrix *mats, int32_t n, const dmuon_step_config *cfg,
                              size_t *offset_out) {
  g_last_error.clear();
  if (!offset_out) return fail(DMUON_ERR_INVALID_ARG, "offset_out is NULL");
  int rc = validate_config(cfg);
  if (rc) return rc;
  if (!(cfg->flags & DMUON_FLAG_CHAIN_LAUNCH))
    return fail(DMUON_ERR_INVALID_ARG, "DMUON_FLAG_CHAIN_LAUNCH is not set");
  rc = validate_shapes(mats, n);
  if (rc) return rc;
  rc = validate_step_shapes(mats, n);
  if (rc) return rc;
  Plan p;
  build_plan(mats, n, *cfg, nullptr, p);
  if (p.off_chain < 0) return fail(DMUON_ERR_INVALID_ARG, "the step has no chained launch");
  // the word after the per-XCD tickets
  *offset_out = static_cast<size_t>(p.off_chain) + sizeof(int32_t) * kXcds;
  return DMUON_OK;
}

int dmuon_workspace_bytes(const dmuon_matrix *mats, int32_t n, const dmuon_step_config *cfg,
                          size_t *out_bytes) {
  g_last_error.clear();
  if (!out_bytes) return fail(DMUON_ERR_INVALID_ARG, "out_bytes is NULL");
  int rc = validate_config(cfg);
  if (rc) return rc;
  rc = validate_shapes(mats, n);
  if (rc) return rc;
  rc = validate_step_shapes(mats, n);
  if (rc) return rc;
  Plan p;
  build_plan(mats, n, *cfg, nullptr, p);
  *out_bytes = static_cast<size_t>(p.total_bytes);
  return DMUON_OK;
}

// packed == nullptr: no packed copy of the updated params.  noalloc: the
// workspace is this device's static scratch (workspace / workspace_bytes
// are ignored) and the tables go through the static host buffer.
static int muon_step_impl(const dmuon_matrix *mats, int32_t n, const dmuon_step_config *cfg,
                          void *workspace, size_t workspace_bytes, void *stream,
                          void *const *events, int32_t n_events, void *packed = nullptr,
                          int32_t packed_dtype = DMUON_BF16, int64_t packed_numel = 0,
                          bool noalloc = false) {
  g_last_error.clear();
  if (n_events < 0 || (n_events > 0 && !events))
    return fail(DMUON_ERR_INVALID_ARG, "bad event list");
  if (packed) {
    if (!dtype_ok(packed_dtype))
      return fail(DMUON_ERR_UNSUPPORTED_DTYPE, "packed dtype %d", packed_dtype);
    if (packed_numel < 0) return fail(DMUON_ERR_INVALID_ARG, "packed_numel < 0");
  }
  int rc = validate_config(cfg);
  if (rc) return rc;
  rc = validate_shapes(mats, n);
  if (rc) return rc;
  rc = validate_step_shapes(mats, n);
  if (rc) return rc;
  if (n == 0) return DMUON_OK;

  std::vector<Interval> iv;
  iv.reserve(4 * n + 1);
  for (int32_t i = 0; i < n; ++i) {
    const dmuon_matrix &d = mats[i];
    if (!d.param || !d.grad || !d.momentum)
      return fail(DMUON_ERR_INVALID_ARG, "matrix %d: NULL param, grad or momentum", i);
    if (!aligned16(d.param) || !aligned16(d.grad) || !aligned16(d.momentum) ||
        (d.orth_out && !aligned16(d.orth_out)))
      return fail(DMUON_ERR_MISALIGNED, "matrix %d: pointers must be 16-byte aligned", i);
    const uintptr_t numel = static_cast<uintptr_t>(d.rows * d.cols);
    auto add = [&](const void *ptr, int64_t es, bool w, const char *what) {
      const uintptr_t lo = reinterpret_cast<uintptr_t>(ptr);
      iv.push_back(Interval{lo, lo + numel * es, w, what, i});
    };
    add(d.param, elem_size(d.param_dtype), true, "param");
    add(d.grad, elem_size(d.grad_dtype), false, "grad");
    add(d.momentum, 4, true, "momentum");
    if (d.orth_out) add(d.orth_out, elem_size(d.param_dtype), true, "orth_out");
    if (packed) {
      if (d.param_dtype != packed_dtype)
        return fail(DMUON_ERR_UNSUPPORTED_DTYPE, "matrix %d: param dtype %d != packed dtype %d", i,
                    d.param_dtype, packed_dtype);
      const int64_t ne = d.rows * d.cols;
      if (d.packed_offset < 0 || d.packed_offset > packed_numel - ne)
        return fail(DMUON_ERR_INVALID_ARG, "matrix %d: [%lld, +%lld) outside packed buffer of %lld", i,
                    (long long)d.packed_offset, (long long)ne, (long long)packed_numel);
      const char *slot = static_cast<const char *>(packed) + d.packed_offset * elem_size(packed_dtype);
      if (!aligned16(slot))
        return fail(DMUON_ERR_MISALIGNED, "matrix %d: packed slot not 16-byte aligned", i);
      add(slot, elem_size(packed_dtype), true, "packed slot");
    }
  }

  rc = check_aliasing(iv);  // caller buffers among themselves
  if (rc) return rc;
  Plan p;
  build_plan(mats, n, *cfg, nullptr, p);
  if (noalloc) {
    if (static_cast<size_t>(p.total_bytes) > kNoAllocScratchBytes)
      return fail(DMUON_ERR_WORKSPACE_TOO_SMALL,
                  "these matrices need %lld bytes of workspace; the static scratch holds %zu",
                  (long long)p.total_bytes, kNoAllocScratchBytes);
    if (static_cast<size_t>(p.table_bytes) > kNoAllocTableBytes)
      return fail(DMUON_ERR_WORKSPACE_TOO_SMALL, "launch tables need %lld bytes; the static staging holds %zu",
                  (long long)p.table_bytes, kNoAllocTableBytes);
    const hipError_t e = noalloc_scratch(&workspace);
    if (e != hipSuccess) return hip_fail(e, "static scratch lookup");
    workspace_bytes = kNoAllocScratchBytes;
  }
  if (workspace_bytes < static_cast<size_t>(p.total_bytes))
    return fail(DMUON_ERR_WORKSPACE_TOO_SMALL, "workspace needs %lld bytes, got %zu",
                (long long)p.total_bytes, workspace_bytes);
  if (!workspace) return fail(DMUON_ERR_INVALID_ARG, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(workspace) & 255u)
    return fail(DMUON_ERR_MISALIGNED, "workspace must be 256-byte aligned");
  {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(workspace);
    iv.push_back(Interval{lo, lo + static_cast<uintptr_t>(p.total_bytes), true, "workspace", -1});
  }
  rc = check_aliasing(iv);  // and against the workspace
  if (rc) return rc;

  // ---- validated: plan with real addresses, upload tables, launch ----
  char *ws = static_cast<char *>(workspace);
  build_plan(mats, n, *cfg, ws, p);
  if (!plan_consistent(p)) return fail(DMUON_ERR_INVALID_ARG, "internal error: inconsistent launch plan");
  if (packed)
    for (int32_t i = 0; i < n; ++i)
      p.mats[i].packed = static_cast<char *>(packed) + mats[i].packed_offset * elem_size(packed_dtype);
  std::vector<char> tables(static_cast<size_t>(p.table_bytes), 0);
  for (size_t t = 0; t < p.off_table.size(); ++t) {
    const std::vector<MatDev> tab = table_contents(p, t);
    if (!tab.empty()) std::memcpy(tables.data() + p.off_table[t], tab.data(), sizeof(MatDev) * tab.size());
  }
  for (size_t l = 0; l < p.lists.size(); ++l)
    if (!p.lists[l].empty())
      std::memcpy(tables.data() + p.off_list[l], p.lists[l].data(), sizeof(TileEntry) * p.lists[l].size());

  hipStream_t s = static_cast<hipStream_t>(stream);
  rc = noalloc ? upload_static(ws, tables, s) : upload(ws, tables, s);
  if (rc) return rc;

  auto dtab = [&](int32_t t) { return reinterpret_cast<const MatDev *>(ws + p.off_table[t]); };
  const MatDev *dm = dtab(0);
  const StepScalars sc{cfg->a, cfg->b, cfg->c, cfg->lr, cfg->momentum, cfg->eps,
                       (cfg->flags & DMUON_FLAG_NESTEROV) ? 1 : 0, 0};

  // events[0] before the first launch, events[j] after launch j
  int32_t ev = 0;
  auto mark = [&]() -> int {
    if (ev < n_events) {
      hipError_t e = hipEventRecord(static_cast<hipEvent_t>(events[ev]), s);
      if (e != hipSuccess) return hip_fail(e, "hipEventRecord (trace)");
    }
    ++ev;
    return DMUON_OK;
  };
  auto launched = [&](hipError_t e, const char *what) -> int {
    const int r = check_launch(e, what);
    return r ? r : mark();
  };

  if ((rc = mark())) return rc;
  for (const Launch &l : p.prog) {
    switch (l.kind) {
      case kLkMomentumSumsq:
        rc = launched(launch_momentum_sumsq(dm, n, p.ew_total, sc, s), "momentum_sumsq launch");
        break;
      case kLkMomentumOrient:
        rc = launched(launch_momentum_orient(dm, n, p.tr_total, sc, s), "momentum_orient launch");
        break;
      case kLkNorm:
        rc = launched(launch_finalize_norm(dm, n, cfg->eps, s), "finalize_norm launch");
        break;
      case kLkUpdateDirect:
        rc = launched(launch_update_direct(dm, n, p.ew_total, sc, s), "update_direct launch");
        break;
      default: {
        const GemmMode mode = l.kind == kLkGram         ? kModeGram
                              : l.kind == kLkSquare     ? kModeSquare
                              : l.kind == kLkGramSquare ? kModeGramSquare
                              : l.kind == kLkApply      ? kModeApply
                                                        : kModeFinal;
        const TileEntry *tl = reinterpret_cast<const TileEntry *>(ws + p.off_list[l.list]);
        float *splitk = p.off_splitk >= 0 ? reinterpret_cast<float *>(ws + p.off_splitk) : nullptr;
        if (l.kind == kLkChain) {
          int32_t *const sync = reinterpret_cast<int32_t *>(ws + p.off_chain);
          rc = check_launch(launch_zero_i32(sync, kChainCounters + p.chain_counters, s), "chained launch reset");
          if (!rc)
            rc = launched(launch_ns_chain(dtab(l.table), tl, p.list_xcd[l.list], sc, sync, s),
                          "chained Newton-Schulz launch");
        } else if (l.tile == 128)
          rc = launched(launch_ns_small_square(dtab(l.table), tl, p.list_xcd[l.list], sc, s),
                        "Newton-Schulz stage launch (128-tiles)");
        else
          rc = launched(launch_ns_stage(mode, l.fp32, l.role, dtab(l.table), tl, p.list_xcd[l.list], sc, splitk, s),
                        "Newton-Schulz stage launch");
      }
    }
    if (rc) return rc;
  }
  return DMUON_OK;
}

int dmuon_step_launches(const dmuon_matrix *mats, int32_t n, const dmuon_step_config *cfg,
                        dmuon_launch_info *out, int32_t cap, int32_t *count) {
  g_last_error.clear();
  if (!count) return fail(DMUON_ERR_INVALID_ARG, "count is NULL");
  if (cap < 0 || (cap > 0 && !out)) return fail(DMUON_ERR_INVALID_ARG, "bad output array");
  int rc = validate_config(cfg);
  if (rc) return rc;
  rc = validate_shapes(mats, n);
  if (rc) return rc;
  rc = validate_step_shapes(mats, n);
  if (rc) return rc;
  if (n == 0) {
    *count = 0;
    return DMUON_OK;
  }
  Plan p;
  build_plan(mats, n, *cfg, nullptr, p);
  if (!plan_consistent(p)) return fail(DMUON_ERR_INVALID_ARG, "internal error: inconsistent launch plan");
  if (!plan_covers(p)) return fail(DMUON_ERR_INVALID_ARG, "internal error: a launch misses or repeats a tile");
  *count = static_cast<int32_t>(p.prog.size());
  for (int32_t j = 0; j < cap && j < *count; ++j) {
    out[j].kind = p.prog[j].kind;
    const bool gemm = p.prog[j].kind >= kLkGram;
    out[j].tile = gemm ? p.prog[j].tile : 0;
    out[j].flops = p.prog[j].flops;
  }
  return DMUON_OK;
}

int dmuon_muon_step(const dmuon_matrix *mats, int32_t n, const dmuon_step_config *cfg,
                    void *workspace, size_t workspace_bytes, void *stream) {
  return muon_step_impl(mats, n, cfg, workspace, workspace_bytes, stream, nullptr, 0);
}

int dmuon_muon_step_traced(const dmuon_matrix *mats, int32_t n, const dmuon_step_config *cfg,
                           void *workspace, size_t workspace_bytes, void *stream,
                           void *const *events, int32_t n_events) {
  return muon_step_impl(mats, n, cfg, workspace, workspace_bytes, stream, events, n_events);
}

int dmuon_muon_step_packed(const dmuon_matrix *mats, int32_t n, const dmuon_step_config *cfg,
                           void *workspace, size_t workspace_bytes, void *packed,
                           int32_t packed_dtype, int64_t packed_numel, void *stream,
                           void *const *events, int32_t n_events) {
  if (!packed) {
    g_last_error.clear();
    return fail(DMUON_ERR_INVALID_ARG, "packed is NULL");
  }
  return muon_step_impl(mats, n, cfg, workspace, workspace_bytes, stream, events, n_events, packed,
                        packed_dtype, packed_numel);
}

int dmuon_muon_step_noalloc(const dmuon_matrix *mats, int32_t n, const dmuon_step_config *cfg,
                            void *stream) {
  return muon_step_impl(mats, n, cfg, nullptr, 0, stream, nullptr, 0, nullptr, DMUON_BF16, 0, true);
}

// ------------------------------------------------------------------ AdamW --
int dmuon_adamw_step(const dmuon_tensor *tensors, int32_t n, const dmuon_adamw_config *cfg,
                     void *stream) {
  g_last_error.clear();
  if (!cfg) return fail(DMUON_ERR_INVALID_ARG, "cfg is NULL");
  const float vals[] = {cfg->lr, cfg->beta1, cfg->beta2, cfg->eps, cfg->weight_decay};
  for (float v : vals)
    if (!std::isfinite(v)) return fail(DMUON_ERR_INVALID_ARG, "non-finite AdamW value");
  if (cfg->beta1 < 0.f || cfg->beta1 >= 1.f || cfg->beta2 < 0.f || cfg->beta2 >= 1.f)
    return fail(DMUON_ERR_INVALID_ARG, "betas must lie in [0, 1)");
  if (cfg->eps <= 0.f) return fail(DMUON_ERR_INVALID_ARG, "eps must be > 0");
  if (cfg->step < 1) return fail(DMUON_ERR_INVALID_ARG, "step must be >= 1");
  if (n < 0) return fail(DMUON_ERR_INVALID_ARG, "n < 0");
  if (n == 0) return DMUON_OK;
  if (!tensors) return fail(DMUON_ERR_INVALID_ARG, "tensors is NULL");
  std::vector<Interval> iv;
  for (int32_t i = 0; i < n; ++i) {
    const dmuon_tensor &t = tensors[i];
    if (t.numel < 1 || t.numel > kMaxNumel)
      return fail(DMUON_ERR_INVALID_ARG, "tensor %d: numel %lld", i, (long long)t.numel);
    if (!dtype_ok(t.param_dtype) || !dtype_ok(t.grad_dtype))
      return fail(DMUON_ERR_UNSUPPORTED_DTYPE, "tensor %d: dtype codes %d/%d", i, t.param_dtype,
                  t.grad_dtype);
    if (!t.param || !t.grad || !t.exp_avg || !t.exp_avg_sq)
      return fail(DMUON_ERR_INVALID_ARG, "tensor %d: NULL pointer", i);
    if (!aligned16(t.param) || !aligned16(t.grad) || !aligned16(t.exp_avg) ||
        !aligned16(t.exp_avg_sq))
      return fail(DMUON_ERR_MISALIGNED, "tensor %d: pointers must be 16-byte aligned", i);
    const uintptr_t ne = static_cast<uintptr_t>(t.numel);
    auto add = [&](const void *ptr, int64_t es, bool w, const char *what) {
      const uintptr_t lo = reinterpret_cast<uintptr_t>(ptr);
      iv.push_back(Interval{lo, lo + ne * es, w, what, i});
    };
    add(t.param, elem_size(t.param_dtype), true, "param");
    add(t.grad, elem_size(t.grad_dtype), false, "grad");
    add(t.exp_avg, 4, true, "exp_avg");
    add(t.exp_avg_sq, 4, true, "exp_avg_sq");
  }
  int rc = check_aliasing(iv);
  if (rc) return rc;
  const double lr = cfg->lr, b1 = cfg->beta1, b2 = cfg->beta2;
  AdamScalars sc;
  sc.decay = static_cast<float>(1.0 - lr * cfg->weight_decay);
  sc.beta1 = cfg->beta1;
  sc.beta2 = cfg->beta2;
  sc.step_size = static_cast<float>(lr / (1.0 - std::pow(b1, cfg->step)));
  sc.inv_sqrt_bc2 = static_cast<float>(1.0 / std::sqrt(1.0 - std::pow(b2, cfg->step)));
  sc.eps = cfg->eps;
  hipStream_t s = static_cast<hipStream_t>(stream);
  AdamBatch b;
  std::memset(&b, 0, sizeof b);
  for (int32_t i = 0; i < n; ++i) {
    const dmuon_tensor &t = tensors[i];
    const int k = b.n;
    b.param[k] = t.param;
    b.grad[k] = t.grad;
    b.m[k] = t.exp_avg;
    b.v[k] = t.exp_avg_sq;
    b.numel[k] = t.numel;
    b.param_dt[k] = t.param_dtype;
    b.grad_dt[k] = t.grad_dtype;
    b.first_block[k + 1] = b.first_block[k] + (t.numel + kAdamChunk - 1) / kAdamChunk;
    b.n = k + 1;
    if (b.n == kAdamBatch || i + 1 == n) {
      if (b.first_block[b.n] > 0x7fffffff) return fail(DMUON_ERR_INVALID_ARG, "AdamW batch too large");
      rc = check_launch(launch_adamw_batch(b, sc, s), "adamw launch");
      if (rc) return rc;
      std::memset(&b, 0, sizeof b);
    }
  }
  return DMUON_OK;
}

// ------------------------------------------------------------ pack/unpack --
static int pack_common(const dmuon_matrix *mats, int32_t n, int32_t field, void *packed_rw,
                       const void *packed, int32_t packed_dtype, int64_t packed_numel,
                       void *stream, bool to_packed) {
  g_last_error.clear();
  if (n < 0) return fail(DMUON_ERR_INVALID_ARG, "n < 0");
  if (n == 0) return DMUON_OK;
  if (!mats || !packed) return fail(DMUON_ERR_INVALID_ARG, "NULL mats or packed");
  if (field != DMUON_FIELD_PARAM && field != DMUON_FIELD_GRAD)
    return fail(DMUON_ERR_INVALID_ARG, "field %d", field);
  if (!dtype_ok(packed_dtype)) return fail(DMUON_ERR_UNSUPPORTED_DTYPE, "packed dtype %d", packed_dtype);
  if (packed_numel < 0) return fail(DMUON_ERR_INVALID_ARG, "packed_numel < 0");
  const int64_t es = elem_size(packed_dtype);
  std::vector<Interval> iv;
  for (int32_t i = 0; i < n; ++i) {
    const dmuon_matrix &d = mats[i];
    if (d.rows < 1 || d.cols < 1 || d.rows >= kMaxDim || d.cols >= kMaxDim ||
        d.rows * d.cols > kMaxNumel)
      return fail(DMUON_ERR_INVALID_ARG, "matrix %d: bad shape", i);
    const int32_t fdt = field == DMUON_FIELD_PARAM ? d.param_dtype : d.grad_dtype;
    if (fdt != packed_dtype)
      return fail(DMUON_ERR_UNSUPPORTED_DTYPE, "matrix %d: field dtype %d != packed dtype %d", i,
                  fdt, packed_dtype);
    const void *fp = field == DMUON_FIELD_PARAM ? d.param : d.grad;
    if (!fp) return fail(DMUON_ERR_INVALID_ARG, "matrix %d: NULL field pointer", i);
    const int64_t numel = d.rows * d.cols;
    if (d.packed_offset < 0 || d.packed_offset > packed_numel - numel)
      return fail(DMUON_ERR_INVALID_ARG, "matrix %d: [%lld, +%lld) outside packed buffer of %lld", i,
                  (long long)d.packed_offset, (long long)numel, (long long)packed_numel);
    const char *pp = static_cast<const char *>(packed) + d.packed_offset * es;
    if (!aligned16(fp) || !aligned16(pp))
      return fail(DMUON_ERR_MISALIGNED, "matrix %d: field or packed slot not 16-byte aligned", i);
    const uintptr_t flo = reinterpret_cast<uintptr_t>(fp), plo = reinterpret_cast<uintptr_t>(pp);
    const uintptr_t bytes = static_cast<uintptr_t>(numel * es);
    iv.push_back(Interval{flo, flo + bytes, !to_packed, "field", i});
    iv.push_back(Interval{plo, plo + bytes, to_packed, "packed slot", i});
  }
  int rc = check_aliasing(iv);
  if (rc) return rc;
  (void)packed_rw;
  hipStream_t s = static_cast<hipStream_t>(stream);
  PackBatch b;
  std::memset(&b, 0, sizeof b);
  for (int32_t i = 0; i < n; ++i) {
    const dmuon_matrix &d = mats[i];
    const void *fp = field == DMUON_FIELD_PARAM ? d.param : d.grad;
    char *pp = const_cast<char *>(static_cast<const char *>(packed)) + d.packed_offset * es;
    const int64_t bytes = d.rows * d.cols * es;
    const int k = b.n;
    b.src[k] = to_packed ? fp : pp;
    b.dst[k] = to_packed ? static_cast<void *>(pp) : const_cast<void *>(fp);
    b.bytes[k] = bytes;
    b.first_block[k + 1] = b.first_block[k] + (bytes + kPackBlockBytes - 1) / kPackBlockBytes;
    b.n = k + 1;
    if (b.n == kPackBatch || i + 1 == n) {
      if (b.first_block[b.n] > 0x7fffffff) return fail(DMUON_ERR_INVALID_ARG, "pack batch too large");
      rc = check_launch(launch_pack_batch(b, s), "pack launch");
      if (rc) return rc;
      std::memset(&b, 0, sizeof b);
    }
  }
  return DMUON_OK;
}

int dmuon_pack(const dmuon_matrix *mats, int32_t n, int32_t field, void *packed,
               int32_t packed_dtype, int64_t packed_numel, void *stream) {
  return pack_common(mats, n, field, packed, packed, packed_dtype, packed_numel, stream, true);
}

int dmuon_unpack(const dmuon_matrix *mats, int32_t n, int32_t field, const void *packed,
                 int32_t packed_dtype, int64_t packed_numel, void *stream) {
  return pack_common(mats, n, field, nullptr, packed, packed_dtype, packed_numel, stream, false);
}

}  // extern "C"

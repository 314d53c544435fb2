// Host side of the C ABI declared in include/dflash.h: argument validation,
// the RoPE table, workspace carving and the kernel sequence of one step.
//
// One step, all on the caller's stream:
//   HK1 grouped GEMM   block rows -> q|k|v, context rows -> k|v; with enough
//                      tiles its epilogue also does HK2's work, else fp32 out
//   HK2 norm_rope      per-head RMSNorm + RoPE + Q pack + cache append
//   HK3 attention      split-KV non-causal GQA over the cache
//   HK4 merge          the pairs HK3 split over several work-groups
//   HK1 GEMM           o_proj
// then the host lengths become T_b = L_b + n_b + bs.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "dflash.h"
#include "kernels.h"

using namespace dflash;

namespace {

constexpr size_t kAlign = 256;
constexpr int kMaxKSlices = 4;  // k splits of the projection GEMM for small M
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Pending {
  int kernel;
  hipEvent_t start, stop;
};

// Workspace regions of one step (byte offsets from the workspace base).
struct Carve {
  size_t qkv, ctxkv, qpack, obuf, part_o, part_ml;
  size_t xq, xs, cq, cs, oq, os;  // MXFP8 rows and step-major scales of the block, context, attention output
  size_t total;
};

}  // namespace

// Scratch of dflash_attn_step_noalloc: a file-scope device array, one copy on
// every device the library runs on, held until the process ends. In host code
// its name is only a host-side stand-in: its device address on each device
// comes from hipGetSymbolAddress (taken once per device, with that device
// current, when a layer is created there) and only that address is used.
static __device__ __align__(256) unsigned char scratch[DFLASH_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t kNoAllocScratchBytes = DFLASH_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Resolve `scratch` on the current device (`device`) once; a failure leaves
// the no-allocation step unavailable there and clears HIP's sticky error so
// that it is not reported by a later, unrelated launch.
void resolve_noalloc_scratch(int device) {
  if (device < 0 || device >= kMaxDevices) return;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[device]) return;
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess && p) {
    g_scratch_ptr[device] = p;
  } else {
    (void)hipGetLastError();
  }
}

void* noalloc_scratch(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  return g_scratch_ptr[device];
}

}  // namespace

struct dflash_layer {
  dflash_config cfg;
  dflash_weights w;
  int device = 0;
  int num_cus = 256;
  float* cos_sin = nullptr;  // [max_pos][d/2] cos, then [max_pos][d/2] sin
  int32_t* err = nullptr;
  int profiling = 0;  // DFLASH_PROFILE_*
  int append_mode = DFLASH_APPEND_AUTO;
  bool mx = false;                 // MXFP8 projections (dflash_layer_create_mxfp8): w holds E4M3 codes
  uint8_t* wqkv_scale = nullptr;   // their scales, repacked step-major (owned)
  uint8_t* wo_scale = nullptr;
  std::vector<Pending> pending;
  std::vector<hipEvent_t> event_pool;
  double ms[DFLASH_K_COUNT] = {};
  int64_t count[DFLASH_K_COUNT] = {};
};

struct dflash_decoder {
  dflash_decoder_config cfg;
  dflash_decoder_weights w;
  dflash_layer* attn = nullptr;
  int num_cus = 256;
};

struct dflash_ctxkv {
  dflash_ctxkv_config cfg;
  dflash_ctxkv_weights w;      // with mx, w.w_kv holds E4M3 codes
  bool mx = false;             // MXFP8 weights (dflash_ctxkv_create_mxfp8)
  uint8_t* w_scale = nullptr;  // their scales, repacked step-major (owned)
  const void* w_fc = nullptr;  // optional fc weight [hidden][fc_in] (borrowed)
  int32_t fc_in = 0;
  int num_cus = 256;
  int append_mode = DFLASH_APPEND_AUTO;
  float* cos_sin = nullptr;
  int32_t* err = nullptr;
};

namespace {

int elem_size(const dflash_config& c) { return c.dtype == DFLASH_BF16 ? 2 : 4; }

// Attention work-groups for N flat tiles: as many as the CUs hold at once
// (the kernel's LDS ring bounds that), fewer when the tiles are few.
int64_t attn_groups(const dflash_layer* L, int64_t n_tiles, int64_t n_pairs) {
  int64_t cap = (int64_t)L->num_cus * attn_wgs_per_cu(L->cfg.dtype, L->cfg.head_dim);
  cap = std::min<int64_t>(cap, kMaxGroups);
  // A work-group with 64 KB of K and V in flight streams ~32 GB/s, so about
  // 200 of them saturate HBM and more only add contention. Measured with
  // bf16, head_dim 128, attention alone, 192 / 208 / 224 work-groups (two
  // alternations on one box): C3 92.3-93.2 / 90.1-90.3 / 90.6-90.8 us, C4
  // 87.0-87.1 / 82.0-82.7 / 84.1-84.4, C5 (window 4096) 48.5 / 47.4-47.8 /
  // 46.9-47.1; on another box 208 / 224: C3 90.0-90.3 / 90.6-90.7, C4
  // 81.0-81.6 / 83.7-84.8, C5 47.9-48.0 / 46.8. All 256 had been slower still
  // (C3 attention + merge 99.9 against 97.8 us at 192 with an earlier
  // kernel). So 13/16 of the CUs, and 7/8 when the ranges would be short
  // (under 48 tiles at 13/16, C5's ~40), where the ramp weighs more. Kernel
  // shapes with less in flight keep every work-group.
  if (attn_kv_in_flight(L->cfg.dtype, L->cfg.head_dim) >= 64 * 1024)
    cap = n_tiles < 48 * (cap * 13 / 16) ? cap * 7 / 8 : cap * 13 / 16;
  // At least 4 tiles a range: a range of one or two tiles is mostly its own
  // ramp, and every range a pair is cut into is one more part for the merge
  // (one sequence at 2080 keys: step 0.0524 ms with 1 tile a range, 0.0476 with
  // 4, 0.0493 with 8), but never fewer ranges than pairs while there are tiles
  // for them (a few short pairs on one range would run one after another). Then
  // a multiple of nkv when there are enough, so every head gets the same ranges.
  constexpr int64_t kMinTilesPerRange = 4;
  int64_t g = std::max<int64_t>(n_tiles / kMinTilesPerRange, std::min<int64_t>(n_tiles, n_pairs));
  g = std::min<int64_t>(cap, std::max<int64_t>(g, 1));
  if (g >= L->cfg.n_kv_heads) g -= g % L->cfg.n_kv_heads;
  return std::max<int64_t>(1, g);
}

}  // namespace

void dflash::attn_bounds(int G, int nkv, int B, const int32_t* tile_cnt, int64_t* bnd) {
  // One list of pairs is cut: a single head's B pairs when G is a multiple of
  // nkv (every head then splits at the same places), else all nkv B pairs.
  const bool by_head = nkv > 1 && G % nkv == 0;
  const int ranges = by_head ? G / nkv : G, copies = by_head ? 1 : nkv;
  int64_t per_head = 0;
  for (int b = 0; b < B; ++b) per_head += tile_cnt[b];
  const int64_t tiles = per_head * copies;
  // Costs in quarter tiles: a pair's start, then its tiles.
  const int64_t total = 4 * tiles + (int64_t)kPairStartQuarters * copies * B;
  int64_t cut[kMaxGroups + 1];
  cut[0] = 0;
  int r = 1;
  int64_t flat = 0, cost = 0;  // flat tile and cost before the current pair
  for (int c = 0; c < copies && r < ranges; ++c)
    for (int b = 0; b < B && r < ranges; ++b) {
      const int64_t t = tile_cnt[b], first = cost + kPairStartQuarters;  // cost where its tile 0 starts
      const int64_t end = first + 4 * t;
      // range r starts at the first tile that begins at or after r total / ranges
      for (; r < ranges && ((int64_t)r * total + ranges - 1) / ranges <= end - 4; ++r) {
        const int64_t x = ((int64_t)r * total + ranges - 1) / ranges;
        cut[r] = flat + (x <= first ? 0 : (x - first + 3) / 4);
      }
      flat += t;
      cost = end;
    }
  for (; r < ranges; ++r) cut[r] = tiles;
  cut[ranges] = tiles;
  // at least one tile a range: push starts forward, then pull back from the end
  for (int i = 1; i < ranges; ++i) cut[i] = std::max(cut[i], cut[i - 1] + 1);
  for (int i = ranges - 1; i >= 1; --i) cut[i] = std::min(cut[i], cut[i + 1] - 1);
  for (int j = 0; j < (by_head ? nkv : 1); ++j)
    for (int i = 0; i < ranges; ++i) bnd[j * ranges + i] = j * per_head + cut[i];
  bnd[G] = per_head * nkv;
}

void dflash::attn_range_map(int G, int nkv, uint8_t* range_of) {
  // The ranges in the order the XCDs take them: (i, j) when every head has
  // G / nkv ranges, else plain order.
  int order[kMaxGroups];
  int n = 0;
  if (nkv > 1 && G % nkv == 0) {
    const int per = G / nkv;
    for (int i = 0; i < per; ++i)
      for (int j = 0; j < nkv; ++j) order[n++] = j * per + i;
  } else {
    for (int w = 0; w < G; ++w) order[n++] = w;
  }
  // The XCDs take work-groups round-robin: XCD x runs bid = x, x + kXcds, ...
  // (only locality depends on kXcds; any value gives a permutation)
  constexpr int kXcds = 8;  // MI355X
  int next = 0;
  for (int x = 0; x < kXcds; ++x)
    for (int bid = x; bid < G; bid += kXcds) range_of[bid] = (uint8_t)order[next++];
}

namespace {

// What one step runs, as far as its scratch depends on it: the projection's
// form (fused epilogue or fp32 slices for the separate kernel), the attention
// work-groups and o_proj's k slices.
struct StepPlan {
  bool fused;
  int qkv_kslices, groups, o_kslices;
};

// Without a plan: a bound for any step of `batch` sequences and `total_ctx`
// context rows (what dflash_workspace_bytes reports). With one: exactly the
// regions that step uses (the scratch of dflash_attn_step_noalloc).
Carve carve(const dflash_layer* L, int64_t batch, int64_t total_ctx, const StepPlan* plan = nullptr) {
  const dflash_config& c = L->cfg;
  const int64_t d = c.head_dim, g = c.n_q_heads / c.n_kv_heads;
  const int64_t mq = batch * c.block_size, es = elem_size(c);
  const int64_t nqkv = (int64_t)(c.n_q_heads + 2 * c.n_kv_heads) * d, nkv2 = 2 * (int64_t)c.n_kv_heads * d;
  const int64_t gmax = plan ? plan->groups
                            : std::min<int64_t>((int64_t)L->num_cus * attn_wgs_per_cu(c.dtype, c.head_dim), kMaxGroups);
  const int64_t ks = plan ? (plan->fused ? 0 : plan->qkv_kslices) : kMaxKSlices;
  // fp32 q|k|v slices of the separate path; o_proj's k slices reuse the region
  int64_t qkv_bytes = ks * mq * nqkv * 4;
  if (plan && plan->o_kslices > 1) qkv_bytes = std::max<int64_t>(qkv_bytes, plan->o_kslices * mq * c.hidden * 4);
  Carve w{};
  size_t off = 0;
  w.qkv = off;     off += align_up(qkv_bytes);
  w.ctxkv = off;   off += align_up(ks * (plan ? total_ctx : std::max<int64_t>(total_ctx, 1)) * nkv2 * 4);
  // The attention kernel fetches whole 64-row query tiles: slack past the end.
  w.qpack = off;   off += align_up(batch * c.n_kv_heads * c.block_size * g * d * es + kMaxQueryRows * d * 4);
  w.obuf = off;    off += align_up(mq * c.n_q_heads * d * es);
  w.part_o = off;  off += align_up(2 * gmax * kMaxQueryRows * d * es);
  w.part_ml = off; off += align_up(2 * gmax * kMaxQueryRows * 2 * 4);
  if (L->mx) {
    const int64_t mc = std::max<int64_t>(total_ctx, 1), od = (int64_t)c.n_q_heads * d;
    w.xq = off; off += align_up(mq * c.hidden);
    w.xs = off; off += align_up(mq * c.hidden / 32);
    w.cq = off; off += align_up(mc * c.hidden);
    w.cs = off; off += align_up(mc * c.hidden / 32);
    w.oq = off; off += align_up(mq * od);
    w.os = off; off += align_up(mq * od / 32);
  }
  w.total = off;
  return w;
}

// Tile shape of a projection launch (one or two problems of m x n outputs).
// A work-group streams BM + BN rows of k per tile and a CU runs one at a time,
// so among the shapes that give at least ~3/4 of a work-group per CU the one
// with the fewest rounds x (BM + BN) wins (ties: the earlier, larger shape);
// problems too small for any use 64 x 64 tiles and, when fp32 partial sums are
// allowed, split k so that the launch still covers the CUs.
struct TileChoice {
  int bm, bn, tiles, kslices;
};
TileChoice choose_tiles(int num_cus, int m0, int n0, int m1, int n1, bool allow_split) {
  static const int cand[4][2] = {{128, 128}, {128, 64}, {64, 128}, {64, 64}};
  const int target = num_cus * 3 / 4;
  auto count = [&](int bm, int bn) {
    int t = ((m0 + bm - 1) / bm) * ((n0 + bn - 1) / bn);
    if (m1 > 0) t += ((m1 + bm - 1) / bm) * ((n1 + bn - 1) / bn);
    return t;
  };
  int best = -1;
  long best_cost = 0;
  for (int i = 0; i < 4; ++i) {
    const int t = count(cand[i][0], cand[i][1]);
    if (t < target) continue;
    const long cost = (long)((t + num_cus - 1) / num_cus) * (cand[i][0] + cand[i][1]);
    if (best < 0 || cost < best_cost) {
      best = i;
      best_cost = cost;
    }
  }
  if (best >= 0) return {cand[best][0], cand[best][1], count(cand[best][0], cand[best][1]), 1};
  const int t = count(64, 64);
  int ks = 1;
  if (allow_split) ks = std::min(kMaxKSlices, std::max(1, (num_cus + t - 1) / t));
  return {64, 64, t, ks};
}
TileChoice choose_tiles(const dflash_layer* L, int m0, int n0, int m1, int n1, bool allow_split) {
  return choose_tiles(L->num_cus, m0, n0, m1, n1, allow_split);
}

// Tile shape and k split of a plain projection with a deep k (m x n outputs,
// k deep, es-byte elements). Its work-groups are bound by the bytes each
// streams into LDS, so a launch is modelled as rounds x (a ~15 us ramp and
// epilogue + (BM + BN) (k / ks) es bytes at ~100 GB/s per CU), plus, with a k
// split, ~3 us for the summing launch and the fp32 partials' round trip at
// ~8 TB/s. Fitted to measured launches on gfx950 (decoder down_proj 512 x 4096
// x 12288: 128 x 64 unsplit 397 us per decoder step, 128 x 128 in two slices
// 386 us, 256 x 128 in four slices 8 us less again; fc projection 281 x 4096
// x 12288: 128 x 64 62.7 us, 128 x 128 in two slices 53.0 us, 128 x 128
// unsplit 80.3 us, 256 x 128 in four slices 62.5 us; 4096 x 4096 x 12288:
// 128 x 128 440 us, 256 x 128 431 us). 256-row tiles (bf16 only) are offered
// only when they cover m exactly: the half-empty second row tile of m = 281
// measured slower than the model says. Ties keep the larger tiles and the
// fewer slices. only_bn != 0 restricts the tiles to that width.
TileChoice choose_tiles_fill(int num_cus, int m, int n, int k, int es, int max_ks, int only_bn = 0) {
  static const int cand[5][2] = {{256, 128}, {128, 128}, {128, 64}, {64, 128}, {64, 64}};
  const int steps = k * es / 128;  // 128-byte k steps
  TileChoice best{64, 64, ((m + 63) / 64) * ((n + 63) / 64), 1};
  double best_t = -1.0;
  for (int i = (es == 2 && m % 256 == 0) ? 0 : 1; i < 5; ++i)
    for (int ks = 1; ks <= std::max(1, std::min(max_ks, steps)); ++ks) {
      const int bm = cand[i][0], bn = cand[i][1];
      if (only_bn && bn != only_bn) continue;
      const int64_t tiles = (int64_t)((m + bm - 1) / bm) * ((n + bn - 1) / bn);
      const int64_t rounds = (tiles * ks + num_cus - 1) / num_cus;
      double t = (double)rounds * (15.0 + (double)(bm + bn) * ((double)k / ks) * es / 1e5);
      if (ks > 1) t += 3.0 + 2.0 * ks * (double)m * n * 4 / 8e6;
      if (best_t < 0 || t < best_t - 1e-9) {
        best_t = t;
        best = TileChoice{bm, bn, (int)tiles, ks};
      }
    }
  return best;
}

// The gate/up SwiGLU projection (m rows, 2 i columns, k = h, no k split):
// one launch of bm x 128 tiles (64 gate + 64 up columns), one launch of
// 256 x 192 tiles (bn = 192: bf16, m % 256 == 0, i % 96 == 0), or two
// launches of 128-column tiles over disjoint column ranges: the first c1
// column tiles in bm-row tiles filling whole rounds of the CUs, the rest in
// bm2-row tiles. Priced with the fill model of choose_tiles_fill plus ~3 us
// for a second launch. At m = 512, i = 12288 (C3's decoder) 256 x 128 tiles
// take 384 work-groups, a round and a half (122.6 us by the kernel trace);
// 256 x 128 tiles over the first 128 column tiles and 128 x 128 over the
// other 64 fill two whole rounds (63.4 + 41.2 us); 256 x 192 tiles fill one.
// Every form gives the same bits: no output's sum changes order with the
// tile's shape. The split needs i % 64 == 0 so that both launches cover whole
// tiles.
struct SwigluPlan {
  int bm, bn, c1, bm2;  // c1 == the column tiles of width bn: one launch
};
SwigluPlan swiglu_plan(int num_cus, int m, int i, int h, int es) {
  const int tn = (2 * i + 127) / 128;
  const double fill = (double)h * es / 1e5;
  auto cost = [&](int bm, int cols) {
    const int64_t tiles = (int64_t)((m + bm - 1) / bm) * cols;
    return (double)((tiles + num_cus - 1) / num_cus) * (15.0 + (bm + 128) * fill);
  };
  const int first = es == 2 && m % 256 == 0 ? 0 : 1;
  static const int rows[3] = {256, 128, 64};
  SwigluPlan best{64, 128, tn, 64};
  double best_t = -1.0;
  for (int a = first; a < 3; ++a) {
    const double t = cost(rows[a], tn);
    if (best_t < 0 || t < best_t - 1e-9) { best_t = t; best = SwigluPlan{rows[a], 128, tn, rows[a]}; }
  }
  if (first == 0 && i % 96 == 0 && h % 32 == 0) {
    const int tw = 2 * i / 192;
    const int64_t tiles = (int64_t)(m / 256) * tw;
    const double t = (double)((tiles + num_cus - 1) / num_cus) * (15.0 + (256 + 192) * fill);
    if (t < best_t - 1e-9) { best_t = t; best = SwigluPlan{256, 192, tw, 256}; }
  }
  if (i % 64 != 0) return best;
  for (int a = first; a < 3; ++a) {
    const int mt = (m + rows[a] - 1) / rows[a];
    const int c1 = (int)(((int64_t)tn * mt / num_cus) * num_cus / mt);  // whole rounds
    if (c1 <= 0 || c1 >= tn || ((int64_t)c1 * mt) % num_cus != 0) continue;
    for (int b = a + 1; b < 3; ++b) {
      const double t = cost(rows[a], c1) + cost(rows[b], tn - c1) + 3.0;
      if (t < best_t - 1e-9) { best_t = t; best = SwigluPlan{rows[a], 128, c1, rows[b]}; }
    }
  }
  return best;
}

// Workspace of a context precompute of mc rows: hidden_norm-ed rows in the
// element type, then the fp32 projection [k slices][mc][L * 2 * nkv * d]. With
// MXFP8 weights: the hidden_norm-ed rows as E4M3 codes [mc][H] and their E8M0
// scales [mc][H / 32] (the projection always appends in its epilogue).
struct CtxCarve {
  size_t normed, proj, scales, total;
};
CtxCarve ctx_carve(const dflash_ctxkv_config& c, int64_t mc, bool mx) {
  const int64_t es = c.dtype == DFLASH_BF16 ? 2 : 4, m = std::max<int64_t>(mc, 1);
  const int64_t n = (int64_t)c.n_layers * 2 * c.n_kv_heads * c.head_dim;
  CtxCarve w{};
  size_t off = 0;
  if (mx) {
    w.normed = off; off += align_up(m * c.hidden);
    w.scales = off; off += align_up(m * c.hidden / 32);
  } else {
    w.normed = off; off += align_up(m * c.hidden * es);
    w.proj = off;   off += align_up(kMaxKSlices * m * n * 4);
  }
  w.total = off;
  return w;
}

int validate_config(const dflash_config* c) {
  if (c->hidden <= 0 || c->n_q_heads <= 0 || c->n_kv_heads <= 0 || c->block_size <= 0 ||
      c->max_position <= 0 || c->sliding_window < 0)
    return DFLASH_ERR_SHAPE;
  if (c->n_q_heads % c->n_kv_heads) return DFLASH_ERR_SHAPE;
  if (c->n_kv_heads > kMaxKvHeads) return DFLASH_ERR_UNSUPPORTED;
  if (c->hidden % 64) return DFLASH_ERR_SHAPE;
  if (!(c->rope_theta > 0.0) || !(c->rms_eps >= 0.0)) return DFLASH_ERR_ARG;
  if (c->dtype != DFLASH_F32 && c->dtype != DFLASH_BF16) return DFLASH_ERR_ARG;
  if (c->head_dim != 64 && c->head_dim != 128) return DFLASH_ERR_UNSUPPORTED;
  if ((int64_t)c->block_size * (c->n_q_heads / c->n_kv_heads) > kMaxQueryRows)
    return DFLASH_ERR_UNSUPPORTED;
  return DFLASH_OK;
}

// RoPE cos/sin of pos * theta^(-2t/d) for t < d/2, angle and trig in float64,
// uploaded as fp32 [max_pos][d/2] cos then [max_pos][d/2] sin.
bool upload_rope_table(int max_pos, int d, double theta, float** out) {
  const int half = d / 2;
  const size_t n = (size_t)max_pos * half;
  std::vector<float> table(2 * n);
  std::vector<double> inv(half);
  for (int t = 0; t < half; ++t) inv[t] = std::pow(theta, -2.0 * t / d);
  for (int64_t p = 0; p < max_pos; ++p)
    for (int t = 0; t < half; ++t) {
      const double ang = (double)p * inv[t];
      table[(size_t)p * half + t] = (float)std::cos(ang);
      table[n + (size_t)p * half + t] = (float)std::sin(ang);
    }
  *out = nullptr;
  if (hipMalloc(out, 2 * n * sizeof(float)) != hipSuccess) {
    *out = nullptr;
    return false;
  }
  return hipMemcpy(*out, table.data(), 2 * n * sizeof(float), hipMemcpyHostToDevice) == hipSuccess;
}

// Host checks of a cache's layout; rows_needed[b] rows of sequence b are
// touched. For a paged cache every block holding such a row must name a
// physical block in the pools (per the host mirror of the table).
int check_layout(const dflash_kv_cache* c, const int64_t* rows_needed) {
  if (!c->block_table) return DFLASH_OK;
  if (!c->block_table_host || c->max_blocks <= 0 || c->num_blocks <= 0) return DFLASH_ERR_ARG;
  if ((int64_t)c->max_blocks * kKeyTile != c->capacity) return DFLASH_ERR_SHAPE;
  for (int b = 0; b < c->batch; ++b) {
    const int64_t nb = (rows_needed[b] + kKeyTile - 1) / kKeyTile;
    for (int64_t i = 0; i < nb; ++i) {
      const int32_t p = c->block_table_host[(int64_t)b * c->max_blocks + i];
      if (p < 0 || p >= c->num_blocks) return DFLASH_ERR_RANGE;
    }
  }
  return DFLASH_OK;
}

CacheMap cache_map(const dflash_kv_cache* c, int nkv) {
  CacheMap m;
  m.bt = c->block_table;
  m.bt_stride = c->block_table ? c->max_blocks : 0;
  m.num_blocks = c->block_table ? c->num_blocks : 0;
  m.cap = c->capacity;
  m.nkv = nkv;
  return m;
}

hipEvent_t pooled_event(dflash_layer* L) {
  if (!L->event_pool.empty()) {
    hipEvent_t e = L->event_pool.back();
    L->event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  hipEventCreate(&e);
  return e;
}
// Events of the profiling mode `mode` (per-kernel pairs, or the one pair
// around the attention and its merge); nothing in the other modes.
void record(dflash_layer* L, hipEvent_t* start, hipStream_t s, int mode = DFLASH_PROFILE_KERNELS) {
  if (L->profiling != mode) return;
  *start = pooled_event(L);
  hipEventRecord(*start, s);
}
void record_end(dflash_layer* L, int kernel, hipEvent_t start, hipStream_t s, int mode = DFLASH_PROFILE_KERNELS) {
  if (L->profiling != mode) return;
  hipEvent_t stop = pooled_event(L);
  hipEventRecord(stop, s);
  L->pending.push_back({kernel, start, stop});
}

// Sequences b0 .. b0 + nb - 1 of a cache as a cache of their own: the same
// pools (paged: the table rows of those sequences) or the contiguous layout's
// slabs of those sequences, and their lengths.
dflash_kv_cache cache_view(const dflash_kv_cache* c, int b0, int nb, int nkv, int d, int es) {
  dflash_kv_cache v = *c;
  v.batch = nb;
  v.len = c->len + b0;
  if (c->block_table) {
    v.block_table = c->block_table + (size_t)b0 * c->max_blocks;
    v.block_table_host = c->block_table_host ? c->block_table_host + (size_t)b0 * c->max_blocks : nullptr;
  } else {
    const size_t seq_bytes = (size_t)c->capacity * nkv * d * es;
    v.k = static_cast<char*>(c->k) + (size_t)b0 * seq_bytes;
    v.v = static_cast<char*>(c->v) + (size_t)b0 * seq_bytes;
  }
  return v;
}

}  // namespace

// A paged cache's free physical blocks (a stack: the last entry is taken
// next) and the table entries changed since the last upload.
struct dflash_block_pool {
  int32_t num_blocks = 0;
  std::vector<int32_t> free;
  std::vector<std::pair<int32_t, int32_t>> pending;  // (flat index, value)
};

namespace {

bool pool_cache_ok(const dflash_kv_cache* c, const dflash_block_pool* p) {
  return c && p && c->block_table && c->block_table_host && c->batch >= 1 && c->max_blocks > 0 &&
         c->num_blocks == p->num_blocks;
}

// Table entries in use by sequence b (the non-negative ones).
int32_t blocks_in_use(const dflash_kv_cache* c, int b) {
  const int32_t* row = c->block_table_host + (int64_t)b * c->max_blocks;
  int32_t n = 0;
  for (int32_t i = 0; i < c->max_blocks; ++i) n += row[i] >= 0;
  return n;
}

void set_entry(dflash_kv_cache* c, dflash_block_pool* p, int64_t idx, int32_t v) {
  const_cast<int32_t*>(c->block_table_host)[idx] = v;
  p->pending.push_back({(int32_t)idx, v});
}

// Back rows [0, rows[b]) of every sequence b with rows[b] >= 0 by blocks:
// sequence by sequence (0 first), each new logical block taking the pool's
// next block. All or nothing: DFLASH_ERR_SHAPE past max_blocks,
// DFLASH_ERR_CAPACITY when the pool holds too few.
int reserve_rows(dflash_kv_cache* c, dflash_block_pool* p, const int64_t* rows) {
  int64_t total = 0;
  for (int b = 0; b < c->batch; ++b) {
    if (rows[b] < 0) continue;
    const int64_t need = (rows[b] + kKeyTile - 1) / kKeyTile;
    if (need > c->max_blocks) return DFLASH_ERR_SHAPE;
    total += std::max<int64_t>(0, need - blocks_in_use(c, b));
  }
  if (total > (int64_t)p->free.size()) return DFLASH_ERR_CAPACITY;
  for (int b = 0; b < c->batch; ++b) {
    if (rows[b] < 0) continue;
    const int64_t need = (rows[b] + kKeyTile - 1) / kKeyTile;
    for (int64_t i = blocks_in_use(c, b); i < need; ++i) {
      set_entry(c, p, (int64_t)b * c->max_blocks + i, p->free.back());
      p->free.pop_back();
    }
  }
  return DFLASH_OK;
}

// Return the blocks of every sequence b with rows[b] >= 0 past its first
// ceil(rows[b] / 64) to the pool: sequence by sequence, last block first.
int release_rows(dflash_kv_cache* c, dflash_block_pool* p, const int64_t* rows) {
  for (int b = 0; b < c->batch; ++b) {
    if (rows[b] < 0) continue;
    const int64_t keep = (rows[b] + kKeyTile - 1) / kKeyTile;
    for (int64_t i = c->max_blocks - 1; i >= keep; --i) {
      const int64_t idx = (int64_t)b * c->max_blocks + i;
      const int32_t blk = c->block_table_host[idx];
      if (blk < 0) continue;
      p->free.push_back(blk);
      set_entry(c, p, idx, -1);
    }
  }
  return DFLASH_OK;
}

}  // namespace

extern "C" {

const char* dflash_status_string(int status) {
  switch (status) {
    case DFLASH_OK: return "ok";
    case DFLASH_ERR_ARG: return "invalid argument";
    case DFLASH_ERR_SHAPE: return "inconsistent or non-divisible shape";
    case DFLASH_ERR_CAPACITY: return "step would exceed the cache capacity";
    case DFLASH_ERR_RANGE: return "value out of range (crop length, position or block-table entry)";
    case DFLASH_ERR_UNSUPPORTED: return "configuration not supported by the kernels";
    case DFLASH_ERR_HIP: return "HIP runtime error";
    case DFLASH_ERR_WORKSPACE: return "workspace missing or too small";
    default: return "unknown status";
  }
}

int dflash_layer_create(const dflash_config* cfg, const dflash_weights* weights,
                        dflash_layer** out) {
  if (!cfg || !weights || !out) return DFLASH_ERR_ARG;
  *out = nullptr;
  if (!weights->w_qkv || !weights->w_o || !weights->q_norm || !weights->k_norm) return DFLASH_ERR_ARG;
  const int st = validate_config(cfg);
  if (st != DFLASH_OK) return st;

  dflash_layer* L = new (std::nothrow) dflash_layer();
  if (!L) return DFLASH_ERR_HIP;
  L->cfg = *cfg;
  L->w = *weights;
  if (hipGetDevice(&L->device) != hipSuccess) { delete L; return DFLASH_ERR_HIP; }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, L->device) == hipSuccess && cus > 0)
    L->num_cus = cus;
  resolve_noalloc_scratch(L->device);

  if (!upload_rope_table(cfg->max_position, cfg->head_dim, cfg->rope_theta, &L->cos_sin) ||
      hipMalloc(&L->err, sizeof(int32_t)) != hipSuccess ||
      hipMemset(L->err, 0, sizeof(int32_t)) != hipSuccess) {
    if (L->cos_sin) hipFree(L->cos_sin);
    if (L->err) hipFree(L->err);
    delete L;
    return DFLASH_ERR_HIP;
  }
  *out = L;
  return DFLASH_OK;
}

void dflash_layer_destroy(dflash_layer* L) {
  if (!L) return;
  hipDeviceSynchronize();
  for (auto& p : L->pending) {
    hipEventDestroy(p.start);
    hipEventDestroy(p.stop);
  }
  for (hipEvent_t e : L->event_pool) hipEventDestroy(e);
  hipFree(L->cos_sin);
  hipFree(L->err);
  if (L->wqkv_scale) hipFree(L->wqkv_scale);
  if (L->wo_scale) hipFree(L->wo_scale);
  delete L;
}

int dflash_layer_create_mxfp8(const dflash_config* cfg, const dflash_mxfp8_weights* weights,
                              dflash_layer** out) {
  if (!cfg || !weights || !out) return DFLASH_ERR_ARG;
  *out = nullptr;
  if (!weights->w_qkv_scale || !weights->w_o_scale) return DFLASH_ERR_ARG;
  if (reinterpret_cast<uintptr_t>(weights->w_qkv_scale) % 4 || reinterpret_cast<uintptr_t>(weights->w_o_scale) % 4)
    return DFLASH_ERR_ARG;
  if (cfg->dtype != DFLASH_BF16) return DFLASH_ERR_UNSUPPORTED;
  if (cfg->hidden % 128 || ((int64_t)cfg->n_q_heads * cfg->head_dim) % 128) return DFLASH_ERR_SHAPE;
  dflash_weights w;
  w.w_qkv = weights->w_qkv;
  w.w_o = weights->w_o;
  w.q_norm = weights->q_norm;
  w.k_norm = weights->k_norm;
  dflash_layer* L = nullptr;
  const int st = dflash_layer_create(cfg, &w, &L);
  if (st != DFLASH_OK) return st;
  L->mx = true;
  const int64_t nqkv = (int64_t)(cfg->n_q_heads + 2 * cfg->n_kv_heads) * cfg->head_dim;
  const int64_t od = (int64_t)cfg->n_q_heads * cfg->head_dim;
  const bool ok = hipMalloc(&L->wqkv_scale, (size_t)nqkv * cfg->hidden / 32) == hipSuccess &&
                  hipMalloc(&L->wo_scale, (size_t)cfg->hidden * od / 32) == hipSuccess &&
                  launch_scales_step_major(weights->w_qkv_scale, L->wqkv_scale, (int)nqkv, cfg->hidden, nullptr) ==
                      hipSuccess &&
                  launch_scales_step_major(weights->w_o_scale, L->wo_scale, cfg->hidden, (int)od, nullptr) ==
                      hipSuccess &&
                  hipDeviceSynchronize() == hipSuccess;
  if (!ok) {
    dflash_layer_destroy(L);
    return DFLASH_ERR_HIP;
  }
  *out = L;
  return DFLASH_OK;
}

size_t dflash_workspace_bytes(const dflash_layer* L, int32_t batch, int64_t total_ctx,
                              int64_t total_keys) {
  if (!L || batch < 1 || batch > DFLASH_MAX_BATCH || total_ctx < 0 || total_keys < 0) return 0;
  // a larger batch runs in runs of at most kMaxBatch sequences sharing it
  return carve(L, std::min<int32_t>(batch, kMaxBatch), total_ctx).total;
}

int dflash_workspace_offset(const dflash_layer* L, int32_t batch, int64_t total_ctx, int32_t region,
                            size_t* offset) {
  if (!L || !offset || batch < 1 || batch > kMaxBatch || total_ctx < 0) return DFLASH_ERR_ARG;
  const Carve wc = carve(L, batch, total_ctx);
  switch (region) {
    case DFLASH_WS_ATTN_OUT: *offset = wc.obuf; return DFLASH_OK;
    case DFLASH_WS_ATTN_OUT_MX:
      if (!L->mx) return DFLASH_ERR_ARG;
      *offset = wc.oq;
      return DFLASH_OK;
    case DFLASH_WS_ATTN_OUT_MX_SCALES:
      if (!L->mx) return DFLASH_ERR_ARG;
      *offset = wc.os;
      return DFLASH_OK;
    default: return DFLASH_ERR_ARG;
  }
}

// The layer step; with validate_only it returns after the host-side checks,
// having enqueued nothing (the decoder layer checks before its first launch).
// With noalloc the scratch is the library's per-device buffer (exactly what
// this step uses, refused past its size) instead of the caller's workspace.
static int attn_step_impl(dflash_layer* L, const void* hidden_states, const void* target_hidden,
                          const int32_t* ctx_offsets, const int32_t* positions, dflash_kv_cache* cache,
                          void* out, void* workspace, size_t workspace_bytes, void* stream,
                          bool validate_only, bool noalloc = false) {
  if (!L || !hidden_states || !ctx_offsets || !cache || !out) return DFLASH_ERR_ARG;
  if (!cache->k || !cache->v || !cache->len) return DFLASH_ERR_ARG;
  const dflash_config& c = L->cfg;
  const int B = cache->batch;
  if (B < 1 || B > kMaxBatch) return DFLASH_ERR_ARG;
  if (cache->capacity <= 0 || cache->capacity % kKeyTile) return DFLASH_ERR_SHAPE;
  if (cache->capacity > kMaxCapacity) return DFLASH_ERR_SHAPE;
  if (ctx_offsets[0] != 0) return DFLASH_ERR_SHAPE;
  const int bs = c.block_size, d = c.head_dim, nq = c.n_q_heads, nkv = c.n_kv_heads;
  const int g = nq / nkv, R = bs * g;

  const int64_t kt = attn_key_tile(c.dtype, d);
  SeqTable seq;
  std::memset(&seq, 0, sizeof(seq));
  seq.batch = B;
  int64_t n_tiles = 0;
  int32_t tile_lo[kMaxBatch], tile_cnt[kMaxBatch];  // each sequence's attention key tiles
  for (int b = 0; b < B; ++b) {
    const int64_t n = (int64_t)ctx_offsets[b + 1] - ctx_offsets[b];
    if (n < 0) return DFLASH_ERR_SHAPE;
    if (cache->len[b] < 0) return DFLASH_ERR_SHAPE;
    const int64_t T = (int64_t)cache->len[b] + n + bs;
    if (T > cache->capacity) return DFLASH_ERR_CAPACITY;
    seq.len[b] = cache->len[b];
    seq.ctx_off[b] = ctx_offsets[b];
    int64_t first = 0;
    if (c.sliding_window > 0) first = std::max<int64_t>(0, T - bs - c.sliding_window + 1);
    tile_lo[b] = (int32_t)(first / kt);
    tile_cnt[b] = (int32_t)((T + kt - 1) / kt - first / kt);
    n_tiles += (int64_t)nkv * tile_cnt[b];
  }
  seq.ctx_off[B] = ctx_offsets[B];
  // Without a position array every window takes len_b, len_b + 1, ...: all
  // of them must lie inside the RoPE table.
  if (!positions)
    for (int b = 0; b < B; ++b)
      if ((int64_t)cache->len[b] + (ctx_offsets[b + 1] - ctx_offsets[b]) + bs > c.max_position)
        return DFLASH_ERR_RANGE;
  const int64_t Mc = ctx_offsets[B];
  if (Mc > 0 && !target_hidden) return DFLASH_ERR_ARG;
  {
    int64_t rows[kMaxBatch];
    for (int b = 0; b < B; ++b) rows[b] = (int64_t)cache->len[b] + (ctx_offsets[b + 1] - ctx_offsets[b]) + bs;
    const int lst = check_layout(cache, rows);
    if (lst != DFLASH_OK) return lst;
  }
  if (L->mx && L->append_mode == DFLASH_APPEND_SEPARATE) return DFLASH_ERR_UNSUPPORTED;
  if (L->mx && (reinterpret_cast<uintptr_t>(hidden_states) % 16 ||
                (Mc > 0 && reinterpret_cast<uintptr_t>(target_hidden) % 16)))
    return DFLASH_ERR_ARG;

  // What the step runs: host decisions that also size its scratch.
  const int es = elem_size(c);
  const int Mq = B * bs, H = c.hidden;
  const int Nqkv = (nq + 2 * nkv) * d, Nkv = 2 * nkv * d;
  // HK1: block q|k|v and context k|v in one launch; with the append fused into
  // its epilogue (one head per tile, no k split) it also does HK2's work.
  const int nt64 = ((Mq + 63) / 64) * (Nqkv / d) + (int)((Mc + 63) / 64) * (Nkv / d);
  const int nt128 = ((Mq + 127) / 128) * (Nqkv / d) + (int)((Mc + 127) / 128) * (Nkv / d);
  const int target = L->num_cus * 3 / 4;
  const int fused_tiles = nt128 >= target ? nt128 : nt64;
  // AUTO fuses unless the fused tiles (full k each) would fill at most half
  // the CUs with a deep k: then the separate path's k split or smaller tiles
  // cover the CUs, which saves more than its norm / RoPE / append launch costs.
  // Measured at H = 4096, 32 / 8 heads, bf16: one sequence 0.0427 against
  // 0.0505 ms fused, 4 sequences 0.0473 against 0.0543, 8 sequences (128 fused
  // tiles) 0.0537 against 0.0578, 12 sequences (192 fused tiles) 0.0705
  // against 0.0649; at H = 256 the launch dominates (C1 0.0306 against 0.0287).
  const bool fused = L->mx || L->append_mode == DFLASH_APPEND_FUSED ||
                     (L->append_mode == DFLASH_APPEND_AUTO && (fused_tiles > L->num_cus / 2 || H < 2048));
  const TileChoice tq = fused ? TileChoice{nt128 >= target ? 128 : 64, d, fused_tiles, 1}
                              : choose_tiles(L, Mq, Nqkv, (int)Mc, Nkv, true);
  const int G = (int)attn_groups(L, n_tiles, (int64_t)B * nkv);
  // the attention's ranges (their tile counts ride in 16 bits)
  int64_t bnd[kMaxGroups + 1];
  attn_bounds(G, nkv, B, tile_cnt, bnd);
  for (int w = 0; w < G; ++w)
    if (bnd[w + 1] - bnd[w] > 0xffff) return DFLASH_ERR_UNSUPPORTED;
  // o_proj: too few rows for the CUs (a small batch) and a weight large enough
  // that streaming it dominates (>= 4 MB; below that the extra launch costs
  // more): k split over fp32 slices in the q|k|v region of the scratch (its
  // contents are consumed by then), summed into out with one rounding.
  const bool o_big = (int64_t)H * nq * d * elem_size(c) >= (4 << 20);
  const TileChoice to = choose_tiles(L, Mq, H, 0, 0, !L->mx && o_big);
  const bool o_split = to.kslices > 1 && (int64_t)to.kslices * H <= (int64_t)kMaxKSlices * Nqkv;

  Carve wc;
  if (noalloc) {
    const StepPlan plan{fused, tq.kslices, G, o_split ? to.kslices : 1};
    wc = carve(L, B, Mc, &plan);
    if (wc.total > kNoAllocScratchBytes) return DFLASH_ERR_WORKSPACE;
    workspace = noalloc_scratch(L->device);
    if (!workspace) return DFLASH_ERR_HIP;
  } else {
    if (!workspace) return DFLASH_ERR_WORKSPACE;
    wc = carve(L, B, Mc);
    if (workspace_bytes < wc.total || reinterpret_cast<uintptr_t>(workspace) % kAlign)
      return DFLASH_ERR_WORKSPACE;
  }
  if (validate_only) return DFLASH_OK;

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  float* qkv = reinterpret_cast<float*>(ws + wc.qkv);
  float* ctxkv = reinterpret_cast<float*>(ws + wc.ctxkv);
  void* qpack = ws + wc.qpack;
  void* obuf = ws + wc.obuf;

  GemmArgs ga;
  std::memset(&ga, 0, sizeof(ga));
  ga.nprob = 1;
  ga.p[0] = {hidden_states, L->w.w_qkv, qkv, Mq, Nqkv, H, H, H, Nqkv,
             (Nqkv + tq.bn - 1) / tq.bn, 0, (int64_t)Mq * Nqkv};
  if (Mc > 0) {
    const char* wkv = static_cast<const char*>(L->w.w_qkv) + (size_t)nq * d * H * es;
    ga.p[1] = {target_hidden, wkv, ctxkv, (int32_t)Mc, Nkv, H, H, H, Nkv,
               (Nkv + tq.bn - 1) / tq.bn, ((Mq + tq.bm - 1) / tq.bm) * ga.p[0].tiles_n,
               (int64_t)Mc * Nkv};
    ga.nprob = 2;
  }
  // HK2 (or the fused epilogue)
  NormRopeArgs na;
  std::memset(&na, 0, sizeof(na));
  na.qkv = qkv;
  na.ctxkv = ctxkv;
  na.qkv_slice = (int64_t)Mq * Nqkv;
  na.ctx_slice = (int64_t)Mc * Nkv;
  na.kslices = tq.kslices;
  na.positions = positions;
  na.cos_sin = L->cos_sin;
  na.q_norm = L->w.q_norm;
  na.k_norm = L->w.k_norm;
  na.qpack = qpack;
  na.kc = cache->k;
  na.vc = cache->v;
  na.err = L->err;
  na.nq = nq; na.nkv = nkv; na.bs = bs; na.cap = cache->capacity; na.max_pos = c.max_position;
  na.eps = (float)c.rms_eps;
  na.qscale = (float)(1.0 / std::sqrt((double)d) * 1.4426950408889634);
  na.ctx_ld = (int64_t)Nkv;
  na.ctx_layer_off = 0;
  na.map = cache_map(cache, nkv);
  na.seq = seq;
  hipEvent_t ev;
  record(L, &ev, s);
  if (L->mx) {
    // MXFP8: the block and context rows quantised once (scales step-major,
    // planes of their own rows), then the block-scaled q|k|v + context k|v
    // projection with the same epilogue. The weight's scale planes hold all
    // its q|k|v rows; the context problem starts at its k rows.
    uint8_t* xq = reinterpret_cast<uint8_t*>(ws + wc.xq);
    uint8_t* xs = reinterpret_cast<uint8_t*>(ws + wc.xs);
    uint8_t* cq = reinterpret_cast<uint8_t*>(ws + wc.cq);
    uint8_t* cs = reinterpret_cast<uint8_t*>(ws + wc.cs);
    if (launch_rows_mx2(hidden_states, xq, xs, Mq, target_hidden, cq, cs, (int)Mc, H, s) != hipSuccess)
      return DFLASH_ERR_HIP;
    ga.p[0].a = xq;
    ga.p[0].sa = xs;
    ga.p[0].sb = L->wqkv_scale;
    ga.p[0].sb_plane = (int64_t)Nqkv * 4;
    if (Mc > 0) {
      ga.p[1].a = cq;
      ga.p[1].b = static_cast<const char*>(L->w.w_qkv) + (size_t)nq * d * H;
      ga.p[1].sa = cs;
      ga.p[1].sb = L->wqkv_scale + (size_t)nq * d * 4;
      ga.p[1].sb_plane = (int64_t)Nqkv * 4;
    }
    if (launch_gemm_append_mx(d, ga, na, tq.tiles, tq.bm, s) != hipSuccess) return DFLASH_ERR_HIP;
    record_end(L, DFLASH_K_GEMM_QKV, ev, s);
  } else if (fused) {
    if (launch_gemm_append(c.dtype, d, ga, na, tq.tiles, tq.bm, s) != hipSuccess) return DFLASH_ERR_HIP;
    record_end(L, DFLASH_K_GEMM_QKV, ev, s);
  } else {
    if (launch_gemm(c.dtype, true, ga, tq.tiles, tq.bm, tq.bn, tq.kslices, s) != hipSuccess)
      return DFLASH_ERR_HIP;
    record_end(L, DFLASH_K_GEMM_QKV, ev, s);
    record(L, &ev, s);
    int max_new = 0;
    for (int b = 0; b < B; ++b) max_new = std::max(max_new, ctx_offsets[b + 1] - ctx_offsets[b] + bs);
    if (launch_norm_rope(c.dtype, d, na, B * nkv, max_new, 1, s) != hipSuccess) return DFLASH_ERR_HIP;
    record_end(L, DFLASH_K_NORM_ROPE, ev, s);
  }

  // HK3 (+ HK4)
  AttnArgs aa;
  aa.q = qpack;
  aa.kc = cache->k;
  aa.vc = cache->v;
  aa.o = obuf;
  aa.part_o = ws + wc.part_o;
  aa.part_ml = reinterpret_cast<float*>(ws + wc.part_ml);
  aa.nq = nq; aa.nkv = nkv; aa.bs = bs; aa.R = R; aa.cap = cache->capacity;
  // A window at least the capacity keeps every key (|query - key| < T_b <= capacity).
  aa.window = c.sliding_window >= cache->capacity ? 0 : c.sliding_window;
  aa.total_tiles = n_tiles;
  aa.G = G;
  // an MXFP8 layer's attention writes o_proj's MXFP8 input directly
  aa.mxo = L->mx ? MxOut{reinterpret_cast<uint8_t*>(ws + wc.oq), reinterpret_cast<uint8_t*>(ws + wc.os), nq * d, Mq}
                 : MxOut{nullptr, nullptr, 0, 0};
  aa.map = cache_map(cache, nkv);
  aa.seq = seq;
  attn_range_map(aa.G, nkv, aa.range_of);
  for (int bid = 0; bid < aa.G; ++bid) {
    const int w = aa.range_of[bid];
    aa.count[bid] = (uint16_t)(bnd[w + 1] - bnd[w]);
  }
  // Each work-group's first (pair, tile): walk the pairs in flat order.
  {
    int64_t f = 0;
    int w = 0;
    for (int j = 0; j < nkv && w < aa.G; ++j)
      for (int b = 0; b < B && w < aa.G; ++b) {
        const int64_t end = f + tile_cnt[b];
        for (; w < aa.G && bnd[w] < end; ++w)
          aa.start[w] = (uint32_t)(b * nkv + j) | ((uint32_t)(tile_lo[b] + (bnd[w] - f)) << 16);
        f = end;
      }
  }
  hipEvent_t span = nullptr;
  record(L, &span, s, DFLASH_PROFILE_ATTN_SPAN);
  record(L, &ev, s);
  if (launch_attn(c.dtype, d, aa, s) != hipSuccess) return DFLASH_ERR_HIP;
  record_end(L, DFLASH_K_ATTN, ev, s);

  // HK4 over the pairs that straddle a range boundary.
  MergeArgs ma;
  ma.part_o = aa.part_o;
  ma.part_ml = aa.part_ml;
  ma.o = obuf;
  ma.mxo = aa.mxo;
  ma.nq = nq; ma.nkv = nkv; ma.bs = bs; ma.R = R;
  ma.n_split = 0;
  {
    // owner of flat tile x: the last range starting at or before it (pairs
    // come in flat order, so the owner only moves forward)
    int w0 = 0;
    int64_t f = 0;
    for (int j = 0; j < nkv; ++j)
      for (int b = 0; b < B; ++b) {
        const int64_t e = f + tile_cnt[b];
        while (w0 + 1 < aa.G && bnd[w0 + 1] <= f) ++w0;
        int w1 = w0;
        while (w1 + 1 < aa.G && bnd[w1 + 1] <= e - 1) ++w1;
        if (w0 != w1) {
          ma.pair[ma.n_split] = b * nkv + j;
          ma.first_slot[ma.n_split] = (int16_t)(2 * w0 + (f != bnd[w0] ? 1 : 0));
          ma.nparts[ma.n_split] = (int16_t)(w1 - w0 + 1);
          ++ma.n_split;
        }
        f = e;
      }
  }
  if (ma.n_split > 0) {
    record(L, &ev, s);
    if (launch_merge(c.dtype, d, ma, s) != hipSuccess) return DFLASH_ERR_HIP;
    record_end(L, DFLASH_K_MERGE, ev, s);
  }
  record_end(L, DFLASH_K_ATTN_MERGE, span, s, DFLASH_PROFILE_ATTN_SPAN);

  // HK1: o_proj (k split as decided above)
  const int64_t o_slice = (int64_t)Mq * H;
  GemmArgs go;
  std::memset(&go, 0, sizeof(go));
  go.nprob = 1;
  go.p[0] = {obuf, L->w.w_o, out, Mq, H, nq * d, nq * d, nq * d, H, (H + to.bn - 1) / to.bn, 0, 0};
  record(L, &ev, s);
  if (L->mx) {
    // the attention and merge wrote the MXFP8 rows of its output (aa.mxo)
    go.p[0].a = aa.mxo.codes;
    go.p[0].sa = aa.mxo.scales;
    go.p[0].sb = L->wo_scale;
    if (launch_gemm_mx(go, to.tiles, to.bm, to.bn, s) != hipSuccess) return DFLASH_ERR_HIP;
  } else if (o_split) {
    float* part = reinterpret_cast<float*>(ws + wc.qkv);
    go.p[0].c = part;
    go.p[0].slice_stride = o_slice;
    if (launch_gemm(c.dtype, true, go, to.tiles, to.bm, to.bn, to.kslices, s) != hipSuccess) return DFLASH_ERR_HIP;
    if (launch_sum_slices(c.dtype == DFLASH_BF16 ? 1 : 0, part, to.kslices, o_slice, out, o_slice, s) != hipSuccess)
      return DFLASH_ERR_HIP;
  } else if (launch_gemm(c.dtype, false, go, to.tiles, to.bm, to.bn, 1, s) != hipSuccess) {
    return DFLASH_ERR_HIP;
  }
  record_end(L, DFLASH_K_GEMM_O, ev, s);

  for (int b = 0; b < B; ++b) cache->len[b] += (ctx_offsets[b + 1] - ctx_offsets[b]) + bs;
  return DFLASH_OK;
}

static_assert(kMaxBatch == DFLASH_LAUNCH_BATCH, "one launch plans for DFLASH_LAUNCH_BATCH sequences");

// A step of more sequences than one launch plans for (kMaxBatch): the
// sequences are independent, so it runs as consecutive steps over runs of at
// most kMaxBatch of them, each on a view of the cache and of the step's rows
// sharing the workspace, after every run has passed the host-side checks.
static int attn_step_any(dflash_layer* L, const void* hidden_states, const void* target_hidden,
                         const int32_t* ctx_offsets, const int32_t* positions, dflash_kv_cache* cache, void* out,
                         void* workspace, size_t workspace_bytes, void* stream, bool validate_only,
                         bool noalloc = false) {
  if (!L || !cache || !ctx_offsets) return DFLASH_ERR_ARG;
  const int B = cache->batch;
  if (B <= kMaxBatch)
    return attn_step_impl(L, hidden_states, target_hidden, ctx_offsets, positions, cache, out, workspace,
                          workspace_bytes, stream, validate_only, noalloc);
  if (B > DFLASH_MAX_BATCH || !hidden_states || !out || !cache->len) return DFLASH_ERR_ARG;
  if (ctx_offsets[0] != 0) return DFLASH_ERR_SHAPE;
  const dflash_config& c = L->cfg;
  const size_t row_bytes = (size_t)c.hidden * elem_size(c);
  for (int pass = 0; pass < (validate_only ? 1 : 2); ++pass)
    for (int b0 = 0; b0 < B; b0 += kMaxBatch) {
      const int nb = std::min(kMaxBatch, B - b0);
      int32_t offs[kMaxBatch + 1];
      for (int i = 0; i <= nb; ++i) offs[i] = ctx_offsets[b0 + i] - ctx_offsets[b0];
      dflash_kv_cache view = cache_view(cache, b0, nb, c.n_kv_heads, c.head_dim, elem_size(c));
      const size_t row0 = (size_t)b0 * c.block_size;
      const int st = attn_step_impl(
          L, static_cast<const char*>(hidden_states) + row0 * row_bytes,
          target_hidden ? static_cast<const char*>(target_hidden) + (size_t)ctx_offsets[b0] * row_bytes : nullptr,
          offs, positions ? positions + ctx_offsets[b0] + row0 : nullptr, &view,
          static_cast<char*>(out) + row0 * row_bytes, workspace, workspace_bytes, stream, pass == 0, noalloc);
      if (st != DFLASH_OK) return st;
    }
  return DFLASH_OK;
}

int dflash_attn_step(dflash_layer* L, const void* hidden_states, const void* target_hidden,
                     const int32_t* ctx_offsets, const int32_t* positions, dflash_kv_cache* cache,
                     void* out, void* workspace, size_t workspace_bytes, void* stream) {
  return attn_step_any(L, hidden_states, target_hidden, ctx_offsets, positions, cache, out, workspace,
                       workspace_bytes, stream, false);
}

int dflash_attn_step_noalloc(dflash_layer* L, const void* hidden_states, const void* target_hidden,
                             const int32_t* ctx_offsets, const int32_t* positions, dflash_kv_cache* cache,
                             void* out, void* stream) {
  return attn_step_any(L, hidden_states, target_hidden, ctx_offsets, positions, cache, out, nullptr, 0, stream,
                       false, true);
}

int dflash_cache_crop(dflash_kv_cache* cache, int32_t seq, int32_t new_len) {
  if (!cache || !cache->len || seq < 0 || seq >= cache->batch) return DFLASH_ERR_ARG;
  if (new_len < 0 || new_len > cache->len[seq]) return DFLASH_ERR_RANGE;
  cache->len[seq] = new_len;
  return DFLASH_OK;
}

int dflash_cache_crop_all(dflash_kv_cache* cache, const int32_t* new_len) {
  if (!cache || !cache->len || !new_len || cache->batch < 0) return DFLASH_ERR_ARG;
  for (int b = 0; b < cache->batch; ++b)
    if (new_len[b] < 0 || new_len[b] > cache->len[b]) return DFLASH_ERR_RANGE;
  for (int b = 0; b < cache->batch; ++b) cache->len[b] = new_len[b];
  return DFLASH_OK;
}

// ------------------------------------------------------------ block pool

int dflash_block_pool_create(int32_t num_blocks, dflash_block_pool** out) {
  if (!out) return DFLASH_ERR_ARG;
  *out = nullptr;
  if (num_blocks <= 0) return DFLASH_ERR_SHAPE;
  dflash_block_pool* p = new (std::nothrow) dflash_block_pool();
  if (!p) return DFLASH_ERR_HIP;
  p->num_blocks = num_blocks;
  p->free.resize(num_blocks);
  for (int32_t i = 0; i < num_blocks; ++i) p->free[i] = num_blocks - 1 - i;  // block 0 is taken first
  *out = p;
  return DFLASH_OK;
}

void dflash_block_pool_destroy(dflash_block_pool* p) { delete p; }

int32_t dflash_block_pool_free_count(const dflash_block_pool* p) { return p ? (int32_t)p->free.size() : -1; }

int dflash_block_pool_get_free(const dflash_block_pool* p, int32_t* blocks, int32_t capacity) {
  if (!p || (!blocks && !p->free.empty())) return DFLASH_ERR_ARG;
  if (capacity < (int32_t)p->free.size()) return DFLASH_ERR_SHAPE;
  std::copy(p->free.begin(), p->free.end(), blocks);
  return DFLASH_OK;
}

int dflash_block_pool_set_free(dflash_block_pool* p, const int32_t* blocks, int32_t n) {
  if (!p || n < 0 || (n > 0 && !blocks)) return DFLASH_ERR_ARG;
  if (n > p->num_blocks) return DFLASH_ERR_SHAPE;
  std::vector<char> seen(p->num_blocks, 0);
  for (int32_t i = 0; i < n; ++i) {
    if (blocks[i] < 0 || blocks[i] >= p->num_blocks || seen[blocks[i]]) return DFLASH_ERR_RANGE;
    seen[blocks[i]] = 1;
  }
  p->free.assign(blocks, blocks + n);
  return DFLASH_OK;
}

int dflash_cache_reserve(dflash_kv_cache* c, dflash_block_pool* p, int32_t seq, int64_t rows) {
  if (!pool_cache_ok(c, p) || seq < 0 || seq >= c->batch) return DFLASH_ERR_ARG;
  std::vector<int64_t> all(c->batch, -1);
  all[seq] = rows;
  return reserve_rows(c, p, all.data());
}

int dflash_cache_reserve_all(dflash_kv_cache* c, dflash_block_pool* p, const int64_t* rows) {
  if (!pool_cache_ok(c, p) || !rows) return DFLASH_ERR_ARG;
  return reserve_rows(c, p, rows);
}

int dflash_cache_release(dflash_kv_cache* c, dflash_block_pool* p, int32_t seq, int64_t rows) {
  if (!pool_cache_ok(c, p) || seq < 0 || seq >= c->batch) return DFLASH_ERR_ARG;
  std::vector<int64_t> all(c->batch, -1);
  all[seq] = rows;
  return release_rows(c, p, all.data());
}

int dflash_cache_release_all(dflash_kv_cache* c, dflash_block_pool* p, const int64_t* rows) {
  if (!pool_cache_ok(c, p) || !rows) return DFLASH_ERR_ARG;
  return release_rows(c, p, rows);
}

int dflash_cache_push_table(dflash_kv_cache* c, dflash_block_pool* p, void* stream) {
  if (!pool_cache_ok(c, p)) return DFLASH_ERR_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t* table = const_cast<int32_t*>(c->block_table);
  // One entry per index, its latest value: a patch kernel writes its entries
  // concurrently, so an index released and taken again since the last push
  // (two pending values) must go up once.
  const size_t n_entries = (size_t)c->batch * c->max_blocks;
  std::vector<char> seen(n_entries, 0);
  std::vector<std::pair<int32_t, int32_t>> latest;
  latest.reserve(p->pending.size());
  for (size_t k = p->pending.size(); k-- > 0;) {
    const auto& e = p->pending[k];
    if (e.first < 0 || (size_t)e.first >= n_entries) return DFLASH_ERR_ARG;
    if (seen[e.first]) continue;
    seen[e.first] = 1;
    latest.push_back(e);
  }
  size_t i = 0;
  while (i < latest.size()) {
    TablePatch patch;
    int n = 0;
    for (; n < kTablePatch && i < latest.size(); ++n, ++i) {
      patch.idx[n] = latest[i].first;
      patch.val[n] = latest[i].second;
    }
    if (launch_table_patch(table, patch, n, s) != hipSuccess) return DFLASH_ERR_HIP;
  }
  p->pending.clear();
  return DFLASH_OK;
}

int32_t dflash_block_pool_pending(const dflash_block_pool* p) { return p ? (int32_t)p->pending.size() : -1; }

int dflash_block_pool_drop_pending(dflash_block_pool* p) {
  if (!p) return DFLASH_ERR_ARG;
  p->pending.clear();
  return DFLASH_OK;
}

int dflash_layer_poll_error(dflash_layer* L, void* stream) {
  if (!L) return DFLASH_ERR_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t flag = 0;
  if (hipStreamSynchronize(s) != hipSuccess) return DFLASH_ERR_HIP;
  if (hipMemcpy(&flag, L->err, sizeof(flag), hipMemcpyDeviceToHost) != hipSuccess) return DFLASH_ERR_HIP;
  if (flag) {
    if (hipMemset(L->err, 0, sizeof(int32_t)) != hipSuccess) return DFLASH_ERR_HIP;
    return DFLASH_ERR_RANGE;
  }
  return DFLASH_OK;
}

int dflash_layer_set_append_mode(dflash_layer* L, int32_t mode) {
  if (!L || mode < DFLASH_APPEND_AUTO || mode > DFLASH_APPEND_SEPARATE) return DFLASH_ERR_ARG;
  L->append_mode = mode;
  return DFLASH_OK;
}

int dflash_layer_set_profiling(dflash_layer* L, int32_t enable) {
  if (!L || enable < DFLASH_PROFILE_OFF || enable > DFLASH_PROFILE_ATTN_SPAN) return DFLASH_ERR_ARG;
  if (hipDeviceSynchronize() != hipSuccess) return DFLASH_ERR_HIP;
  for (auto& p : L->pending) {
    L->event_pool.push_back(p.start);
    L->event_pool.push_back(p.stop);
  }
  L->pending.clear();
  std::fill(L->ms, L->ms + DFLASH_K_COUNT, 0.0);
  std::fill(L->count, L->count + DFLASH_K_COUNT, 0);
  L->profiling = enable;
  return DFLASH_OK;
}

int dflash_layer_kernel_times(dflash_layer* L, double* ms, int64_t* count) {
  if (!L || !ms || !count) return DFLASH_ERR_ARG;
  for (auto& p : L->pending) {
    if (hipEventSynchronize(p.stop) != hipSuccess) return DFLASH_ERR_HIP;
    float t = 0.f;
    if (hipEventElapsedTime(&t, p.start, p.stop) != hipSuccess) return DFLASH_ERR_HIP;
    L->ms[p.kernel] += t;
    L->count[p.kernel] += 1;
    L->event_pool.push_back(p.start);
    L->event_pool.push_back(p.stop);
  }
  L->pending.clear();
  for (int k = 0; k < DFLASH_K_COUNT; ++k) {
    ms[k] = L->ms[k];
    count[k] = L->count[k];
  }
  return DFLASH_OK;
}

namespace {
int ctxkv_create_impl(const dflash_ctxkv_config* cfg, const dflash_ctxkv_weights* weights, const uint8_t* w_scale,
                      bool mx, dflash_ctxkv** out) {
  if (!cfg || !weights || !out) return DFLASH_ERR_ARG;
  *out = nullptr;
  if (!weights->hidden_norm || !weights->w_kv || !weights->k_norm) return DFLASH_ERR_ARG;
  if (reinterpret_cast<uintptr_t>(weights->hidden_norm) % 16 || reinterpret_cast<uintptr_t>(weights->w_kv) % 16)
    return DFLASH_ERR_ARG;
  if (mx && (!w_scale || reinterpret_cast<uintptr_t>(w_scale) % 4)) return DFLASH_ERR_ARG;
  if (cfg->hidden <= 0 || cfg->n_kv_heads <= 0 || cfg->n_layers <= 0 || cfg->max_position <= 0)
    return DFLASH_ERR_SHAPE;
  if (cfg->hidden % (mx ? 128 : 64)) return DFLASH_ERR_SHAPE;
  if (cfg->n_layers > kMaxLayers || cfg->n_kv_heads > kMaxKvHeads) return DFLASH_ERR_UNSUPPORTED;
  if (cfg->head_dim != 64 && cfg->head_dim != 128) return DFLASH_ERR_UNSUPPORTED;
  if (!(cfg->rope_theta > 0.0) || !(cfg->rms_eps >= 0.0)) return DFLASH_ERR_ARG;
  if (cfg->dtype != DFLASH_F32 && cfg->dtype != DFLASH_BF16) return DFLASH_ERR_ARG;
  if (mx && cfg->dtype != DFLASH_BF16) return DFLASH_ERR_UNSUPPORTED;
  dflash_ctxkv* h = new (std::nothrow) dflash_ctxkv();
  if (!h) return DFLASH_ERR_HIP;
  h->cfg = *cfg;
  h->w = *weights;
  h->mx = mx;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) { delete h; return DFLASH_ERR_HIP; }
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0)
    h->num_cus = cus;
  // MXFP8: the weight scales [N][H / 32] repacked step-major for the GEMM's
  // scale loads (the caller's array is only read here).
  const int64_t n_rows = (int64_t)cfg->n_layers * 2 * cfg->n_kv_heads * cfg->head_dim;
  bool ok = upload_rope_table(cfg->max_position, cfg->head_dim, cfg->rope_theta, &h->cos_sin) &&
            hipMalloc(&h->err, sizeof(int32_t)) == hipSuccess && hipMemset(h->err, 0, sizeof(int32_t)) == hipSuccess;
  if (ok && mx)
    ok = hipMalloc(&h->w_scale, (size_t)n_rows * cfg->hidden / 32) == hipSuccess &&
         launch_scales_step_major(w_scale, h->w_scale, (int)n_rows, cfg->hidden, nullptr) == hipSuccess;
  if (!ok || hipDeviceSynchronize() != hipSuccess) {
    if (h->cos_sin) hipFree(h->cos_sin);
    if (h->err) hipFree(h->err);
    if (h->w_scale) hipFree(h->w_scale);
    delete h;
    return DFLASH_ERR_HIP;
  }
  *out = h;
  return DFLASH_OK;
}
}  // namespace

int dflash_ctxkv_create(const dflash_ctxkv_config* cfg, const dflash_ctxkv_weights* weights,
                        dflash_ctxkv** out) {
  return ctxkv_create_impl(cfg, weights, nullptr, false, out);
}

int dflash_ctxkv_create_mxfp8(const dflash_ctxkv_config* cfg, const dflash_ctxkv_mxfp8_weights* weights,
                              dflash_ctxkv** out) {
  if (!weights) return DFLASH_ERR_ARG;
  dflash_ctxkv_weights w;
  w.hidden_norm = weights->hidden_norm;
  w.w_kv = weights->w_kv;
  w.k_norm = weights->k_norm;
  return ctxkv_create_impl(cfg, &w, static_cast<const uint8_t*>(weights->w_kv_scale), true, out);
}

int dflash_ctxkv_set_fc(dflash_ctxkv* h, const void* w_fc, int32_t fc_in) {
  if (!h) return DFLASH_ERR_ARG;
  if (!w_fc) {
    h->w_fc = nullptr;
    h->fc_in = 0;
    return DFLASH_OK;
  }
  if (reinterpret_cast<uintptr_t>(w_fc) % 16) return DFLASH_ERR_ARG;
  if (fc_in <= 0 || fc_in % 64) return DFLASH_ERR_SHAPE;
  h->w_fc = w_fc;
  h->fc_in = fc_in;
  return DFLASH_OK;
}

size_t dflash_ctxkv_combine_workspace_bytes(const dflash_ctxkv* h, int64_t rows) {
  if (!h || rows < 0) return 0;
  return align_up((size_t)kMaxKSlices * (size_t)std::max<int64_t>(rows, 1) * h->cfg.hidden * 4);
}

int dflash_ctxkv_combine(dflash_ctxkv* h, const void* aux_states, int64_t rows, void* context_states,
                         void* workspace, size_t workspace_bytes, void* stream) {
  if (!h) return DFLASH_ERR_ARG;
  if (rows < 0 || rows > INT32_MAX) return DFLASH_ERR_SHAPE;
  if (rows == 0) return DFLASH_OK;
  if (!h->w_fc || !aux_states || !context_states) return DFLASH_ERR_ARG;
  if (reinterpret_cast<uintptr_t>(aux_states) % 16 || reinterpret_cast<uintptr_t>(context_states) % 16)
    return DFLASH_ERR_ARG;
  const dflash_ctxkv_config& c = h->cfg;
  const int H = c.hidden, K = h->fc_in;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // Few rows and a long k: split k over fp32 slices in the workspace and sum
  // them (one rounding to the dtype); otherwise the GEMM rounds directly.
  const TileChoice t = choose_tiles_fill(h->num_cus, (int)rows, H, K, c.dtype == DFLASH_BF16 ? 2 : 4, kMaxKSlices);
  GemmArgs ga;
  std::memset(&ga, 0, sizeof(ga));
  ga.nprob = 1;
  const int64_t slice = rows * (int64_t)H;
  if (t.kslices == 1) {
    ga.p[0] = {aux_states, h->w_fc, context_states, (int32_t)rows, H, K, K, K, H, (H + t.bn - 1) / t.bn, 0, 0};
    if (launch_gemm(c.dtype, c.dtype == DFLASH_F32, ga, t.tiles, t.bm, t.bn, 1, s) != hipSuccess)
      return DFLASH_ERR_HIP;
    return DFLASH_OK;
  }
  if (!workspace) return DFLASH_ERR_WORKSPACE;
  if (workspace_bytes < (size_t)t.kslices * slice * 4 || reinterpret_cast<uintptr_t>(workspace) % kAlign)
    return DFLASH_ERR_WORKSPACE;
  float* part = static_cast<float*>(workspace);
  ga.p[0] = {aux_states, h->w_fc, part, (int32_t)rows, H, K, K, K, H, (H + t.bn - 1) / t.bn, 0, slice};
  if (launch_gemm(c.dtype, true, ga, t.tiles, t.bm, t.bn, t.kslices, s) != hipSuccess) return DFLASH_ERR_HIP;
  if (launch_sum_slices(c.dtype == DFLASH_BF16 ? 1 : 0, part, t.kslices, slice, context_states, slice, s) !=
      hipSuccess)
    return DFLASH_ERR_HIP;
  return DFLASH_OK;
}

int dflash_mxfp8_quantize(const void* x, int64_t rows, int32_t cols, void* codes, void* scales, void* stream) {
  if (rows < 0 || rows > INT32_MAX || cols <= 0 || cols % 128) return DFLASH_ERR_SHAPE;
  if (rows == 0) return DFLASH_OK;
  if (!x || !codes || !scales) return DFLASH_ERR_ARG;
  if (reinterpret_cast<uintptr_t>(x) % 16 || reinterpret_cast<uintptr_t>(codes) % 16) return DFLASH_ERR_ARG;
  if (launch_rms_rows_mx(x, nullptr, static_cast<uint8_t*>(codes), static_cast<uint8_t*>(scales), (int)rows, cols,
                         0.f, 0, static_cast<hipStream_t>(stream)) != hipSuccess)
    return DFLASH_ERR_HIP;
  return DFLASH_OK;
}

void dflash_ctxkv_destroy(dflash_ctxkv* h) {
  if (!h) return;
  hipDeviceSynchronize();
  hipFree(h->cos_sin);
  hipFree(h->err);
  if (h->w_scale) hipFree(h->w_scale);
  delete h;
}

size_t dflash_ctxkv_workspace_bytes(const dflash_ctxkv* h, int64_t total_ctx) {
  if (!h || total_ctx < 0) return 0;
  return ctx_carve(h->cfg, total_ctx, h->mx).total;
}

int dflash_ctxkv_workspace_offset(const dflash_ctxkv* h, int64_t total_ctx, int32_t region, size_t* offset) {
  if (!h || !offset || total_ctx < 0) return DFLASH_ERR_ARG;
  const CtxCarve wc = ctx_carve(h->cfg, total_ctx, h->mx);
  switch (region) {
    case DFLASH_CTX_WS_NORMED: *offset = wc.normed; return DFLASH_OK;
    case DFLASH_CTX_WS_NORMED_MX_SCALES:
      if (!h->mx) return DFLASH_ERR_ARG;
      *offset = wc.scales;
      return DFLASH_OK;
    default: return DFLASH_ERR_ARG;
  }
}

}  // extern "C"

// The precompute for at most kMaxBatch sequences; with validate_only it
// returns after the host-side checks, having enqueued nothing.
static int ctxkv_append_impl(dflash_ctxkv* h, const void* context_states, const int32_t* ctx_offsets,
                             const int32_t* positions, dflash_kv_cache* const* caches, void* workspace,
                             size_t workspace_bytes, void* stream, bool validate_only) {
  if (!h || !ctx_offsets || !caches) return DFLASH_ERR_ARG;
  const dflash_ctxkv_config& c = h->cfg;
  const int nl = c.n_layers, nkv = c.n_kv_heads, d = c.head_dim, H = c.hidden;
  for (int l = 0; l < nl; ++l)
    if (!caches[l] || !caches[l]->k || !caches[l]->v || !caches[l]->len) return DFLASH_ERR_ARG;
  const dflash_kv_cache* c0 = caches[0];
  const int B = c0->batch;
  if (B < 1 || B > kMaxBatch) return DFLASH_ERR_ARG;
  if (c0->capacity <= 0 || c0->capacity % kKeyTile || c0->capacity > kMaxCapacity) return DFLASH_ERR_SHAPE;
  for (int l = 1; l < nl; ++l) {
    if (caches[l]->batch != B || caches[l]->capacity != c0->capacity) return DFLASH_ERR_SHAPE;
    // every layer paged or none; a paged layer may have its own table and pools
    if ((caches[l]->block_table == nullptr) != (c0->block_table == nullptr)) return DFLASH_ERR_SHAPE;
    for (int b = 0; b < B; ++b)
      if (caches[l]->len[b] != c0->len[b]) return DFLASH_ERR_SHAPE;
  }
  if (ctx_offsets[0] != 0) return DFLASH_ERR_SHAPE;
  SeqTable seq;
  std::memset(&seq, 0, sizeof(seq));
  seq.batch = B;
  int max_new = 0;
  for (int b = 0; b < B; ++b) {
    const int64_t n = (int64_t)ctx_offsets[b + 1] - ctx_offsets[b];
    if (n < 0 || c0->len[b] < 0) return DFLASH_ERR_SHAPE;
    if ((int64_t)c0->len[b] + n > c0->capacity) return DFLASH_ERR_CAPACITY;
    seq.len[b] = c0->len[b];
    seq.ctx_off[b] = ctx_offsets[b];
    max_new = std::max<int>(max_new, (int)n);
  }
  seq.ctx_off[B] = ctx_offsets[B];
  const int64_t Mc = ctx_offsets[B];
  {
    int64_t rows[kMaxBatch];
    for (int b = 0; b < B; ++b) rows[b] = (int64_t)c0->len[b] + (ctx_offsets[b + 1] - ctx_offsets[b]);
    for (int l = 0; l < nl; ++l) {
      const int lst = check_layout(caches[l], rows);
      if (lst != DFLASH_OK) return lst;
    }
  }
  if (!positions)
    for (int b = 0; b < B; ++b)
      if ((int64_t)c0->len[b] + (ctx_offsets[b + 1] - ctx_offsets[b]) > c.max_position) return DFLASH_ERR_RANGE;
  if (Mc == 0) return DFLASH_OK;
  if (!context_states || reinterpret_cast<uintptr_t>(context_states) % 16) return DFLASH_ERR_ARG;
  if (!workspace) return DFLASH_ERR_WORKSPACE;
  if (h->mx && h->append_mode == DFLASH_APPEND_SEPARATE) return DFLASH_ERR_UNSUPPORTED;
  const CtxCarve wc = ctx_carve(c, Mc, h->mx);
  if (workspace_bytes < wc.total || reinterpret_cast<uintptr_t>(workspace) % kAlign)
    return DFLASH_ERR_WORKSPACE;

  if (validate_only) return DFLASH_OK;

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  void* normed = ws + wc.normed;
  float* proj = reinterpret_cast<float*>(ws + wc.proj);
  const int N = nl * 2 * nkv * d;

  // hidden_norm over each raw context row (as MXFP8 rows for MXFP8 weights)
  if (h->mx) {
    if (launch_rms_rows_mx(context_states, h->w.hidden_norm, static_cast<uint8_t*>(normed),
                           reinterpret_cast<uint8_t*>(ws + wc.scales), (int)Mc, H, (float)c.rms_eps, (int)Mc,
                           s) != hipSuccess)
      return DFLASH_ERR_HIP;
  } else if (launch_rms_rows(c.dtype, context_states, nullptr, h->w.hidden_norm, nullptr, normed, (int)Mc, H,
                             (float)c.rms_eps, s) != hipSuccess) {
    return DFLASH_ERR_HIP;
  }
  // Every layer's K and V in one projection. With enough 64-row tiles (one
  // head each) its epilogue normalises, rotates and appends (no fp32 rows);
  // otherwise fp32 rows (k split when M is small) go to HK2 over the layers.
  const int heads = nl * 2 * nkv;
  const int t64 = (int)((Mc + 63) / 64) * heads, t128 = (int)((Mc + 127) / 128) * heads;
  const bool fused = h->mx || h->append_mode == DFLASH_APPEND_FUSED ||
                     (h->append_mode == DFLASH_APPEND_AUTO && t64 >= h->num_cus * 3 / 4);
  NormRopeArgs na;
  std::memset(&na, 0, sizeof(na));
  na.positions = positions;
  na.cos_sin = h->cos_sin;
  na.q_norm = h->w.k_norm;
  na.k_norm = h->w.k_norm;
  na.kc = c0->k;
  na.vc = c0->v;
  for (int l = 0; l < nl; ++l) {
    na.layer_kc[l] = caches[l]->k;
    na.layer_vc[l] = caches[l]->v;
    na.layer_bt[l] = caches[l]->block_table;
    na.layer_nb[l] = caches[l]->block_table ? caches[l]->num_blocks : 0;
  }
  na.err = h->err;
  na.nq = nkv; na.nkv = nkv; na.bs = 0; na.cap = c0->capacity; na.max_pos = c.max_position;
  na.eps = (float)c.rms_eps;
  na.qscale = 1.0f;
  na.ctx_ld = N;
  na.ctx_layer_off = (int64_t)2 * nkv * d;
  na.map = cache_map(c0, nkv);
  na.seq = seq;
  GemmArgs ga;
  std::memset(&ga, 0, sizeof(ga));
  if (fused) {
    // the context problem is the second one (an empty first problem)
    const long r64 = (long)((t64 + h->num_cus - 1) / h->num_cus) * (64 + d);
    const long r128 = (long)((t128 + h->num_cus - 1) / h->num_cus) * (128 + d);
    const int bm = r128 <= r64 ? 128 : 64, tiles = bm == 128 ? t128 : t64;
    ga.nprob = 2;
    ga.p[0] = {normed, h->w.w_kv, nullptr, 0, N, H, H, H, N, heads, 0, 0};
    ga.p[1] = {normed, h->w.w_kv, proj, (int32_t)Mc, N, H, H, H, N, heads, 0, Mc * N};
    na.qkv = proj;
    na.ctxkv = proj;
    na.qpack = proj;
    if (h->mx) {
      // E4M3 rows of H bytes; the scales of both operands ride in the problem
      ga.p[1].sa = reinterpret_cast<const uint8_t*>(ws + wc.scales);
      ga.p[1].sb = h->w_scale;
      if (launch_gemm_append_mx(d, ga, na, tiles, bm, s) != hipSuccess) return DFLASH_ERR_HIP;
    } else if (launch_gemm_append(c.dtype, d, ga, na, tiles, bm, s) != hipSuccess) {
      return DFLASH_ERR_HIP;
    }
  } else {
    const TileChoice t = choose_tiles(h->num_cus, (int)Mc, N, 0, 0, true);
    ga.nprob = 1;
    ga.p[0] = {normed, h->w.w_kv, proj, (int32_t)Mc, N, H, H, H, N, (N + t.bn - 1) / t.bn, 0, Mc * N};
    if (launch_gemm(c.dtype, true, ga, t.tiles, t.bm, t.bn, t.kslices, s) != hipSuccess) return DFLASH_ERR_HIP;
    na.qkv = proj;
    na.ctxkv = proj;
    na.qkv_slice = Mc * N;
    na.ctx_slice = Mc * N;
    na.kslices = t.kslices;
    na.qpack = proj;
    if (launch_norm_rope(c.dtype, d, na, B * nkv, max_new, nl, s) != hipSuccess) return DFLASH_ERR_HIP;
  }

  for (int l = 0; l < nl; ++l)
    for (int b = 0; b < B; ++b) caches[l]->len[b] += ctx_offsets[b + 1] - ctx_offsets[b];
  return DFLASH_OK;
}

extern "C" {

int dflash_ctxkv_append(dflash_ctxkv* h, const void* context_states, const int32_t* ctx_offsets,
                        const int32_t* positions, dflash_kv_cache* const* caches, void* workspace,
                        size_t workspace_bytes, void* stream) {
  if (!h || !ctx_offsets || !caches || !caches[0]) return DFLASH_ERR_ARG;
  const int B = caches[0]->batch;
  if (B <= kMaxBatch)
    return ctxkv_append_impl(h, context_states, ctx_offsets, positions, caches, workspace, workspace_bytes, stream,
                             false);
  // more sequences than one launch plans for: runs of at most kMaxBatch on
  // views of every layer's cache, all checked before the first runs
  const dflash_ctxkv_config& c = h->cfg;
  if (B > DFLASH_MAX_BATCH || c.n_layers > kMaxLayers) return DFLASH_ERR_ARG;
  if (ctx_offsets[0] != 0) return DFLASH_ERR_SHAPE;
  for (int l = 0; l < c.n_layers; ++l)
    if (!caches[l] || !caches[l]->len || caches[l]->batch != B) return caches[l] ? DFLASH_ERR_SHAPE : DFLASH_ERR_ARG;
  const int es = c.dtype == DFLASH_BF16 ? 2 : 4;
  const size_t row_bytes = (size_t)c.hidden * es;
  for (int pass = 0; pass < 2; ++pass)
    for (int b0 = 0; b0 < B; b0 += kMaxBatch) {
      const int nb = std::min(kMaxBatch, B - b0);
      int32_t offs[kMaxBatch + 1];
      for (int i = 0; i <= nb; ++i) offs[i] = ctx_offsets[b0 + i] - ctx_offsets[b0];
      dflash_kv_cache views[kMaxLayers];
      dflash_kv_cache* vp[kMaxLayers];
      for (int l = 0; l < c.n_layers; ++l) {
        views[l] = cache_view(caches[l], b0, nb, c.n_kv_heads, c.head_dim, es);
        vp[l] = &views[l];
      }
      const int st = ctxkv_append_impl(
          h, context_states ? static_cast<const char*>(context_states) + (size_t)ctx_offsets[b0] * row_bytes : nullptr,
          offs, positions ? positions + ctx_offsets[b0] : nullptr, vp, workspace, workspace_bytes, stream, pass == 0);
      if (st != DFLASH_OK) return st;
    }
  return DFLASH_OK;
}

int dflash_ctxkv_set_append_mode(dflash_ctxkv* h, int32_t mode) {
  if (!h || mode < DFLASH_APPEND_AUTO || mode > DFLASH_APPEND_SEPARATE) return DFLASH_ERR_ARG;
  h->append_mode = mode;
  return DFLASH_OK;
}

int dflash_ctxkv_poll_error(dflash_ctxkv* h, void* stream) {
  if (!h) return DFLASH_ERR_ARG;
  int32_t flag = 0;
  if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess) return DFLASH_ERR_HIP;
  if (hipMemcpy(&flag, h->err, sizeof(flag), hipMemcpyDeviceToHost) != hipSuccess) return DFLASH_ERR_HIP;
  if (flag) {
    if (hipMemset(h->err, 0, sizeof(int32_t)) != hipSuccess) return DFLASH_ERR_HIP;
    return DFLASH_ERR_RANGE;
  }
  return DFLASH_OK;
}

// ---------------------------------------------------------------- decoder layer

namespace {
// Workspace of a decoder step: the attention's, then input_layernorm output a,
// attention output, residual h, post_attention_layernorm output m ([Mq, H]
// each) and the MLP activation [Mq, I], all in the element type.
struct DecCarve {
  size_t attn, a, att, h, m, act, total;
};
// down_proj's tiles; k slices only where their fp32 partials fit the attention
// step's scratch region.
TileChoice down_tiles(const dflash_decoder* D, int m, int n, int k, size_t scratch_bytes) {
  const int es = D->cfg.attn.dtype == DFLASH_BF16 ? 2 : 4;
  const int fit = (int)std::min<size_t>(kMaxKSlices, scratch_bytes / ((size_t)m * n * 4));
  return choose_tiles_fill(D->num_cus, m, n, k, es, fit);
}
DecCarve dec_carve(const dflash_decoder* D, int64_t batch, int64_t total_ctx) {
  const dflash_config& c = D->cfg.attn;
  const int64_t es = c.dtype == DFLASH_BF16 ? 2 : 4, mq = batch * c.block_size;
  DecCarve w{};
  size_t off = 0;
  w.attn = off; off += align_up(carve(D->attn, std::min<int64_t>(batch, kMaxBatch), total_ctx).total);
  w.a = off;    off += align_up(mq * c.hidden * es);
  w.att = off;  off += align_up(mq * c.hidden * es);
  w.h = off;    off += align_up(mq * c.hidden * es);
  w.m = off;    off += align_up(mq * c.hidden * es);
  w.act = off;  off += align_up(mq * D->cfg.intermediate * es);
  w.total = off;
  return w;
}
}  // namespace

int dflash_decoder_create(const dflash_decoder_config* cfg, const dflash_decoder_weights* weights,
                          dflash_decoder** out) {
  if (!cfg || !weights || !out) return DFLASH_ERR_ARG;
  *out = nullptr;
  if (!weights->input_norm || !weights->post_norm || !weights->w_gate_up || !weights->w_down)
    return DFLASH_ERR_ARG;
  for (const void* p : {weights->input_norm, weights->post_norm})
    if (reinterpret_cast<uintptr_t>(p) % 16) return DFLASH_ERR_ARG;
  if (cfg->intermediate <= 0 || cfg->intermediate % 64) return DFLASH_ERR_SHAPE;
  dflash_decoder* D = new (std::nothrow) dflash_decoder();
  if (!D) return DFLASH_ERR_HIP;
  D->cfg = *cfg;
  D->w = *weights;
  const int st = dflash_layer_create(&cfg->attn, &weights->attn, &D->attn);
  if (st != DFLASH_OK) {
    delete D;
    return st;
  }
  D->num_cus = D->attn->num_cus;
  *out = D;
  return DFLASH_OK;
}

void dflash_decoder_destroy(dflash_decoder* D) {
  if (!D) return;
  dflash_layer_destroy(D->attn);
  delete D;
}

size_t dflash_decoder_workspace_bytes(const dflash_decoder* D, int32_t batch, int64_t total_ctx) {
  if (!D || batch < 1 || batch > DFLASH_MAX_BATCH || total_ctx < 0) return 0;
  return dec_carve(D, batch, total_ctx).total;
}

int dflash_decoder_workspace_offset(const dflash_decoder* D, int32_t batch, int64_t total_ctx, int32_t region,
                                    size_t* offset) {
  if (!D || !offset || batch < 1 || batch > DFLASH_MAX_BATCH || total_ctx < 0) return DFLASH_ERR_ARG;
  const DecCarve wc = dec_carve(D, batch, total_ctx);
  switch (region) {
    case DFLASH_DEC_WS_A: *offset = wc.a; return DFLASH_OK;
    case DFLASH_DEC_WS_ATT: *offset = wc.att; return DFLASH_OK;
    case DFLASH_DEC_WS_H: *offset = wc.h; return DFLASH_OK;
    case DFLASH_DEC_WS_M: *offset = wc.m; return DFLASH_OK;
    case DFLASH_DEC_WS_ACT: *offset = wc.act; return DFLASH_OK;
    default: return DFLASH_ERR_ARG;
  }
}

int dflash_decoder_step(dflash_decoder* D, const void* x, const void* target_hidden, const int32_t* ctx_offsets,
                        const int32_t* positions, dflash_kv_cache* cache, void* out, void* workspace,
                        size_t workspace_bytes, void* stream) {
  if (!D || !x || !out || !ctx_offsets || !cache) return DFLASH_ERR_ARG;
  if (reinterpret_cast<uintptr_t>(x) % 16 || reinterpret_cast<uintptr_t>(out) % 16) return DFLASH_ERR_ARG;
  const dflash_config& c = D->cfg.attn;
  const int B = cache->batch;
  if (B < 1 || B > DFLASH_MAX_BATCH) return DFLASH_ERR_ARG;
  if (!workspace) return DFLASH_ERR_WORKSPACE;
  const int64_t Mc = ctx_offsets[B];
  if (Mc < 0) return DFLASH_ERR_SHAPE;
  const DecCarve wc = dec_carve(D, B, Mc);
  if (workspace_bytes < wc.total || reinterpret_cast<uintptr_t>(workspace) % kAlign) return DFLASH_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  void* a = ws + wc.a;
  void* att = ws + wc.att;
  void* h = ws + wc.h;
  void* m = ws + wc.m;
  void* act = ws + wc.act;
  const size_t attn_bytes = wc.a - wc.attn;
  // every check of the attention step before anything is enqueued
  int st = attn_step_any(D->attn, a, target_hidden, ctx_offsets, positions, cache, att, ws + wc.attn, attn_bytes,
                         stream, true);
  if (st != DFLASH_OK) return st;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const int H = c.hidden, I = D->cfg.intermediate, Mq = B * c.block_size;
  const float eps = (float)c.rms_eps;
  // input_layernorm, then the attention layer step (its o_proj output in att)
  if (launch_rms_rows(c.dtype, x, nullptr, D->w.input_norm, nullptr, a, Mq, H, eps, s) != hipSuccess)
    return DFLASH_ERR_HIP;
  st = attn_step_any(D->attn, a, target_hidden, ctx_offsets, positions, cache, att, ws + wc.attn, attn_bytes,
                     stream, false);
  if (st != DFLASH_OK) return st;
  // h = x + att (the residual stream), m = post_attention_layernorm(h)
  if (launch_rms_rows(c.dtype, x, att, D->w.post_norm, h, m, Mq, H, eps, s) != hipSuccess) return DFLASH_ERR_HIP;
  // act = silu(m Wg^T) * (m Wu^T), no k split (the activation needs whole
  // sums): 256 x 192 tiles, or 128-column tiles (64 gate + 64 up) in one or two
  // launches, as swiglu_plan picks
  {
    const int tn = (2 * I + 127) / 128, es = (int)elem_size(c);
    const SwigluPlan sp = swiglu_plan(D->num_cus, Mq, I, H, es);
    GemmArgs ga;
    std::memset(&ga, 0, sizeof(ga));
    ga.nprob = 1;
    if (sp.bn == 192) {
      ga.p[0] = {m, D->w.w_gate_up, act, Mq, 2 * I, H, H, H, I, sp.c1, 0, 0};
      ga.p[0].b_pair = I;
      if (launch_gemm_swiglu_wide(ga, (Mq / 256) * sp.c1, s) != hipSuccess) return DFLASH_ERR_HIP;
    } else {
      ga.p[0] = {m, D->w.w_gate_up, act, Mq, sp.c1 < tn ? 2 * sp.c1 * 64 : 2 * I, H, H, H, I, sp.c1, 0, 0};
      ga.p[0].b_pair = I;
      if (launch_gemm_swiglu(c.dtype, ga, ((Mq + sp.bm - 1) / sp.bm) * sp.c1, sp.bm, s) != hipSuccess)
        return DFLASH_ERR_HIP;
      if (sp.c1 < tn) {
        // the other column tiles: gate rows and output columns from c1 * 64 on
        // (the up rows stay b_pair = I past their gate rows)
        const int c2 = tn - sp.c1;
        ga.p[0].b = static_cast<const char*>(D->w.w_gate_up) + (size_t)sp.c1 * 64 * H * es;
        ga.p[0].c = static_cast<char*>(act) + (size_t)sp.c1 * 64 * es;
        ga.p[0].n = 2 * c2 * 64;
        ga.p[0].tiles_n = c2;
        if (launch_gemm_swiglu(c.dtype, ga, ((Mq + sp.bm2 - 1) / sp.bm2) * c2, sp.bm2, s) != hipSuccess)
          return DFLASH_ERR_HIP;
      }
    }
  }
  // out = h + act Wd^T
  {
    const TileChoice t = down_tiles(D, Mq, H, I, attn_bytes);
    GemmArgs ga;
    std::memset(&ga, 0, sizeof(ga));
    ga.nprob = 1;
    ga.p[0] = {act, D->w.w_down, out, Mq, H, I, I, I, H, (H + t.bn - 1) / t.bn, 0, 0};
    if (t.kslices > 1) {
      // fp32 k slices in the attention step's scratch (consumed by now), summed
      // with the residual into out (one rounding)
      const int64_t slice = (int64_t)Mq * H;
      float* part = reinterpret_cast<float*>(ws + wc.attn);
      ga.p[0].c = part;
      ga.p[0].slice_stride = slice;
      if (launch_gemm(c.dtype, true, ga, t.tiles, t.bm, t.bn, t.kslices, s) != hipSuccess) return DFLASH_ERR_HIP;
      if (launch_sum_slices(c.dtype == DFLASH_BF16 ? 1 : 0, part, t.kslices, slice, out, slice, s, h) != hipSuccess)
        return DFLASH_ERR_HIP;
    } else {
      ga.p[0].r = h;
      if (launch_gemm(c.dtype, false, ga, t.tiles, t.bm, t.bn, 1, s) != hipSuccess) return DFLASH_ERR_HIP;
    }
  }
  return DFLASH_OK;
}

dflash_layer* dflash_decoder_attention(dflash_decoder* D) { return D ? D->attn : nullptr; }

int dflash_rms_norm(const void* x, const void* gain, void* out, int32_t rows, int32_t hidden, double eps,
                    int32_t dtype, void* stream) {
  if (!x || !gain || !out || rows < 0 || hidden <= 0 || hidden % 64 || !(eps >= 0.0)) return DFLASH_ERR_ARG;
  if (dtype != DFLASH_F32 && dtype != DFLASH_BF16) return DFLASH_ERR_ARG;
  for (const void* p : {x, gain, static_cast<const void*>(out)})
    if (reinterpret_cast<uintptr_t>(p) % 16) return DFLASH_ERR_ARG;
  if (launch_rms_rows(dtype, x, nullptr, gain, nullptr, out, rows, hidden, (float)eps,
                      static_cast<hipStream_t>(stream)) != hipSuccess)
    return DFLASH_ERR_HIP;
  return DFLASH_OK;
}

}  // extern "C"

// Host-side check of libdflash's C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer, with device memory, copies and launches served
// by the host stand-in of hip_stub.cpp (no GPU is needed or touched).
//
// It drives every entry point of include/dflash.h through its argument
// checks, its workspace and scratch carving, its paged-table checks and its
// launch planning, over fixed edge cases and seeded random shapes, and checks
//   - the status of every call, and that a rejected call launches nothing and
//     changes no length;
//   - the shape of every launch (work-group size a positive multiple of the
//     64-lane wavefront and at most 1024, grid within the hardware limits);
//   - the workspace offsets the library reports lie inside its workspace;
//   - after every create that fails part-way (a failing hipMalloc is injected
//     at each allocation in turn) and after every destroy, that no device
//     allocation is left behind.
// The sanitizers check the library's host code itself (bounds of its fixed
// per-sequence tables, the merge list, integer overflow in size arithmetic).
// Exit status 0 when every check holds.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "dflash.h"
#include "hip_stub.h"

extern "C" int hipMalloc(void** p, size_t bytes);
extern "C" int hipFree(void* p);
// plan_check.cpp: the attention plan in the captured argument blocks
extern "C" int plan_check(const void* attn_bytes, size_t attn_size, const void* merge_bytes, size_t merge_size,
                          int key_tile, char* msg, size_t msg_size);
extern "C" size_t plan_arg_size(int which);
namespace dflash {
void attn_bounds(int G, int nkv, int B, const int32_t* tile_cnt, int64_t* bnd);
}

namespace {

int g_failures = 0, g_checks = 0;
size_t g_launches_checked = 0, g_plans_checked = 0;

#define CHECK(cond, ...)                                                  \
  do {                                                                    \
    ++g_checks;                                                           \
    if (!(cond)) {                                                        \
      ++g_failures;                                                       \
      std::fprintf(stderr, "FAIL %s:%d: %s: ", __FILE__, __LINE__, #cond); \
      std::fprintf(stderr, __VA_ARGS__);                                  \
      std::fprintf(stderr, "\n");                                         \
    }                                                                     \
  } while (0)

struct Rng {  // a 64-bit linear congruential generator (Knuth's MMIX constants)
  uint64_t s;
  explicit Rng(uint64_t seed) : s(seed * 2 + 1) {}
  uint32_t next() {
    s = s * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(s >> 33);
  }
  int range(int lo, int hi) { return lo + (int)(next() % (uint32_t)(hi - lo + 1)); }  // [lo, hi]
};

void* dev(size_t bytes) {
  void* p = nullptr;
  if (hipMalloc(&p, bytes ? bytes : 1) != 0) {
    std::fprintf(stderr, "stub allocation of %zu bytes failed\n", bytes);
    std::exit(2);
  }
  return p;
}
void* dev_zero(size_t bytes) {
  void* p = dev(bytes);
  std::memset(p, 0, bytes);
  return p;
}

// Every launch since the last clear: a sane shape; with key_tile > 0 also the
// plan of every attention launch and of the merge launch that follows it.
void check_launches(const char* what, int key_tile = 0) {
  const size_t n = stub_launch_count();
  if (key_tile > 0) {
    std::vector<unsigned char> attn(plan_arg_size(0)), merge(plan_arg_size(1));
    for (size_t i = 0; i < n; ++i) {
      if (!std::strstr(stub_launch(i).name, "attn_splitkv_kernel")) continue;
      const size_t na = stub_launch_first_arg(i, attn.data(), attn.size());
      const bool merged = i + 1 < n && std::strstr(stub_launch(i + 1).name, "attn_merge_kernel");
      const size_t nm = merged ? stub_launch_first_arg(i + 1, merge.data(), merge.size()) : 0;
      char msg[256] = "";
      const int rc = plan_check(attn.data(), na, merged ? merge.data() : nullptr, nm, key_tile, msg, sizeof(msg));
      CHECK(rc == 0, "%s: attention plan of launch %zu: %s", what, i, msg);
      ++g_plans_checked;
    }
  }
  for (size_t i = 0; i < n; ++i) {
    const StubLaunch l = stub_launch(i);
    const uint64_t threads = (uint64_t)l.block[0] * l.block[1] * l.block[2];
    CHECK(threads >= 64 && threads <= 1024 && threads % 64 == 0, "%s: %s block %ux%ux%u", what, l.name,
          l.block[0], l.block[1], l.block[2]);
    CHECK(l.grid[0] >= 1 && l.grid[1] >= 1 && l.grid[2] >= 1 && l.grid[0] <= 0x7fffffffu && l.grid[1] <= 65535 &&
              l.grid[2] <= 65535,
          "%s: %s grid %ux%ux%u", what, l.name, l.grid[0], l.grid[1], l.grid[2]);
    CHECK(l.shmem <= 160 * 1024, "%s: %s dynamic LDS %zu", what, l.name, l.shmem);
    CHECK(std::strcmp(l.name, "<unregistered>") != 0, "%s: launch of an unregistered kernel", what);
  }
  g_launches_checked += n;
  stub_clear_launches();
}

// ------------------------------------------------------------------ caches
struct Cache {
  dflash_kv_cache c{};
  std::vector<int32_t> len, table;
  void* k = nullptr;
  void* v = nullptr;
  void* dtable = nullptr;
  Cache(int batch, int nkv, int d, int es, int capacity, bool paged, int spare_blocks, Rng* rng) {
    len.assign(batch, 0);
    c.len = len.data();
    c.batch = batch;
    c.capacity = capacity;
    const int per = capacity / 64;
    if (!paged) {
      k = dev((size_t)batch * capacity * nkv * d * es);
      v = dev((size_t)batch * capacity * nkv * d * es);
    } else {
      const int nb = batch * per + spare_blocks;
      k = dev((size_t)nb * 64 * nkv * d * es);
      v = dev((size_t)nb * 64 * nkv * d * es);
      std::vector<int32_t> perm(nb);
      for (int i = 0; i < nb; ++i) perm[i] = i;
      for (int i = nb - 1; i > 0; --i) std::swap(perm[i], perm[rng->range(0, i)]);
      table.assign((size_t)batch * per, -1);
      for (size_t i = 0; i < table.size(); ++i) table[i] = perm[i];
      dtable = dev(table.size() * 4);
      std::memcpy(dtable, table.data(), table.size() * 4);
      c.block_table = static_cast<const int32_t*>(dtable);
      c.block_table_host = table.data();
      c.max_blocks = per;
      c.num_blocks = nb;
    }
    c.k = k;
    c.v = v;
  }
  Cache(const Cache&) = delete;
  Cache& operator=(const Cache&) = delete;
  ~Cache() {
    hipFree(k);
    hipFree(v);
    hipFree(dtable);
  }
};

// ------------------------------------------------------------------ layers
struct LayerBufs {
  void* wqkv = nullptr;
  void* wo = nullptr;
  void* qn = nullptr;
  void* kn = nullptr;
  void* wqkv_s = nullptr;
  void* wo_s = nullptr;
  ~LayerBufs() {
    hipFree(wqkv);
    hipFree(wo);
    hipFree(qn);
    hipFree(kn);
    hipFree(wqkv_s);
    hipFree(wo_s);
  }
};

dflash_config config(int H, int nq, int nkv, int d, int bs, int dtype, int window = 0) {
  dflash_config c{};
  c.hidden = H;
  c.n_q_heads = nq;
  c.n_kv_heads = nkv;
  c.head_dim = d;
  c.block_size = bs;
  c.sliding_window = window;
  c.max_position = 1 << 16;
  c.dtype = dtype;
  c.rope_theta = 1e6;
  c.rms_eps = 1e-6;
  return c;
}

dflash_layer* make_layer(const dflash_config& c, LayerBufs& b, bool mx) {
  const int es = c.dtype == DFLASH_BF16 ? 2 : 4;
  const size_t nqkv = (size_t)(c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim, od = (size_t)c.n_q_heads * c.head_dim;
  dflash_layer* L = nullptr;
  if (!mx) {
    b.wqkv = dev_zero(nqkv * c.hidden * es);
    b.wo = dev_zero((size_t)c.hidden * od * es);
    b.qn = dev_zero(c.head_dim * es);
    b.kn = dev_zero(c.head_dim * es);
    dflash_weights w{b.wqkv, b.wo, b.qn, b.kn};
    const int st = dflash_layer_create(&c, &w, &L);
    CHECK(st == DFLASH_OK && L, "create H=%d nq=%d nkv=%d d=%d bs=%d: %d", c.hidden, c.n_q_heads, c.n_kv_heads,
          c.head_dim, c.block_size, st);
  } else {
    b.wqkv = dev_zero(nqkv * c.hidden);
    b.wqkv_s = dev_zero(nqkv * c.hidden / 32);
    b.wo = dev_zero((size_t)c.hidden * od);
    b.wo_s = dev_zero((size_t)c.hidden * od / 32);
    b.qn = dev_zero(c.head_dim * 2);
    b.kn = dev_zero(c.head_dim * 2);
    dflash_mxfp8_weights w{b.wqkv, b.wqkv_s, b.wo, b.wo_s, b.qn, b.kn};
    const int st = dflash_layer_create_mxfp8(&c, &w, &L);
    CHECK(st == DFLASH_OK && L, "create_mxfp8 H=%d: %d", c.hidden, st);
  }
  return L;
}

// One layer step (or a noalloc step) over `cache` with per-sequence new
// context rows n[b]; checks the status against `expect` and the effects.
struct StepIO {
  void* hs = nullptr;
  void* th = nullptr;
  void* pos = nullptr;
  void* out = nullptr;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  ~StepIO() {
    hipFree(hs);
    hipFree(th);
    hipFree(pos);
    hipFree(out);
    hipFree(ws);
  }
};

// expect: a status, or kAnyStatus for "runs, or (noalloc only) does not fit
// the scratch".
constexpr int kAnyStatus = -1;

int run_step(dflash_layer* L, const dflash_config& c, Cache& cache, const std::vector<int32_t>& offs, bool noalloc,
             int expect, const char* what, size_t ws_shrink = 0) {
  const int es = c.dtype == DFLASH_BF16 ? 2 : 4, B = cache.c.batch, bs = c.block_size;
  const int64_t mc = offs[B];
  int64_t keys = 0;
  for (int b = 0; b < B; ++b) keys += cache.len[b] + (offs[b + 1] - offs[b]) + bs;
  StepIO io;
  io.hs = dev((size_t)B * bs * c.hidden * es);
  io.th = mc ? dev((size_t)mc * c.hidden * es) : nullptr;
  io.pos = dev_zero((size_t)(mc + (int64_t)B * bs) * 4);
  io.out = dev((size_t)B * bs * c.hidden * es);
  if (!noalloc) {
    const size_t need = dflash_workspace_bytes(L, B, mc, keys);
    CHECK(need > 0, "%s: workspace bytes", what);
    io.ws_bytes = need - std::min(need, ws_shrink);
    io.ws = dev(io.ws_bytes);
    for (int r = DFLASH_WS_ATTN_OUT; r <= DFLASH_WS_ATTN_OUT_MX_SCALES; ++r) {
      size_t off = 0;
      if (dflash_workspace_offset(L, B, mc, r, &off) == DFLASH_OK) {
        const size_t rows = (size_t)B * bs, od = (size_t)c.n_q_heads * c.head_dim;
        const size_t bytes = r == DFLASH_WS_ATTN_OUT ? rows * od * es : (r == DFLASH_WS_ATTN_OUT_MX ? rows * od
                                                                                              : rows * od / 32);
        CHECK(off % 16 == 0 && off + bytes <= need, "%s: region %d at %zu + %zu of %zu", what, r, off, bytes, need);
      }
    }
  }
  const std::vector<int32_t> before = cache.len;
  stub_clear_launches();
  const int st = noalloc ? dflash_attn_step_noalloc(L, io.hs, io.th, offs.data(), static_cast<int32_t*>(io.pos),
                                                    &cache.c, io.out, nullptr)
                         : dflash_attn_step(L, io.hs, io.th, offs.data(), static_cast<int32_t*>(io.pos), &cache.c,
                                            io.out, io.ws, io.ws_bytes, nullptr);
  if (expect == kAnyStatus)
    CHECK(st == DFLASH_OK || (noalloc && st == DFLASH_ERR_WORKSPACE), "%s: status %d", what, st);
  else
    CHECK(st == expect, "%s: status %d, expected %d", what, st, expect);
  if (st == DFLASH_OK) {
    CHECK(stub_launch_count() >= 3, "%s: %zu launches", what, stub_launch_count());
    for (int b = 0; b < B; ++b)
      CHECK(cache.len[b] == before[b] + (offs[b + 1] - offs[b]) + bs, "%s: len[%d] %d from %d", what, b,
            cache.len[b], before[b]);
  } else {
    CHECK(stub_launch_count() == 0, "%s: rejected step launched %zu kernels", what, stub_launch_count());
    CHECK(cache.len == before, "%s: rejected step changed a length", what);
  }
  check_launches(what, c.dtype == DFLASH_F32 && c.head_dim == 128 ? 32 : 64);
  return st;
}

std::vector<int32_t> offsets(const std::vector<int>& n) {
  std::vector<int32_t> o(n.size() + 1, 0);
  for (size_t b = 0; b < n.size(); ++b) o[b + 1] = o[b] + n[b];
  return o;
}

// ------------------------------------------------------------------ tests
void test_status_strings() {
  for (int s = -1; s <= 8; ++s) CHECK(dflash_status_string(s) && dflash_status_string(s)[0], "string %d", s);
}

void test_layer_create_rejections() {
  const size_t live = stub_live_allocations();
  LayerBufs b;
  b.wqkv = dev_zero(64);
  b.wo = dev_zero(64);
  b.qn = dev_zero(64);
  b.kn = dev_zero(64);
  dflash_weights w{b.wqkv, b.wo, b.qn, b.kn};
  struct Bad {
    dflash_config c;
    int expect;
  } bad[] = {
      {config(512, 6, 4, 128, 16, DFLASH_BF16), DFLASH_ERR_SHAPE},        // n_q % n_kv
      {config(512, 8, 2, 96, 16, DFLASH_BF16), DFLASH_ERR_UNSUPPORTED},   // head_dim 96
      {config(512, 32, 4, 128, 16, DFLASH_BF16), DFLASH_ERR_UNSUPPORTED}, // bs * g = 128 > 64
      {config(520, 8, 2, 128, 16, DFLASH_BF16), DFLASH_ERR_SHAPE},        // hidden % 64
      {config(512, 8, 2, 128, 16, 7), DFLASH_ERR_ARG},                    // dtype
      {config(512, 8, 2, 128, 0, DFLASH_BF16), DFLASH_ERR_SHAPE},         // block_size 0
      {config(512, 512, 512, 64, 1, DFLASH_BF16), DFLASH_ERR_UNSUPPORTED},// n_kv > 256
      {config(512, 8, 2, 128, 16, DFLASH_BF16, -1), DFLASH_ERR_SHAPE},    // window < 0
  };
  for (auto& x : bad) {
    dflash_layer* L = reinterpret_cast<dflash_layer*>(&b);  // must be reset to NULL
    const int st = dflash_layer_create(&x.c, &w, &L);
    CHECK(st == x.expect && L == nullptr, "bad config: status %d expected %d", st, x.expect);
  }
  dflash_config c = config(512, 8, 2, 128, 16, DFLASH_BF16);
  c.rope_theta = 0;
  dflash_layer* L = nullptr;
  CHECK(dflash_layer_create(&c, &w, &L) == DFLASH_ERR_ARG && !L, "theta 0");
  c = config(512, 8, 2, 128, 16, DFLASH_BF16);
  CHECK(dflash_layer_create(nullptr, &w, &L) == DFLASH_ERR_ARG, "null cfg");
  CHECK(dflash_layer_create(&c, nullptr, &L) == DFLASH_ERR_ARG, "null weights");
  CHECK(dflash_layer_create(&c, &w, nullptr) == DFLASH_ERR_ARG, "null out");
  dflash_weights w0 = w;
  w0.k_norm = nullptr;
  CHECK(dflash_layer_create(&c, &w0, &L) == DFLASH_ERR_ARG && !L, "null k_norm");
  // MXFP8: bf16 only, hidden % 128, scale pointers present
  dflash_mxfp8_weights mw{b.wqkv, b.wqkv, b.wo, b.wo, b.qn, b.kn};
  dflash_config cf = config(512, 8, 2, 128, 16, DFLASH_F32);
  CHECK(dflash_layer_create_mxfp8(&cf, &mw, &L) == DFLASH_ERR_UNSUPPORTED && !L, "mxfp8 fp32");
  dflash_config ch = config(576, 8, 2, 128, 16, DFLASH_BF16);
  CHECK(dflash_layer_create_mxfp8(&ch, &mw, &L) == DFLASH_ERR_SHAPE && !L, "mxfp8 hidden 576");
  mw.w_o_scale = nullptr;
  CHECK(dflash_layer_create_mxfp8(&c, &mw, &L) == DFLASH_ERR_ARG && !L, "mxfp8 null scale");
  dflash_layer_destroy(nullptr);
  CHECK(stub_live_allocations() == live + 4, "rejected creates left %zu allocations",
        stub_live_allocations() - live - 4);
  check_launches("create rejections");
}

// A failing hipMalloc at each allocation of create in turn: HIP error, no
// handle, nothing left allocated.
void test_create_allocation_failures() {
  for (int mx = 0; mx < 2; ++mx) {
    LayerBufs b;
    const dflash_config c = config(512, 8, 2, 128, 16, DFLASH_BF16);
    dflash_layer* L = make_layer(c, b, mx);
    dflash_layer_destroy(L);
    const size_t live = stub_live_allocations();
    dflash_weights w{b.wqkv, b.wo, b.qn, b.kn};
    dflash_mxfp8_weights mw{b.wqkv, b.wqkv_s, b.wo, b.wo_s, b.qn, b.kn};
    int failed = 0;
    for (int k = 0; k < 16; ++k) {
      stub_fail_malloc_after(k);
      L = nullptr;
      const int st = mx ? dflash_layer_create_mxfp8(&c, &mw, &L) : dflash_layer_create(&c, &w, &L);
      stub_fail_malloc_after(-1);
      if (st == DFLASH_OK) {
        dflash_layer_destroy(L);
        break;
      }
      ++failed;
      CHECK(st == DFLASH_ERR_HIP && !L, "alloc failure %d: status %d", k, st);
      CHECK(stub_live_allocations() == live, "alloc failure %d (mx %d): %zu allocations left", k, mx,
            stub_live_allocations() - live);
    }
    CHECK(failed >= 2, "create made only %d allocations", failed);
    CHECK(stub_live_allocations() == live, "destroy left allocations");
  }
  check_launches("create failures");
}

void test_layer_steps_fixed() {
  const size_t live = stub_live_allocations();
  Rng rng(11);
  for (int dtype : {DFLASH_BF16, DFLASH_F32}) {
    for (int d : {64, 128}) {
      LayerBufs b;
      const dflash_config c = config(512, 8, 2, d, 16, dtype);
      const int es = dtype == DFLASH_BF16 ? 2 : 4;
      dflash_layer* L = make_layer(c, b, false);
      for (int paged = 0; paged < 2; ++paged) {
        Cache cache(3, 2, d, es, 320, paged, 4, &rng);
        cache.len = {0, 100, 200};
        cache.c.len = cache.len.data();
        run_step(L, c, cache, offsets({5, 0, 9}), false, DFLASH_OK, "ragged step");
        run_step(L, c, cache, offsets({0, 0, 0}), false, DFLASH_OK, "no context rows");
        run_step(L, c, cache, offsets({0, 0, 0}), true, DFLASH_OK, "noalloc step");
        // lengths 53, 148, 257 after the three steps above: 257 + 60 + 16 > 320
        run_step(L, c, cache, offsets({0, 0, 60}), false, DFLASH_ERR_CAPACITY, "past capacity");
        run_step(L, c, cache, offsets({1, 1, 1}), false, DFLASH_ERR_WORKSPACE, "workspace short", 256);
        std::vector<int32_t> bad = offsets({1, 2, 3});
        bad[2] = 0;  // decreasing
        run_step(L, c, cache, bad, false, DFLASH_ERR_SHAPE, "decreasing offsets");
        bad = offsets({1, 2, 3});
        bad[0] = 1;
        run_step(L, c, cache, bad, false, DFLASH_ERR_SHAPE, "offsets[0] != 0");
        for (int mode : {DFLASH_APPEND_FUSED, DFLASH_APPEND_SEPARATE, DFLASH_APPEND_AUTO}) {
          CHECK(dflash_layer_set_append_mode(L, mode) == DFLASH_OK, "mode %d", mode);
          CHECK(dflash_cache_crop_all(&cache.c, std::vector<int32_t>{0, 10, 20}.data()) == DFLASH_OK, "crop");
          run_step(L, c, cache, offsets({3, 7, 1}), mode == DFLASH_APPEND_SEPARATE, DFLASH_OK, "append mode");
        }
        if (paged) {
          const int32_t keep = cache.table[1];
          cache.table[1] = cache.c.num_blocks;  // sequence 0's second block: past the pools
          CHECK(dflash_cache_crop_all(&cache.c, std::vector<int32_t>{0, 0, 0}.data()) == DFLASH_OK, "crop");
          run_step(L, c, cache, offsets({60, 0, 0}), false, DFLASH_ERR_RANGE, "table entry past the pools");
          cache.table[1] = -1;
          run_step(L, c, cache, offsets({60, 0, 0}), true, DFLASH_ERR_RANGE, "missing table entry");
          cache.table[1] = keep;
          run_step(L, c, cache, offsets({60, 0, 0}), false, DFLASH_OK, "table restored");
        }
      }
      CHECK(dflash_layer_set_append_mode(L, 3) == DFLASH_ERR_ARG, "bad mode");
      // profiling: every kernel of a step counted once
      CHECK(dflash_layer_set_profiling(L, 1) == DFLASH_OK, "profiling on");
      {
        Cache cache(2, 2, d, es, 128, false, 0, &rng);
        run_step(L, c, cache, offsets({4, 4}), false, DFLASH_OK, "profiled step");
        double ms[DFLASH_K_COUNT];
        int64_t cnt[DFLASH_K_COUNT];
        CHECK(dflash_layer_kernel_times(L, ms, cnt) == DFLASH_OK, "kernel times");
        CHECK(cnt[DFLASH_K_GEMM_QKV] == 1 && cnt[DFLASH_K_ATTN] == 1 && cnt[DFLASH_K_GEMM_O] == 1,
              "kernel counts %lld %lld %lld", (long long)cnt[0], (long long)cnt[2], (long long)cnt[4]);
      }
      // one span around the attention and its merge, nothing per kernel
      CHECK(dflash_layer_set_profiling(L, DFLASH_PROFILE_ATTN_SPAN) == DFLASH_OK, "span profiling");
      {
        Cache cache(2, 2, d, es, 128, false, 0, &rng);
        run_step(L, c, cache, offsets({4, 4}), false, DFLASH_OK, "span-profiled step");
        double ms[DFLASH_K_COUNT];
        int64_t cnt[DFLASH_K_COUNT];
        CHECK(dflash_layer_kernel_times(L, ms, cnt) == DFLASH_OK, "span times");
        CHECK(cnt[DFLASH_K_ATTN_MERGE] == 1 && cnt[DFLASH_K_ATTN] == 0 && cnt[DFLASH_K_GEMM_QKV] == 0,
              "span counts %lld %lld", (long long)cnt[DFLASH_K_ATTN_MERGE], (long long)cnt[DFLASH_K_ATTN]);
      }
      CHECK(dflash_layer_set_profiling(L, 3) == DFLASH_ERR_ARG, "unknown profiling mode");
      CHECK(dflash_layer_set_profiling(L, 0) == DFLASH_OK, "profiling off");
      CHECK(dflash_layer_poll_error(L, nullptr) == DFLASH_OK, "poll");
      dflash_layer_destroy(L);
    }
  }
  CHECK(stub_live_allocations() == live, "fixed steps left %zu allocations", stub_live_allocations() - live);
}

void test_crop() {
  Rng rng(3);
  Cache cache(3, 1, 64, 2, 128, false, 0, &rng);
  cache.len = {10, 20, 30};
  cache.c.len = cache.len.data();
  CHECK(dflash_cache_crop(&cache.c, 1, 5) == DFLASH_OK && cache.len[1] == 5, "crop");
  CHECK(dflash_cache_crop(&cache.c, 1, 6) == DFLASH_ERR_RANGE && cache.len[1] == 5, "crop grows");
  CHECK(dflash_cache_crop(&cache.c, 3, 0) == DFLASH_ERR_ARG, "crop seq past batch");
  CHECK(dflash_cache_crop(&cache.c, -1, 0) == DFLASH_ERR_ARG, "crop seq -1");
  CHECK(dflash_cache_crop(nullptr, 0, 0) == DFLASH_ERR_ARG, "crop null");
  const int32_t bad[3] = {1, 2, 31};
  CHECK(dflash_cache_crop_all(&cache.c, bad) == DFLASH_ERR_RANGE && cache.len[0] == 10 && cache.len[1] == 5,
        "crop_all all-or-nothing");
  const int32_t good[3] = {1, 2, 3};
  CHECK(dflash_cache_crop_all(&cache.c, good) == DFLASH_OK && cache.len[2] == 3, "crop_all");
  CHECK(dflash_cache_crop_all(&cache.c, nullptr) == DFLASH_ERR_ARG, "crop_all null");
}

// Seeded random shapes: batch up to the maximum, ragged lengths up to the
// capacity, empty contexts, windows, both layouts, both entry points.
void test_layer_steps_random(int cases) {
  const size_t live = stub_live_allocations();
  Rng rng(2024);
  for (int t = 0; t < cases; ++t) {
    const int d = rng.range(0, 1) ? 128 : 64;
    const int nkv = rng.range(1, 4), g = 1 << rng.range(0, 3);
    const int bs = 1 << rng.range(0, 6 - (g == 1 ? 0 : (g == 2 ? 1 : (g == 4 ? 2 : 3))));
    const int dtype = rng.range(0, 3) ? DFLASH_BF16 : DFLASH_F32;
    const int H = 64 * rng.range(2, 12);
    const bool mx = dtype == DFLASH_BF16 && H % 128 == 0 && (nkv * g * d) % 128 == 0 && rng.range(0, 2) == 0;
    const int window = rng.range(0, 3) == 0 ? rng.range(1, 400) : 0;
    const dflash_config c = config(H, nkv * g, nkv, d, bs, dtype, window);
    LayerBufs b;
    dflash_layer* L = make_layer(c, b, mx);
    if (!L) continue;
    const int pick = rng.range(0, 9);
    const int B = pick < 2 ? rng.range(200, DFLASH_LAUNCH_BATCH) : (pick == 2 ? rng.range(257, 700) : rng.range(1, 24));
    const int capacity = 64 * rng.range(1, B > 256 ? 4 : (B > 64 ? 8 : 24));
    const bool paged = rng.range(0, 1);
    const int es = dtype == DFLASH_BF16 ? 2 : 4;
    Cache cache(B, nkv, d, es, capacity, paged, rng.range(0, 3), &rng);
    std::vector<int> n(B);
    for (int s = 0; s < B; ++s) {  // every window fits: len + n + bs <= capacity (capacity >= 64 >= bs)
      const int room = capacity - bs;
      cache.len[s] = rng.range(0, 3) == 0 ? 0 : rng.range(0, room);
      n[s] = rng.range(0, 2) == 0 ? 0 : rng.range(0, std::min(room - cache.len[s], 70));
    }
    dflash_layer_set_append_mode(L, mx ? DFLASH_APPEND_AUTO : rng.range(0, 2));
    char what[160];
    std::snprintf(what, sizeof(what), "random case %d (B %d cap %d H %d nq %d nkv %d d %d bs %d %s%s%s)", t, B,
                  capacity, H, nkv * g, nkv, d, bs, dtype == DFLASH_BF16 ? "bf16" : "fp32", mx ? " mxfp8" : "",
                  paged ? " paged" : "");
    run_step(L, c, cache, offsets(n), rng.range(0, 2) == 0, kAnyStatus, what);
    dflash_layer_destroy(L);
  }
  CHECK(stub_live_allocations() == live, "random steps left %zu allocations", stub_live_allocations() - live);
}

// ------------------------------------------------------------------ ctxkv
struct CtxBufs {
  void* hn = nullptr;
  void* wkv = nullptr;
  void* kn = nullptr;
  void* wkv_s = nullptr;
  void* wfc = nullptr;
  ~CtxBufs() {
    hipFree(hn);
    hipFree(wkv);
    hipFree(kn);
    hipFree(wkv_s);
    hipFree(wfc);
  }
};

void test_ctxkv() {
  const size_t live = stub_live_allocations();
  Rng rng(7);
  for (int mx = 0; mx < 2; ++mx) {
    dflash_ctxkv_config c{};
    c.hidden = 512;
    c.n_layers = 3;
    c.n_kv_heads = 2;
    c.head_dim = 128;
    c.max_position = 4096;
    c.dtype = DFLASH_BF16;
    c.rope_theta = 1e6;
    c.rms_eps = 1e-6;
    const size_t rows = (size_t)c.n_layers * 2 * c.n_kv_heads * c.head_dim;
    CtxBufs bf;
    bf.hn = dev_zero(c.hidden * 2);
    bf.wkv = dev_zero(rows * c.hidden * (mx ? 1 : 2));
    bf.kn = dev_zero((size_t)c.n_layers * c.head_dim * 2);
    bf.wkv_s = dev_zero(rows * c.hidden / 32);
    dflash_ctxkv* h = nullptr;
    if (mx) {
      dflash_ctxkv_mxfp8_weights w{bf.hn, bf.wkv, bf.wkv_s, bf.kn};
      CHECK(dflash_ctxkv_create_mxfp8(&c, &w, &h) == DFLASH_OK && h, "ctxkv mxfp8 create");
    } else {
      dflash_ctxkv_weights w{bf.hn, bf.wkv, bf.kn};
      dflash_ctxkv_config bad = c;
      bad.n_layers = 17;
      CHECK(dflash_ctxkv_create(&bad, &w, &h) != DFLASH_OK && !h, "17 layers");
      bad = c;
      bad.head_dim = 96;
      CHECK(dflash_ctxkv_create(&bad, &w, &h) == DFLASH_ERR_UNSUPPORTED && !h, "ctxkv head_dim 96");
      CHECK(dflash_ctxkv_create(&c, &w, &h) == DFLASH_OK && h, "ctxkv create");
    }
    if (!h) continue;
    const int B = 4;
    std::vector<int> n = {3, 0, 70, 1};
    const std::vector<int32_t> offs = offsets(n);
    const int64_t mc = offs[B];
    void* states = dev((size_t)mc * c.hidden * 2);
    void* pos = dev_zero((size_t)mc * 4);
    const size_t need = dflash_ctxkv_workspace_bytes(h, mc);
    CHECK(need > 0, "ctxkv workspace");
    void* ws = dev(need);
    for (int r = DFLASH_CTX_WS_NORMED; r <= DFLASH_CTX_WS_NORMED_MX_SCALES; ++r) {
      size_t off = 0;
      if (dflash_ctxkv_workspace_offset(h, mc, r, &off) == DFLASH_OK)
        CHECK(off + (size_t)mc * c.hidden / (r == DFLASH_CTX_WS_NORMED ? (mx ? 1 : 1) : 32) <= need,
              "ctxkv region %d", r);
    }
    for (int tables = 0; tables < 3; ++tables) {  // contiguous, one shared table, a table per layer
      std::vector<Cache*> caches;
      for (int l = 0; l < c.n_layers; ++l) {
        caches.push_back(new Cache(B, c.n_kv_heads, c.head_dim, 2, 256, tables > 0, 2 + l, &rng));
        caches.back()->len = {10, 0, 100, 255 - 1};
        caches.back()->c.len = caches.back()->len.data();
      }
      if (tables == 1)
        for (int l = 1; l < c.n_layers; ++l) {
          caches[l]->c.block_table = caches[0]->c.block_table;
          caches[l]->c.block_table_host = caches[0]->c.block_table_host;
          caches[l]->c.num_blocks = caches[0]->c.num_blocks;
        }
      std::vector<dflash_kv_cache*> descs;
      for (auto* p : caches) descs.push_back(&p->c);
      stub_clear_launches();
      int st = dflash_ctxkv_append(h, states, offs.data(), static_cast<int32_t*>(pos), descs.data(), ws, need,
                                   nullptr);
      CHECK(st == DFLASH_OK, "ctxkv append (tables %d, mx %d): %d", tables, mx, st);
      for (auto* p : caches) CHECK(p->len[2] == 170 && p->len[3] == 255, "ctxkv lengths");
      check_launches("ctxkv append");
      // rejections leave every layer alone
      auto same = [&](const std::vector<std::vector<int32_t>>& lens) {
        for (size_t l = 0; l < caches.size(); ++l)
          if (caches[l]->len != lens[l]) return false;
        return true;
      };
      std::vector<std::vector<int32_t>> lens;
      for (auto* p : caches) lens.push_back(p->len);
      std::vector<int32_t> big = offsets({0, 0, 0, 2});  // 255 + 2 > 256
      st = dflash_ctxkv_append(h, states, big.data(), static_cast<int32_t*>(pos), descs.data(), ws, need, nullptr);
      CHECK(st == DFLASH_ERR_CAPACITY && same(lens) && stub_launch_count() == 0, "ctxkv capacity: %d", st);
      caches[2]->len[0] += 1;
      st = dflash_ctxkv_append(h, states, offs.data(), static_cast<int32_t*>(pos), descs.data(), ws, need, nullptr);
      CHECK(st == DFLASH_ERR_SHAPE && stub_launch_count() == 0, "ctxkv unequal lengths: %d", st);
      caches[2]->len[0] -= 1;
      if (tables == 2) {
        const int32_t keep = caches[2]->table[0];
        caches[2]->table[0] = caches[2]->c.num_blocks;
        st = dflash_ctxkv_append(h, states, offs.data(), static_cast<int32_t*>(pos), descs.data(), ws, need,
                                 nullptr);
        CHECK(st == DFLASH_ERR_RANGE && same(lens) && stub_launch_count() == 0, "ctxkv bad table: %d", st);
        caches[2]->table[0] = keep;
        const int32_t* t = caches[1]->c.block_table;
        caches[1]->c.block_table = nullptr;  // a contiguous layer among paged ones
        st = dflash_ctxkv_append(h, states, offs.data(), static_cast<int32_t*>(pos), descs.data(), ws, need,
                                 nullptr);
        CHECK(st == DFLASH_ERR_SHAPE && same(lens) && stub_launch_count() == 0, "ctxkv mixed layouts: %d", st);
        caches[1]->c.block_table = t;
      }
      st = dflash_ctxkv_append(h, states, offs.data(), static_cast<int32_t*>(pos), descs.data(), ws, need - 1,
                               nullptr);
      CHECK(st == DFLASH_ERR_WORKSPACE && same(lens), "ctxkv workspace short: %d", st);
      for (auto* p : caches) delete p;
    }
    for (int mode : {DFLASH_APPEND_FUSED, DFLASH_APPEND_SEPARATE})
      CHECK(dflash_ctxkv_set_append_mode(h, mode) == DFLASH_OK, "ctxkv mode");
    CHECK(dflash_ctxkv_set_append_mode(h, 9) == DFLASH_ERR_ARG, "ctxkv bad mode");
    // fc combine
    if (!mx) {
      bf.wfc = dev_zero((size_t)c.hidden * 1536 * 2);
      CHECK(dflash_ctxkv_set_fc(h, bf.wfc, 100) == DFLASH_ERR_SHAPE, "fc_in 100");
      CHECK(dflash_ctxkv_set_fc(h, bf.wfc, 1536) == DFLASH_OK, "set_fc");
      for (int64_t r : {1, 7, 300}) {
        void* aux = dev((size_t)r * 1536 * 2);
        void* out = dev((size_t)r * c.hidden * 2);
        const size_t wsb = dflash_ctxkv_combine_workspace_bytes(h, r);
        void* cws = dev(wsb ? wsb : 1);
        stub_clear_launches();
        CHECK(dflash_ctxkv_combine(h, aux, r, out, cws, wsb, nullptr) == DFLASH_OK, "combine %lld", (long long)r);
        check_launches("combine");
        hipFree(aux);
        hipFree(out);
        hipFree(cws);
      }
      CHECK(dflash_ctxkv_combine(h, states, -1, states, ws, need, nullptr) == DFLASH_ERR_SHAPE, "combine rows -1");
    }
    CHECK(dflash_ctxkv_poll_error(h, nullptr) == DFLASH_OK, "ctxkv poll");
    dflash_ctxkv_destroy(h);
    hipFree(states);
    hipFree(pos);
    hipFree(ws);
  }
  dflash_ctxkv_destroy(nullptr);
  CHECK(stub_live_allocations() == live, "ctxkv left %zu allocations", stub_live_allocations() - live);
}

// ------------------------------------------------------------------ decoder
void test_decoder() {
  const size_t live = stub_live_allocations();
  Rng rng(5);
  dflash_decoder_config dc{};
  dc.attn = config(512, 8, 2, 128, 16, DFLASH_BF16);
  dc.intermediate = 1536;
  LayerBufs b;
  b.wqkv = dev_zero((size_t)12 * 128 * 512 * 2);
  b.wo = dev_zero((size_t)512 * 1024 * 2);
  b.qn = dev_zero(256);
  b.kn = dev_zero(256);
  void* in_n = dev_zero(1024);
  void* post_n = dev_zero(1024);
  void* wgu = dev_zero((size_t)2 * 1536 * 512 * 2);
  void* wd = dev_zero((size_t)512 * 1536 * 2);
  dflash_decoder_weights w{{b.wqkv, b.wo, b.qn, b.kn}, in_n, post_n, wgu, wd};
  dflash_decoder* D = nullptr;
  dflash_decoder_config bad = dc;
  bad.intermediate = 100;
  CHECK(dflash_decoder_create(&bad, &w, &D) == DFLASH_ERR_SHAPE && !D, "decoder intermediate 100");
  CHECK(dflash_decoder_create(&dc, &w, &D) == DFLASH_OK && D, "decoder create");
  if (D) {
    CHECK(dflash_decoder_attention(D) != nullptr, "decoder attention");
    for (int B : {1, 5, 256}) {
      Cache cache(B, 2, 128, 2, 128, B == 5, 1, &rng);
      std::vector<int> n(B, 0);
      n[0] = 9;
      const std::vector<int32_t> offs = offsets(n);
      const int64_t mc = offs[B];
      const size_t need = dflash_decoder_workspace_bytes(D, B, mc);
      void* x = dev((size_t)B * 16 * 512 * 2);
      void* th = dev((size_t)mc * 512 * 2);
      void* pos = dev_zero((size_t)(mc + B * 16) * 4);
      void* out = dev((size_t)B * 16 * 512 * 2);
      void* ws = dev(need);
      for (int r = DFLASH_DEC_WS_A; r <= DFLASH_DEC_WS_ACT; ++r) {
        size_t off = 0;
        CHECK(dflash_decoder_workspace_offset(D, B, mc, r, &off) == DFLASH_OK, "decoder region %d", r);
        const size_t bytes = (size_t)B * 16 * (r == DFLASH_DEC_WS_ACT ? 1536 : 512) * 2;
        CHECK(off + bytes <= need, "decoder region %d at %zu + %zu of %zu", r, off, bytes, need);
      }
      CHECK(dflash_decoder_workspace_offset(D, B, mc, 9, nullptr) == DFLASH_ERR_ARG, "decoder bad region");
      stub_clear_launches();
      CHECK(dflash_decoder_step(D, x, th, offs.data(), static_cast<int32_t*>(pos), &cache.c, out, ws, need,
                                nullptr) == DFLASH_OK,
            "decoder step B=%d", B);
      check_launches("decoder step", 64);  // bf16, head_dim 128: 64-key tiles
      CHECK(cache.len[0] == 9 + 16, "decoder step length");
      CHECK(dflash_decoder_step(D, x, th, offs.data(), static_cast<int32_t*>(pos), &cache.c, out, ws, need - 1,
                                nullptr) == DFLASH_ERR_WORKSPACE && stub_launch_count() == 0,
            "decoder workspace short");
      hipFree(x);
      hipFree(th);
      hipFree(pos);
      hipFree(out);
      hipFree(ws);
    }
    dflash_decoder_destroy(D);
  }
  dflash_decoder_destroy(nullptr);
  hipFree(in_n);
  hipFree(post_n);
  hipFree(wgu);
  hipFree(wd);
  CHECK(stub_live_allocations() == live + 4, "decoder left allocations");
}

// The block pool against a plain model of the same rules (a free stack,
// sequence-major reserve, last-block-first release), over random operations.
void test_block_pool() {
  const size_t live = stub_live_allocations();
  Rng rng(99);
  const int B = 7, per = 9, nb = 40;
  Cache cache(B, 1, 64, 2, per * 64, true, 0, &rng);  // pools of B * per blocks; the pool hands out nb < that
  cache.c.num_blocks = nb;
  std::fill(cache.table.begin(), cache.table.end(), -1);
  dflash_block_pool* pool = nullptr;
  CHECK(dflash_block_pool_create(0, &pool) == DFLASH_ERR_SHAPE && !pool, "pool of 0 blocks");
  CHECK(dflash_block_pool_create(nb, &pool) == DFLASH_OK && pool, "pool create");
  CHECK(dflash_block_pool_free_count(pool) == nb, "all free");
  std::vector<int32_t> order(nb);
  for (int i = 0; i < nb; ++i) order[i] = i;
  for (int i = nb - 1; i > 0; --i) std::swap(order[i], order[rng.range(0, i)]);
  std::vector<int32_t> bad = order;
  bad[3] = bad[4];
  CHECK(dflash_block_pool_set_free(pool, bad.data(), nb) == DFLASH_ERR_RANGE, "repeated block");
  CHECK(dflash_block_pool_set_free(pool, order.data(), nb) == DFLASH_OK, "set free");
  std::vector<int32_t> model_free = order, model_table(B * per, -1);
  auto in_use = [&](int b) {
    int n = 0;
    for (int i = 0; i < per; ++i) n += model_table[b * per + i] >= 0;
    return n;
  };
  for (int op = 0; op < 3000; ++op) {
    const int kind = rng.range(0, 3);
    std::vector<int64_t> rows(B, -1);
    if (kind == 0 || kind == 2) {
      const int b = rng.range(0, B - 1);
      rows[b] = rng.range(0, per * 64 + 70);
    } else {
      for (int b = 0; b < B; ++b) rows[b] = rng.range(0, 2) ? rng.range(0, per * 64 + 10) : -1;
    }
    const bool reserve = kind < 2;
    // the model
    int expect = DFLASH_OK;
    if (reserve) {
      int64_t total = 0;
      for (int b = 0; b < B; ++b)
        if (rows[b] >= 0) {
          const int64_t need = (rows[b] + 63) / 64;
          if (need > per) expect = DFLASH_ERR_SHAPE;
          total += std::max<int64_t>(0, need - in_use(b));
        }
      if (expect == DFLASH_OK && total > (int64_t)model_free.size()) expect = DFLASH_ERR_CAPACITY;
      if (expect == DFLASH_OK)
        for (int b = 0; b < B; ++b)
          if (rows[b] >= 0)
            for (int64_t i = in_use(b); i < (rows[b] + 63) / 64; ++i) {
              model_table[b * per + i] = model_free.back();
              model_free.pop_back();
            }
    } else {
      for (int b = 0; b < B; ++b)
        if (rows[b] >= 0)
          for (int64_t i = per - 1; i >= (rows[b] + 63) / 64; --i)
            if (model_table[b * per + i] >= 0) {
              model_free.push_back(model_table[b * per + i]);
              model_table[b * per + i] = -1;
            }
    }
    int st;
    int seq = 0;
    for (int b = 0; b < B; ++b)
      if (rows[b] >= 0) seq = b;
    if (kind == 0) st = dflash_cache_reserve(&cache.c, pool, seq, rows[seq]);
    else if (kind == 1) st = dflash_cache_reserve_all(&cache.c, pool, rows.data());
    else if (kind == 2) st = dflash_cache_release(&cache.c, pool, seq, rows[seq]);
    else st = dflash_cache_release_all(&cache.c, pool, rows.data());
    CHECK(st == expect, "pool op %d kind %d: status %d, expected %d", op, kind, st, expect);
    CHECK(cache.table == model_table, "pool op %d: table differs from the model", op);
    std::vector<int32_t> got(nb);
    const int32_t nfree = dflash_block_pool_free_count(pool);
    CHECK(nfree == (int32_t)model_free.size() &&
              dflash_block_pool_get_free(pool, got.data(), nb) == DFLASH_OK &&
              std::equal(model_free.begin(), model_free.end(), got.begin()),
          "pool op %d: free stack differs from the model", op);
    if (rng.range(0, 9) == 0) {
      stub_clear_launches();
      const int32_t pending = dflash_block_pool_pending(pool);
      CHECK(dflash_cache_push_table(&cache.c, pool, nullptr) == DFLASH_OK, "push table");
      CHECK((int)stub_launch_count() <= (pending + 447) / 448, "push launches %zu for %d entries",
            stub_launch_count(), pending);
      CHECK(dflash_block_pool_pending(pool) == 0, "push clears pending");
      check_launches("push table");
    }
  }
  std::vector<int32_t> small(3);
  CHECK(dflash_block_pool_get_free(pool, small.data(), 3) == DFLASH_ERR_SHAPE || dflash_block_pool_free_count(pool) <= 3,
        "get_free into a short buffer");
  dflash_kv_cache flat = cache.c;
  flat.block_table = nullptr;
  CHECK(dflash_cache_reserve(&flat, pool, 0, 64) == DFLASH_ERR_ARG, "reserve on a contiguous cache");
  CHECK(dflash_cache_reserve(&cache.c, pool, B, 64) == DFLASH_ERR_ARG, "reserve past the batch");
  dflash_block_pool_destroy(pool);
  dflash_block_pool_destroy(nullptr);
  CHECK(stub_live_allocations() == live + 3, "pool test allocations");
}

// Steps without a position array: contiguous positions, refused up front when
// a window would pass max_position.
void test_contiguous_positions() {
  Rng rng(17);
  LayerBufs b;
  dflash_config c = config(512, 8, 2, 128, 16, DFLASH_BF16);
  c.max_position = 300;
  dflash_layer* L = make_layer(c, b, false);
  Cache cache(3, 2, 128, 2, 512, false, 0, &rng);
  cache.len = {10, 200, 260};
  cache.c.len = cache.len.data();
  const std::vector<int32_t> offs = offsets({3, 5, 24});  // 260 + 24 + 16 = 300: the last position 299
  StepIO io;
  io.hs = dev(3 * 16 * 512 * 2);
  io.th = dev(32 * 512 * 2);
  io.out = dev(3 * 16 * 512 * 2);
  io.ws_bytes = dflash_workspace_bytes(L, 3, 32, 600);
  io.ws = dev(io.ws_bytes);
  stub_clear_launches();
  CHECK(dflash_attn_step(L, io.hs, io.th, offs.data(), nullptr, &cache.c, io.out, io.ws, io.ws_bytes, nullptr) ==
            DFLASH_OK,
        "step without positions");
  check_launches("contiguous positions", 64);  // bf16, head_dim 128: 64-key tiles
  cache.len = {10, 200, 261};
  CHECK(dflash_attn_step(L, io.hs, io.th, offs.data(), nullptr, &cache.c, io.out, io.ws, io.ws_bytes, nullptr) ==
                DFLASH_ERR_RANGE &&
            stub_launch_count() == 0 && cache.len[2] == 261,
        "window past max_position refused");
  dflash_layer_destroy(L);
}

void test_free_functions() {
  void* x = dev_zero(300 * 512 * 2);
  void* g = dev_zero(512 * 2);
  void* o = dev(300 * 512 * 2);
  void* codes = dev(300 * 512);
  void* sc = dev(300 * 512 / 32);
  stub_clear_launches();
  CHECK(dflash_rms_norm(x, g, o, 300, 512, 1e-6, DFLASH_BF16, nullptr) == DFLASH_OK, "rms_norm");
  CHECK(dflash_rms_norm(x, g, o, 300, 520, 1e-6, DFLASH_BF16, nullptr) != DFLASH_OK, "rms_norm hidden 520");
  CHECK(dflash_rms_norm(nullptr, g, o, 300, 512, 1e-6, DFLASH_BF16, nullptr) == DFLASH_ERR_ARG, "rms_norm null");
  CHECK(dflash_mxfp8_quantize(x, 300, 512, codes, sc, nullptr) == DFLASH_OK, "quantize");
  CHECK(dflash_mxfp8_quantize(x, 300, 500, codes, sc, nullptr) == DFLASH_ERR_SHAPE, "quantize cols 500");
  CHECK(dflash_mxfp8_quantize(x, -1, 512, codes, sc, nullptr) == DFLASH_ERR_SHAPE, "quantize rows -1");
  CHECK(dflash_mxfp8_quantize(x, 0, 512, codes, sc, nullptr) == DFLASH_OK, "quantize 0 rows");
  check_launches("free functions");
  hipFree(x);
  hipFree(g);
  hipFree(o);
  hipFree(codes);
  hipFree(sc);
}

}  // namespace

// The attention's range cut on its own, over shapes the steps rarely reach:
// as many ranges as tiles (every range one tile), one long pair among many
// short ones, heads that cannot share the cut (G not a multiple of nkv).
void test_attn_bounds() {
  Rng rng(11);
  for (int it = 0; it < 2000; ++it) {
    const int B = rng.range(1, 64), nkv = rng.range(1, 8);
    std::vector<int32_t> tc(B);
    for (int b = 0; b < B; ++b) tc[b] = rng.range(0, 9) == 0 ? rng.range(50, 400) : rng.range(1, 6);
    int64_t per_head = 0;
    for (int b = 0; b < B; ++b) per_head += tc[b];
    const int64_t n = per_head * nkv;
    // 1 <= G <= the tiles, as attn_groups guarantees
    const int G = (int)std::min<int64_t>(std::min<int64_t>(256, n), rng.range(0, 3) == 0 ? n : rng.range(1, 256));
    std::vector<int64_t> bnd(G + 1, -1);
    dflash::attn_bounds(G, nkv, B, tc.data(), bnd.data());
    bool ok = bnd[0] == 0 && bnd[G] == n;
    for (int w = 0; w < G && ok; ++w) ok = bnd[w + 1] > bnd[w];
    if (ok && nkv > 1 && G % nkv == 0) {
      const int per = G / nkv;
      for (int j = 1; j < nkv && ok; ++j)
        for (int i = 0; i < per && ok; ++i) ok = bnd[j * per + i] == j * per_head + bnd[i];
    }
    CHECK(ok, "attn_bounds G=%d nkv=%d B=%d tiles=%lld: not %d non-empty, ordered, per-head ranges", G, nkv, B,
          (long long)n, G);
  }
}

int main(int argc, char** argv) {
  const int random_cases = argc > 1 ? std::atoi(argv[1]) : 200;
  stub_capture_first_arg("attn_splitkv_kernel", plan_arg_size(0));
  stub_capture_first_arg("attn_merge_kernel", plan_arg_size(1));
  const size_t live0 = stub_live_allocations();
  test_status_strings();
  test_attn_bounds();
  test_layer_create_rejections();
  test_create_allocation_failures();
  test_layer_steps_fixed();
  test_crop();
  test_layer_steps_random(random_cases);
  test_ctxkv();
  test_decoder();
  test_block_pool();
  test_contiguous_positions();
  test_free_functions();
  CHECK(stub_live_allocations() == live0, "%zu device allocations left at exit", stub_live_allocations() - live0);
  std::printf("host ABI check: %d checks, %zu launches checked, %zu attention plans checked, %d failures\n", g_checks,
              g_launches_checked, g_plans_checked, g_failures);
  return g_failures ? 1 : 0;
}

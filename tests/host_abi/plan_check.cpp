// Checks the attention plan a layer step handed to its kernels: the argument
// blocks of the split-KV attention launch and of its merge launch, as the host
// stand-in of the HIP runtime captured them. Compiled as HIP host code so that
// it sees the library's own argument structs; no device code runs.
//
// The flattened work is every (KV head j, sequence b) pair in head-major
// order, pair (b, j) owning key tiles [lo_b, hi_b) of sequence b. The checks:
//   - range_of is a permutation of the G ranges;
//   - every range holds at least one tile (count[bid], for the range
//     range_of[bid]) and together they hold every tile exactly once, in order
//     (start[w] is the pair and tile at the flat position where range w
//     begins);
//   - the merge list holds exactly the pairs that more than one range touches,
//     each with the slot of its first part (2 w0, or 2 w0 + 1 when the pair
//     begins after the start of range w0) and its number of parts;
//   - with G a multiple of nkv, every head is cut at the same places.
#include <cstdio>
#include <cstring>
#include <vector>

#include "kernels.h"

using dflash::AttnArgs;
using dflash::MergeArgs;

extern "C" int plan_check(const void* attn_bytes, size_t attn_size, const void* merge_bytes, size_t merge_size,
                          int key_tile, char* msg, size_t msg_size) {
  auto fail = [&](const char* what, long long a, long long b) {
    std::snprintf(msg, msg_size, "%s (%lld, %lld)", what, a, b);
    return 1;
  };
  if (attn_size != sizeof(AttnArgs)) return fail("attention argument size", (long long)attn_size, sizeof(AttnArgs));
  AttnArgs a;
  std::memcpy(&a, attn_bytes, sizeof(a));
  MergeArgs m;
  std::memset(&m, 0, sizeof(m));
  if (merge_bytes) {
    if (merge_size != sizeof(MergeArgs)) return fail("merge argument size", (long long)merge_size, sizeof(MergeArgs));
    std::memcpy(&m, merge_bytes, sizeof(m));
  }
  const int G = a.G, nkv = a.nkv, B = a.seq.batch;
  if (G < 1 || G > dflash::kMaxGroups) return fail("range count", G, dflash::kMaxGroups);
  std::vector<int> seen(G, 0);
  for (int bid = 0; bid < G; ++bid) {
    const int w = a.range_of[bid];
    if (w >= G || seen[w]++) return fail("range_of is not a permutation: work-group, range", bid, w);
  }
  // each sequence's key tiles
  std::vector<int> lo(B), cnt(B);
  for (int b = 0; b < B; ++b) {
    const int T = a.seq.len[b] + (a.seq.ctx_off[b + 1] - a.seq.ctx_off[b]) + a.bs;
    int first = 0;
    if (a.window > 0) first = T - a.bs - a.window + 1 > 0 ? T - a.bs - a.window + 1 : 0;
    lo[b] = first / key_tile;
    cnt[b] = (T + key_tile - 1) / key_tile - lo[b];
  }
  // the flat tiles in order, and the range that owns each
  std::vector<int> owner;
  std::vector<int> pair_of, tile_of;
  for (int j = 0; j < nkv; ++j)
    for (int b = 0; b < B; ++b)
      for (int t = 0; t < cnt[b]; ++t) {
        pair_of.push_back(b * nkv + j);
        tile_of.push_back(lo[b] + t);
      }
  const long long n = (long long)pair_of.size();
  if (n != a.total_tiles) return fail("total tiles", a.total_tiles, n);
  long long f = 0;
  owner.assign(n, -1);
  // each range's tile count, from the work-group that runs it
  std::vector<int> count(G, 0);
  for (int bid = 0; bid < G; ++bid) count[a.range_of[bid]] = a.count[bid];
  for (int w = 0; w < G; ++w) {
    if (count[w] < 1) return fail("empty range", w, count[w]);
    if (f + count[w] > n) return fail("ranges past the last tile: range, end", w, f + count[w]);
    const unsigned want = (unsigned)pair_of[f] | ((unsigned)tile_of[f] << 16);
    if (a.start[w] != want) return fail("start word of range", w, (long long)a.start[w]);
    for (int k = 0; k < count[w]; ++k) owner[f + k] = w;
    f += count[w];
  }
  if (f != n) return fail("ranges cover fewer tiles than there are", f, n);
  if (G % nkv == 0 && nkv > 1) {
    const int per = G / nkv;
    for (int j = 1; j < nkv; ++j)
      for (int i = 0; i < per; ++i)
        if (count[j * per + i] != count[i]) return fail("heads cut differently: head, range", j, i);
  }
  // the merge list
  int n_split = 0;
  f = 0;
  for (int j = 0; j < nkv; ++j)
    for (int b = 0; b < B; ++b) {
      const long long e = f + cnt[b];
      const int w0 = owner[f], w1 = owner[e - 1];
      if (w0 != w1) {
        if (!merge_bytes) return fail("split pair but no merge launch: pair", b * nkv + j, w0);
        int k = -1;
        for (int s = 0; s < m.n_split; ++s)
          if (m.pair[s] == b * nkv + j) k = s;
        if (k < 0) return fail("split pair missing from the merge list", b * nkv + j, w0);
        const bool starts_range = f == 0 || owner[f - 1] != w0;
        if (m.first_slot[k] != 2 * w0 + (starts_range ? 0 : 1)) return fail("first slot of pair", b * nkv + j, m.first_slot[k]);
        if (m.nparts[k] != w1 - w0 + 1) return fail("parts of pair", b * nkv + j, m.nparts[k]);
        ++n_split;
      }
      f = e;
    }
  if (merge_bytes && m.n_split != n_split) return fail("merge list length", m.n_split, n_split);
  return 0;
}

// Sizes of the captured argument blocks: 0 the attention's, 1 the merge's.
extern "C" size_t plan_arg_size(int which) { return which == 0 ? sizeof(AttnArgs) : sizeof(MergeArgs); }

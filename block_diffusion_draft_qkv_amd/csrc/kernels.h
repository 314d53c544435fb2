// Internal launch interface between the C-ABI host code and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace dflash {

// ---------------------------------------------------------------- projections
// C[m][n] = sum_k A[m][k] * B[n][k]: both operands row-major with k contiguous
// (an nn.Linear weight is B). Up to two independent problems per launch, one
// BM x BN tile per work-group; gridDim.y splits k, slice s of a problem's fp32
// partial sums going to c + s * slice_stride elements.
struct GemmProblem {
  const void* a;
  const void* b;
  void* c;
  int32_t m, n, k;
  int32_t lda, ldb, ldc;
  int32_t tiles_n;       // ceil(n / BN)
  int32_t tile_begin;    // first flat tile index of this problem in the launch
  int64_t slice_stride;  // elements between k-slice outputs
  // Optional, plain GEMM without a k split: C = A W^T + R (R [m][ldc] in the
  // output type, rounded once after the sum).
  const void* r = nullptr;
  // SwiGLU GEMM: W rows [0, b_pair) are the gate rows, [b_pair, 2 b_pair) the
  // up rows; output column j of a tile pairs gate row j and up row b_pair + j.
  int32_t b_pair = 0;
  // MXFP8 operands (gemm_append with the MX flag): a and b hold E4M3 codes
  // ([m][lda], [n][ldb] bytes) and sa / sb their E8M0 scales, one byte per 32
  // consecutive k, step-major: [k / 128][plane rows][4 bytes], the problem's
  // rows at the start of each plane; sa_plane / sb_plane are the bytes between
  // planes (0: 4 m and 4 n, planes of exactly the problem's rows).
  const uint8_t* sa = nullptr;
  const uint8_t* sb = nullptr;
  int64_t sa_plane = 0;
  int64_t sb_plane = 0;
};
struct GemmArgs {
  GemmProblem p[2];
  int32_t nprob;
};
// dtype: 0 fp32, 1 bf16 (A, B element type). out_f32: C is fp32, else C has
// the element type of A and B (then kslices must be 1). (bm, bn) in
// {64, 128}^2, or 256 x 128 for bf16.
hipError_t launch_gemm(int dtype, bool out_f32, const GemmArgs& args, int total_tiles, int bm, int bn,
                       int kslices, hipStream_t stream);

// ------------------------------------------------------------- cache layout
// Where cache row `row` of sequence b, KV head j lives. Rows come in 64-row
// blocks of every head, K [blocks][nkv][64][d] and V transposed within the
// block [blocks][nkv][d][64]. Contiguous: sequence b owns blocks
// b * (cap / 64) ... in order. Paged (bt != nullptr): logical block i of
// sequence b is physical block bt[b * bt_stride + i]; table entries are
// clamped into [0, num_blocks) (the host checks its mirror of the table; the
// clamp keeps a stale device table inside the pools).
struct CacheMap {
  const int32_t* bt;
  int32_t bt_stride, num_blocks, cap, nkv;
  __device__ inline int clamp_block(int p) const {
    return p < 0 ? 0 : (p >= num_blocks ? num_blocks - 1 : p);
  }
  __device__ inline int phys(int b, int row) const {
    return clamp_block(bt[(size_t)b * bt_stride + row / kKeyTile]);
  }
  // The raw table entry for wave-uniform b and row, read through the
  // constant address space: the table does not change while a kernel runs,
  // so the load is a scalar one and its wait (lgkmcnt) leaves the
  // vector-memory counter, which LDS-DMA streams pace themselves by, alone.
  // Clamp it with clamp_block where it is used, so the wait lands there.
  __device__ inline int entry_uniform(int b, int row) const {
    using ctab = const __attribute__((address_space(4))) int32_t;
    return ((ctab*)bt)[(size_t)b * bt_stride + row / kKeyTile];
  }
  // Both layouts are block-major: block p holds rows of every KV head,
  // K [p][nkv][64][d] and V^T [p][nkv][d][64]. A paged cache's block comes
  // from its table; a contiguous cache's row `row` of sequence b is in block
  // b * (cap / 64) + row / 64.
  __device__ inline size_t block_of(int b, int row) const {
    if (bt) return (size_t)phys(b, row);
    return (size_t)b * (cap / kKeyTile) + row / kKeyTile;
  }
  // element offset of K row `row`
  __device__ inline size_t k_row(int b, int j, int row, int d) const {
    return ((block_of(b, row) * nkv + j) * kKeyTile + row % kKeyTile) * d;
  }
  // element offset of V^T (dim 0, row `row`); dim dd adds dd * vstride()
  __device__ inline size_t v_col(int b, int j, int row, int d) const {
    return (block_of(b, row) * nkv + j) * d * kKeyTile + row % kKeyTile;
  }
  __device__ static constexpr int vstride() { return kKeyTile; }
};

// ------------------------------------------------- norm + RoPE + append + Q
struct NormRopeArgs {
  const float* qkv;        // [kslices][B*bs][(nq + 2 nkv) d] block projections (fp32)
  const float* ctxkv;      // [kslices][sum n_b][2 nkv d] context projections (fp32)
  int64_t qkv_slice, ctx_slice;  // elements between k slices (summed on read)
  int32_t kslices;
  const int32_t* positions;  // NULL: contiguous, len_b + (row in the window)
  const float* cos_sin;    // cos [max_pos][d/2] then sin [max_pos][d/2]
  const void* q_norm;
  const void* k_norm;
  void* qpack;             // [B*nkv][R][d]: R = bs*g rows ordered (i, hh)
  void* kc;                // cache K (CacheMap layout)
  void* vc;                // cache V^T (CacheMap layout)
  int32_t* err;
  int32_t nq, nkv, bs, cap, max_pos;
  float eps, qscale;
  int64_t ctx_ld;          // elements between context rows of ctxkv (2 nkv d for a layer step)
  // The multi-layer context precompute (bs = 0, no queries) runs grid.z =
  // layers: layer z > 0 reads the columns ctxkv + z * ctx_layer_off, its gain
  // k_norm + z * d and writes the cache layer_kc[z] / layer_vc[z].
  // Layer z > 0 of a paged stack may have its own block table and pool size
  // (layer_bt[z], layer_nb[z]); the table stride, capacity and lengths are
  // every layer's.
  int64_t ctx_layer_off;
  void* layer_kc[kMaxLayers];
  void* layer_vc[kMaxLayers];
  const int32_t* layer_bt[kMaxLayers];
  int32_t layer_nb[kMaxLayers];
  CacheMap map;            // cache layout of layer 0 (and of a layer step)
  SeqTable seq;
  __device__ inline CacheMap map_of(int z) const {
    CacheMap m = map;
    if (z > 0 && m.bt) {
      m.bt = layer_bt[z];
      m.num_blocks = layer_nb[z];
    }
    return m;
  }
};
// grid: B * n_kv (one column of work-groups per sequence and KV head) times
// `layers` (1 for a layer step); max_new_rows: the largest n_b + bs.
hipError_t launch_norm_rope(int dtype, int head_dim, const NormRopeArgs& args, int grid,
                            int max_new_rows, int layers, hipStream_t stream);

// RMSNorm of `rows` rows of h elements (h % 64 == 0) with gain g [h]:
// out = v / sqrt(mean(v^2) + eps) * g with v = x, or v = x + y rounded to the
// element type (then also stored to hout) when y is given; fp32 math, stored in
// the element type; 16-byte aligned rows.
hipError_t launch_rms_rows(int dtype, const void* x, const void* y, const void* g, void* hout, void* out,
                           int rows, int h, float eps, hipStream_t stream);

// Qwen3MLP's gate/up projection with its activation in the epilogue:
// C[m][j] = silu(A W_gate^T)[m][j] * (A W_up^T)[m][j] for j < n = b_pair, with
// W = [W_gate; W_up] stacked ([2 n, k]); one problem, bm x 128 tiles (64 outputs
// per tile), C in the element type.
hipError_t launch_gemm_swiglu(int dtype, const GemmArgs& args, int total_tiles, int bm, hipStream_t stream);
// The same in 256 x 192 tiles (96 gate + 96 up columns; bf16, k % 32 == 0,
// tiles_n = n / 192 with n = 2 b_pair a multiple of 192).
hipError_t launch_gemm_swiglu_wide(const GemmArgs& args, int total_tiles, hipStream_t stream);

// The q|k|v + context k|v projection (args as for launch_gemm, tiles bm x
// head_dim, no k split) doing the work of launch_norm_rope in its epilogue
// (nr's qkv, ctxkv and kslices fields are unused).
// The plain GEMM over MXFP8 operands (sa / sb set, k % 128 == 0, no k split),
// bf16 output: C = A W^T (+ R).
hipError_t launch_gemm_mx(const GemmArgs& args, int total_tiles, int bm, int bn, hipStream_t stream);
// gemm_append over MXFP8 operands (GemmProblem sa / sb set, k % 128 == 0);
// the caches and gains are bf16.
hipError_t launch_gemm_append_mx(int head_dim, const GemmArgs& args, const NormRopeArgs& nr, int total_tiles,
                                 int bm, hipStream_t stream);
// MXFP8 rows of bf16 x [rows][h] (h % 128 == 0): with g, hidden_norm first
// (x / sqrt(mean(x^2) + eps) * g rounded to bf16), without g x itself; codes
// [rows][h] E4M3 bytes and scales [rows][h / 32] E8M0 bytes, or step-major
// [h / 128][step_rows][4] when step_rows > 0 (step_rows >= rows).
hipError_t launch_rms_rows_mx(const void* x, const void* g, uint8_t* codes, uint8_t* scales, int rows, int h,
                              float eps, int step_rows, hipStream_t stream);
// table[idx[i]] = val[i] for i < count (count <= kTablePatch): the entries of a
// paged cache's block table that its block pool changed since the last upload.
constexpr int kTablePatch = 448;
struct TablePatch {
  int32_t idx[kTablePatch];
  int32_t val[kTablePatch];
};
hipError_t launch_table_patch(int32_t* table, const TablePatch& patch, int count, hipStream_t stream);

// out[i] = sum_s in[s * slice_stride + i] (+ residual[i] when given, in the
// dtype) rounded to the dtype (0 fp32, 1 bf16) for i < n (n % 4 == 0, 16-byte
// aligned buffers).
hipError_t launch_sum_slices(int dtype, const float* in, int slices, int64_t slice_stride, void* out, int64_t n,
                             hipStream_t stream, const void* residual = nullptr);
// Two bf16 row sets [rows1][h], [rows2][h] quantised (no norm) in one launch,
// each with step-major scales [h / 128][rows_i][4].
hipError_t launch_rows_mx2(const void* x1, uint8_t* c1, uint8_t* s1, int rows1, const void* x2, uint8_t* c2,
                           uint8_t* s2, int rows2, int h, hipStream_t stream);
// E8M0 scales [n][k / 32] (4-byte aligned) -> step-major [k / 128][n][4].
hipError_t launch_scales_step_major(const void* src, void* dst, int n, int k, hipStream_t stream);
hipError_t launch_gemm_append(int dtype, int head_dim, const GemmArgs& args, const NormRopeArgs& nr,
                              int total_tiles, int bm, hipStream_t stream);

// ------------------------------------------------------------------ attention
// MXFP8 form of the attention output (the o_proj input of a layer whose
// projections are MXFP8): codes [rows][ld] E4M3 bytes, scales step-major
// [ld / 128][rows][4] E8M0 bytes. codes == nullptr: write O in the dtype.
struct MxOut {
  uint8_t* codes;
  uint8_t* scales;
  int32_t ld, rows;
};

// Flattened work: pairs (b, j) in head-major order (j outer, b inner), each
// owning the 64-key tiles [lo_b, hi_b) of sequence b (lo_b > 0 only under a
// sliding window). Range w = range_of[bid] takes the count[bid] flat tiles
// from the one at start[w]; the host cuts the ranges (attn_bounds). With G a multiple of nkv,
// ranges w = j (G / nkv) + i of every head j cover the same sequences and
// tiles, so the nkv work-groups of one i read the nkv neighbouring 16 KB
// pieces of the same cache blocks at about the same time.
struct AttnArgs {
  const void* q;           // qpack
  const void* kc;
  const void* vc;
  void* o;                 // [B*bs][nq d] attention output (pre o_proj)
  void* part_o;            // [2G][64][d] un-normalised partial outputs, in the element type
  float* part_ml;          // [2G][64][2] running max (log2 domain) and sum
  int32_t nq, nkv, bs, R, cap, window, G;
  MxOut mxo;
  int64_t total_tiles;
  CacheMap map;            // cache layout
  SeqTable seq;
  // Start of range w: pair b * nkv + j in bits 0..15, absolute key tile in
  // bits 16..31 (filled by the host, which knows every length).
  uint32_t start[kMaxGroups];
  // Key tiles of the range that work-group bid runs (at least one). Indexed
  // by work-group, not by range: a 16-bit array read at w beside start[w]
  // let the compiler build start[w]'s scalar load from an SGPR base of
  // args + 2 w plus an offset of 2 w, and the scalar unit drops a base's low
  // two bits, so odd ranges read their neighbour's start.
  uint16_t count[kMaxGroups];
  // Range of work-group `bid` (a permutation of [0, G)); see attn_range_map.
  uint8_t range_of[kMaxGroups];
};
// Deals the G ranges to work-groups. Work-groups go to the 8 XCDs round-robin
// (bid % 8); each XCD gets a contiguous run of the ranges in (i, j) order, so
// the nkv heads of one i share an XCD and its L2.
void attn_range_map(int G, int nkv, uint8_t* range_of);
// Cuts the flat tiles of B sequences (tile_cnt[b] key tiles each, for each of
// nkv heads) into G ranges: bnd[w] is the first flat tile of range w, bnd[G]
// the total. The ranges are about equal in tiles plus kPairStartQuarters / 4
// tiles for each pair that starts inside them, every range holds at least one
// tile, and with G a multiple of nkv every head is cut at the same places.
constexpr int kPairStartQuarters = 4;  // a pair start's cost, in quarter tiles
void attn_bounds(int G, int nkv, int B, const int32_t* tile_cnt, int64_t* bnd);
hipError_t launch_attn(int dtype, int head_dim, const AttnArgs& args, hipStream_t stream);
// Attention work-groups one CU holds at once (bounded by the kernel's LDS ring)
// and the keys per attention tile.
int attn_wgs_per_cu(int dtype, int head_dim);
int attn_key_tile(int dtype, int head_dim);
// Bytes of K and V tiles one attention work-group keeps in flight (its ring
// minus the stage being consumed).
int attn_kv_in_flight(int dtype, int head_dim);

// Pairs that the attention split over several work-group ranges (at most
// G - 1: each contains a range boundary), merged by HK4.
struct MergeArgs {
  const void* part_o;
  const float* part_ml;
  void* o;
  MxOut mxo;
  int32_t nq, nkv, bs, R, n_split;
  int32_t pair[kMaxGroups];        // b * nkv + j
  int16_t first_slot[kMaxGroups];  // slot of the pair's first part
  int16_t nparts[kMaxGroups];      // parts (work-group ranges) of the pair
};
// kernel arguments are passed by value: both must fit the 4 KB argument block
static_assert(sizeof(AttnArgs) <= 4096 && sizeof(MergeArgs) <= 4096, "kernel arguments exceed 4 KB");
hipError_t launch_merge(int dtype, int head_dim, const MergeArgs& args, hipStream_t stream);


}  // namespace dflash

// HK2: per-head RMSNorm, RoPE, query packing and KV-cache append.
//
// Grid: one column per (sequence b, KV head j); along y, first the value
// tiles (dispatched first: they take longest), then slices of 16 (d=128) or
// 32 (d=64) key/query rows. For its pair the column
//   * takes the new key rows of the window [context (n_b rows) | block (bs)]
//     from the fp32 projections (summing the GEMM's k slices), RMS-normalises each over head_dim with the
//     k_norm gain, rotates it at its own window position and stores it as
//     cache K row L_b + r ("DFlash源码导读（二）" sections 1-4: k_norm before
//     RoPE, keys over the whole window, cache update);
//   * normalises (q_norm) and rotates the g = nq/nkv query heads of KV head j
//     for every block token i at the window's suffix position n_b + i (NeMo
//     page "draft_qwen3", apply_rotary_pos_emb), scales them by
//     head_dim^-0.5 * log2(e) so that attention scores come out in the log2
//     domain, and packs them as rows i*g + hh of the pair's query tile;
//   * stores the raw value rows transposed into cache V (column L_b + r), via
//     an LDS tile so that global writes run along the key axis.
// A work-group issues the loads of all its rows before using any (inputs and
// positions, then the cos/sin rows those positions select), so each costs two
// memory round trips whatever the row count.
// The same kernel appends the new context rows of every draft layer for the
// multi-layer context precompute (vLLM page "qwen3_dflash",
// precompute_and_store_context_kv: grouped k_norm, RoPE at the context
// positions, per-layer cache insert): then bs = 0 (no block rows, no queries)
// and grid.z runs over the layers, layer z taking its own columns of the
// all-layer projection, its own k_norm gain and its own cache.
// RoPE is neox style (vLLM page "qwen3_dflash": is_neox_style): element t of
// the first half pairs with element t + d/2. One lane owns one such pair, so a
// head is d/2 lanes and the rotation needs no data exchange; the RMS reduction
// is a butterfly over those lanes.
#include "kernels.h"

namespace dflash {

namespace {

template <int D>
__device__ inline float head_sum(float v) {
#pragma unroll
  for (int m = D / 4; m >= 1; m >>= 1) v += shfl_xor(v, m);
  return v;
}

// Row slots per wave: a key/query work-group takes 4 * kNormSlots * (128 / D)
// rows, all of whose loads go out before any is used.
constexpr int kNormSlots = 4;
// k slices the host splits a small-M projection into (at most): their loads
// are all issued before the first add.
constexpr int kSliceLoads = 4;

// x = sum over the k slices of rows src[r][t] and src[r][t + half] (slice sl
// at sl * stride[r]): every load of the first SL slices goes out before any
// add, then the slices are added in order (the rounding of a running sum);
// slices past SL are added one at a time afterwards. The host launches
// SL = kSliceLoads for split projections (few rows: the loads' latency
// matters) and SL = 1 otherwise, whose registers leave room for twice the
// waves (104 against 200 VGPRs at d = 128).
template <int N, int SL>
__device__ inline void sum_slices(const float* const (&src)[N], const int64_t (&stride)[N], int kslices, int t,
                                  int half, float (&x1)[N], float (&x2)[N]) {
  float l1[SL][N], l2[SL][N];
#pragma unroll
  for (int sl = 0; sl < SL; ++sl)
    if (sl < kslices) {
#pragma unroll
      for (int r = 0; r < N; ++r) {
        l1[sl][r] = src[r][sl * stride[r] + t];
        l2[sl][r] = src[r][sl * stride[r] + t + half];
      }
    }
#pragma unroll
  for (int r = 0; r < N; ++r) {
    x1[r] = l1[0][r];
    x2[r] = l2[0][r];
  }
#pragma unroll
  for (int sl = 1; sl < SL; ++sl)
    if (sl < kslices) {
#pragma unroll
      for (int r = 0; r < N; ++r) {
        x1[r] += l1[sl][r];
        x2[r] += l2[sl][r];
      }
    }
  for (int sl = SL; sl < kslices; ++sl)
#pragma unroll
    for (int r = 0; r < N; ++r) {
      x1[r] += src[r][sl * stride[r] + t];
      x2[r] += src[r][sl * stride[r] + t + half];
    }
}

template <typename T, int D, int SL>
__global__ __launch_bounds__(256) void norm_rope_append_kernel(NormRopeArgs a, int yv) {
  constexpr int HALF = D / 2;            // lanes per row
  constexpr int RPW = 64 / HALF;         // rows per wave slot
  constexpr int SLOTS = kNormSlots;
  constexpr int WG_ROWS = 4 * SLOTS * RPW;
  constexpr int VT = 64;                 // value rows per transpose tile
  __shared__ T vt[D][VT + 2];            // values in the cache type (padding spreads banks)

  const int nkv = a.nkv, nq = a.nq, bs = a.bs, g = nq / nkv;
  const int b = blockIdx.x / nkv, j = blockIdx.x % nkv;
  const int L = a.seq.len[b], c0 = a.seq.ctx_off[b], n = a.seq.ctx_off[b + 1] - c0;
  const int nnew = n + bs, pos_off = c0 + b * bs;
  const int R = bs * g;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = lane / HALF, t = lane % HALF;
  const size_t ld_blk = (size_t)(nq + 2 * nkv) * D, ld_ctx = (size_t)a.ctx_ld;
  // Layer z of a multi-layer context precompute (z = 0 for a layer step).
  const int z = blockIdx.z;
  const float* ctxkv = a.ctxkv + (size_t)z * a.ctx_layer_off;
  const CacheMap map = a.map_of(z);
  const size_t pair = (size_t)b * nkv + j;

  if ((int)blockIdx.y >= yv) {
    // Rows of this work-group: jobs [0, nnew) are key rows (context then
    // block), [nnew, nnew + R) are query rows (i, hh) = divmod(job - nnew, g).
    const int yk = (int)blockIdx.y - yv;
    const int base = yk * WG_ROWS + wave * SLOTS * RPW + sub;
    if (yk * WG_ROWS >= nnew + R) return;
    float x1[SLOTS], x2[SLOTS];
    int pidx[SLOTS], kind[SLOTS];  // kind: 0 none, 1 key, 2 query
    const float* src[SLOTS];
    int64_t stride[SLOTS];
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) {
      const int r = base + s * RPW;
      src[s] = a.qkv;  // any valid address for idle slots
      stride[s] = a.qkv_slice;
      kind[s] = 0;
      pidx[s] = pos_off;
      if (r < nnew) {
        kind[s] = 1;
        if (r < n) {
          src[s] = ctxkv + (size_t)(c0 + r) * ld_ctx + (size_t)j * D;
          stride[s] = a.ctx_slice;
        } else {
          src[s] = a.qkv + (size_t)(b * bs + r - n) * ld_blk + (size_t)(nq + j) * D;
        }
        pidx[s] = pos_off + r;
      } else if (r - nnew < R) {
        kind[s] = 2;
        const int i = (r - nnew) / g, hh = (r - nnew) % g;
        src[s] = a.qkv + (size_t)(b * bs + i) * ld_blk + (size_t)(j * g + hh) * D;
        pidx[s] = pos_off + n + i;  // queries sit at the window's suffix
      }
    }
    // The positions, then every k slice of every slot, all in flight together
    // (the cos/sin rows wait only for the positions).
    int p[SLOTS];
#pragma unroll
    for (int s = 0; s < SLOTS; ++s)
      // no position array: contiguous positions from the cached length
      p[s] = a.positions ? a.positions[pidx[s]] : L + (pidx[s] - pos_off);
    sum_slices<SLOTS, SL>(src, stride, a.kslices, t, HALF, x1, x2);
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) {
      if (p[s] < 0 || p[s] >= a.max_pos) {
        if (kind[s] != 0 && t == 0) atomicOr(a.err, 1);
        p[s] = p[s] < 0 ? 0 : a.max_pos - 1;
      }
    }
    const T* kn = static_cast<const T*>(a.k_norm) + (size_t)z * D;
    const T* qn = static_cast<const T*>(a.q_norm);
    const float kg1 = Elem<T>::to_f32(kn[t]), kg2 = Elem<T>::to_f32(kn[t + HALF]);
    const float qg1 = Elem<T>::to_f32(qn[t]), qg2 = Elem<T>::to_f32(qn[t + HALF]);
    const float* cos_t = a.cos_sin;
    const float* sin_t = a.cos_sin + (size_t)a.max_pos * HALF;
    float cs[SLOTS], sn[SLOTS];
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) {
      cs[s] = cos_t[(size_t)p[s] * HALF + t];
      sn[s] = sin_t[(size_t)p[s] * HALF + t];
    }
    T* kbase = static_cast<T*>(z == 0 ? a.kc : a.layer_kc[z]);
    T* qdst = static_cast<T*>(a.qpack) + pair * R * D;
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) {
      // RMSNorm over the head (all lanes of the row take part), then rotate.
      const float ss = head_sum<D>(x1[s] * x1[s] + x2[s] * x2[s]);
      const bool key = kind[s] == 1;
      const float scale = key ? 1.0f : a.qscale;
      const float inv = rsqrtf(ss * (1.0f / D) + a.eps) * scale;
      const float y1 = x1[s] * inv * (key ? kg1 : qg1), y2 = x2[s] * inv * (key ? kg2 : qg2);
      const float o1 = y1 * cs[s] - y2 * sn[s];
      const float o2 = y2 * cs[s] + y1 * sn[s];
      const int r = base + s * RPW;
      T* dst = key ? kbase + map.k_row(b, j, L + r, D) : qdst + (size_t)(r - nnew) * D;
      if (kind[s] != 0) {
        dst[t] = Elem<T>::from_f32(o1);
        dst[t + HALF] = Elem<T>::from_f32(o2);
      }
    }
    return;
  }

  // Values: raw rows of one 64-row tile, written transposed (key index
  // contiguous) through LDS.
  const int r0 = (int)blockIdx.y * VT;
  if (r0 >= nnew) return;
  const int nr = nnew - r0 < VT ? nnew - r0 : VT;
  // Each wave takes rows wave*RPW + sub + k*4*RPW; all of a lane's loads go
  // out before the first LDS write.
  constexpr int VROWS = VT / (4 * RPW);
  const float* vsrc[VROWS];
  int64_t vstride[VROWS];
  float v1[VROWS], v2[VROWS];
#pragma unroll
  for (int k = 0; k < VROWS; ++k) {
    const int rb = wave * RPW + sub + k * 4 * RPW, rr = r0 + rb;
    vsrc[k] = a.qkv;  // any valid address for rows past the tile
    vstride[k] = a.qkv_slice;
    if (rb < nr) {
      if (rr < n) {
        vsrc[k] = ctxkv + (size_t)(c0 + rr) * ld_ctx + (size_t)(nkv + j) * D;
        vstride[k] = a.ctx_slice;
      } else {
        vsrc[k] = a.qkv + (size_t)(b * bs + rr - n) * ld_blk + (size_t)(nq + nkv + j) * D;
      }
    }
  }
  sum_slices<VROWS, SL>(vsrc, vstride, a.kslices, t, HALF, v1, v2);
#pragma unroll
  for (int k = 0; k < VROWS; ++k) {
    const int rb = wave * RPW + sub + k * 4 * RPW;
    if (rb < nr) {
      vt[t][rb] = Elem<T>::from_f32(v1[k]);
      vt[t + HALF][rb] = Elem<T>::from_f32(v2[k]);
    }
  }
  // Where each row's column starts (a paged cache maps rows to blocks).
  __shared__ size_t vcol[VT];
  if (tid < nr) vcol[tid] = map.v_col(b, j, L + r0 + tid, D);
  __syncthreads();
  T* vbase = static_cast<T*>(z == 0 ? a.vc : a.layer_vc[z]);
  const size_t vs = (size_t)CacheMap::vstride();
  for (int idx = tid; idx < D * nr; idx += 256) {
    const int dd = idx / nr, rr = idx % nr;
    vbase[vcol[rr] + (size_t)dd * vs] = vt[dd][rr];
  }
}

template <typename T, int D>
void launch_nr(const NormRopeArgs& args, int yv, dim3 g, dim3 blk, hipStream_t stream) {
  if (args.kslices > 1)
    hipLaunchKernelGGL((norm_rope_append_kernel<T, D, kSliceLoads>), g, blk, 0, stream, args, yv);
  else
    hipLaunchKernelGGL((norm_rope_append_kernel<T, D, 1>), g, blk, 0, stream, args, yv);
}

}  // namespace

hipError_t launch_norm_rope(int dtype, int head_dim, const NormRopeArgs& args, int grid,
                            int max_new_rows, int layers, hipStream_t stream) {
  if (grid <= 0 || layers <= 0) return hipSuccess;
  const int wg_rows = 4 * kNormSlots * (128 / head_dim);
  const int R = args.bs * (args.nq / args.nkv);
  const int yk = (max_new_rows + R + wg_rows - 1) / wg_rows;
  const int yv = (max_new_rows + 63) / 64;
  const dim3 g(grid, yv + yk, layers), blk(256);
  if (dtype == 1) {
    if (head_dim == 128)
      launch_nr<__bf16, 128>(args, yv, g, blk, stream);
    else
      launch_nr<__bf16, 64>(args, yv, g, blk, stream);
  } else {
    if (head_dim == 128)
      launch_nr<float, 128>(args, yv, g, blk, stream);
    else
      launch_nr<float, 64>(args, yv, g, blk, stream);
  }
  return hipGetLastError();
}

}  // namespace dflash

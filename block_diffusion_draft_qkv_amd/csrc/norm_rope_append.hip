// HK2: per-head RMSNorm, RoPE, query packing and KV-cache append.
//
// One work-group per (sequence b, KV head j). For that pair it
//   * takes the new key rows of the window [context (n_b rows) | block (bs)]
//     from the fp32 projections, RMS-normalises each over head_dim with the
//     k_norm gain, rotates it at its own window position and stores it as
//     cache K row L_b + r ("DFlash源码导读（二）" sections 1-4: k_norm before
//     RoPE, keys over the whole window, cache update);
//   * stores the raw value rows transposed into cache V (column L_b + r), via
//     an LDS tile so that global writes run along the key axis, and zeroes V
//     columns T_b .. (T_b rounded up to 64) - 1;
//   * normalises (q_norm) and rotates the g = nq/nkv query heads of KV head j
//     for every block token i at the window's suffix position n_b + i (NeMo
//     page "draft_qwen3", apply_rotary_pos_emb), scales them by
//     head_dim^-0.5 * log2(e) so that attention scores come out in the log2
//     domain, and packs them as rows i*g + hh of the pair's query tile.
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

template <typename T, int D>
__global__ __launch_bounds__(256) void norm_rope_append_kernel(NormRopeArgs a) {
  constexpr int HALF = D / 2;      // lanes per row
  constexpr int RPW = 64 / HALF;   // rows per wave pass
  constexpr int SLOTS = 4 * RPW;   // rows per work-group pass
  constexpr int VT = 64;           // value rows per transpose tile
  __shared__ float vt[D][VT + 1];

  const int nkv = a.nkv, nq = a.nq, bs = a.bs, g = nq / nkv;
  const int b = blockIdx.x / nkv, j = blockIdx.x % nkv;
  const int L = a.seq.len[b], c0 = a.seq.ctx_off[b], n = a.seq.ctx_off[b + 1] - c0;
  const int nnew = n + bs, pos_off = c0 + b * bs;
  const int R = bs * g;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = lane / HALF, t = lane % HALF;
  const int slot = wave * RPW + sub;
  const size_t ld_blk = (size_t)(nq + 2 * nkv) * D, ld_ctx = (size_t)2 * nkv * D;
  const size_t pair = (size_t)b * nkv + j;

  const T* kn = static_cast<const T*>(a.k_norm);
  const T* qn = static_cast<const T*>(a.q_norm);
  const float kg1 = Elem<T>::to_f32(kn[t]), kg2 = Elem<T>::to_f32(kn[t + HALF]);
  const float qg1 = Elem<T>::to_f32(qn[t]), qg2 = Elem<T>::to_f32(qn[t + HALF]);
  const float* cos_t = a.cos_sin;
  const float* sin_t = a.cos_sin + (size_t)a.max_pos * HALF;

  auto position = [&](int idx) {
    int p = a.positions[idx];
    if (p < 0 || p >= a.max_pos) {
      if (t == 0) atomicOr(a.err, 1);
      p = p < 0 ? 0 : a.max_pos - 1;
    }
    return p;
  };
  // RMSNorm over the head (all lanes of the row take part), then rotate.
  auto norm_rope = [&](float x1, float x2, float g1, float g2, int p, float scale, float& o1,
                       float& o2) {
    const float ss = head_sum<D>(x1 * x1 + x2 * x2);
    const float inv = rsqrtf(ss * (1.0f / D) + a.eps) * scale;
    const float y1 = x1 * inv * g1, y2 = x2 * inv * g2;
    const float c = cos_t[(size_t)p * HALF + t], s = sin_t[(size_t)p * HALF + t];
    o1 = y1 * c - y2 * s;
    o2 = y2 * c + y1 * s;
  };

  // Keys: context rows then block rows, appended at L_b.
  T* kdst = static_cast<T*>(a.kc) + (pair * a.cap + L) * D;
  for (int rb = 0; rb < nnew; rb += SLOTS) {
    const int r = rb + slot;
    const bool ok = r < nnew;
    const int rr = ok ? r : nnew - 1;
    const float* src = rr < n ? a.ctxkv + (size_t)(c0 + rr) * ld_ctx + (size_t)j * D
                              : a.qkv + (size_t)(b * bs + rr - n) * ld_blk + (size_t)(nq + j) * D;
    const int p = position(pos_off + rr);
    float o1, o2;
    norm_rope(src[t], src[t + HALF], kg1, kg2, p, 1.0f, o1, o2);
    if (ok) {
      kdst[(size_t)r * D + t] = Elem<T>::from_f32(o1);
      kdst[(size_t)r * D + t + HALF] = Elem<T>::from_f32(o2);
    }
  }

  // Queries of the block at the suffix positions.
  T* qdst = static_cast<T*>(a.qpack) + pair * R * D;
  for (int rb = 0; rb < R; rb += SLOTS) {
    const int r = rb + slot;
    const bool ok = r < R;
    const int rr = ok ? r : R - 1;
    const int i = rr / g, hh = rr % g;
    const float* src = a.qkv + (size_t)(b * bs + i) * ld_blk + (size_t)(j * g + hh) * D;
    const int p = position(pos_off + n + i);
    float o1, o2;
    norm_rope(src[t], src[t + HALF], qg1, qg2, p, a.qscale, o1, o2);
    if (ok) {
      qdst[(size_t)r * D + t] = Elem<T>::from_f32(o1);
      qdst[(size_t)r * D + t + HALF] = Elem<T>::from_f32(o2);
    }
  }

  // Values: raw rows, written transposed (key index contiguous).
  T* vdst = static_cast<T*>(a.vc) + pair * D * a.cap + L;
  for (int r0 = 0; r0 < nnew; r0 += VT) {
    const int nr = nnew - r0 < VT ? nnew - r0 : VT;
    for (int rb = 0; rb < nr; rb += SLOTS) {
      const int r = rb + slot;
      if (r < nr) {
        const int rr = r0 + r;
        const float* src = rr < n ? a.ctxkv + (size_t)(c0 + rr) * ld_ctx + (size_t)(nkv + j) * D
                                  : a.qkv + (size_t)(b * bs + rr - n) * ld_blk + (size_t)(nq + nkv + j) * D;
        vt[t][r] = src[t];
        vt[t + HALF][r] = src[t + HALF];
      }
    }
    __syncthreads();
    for (int idx = tid; idx < D * nr; idx += 256) {
      const int dd = idx / nr, rr = idx % nr;
      vdst[(size_t)dd * a.cap + r0 + rr] = Elem<T>::from_f32(vt[dd][rr]);
    }
    __syncthreads();
  }

  // Zero V from T_b to the end of its 64-key tile: the attention kernel reads
  // whole tiles and needs finite values past T_b (they meet zero weights).
  T* vpad = static_cast<T*>(a.vc) + pair * D * a.cap;
  const int Tb = L + nnew;
  const int pad = (Tb + 63) / 64 * 64 - Tb;
  for (int idx = tid; idx < D * pad; idx += 256) {
    const int dd = idx / pad, k = idx % pad;
    vpad[(size_t)dd * a.cap + Tb + k] = Elem<T>::from_f32(0.f);
  }
}

}  // namespace

hipError_t launch_norm_rope(int dtype, int head_dim, const NormRopeArgs& args, int grid,
                            hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  const dim3 g(grid), blk(256);
  if (dtype == 1) {
    if (head_dim == 128)
      hipLaunchKernelGGL((norm_rope_append_kernel<__bf16, 128>), g, blk, 0, stream, args);
    else
      hipLaunchKernelGGL((norm_rope_append_kernel<__bf16, 64>), g, blk, 0, stream, args);
  } else {
    if (head_dim == 128)
      hipLaunchKernelGGL((norm_rope_append_kernel<float, 128>), g, blk, 0, stream, args);
    else
      hipLaunchKernelGGL((norm_rope_append_kernel<float, 64>), g, blk, 0, stream, args);
  }
  return hipGetLastError();
}

}  // namespace dflash

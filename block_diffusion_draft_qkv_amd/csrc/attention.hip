// HK3: split-KV non-causal grouped-query attention of the draft block over the
// draft KV cache, and HK4: log-sum-exp merge of split partials.
//
// What is computed (NeMo page "draft_qwen3": Qwen3DFlashAttention, scaling,
// _sliding_window_mask; "DFlash源码导读（二）" section on non-causal block
// attention): for sequence b with T_b keys and query head h of KV head
// j = h / g, o = softmax_t(d^-1/2 <q, k_t>) over every cached key t (the block
// included, no causal mask), restricted under a window W to
// |(T_b - bs + i) - t| < W; then o . V.
//
// Layout of the work. The bs*g query rows that share KV head j (row i*g + hh)
// form one tile of up to 64 rows; wave w of the 256-thread work-group owns rows
// 16w .. 16w+15. Keys stream in tiles of 64 through LDS, double-buffered, the
// next tile's global loads in flight while the current one is used:
//   S^T (keys x queries) = K . Q^T     on MFMA, K from LDS, Q held in VGPRs
//   online softmax in the log2 domain  (Q was pre-scaled by d^-1/2 log2 e)
//   O^T (d x queries)   += V^T . P^T   on MFMA, V^T from LDS, P^T from VGPRs
// The S^T accumulator gives every lane one query column and 4 keys per 16-key
// block, which is exactly the P^T operand layout the second product needs, so P
// never leaves registers; V is stored transposed in the cache so V^T tiles are
// plain row reads. For bf16 the key order inside a 32-key step is permuted
// (block 2s row 4q+r <-> key 8q+r, block 2s+1 row 4q+r <-> key 8q+4+r) so a
// lane's 8 P values are 8 consecutive keys, i.e. one 16-byte chunk of V^T.
//
// Split-KV: all (b, j, 64-key tile) items are flattened (b-major) and cut into
// G equal ranges, one per work-group, so every work-group streams the same
// number of key tiles whatever the ragged lengths. A work-group writes a pair
// that lies wholly inside its range straight to the output; a pair cut by a
// range boundary leaves fp32 partials (un-normalised O, running max, sum) in
// slot 2w (the range's first segment) or 2w+1 (its last), which HK4 merges.
#include "kernels.h"

namespace dflash {

namespace {

constexpr float kNegInf = -__builtin_inff();

// Sequence geometry shared by both kernels: per sequence, the first key tile
// and the tile count; an exclusive prefix of the counts.
struct SeqGeom {
  int32_t lo[kMaxBatch];
  int32_t cnt[kMaxBatch];
  int64_t pre[kMaxBatch + 1];
};

__device__ inline void build_geom(const AttnArgs& a, SeqGeom& sg) {
  const int B = a.seq.batch, tid = threadIdx.x;
  for (int b = tid; b < kMaxBatch; b += blockDim.x) {
    int lo = 0, cnt = 0;
    if (b < B) {
      const int T = a.seq.len[b] + (a.seq.ctx_off[b + 1] - a.seq.ctx_off[b]) + a.bs;
      int first = 0;
      if (a.window > 0) {
        first = T - a.bs - a.window + 1;
        if (first < 0) first = 0;
      }
      lo = first / kKeyTile;
      cnt = (T + kKeyTile - 1) / kKeyTile - lo;
    }
    sg.lo[b] = lo;
    sg.cnt[b] = cnt;
    sg.pre[b + 1] = cnt;
  }
  if (tid == 0) sg.pre[0] = 0;
  __syncthreads();
  // inclusive scan of pre[1..kMaxBatch] (Hillis-Steele)
  for (int off = 1; off < kMaxBatch; off <<= 1) {
    int64_t v = 0;
    for (int b = tid; b < kMaxBatch; b += blockDim.x) {
      if (b >= off) v = sg.pre[b + 1 - off];
    }
    __syncthreads();
    for (int b = tid; b < kMaxBatch; b += blockDim.x) {
      if (b >= off) sg.pre[b + 1] += v;
    }
    __syncthreads();
  }
}

__device__ inline int64_t bound_of(int64_t w, int64_t n, int64_t g) { return (w * n) / g; }
__device__ inline int64_t owner_of(int64_t f, int64_t n, int64_t g) { return ((f + 1) * g + n - 1) / n - 1; }

// Which key each lane's S^T accumulator row stands for (see the file comment).
template <typename T> __device__ inline int key_of(int kb, int m);
template <> __device__ inline int key_of<__bf16>(int kb, int m) {
  return 32 * (kb >> 1) + 8 * (m >> 2) + 4 * (kb & 1) + (m & 3);
}
template <> __device__ inline int key_of<float>(int kb, int m) { return 16 * kb + m; }

// LDS chunk swizzle of a K tile row: keeps the 8 rows read by one ds_read_b128
// phase on 8 distinct chunks.
template <typename T> __device__ inline int kswz(int row);
template <> __device__ inline int kswz<__bf16>(int row) { return (row & 3) | ((row >> 1) & 4); }
template <> __device__ inline int kswz<float>(int row) { return row & 7; }

// Zero the elements of a 16-byte chunk whose key index (first + e) is >= end.
template <typename T> __device__ inline u32x4 mask_tail(u32x4 v, int first, int end);
template <> __device__ inline u32x4 mask_tail<float>(u32x4 v, int first, int end) {
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (first + e >= end) v[e] = 0u;
  return v;
}
template <> __device__ inline u32x4 mask_tail<__bf16>(u32x4 v, int first, int end) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t keep = 0u;
    if (first + 2 * w < end) keep |= 0x0000FFFFu;
    if (first + 2 * w + 1 < end) keep |= 0xFFFF0000u;
    v[w] &= keep;
  }
  return v;
}

template <typename T> __device__ inline u32x4 pack_p(const float* p0, const float* p1);
template <> __device__ inline u32x4 pack_p<__bf16>(const float* p0, const float* p1) {
  bf16x8 v;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    v[r] = (__bf16)p0[r];
    v[4 + r] = (__bf16)p1[r];
  }
  return __builtin_bit_cast(u32x4, v);
}

template <typename T, int D>
__global__ __launch_bounds__(256, 2) void attn_splitkv_kernel(AttnArgs a) {
  constexpr int E = Elem<T>::kPerChunk;
  constexpr int CPR = D * (int)sizeof(T) / 16;         // chunks per K row
  constexpr int VCPR = kKeyTile * (int)sizeof(T) / 16; // chunks per V^T row
  constexpr int NC = CPR / 4;                          // reduction blocks over d
  constexpr int K_CH = kKeyTile * CPR, V_CH = D * VCPR;
  constexpr int KPT = K_CH / 256, VPT = V_CH / 256;
  constexpr int DB = D / 16;
  static_assert(K_CH % 256 == 0 && V_CH % 256 == 0, "tile must split over 256 threads");
  __shared__ u32x4 lds[2][K_CH + V_CH];
  __shared__ SeqGeom sg;

  build_geom(a, sg);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = lane >> 4, r16 = lane & 15;
  const int nkv = a.nkv, g = a.nq / nkv, R = a.R;
  const int64_t N = a.total_tiles, G = a.G, w = blockIdx.x;
  const int64_t f0 = bound_of(w, N, G), f1 = bound_of(w + 1, N, G);
  const bool active = wave * 16 < R;
  const int qrow = wave * 16 + r16;
  const bool qvalid = qrow < R;
  const T* __restrict__ Qp = static_cast<const T*>(a.q);
  const T* __restrict__ Kc = static_cast<const T*>(a.kc);
  const T* __restrict__ Vc = static_cast<const T*>(a.vc);

  int64_t f = f0;
  bool first_seg = true;
  while (f < f1) {
    // locate the pair holding flat tile f
    int lo = 0, hi = a.seq.batch;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if ((int64_t)nkv * sg.pre[mid] <= f) lo = mid; else hi = mid;
    }
    const int b = lo;
    const int cnt = sg.cnt[b];
    const int64_t base_b = (int64_t)nkv * sg.pre[b];
    const int j = (int)((f - base_b) / cnt);
    const int tin = (int)((f - base_b) % cnt);
    const int64_t pair_end = base_b + (int64_t)(j + 1) * cnt;
    const int64_t seg_end = f1 < pair_end ? f1 : pair_end;
    const int ntiles = (int)(seg_end - f);
    const bool full = tin == 0 && seg_end == pair_end;
    const int slot = 2 * (int)w + (first_seg ? 0 : 1);
    const int tile0 = sg.lo[b] + tin;

    const int Tb = a.seq.len[b] + (a.seq.ctx_off[b + 1] - a.seq.ctx_off[b]) + a.bs;
    const size_t pair = (size_t)b * nkv + j;
    const T* Kpair = Kc + pair * (size_t)a.cap * D;
    const T* Vpair = Vc + pair * (size_t)D * a.cap;
    const int qpos = Tb - a.bs + (qvalid ? qrow / g : 0);

    u32x4 qf[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c)
      qf[c] = qvalid ? ldg16(Qp + (pair * R + qrow) * D + (size_t)(4 * c + q) * E) : u32x4{0, 0, 0, 0};

    float m_run = kNegInf, l_run = 0.f;
    f32x4 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x4 rk[KPT], rv[VPT];
    auto load_regs = [&](int tile) {
      const int t0 = tile * kKeyTile;
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const int id = tid + 256 * i, row = id / CPR, c = id % CPR;
        rk[i] = ldg16(Kpair + (size_t)(t0 + row) * D + c * E);
      }
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        const int id = tid + 256 * i, row = id / VCPR, c = id % VCPR;
        rv[i] = ldg16(Vpair + (size_t)row * a.cap + t0 + c * E);
      }
    };
    auto store_lds = [&](int buf, int tile) {
      const int t0 = tile * kKeyTile;
      const bool tail = t0 + kKeyTile > Tb;
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const int id = tid + 256 * i, row = id / CPR, c = id % CPR;
        lds[buf][row * CPR + (c ^ kswz<T>(row))] = rk[i];
      }
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        const int id = tid + 256 * i, row = id / VCPR, c = id % VCPR;
        const u32x4 v = tail ? mask_tail<T>(rv[i], t0 + c * E, Tb) : rv[i];
        lds[buf][K_CH + row * VCPR + (c ^ (row & 7))] = v;
      }
    };
    auto compute = [&](int buf, int tile) {
      const int t0 = tile * kKeyTile;
      f32x4 s[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int krow = key_of<T>(kb, r16);
#pragma unroll
        for (int c = 0; c < NC; ++c)
          Mfma<T>::chunk(s[kb], lds[buf][krow * CPR + ((4 * c + q) ^ kswz<T>(krow))], qf[c]);
      }
      if (t0 + kKeyTile > Tb || a.window > 0) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = t0 + key_of<T>(kb, 4 * q + r);
            bool ok = key < Tb;
            if (a.window > 0) {
              const int dlt = qpos - key;
              ok = ok && (dlt < a.window) && (-dlt < a.window);
            }
            if (!ok) s[kb][r] = kNegInf;
          }
      }
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = fmaxf(mx, shfl_xor(mx, 16));
      mx = fmaxf(mx, shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float m_use = m_new == kNegInf ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      m_run = m_new;
      float p[4][4];
      float psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          p[kb][r] = __builtin_amdgcn_exp2f(s[kb][r] - m_use);
          psum += p[kb][r];
        }
      l_run = l_run * alpha + psum;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] *= alpha;
      if constexpr (sizeof(T) == 2) {
        u32x4 pf[2];
        pf[0] = pack_p<T>(p[0], p[1]);
        pf[1] = pack_p<T>(p[2], p[3]);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int vrow = db * 16 + r16;
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
            Mfma<T>::chunk(acc[db], lds[buf][K_CH + vrow * VCPR + ((4 * ks + q) ^ (vrow & 7))], pf[ks]);
        }
      } else {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int vrow = db * 16 + r16;
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            const u32x4 pb = u32x4{__float_as_uint(p[kb][0]), __float_as_uint(p[kb][1]),
                                   __float_as_uint(p[kb][2]), __float_as_uint(p[kb][3])};
            Mfma<T>::chunk(acc[db], lds[buf][K_CH + vrow * VCPR + ((4 * kb + q) ^ (vrow & 7))], pb);
          }
        }
      }
    };

    load_regs(tile0);
    store_lds(0, tile0);
    __syncthreads();
    for (int it = 0; it < ntiles; ++it) {
      const int cur = it & 1;
      const bool more = it + 1 < ntiles;
      if (more) load_regs(tile0 + it + 1);
      if (active) compute(cur, tile0 + it);
      if (more) store_lds(cur ^ 1, tile0 + it + 1);
      __syncthreads();
    }

    if (active) {
      float lt = l_run + shfl_xor(l_run, 16);
      lt += shfl_xor(lt, 32);
      if (qvalid) {
        if (full) {
          const float inv = 1.0f / lt;
          const int i = qrow / g, hh = qrow % g;
          T* orow = static_cast<T*>(a.o) + ((size_t)(b * a.bs + i) * a.nq + (size_t)(j * g + hh)) * D;
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r) orow[db * 16 + 4 * q + r] = Elem<T>::from_f32(acc[db][r] * inv);
        } else {
          float* po = a.part_o + ((size_t)slot * kMaxQueryRows + qrow) * D;
#pragma unroll
          for (int db = 0; db < DB; ++db) *reinterpret_cast<f32x4*>(po + db * 16 + 4 * q) = acc[db];
          if (q == 0) {
            float* pm = a.part_ml + ((size_t)slot * kMaxQueryRows + qrow) * 2;
            pm[0] = m_run;
            pm[1] = lt;
          }
        }
      }
    }
    f = seg_end;
    first_seg = false;
  }
}

// HK4: one work-group per (pair, group of rows). Pairs processed whole by one
// work-group return at once.
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a, int rows_per_group) {
  __shared__ SeqGeom sg;
  build_geom(a, sg);
  const int nkv = a.nkv, g = a.nq / nkv;
  const int b = blockIdx.x / nkv, j = blockIdx.x % nkv;
  const int64_t N = a.total_tiles, G = a.G;
  const int cnt = sg.cnt[b];
  const int64_t s_p = (int64_t)nkv * sg.pre[b] + (int64_t)j * cnt, e_p = s_p + cnt;
  const int64_t w_first = owner_of(s_p, N, G), w_last = owner_of(e_p - 1, N, G);
  if (w_first == w_last) return;

  constexpr int TPR = D / 4;  // threads per row, 4 values each
  const int tid = threadIdx.x;
  const int row = blockIdx.y * rows_per_group + tid / TPR;
  const int d4 = (tid % TPR) * 4;
  if (tid / TPR >= rows_per_group || row >= a.R) return;

  auto slot_of = [&](int64_t wg) {
    return (int)(2 * wg + ((wg == w_first && s_p != bound_of(wg, N, G)) ? 1 : 0));
  };
  float M = kNegInf;
  for (int64_t wg = w_first; wg <= w_last; ++wg)
    M = fmaxf(M, a.part_ml[((size_t)slot_of(wg) * kMaxQueryRows + row) * 2]);
  float den = 0.f;
  f32x4 num = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int64_t wg = w_first; wg <= w_last; ++wg) {
    const size_t sr = (size_t)slot_of(wg) * kMaxQueryRows + row;
    const float wgt = __builtin_amdgcn_exp2f(a.part_ml[sr * 2] - M);
    den += wgt * a.part_ml[sr * 2 + 1];
    num += wgt * *reinterpret_cast<const f32x4*>(a.part_o + sr * D + d4);
  }
  const float inv = 1.0f / den;
  const int i = row / g, hh = row % g;
  T* orow = static_cast<T*>(a.o) + ((size_t)(b * a.bs + i) * a.nq + (size_t)(j * g + hh)) * D;
#pragma unroll
  for (int r = 0; r < 4; ++r) orow[d4 + r] = Elem<T>::from_f32(num[r] * inv);
}

}  // namespace

hipError_t launch_attn(int dtype, int head_dim, const AttnArgs& args, hipStream_t stream) {
  if (args.G <= 0) return hipSuccess;
  const dim3 grid(args.G), block(256);
  if (dtype == 1) {
    if (head_dim == 128)
      hipLaunchKernelGGL((attn_splitkv_kernel<__bf16, 128>), grid, block, 0, stream, args);
    else
      hipLaunchKernelGGL((attn_splitkv_kernel<__bf16, 64>), grid, block, 0, stream, args);
  } else {
    if (head_dim == 128)
      hipLaunchKernelGGL((attn_splitkv_kernel<float, 128>), grid, block, 0, stream, args);
    else
      hipLaunchKernelGGL((attn_splitkv_kernel<float, 64>), grid, block, 0, stream, args);
  }
  return hipGetLastError();
}

hipError_t launch_merge(int dtype, int head_dim, const AttnArgs& args, int merge_groups,
                        hipStream_t stream) {
  const int rows_per_group = 256 / (head_dim / 4);
  const dim3 grid(args.seq.batch * args.nkv, merge_groups), block(256);
  if (dtype == 1) {
    if (head_dim == 128)
      hipLaunchKernelGGL((attn_merge_kernel<__bf16, 128>), grid, block, 0, stream, args, rows_per_group);
    else
      hipLaunchKernelGGL((attn_merge_kernel<__bf16, 64>), grid, block, 0, stream, args, rows_per_group);
  } else {
    if (head_dim == 128)
      hipLaunchKernelGGL((attn_merge_kernel<float, 128>), grid, block, 0, stream, args, rows_per_group);
    else
      hipLaunchKernelGGL((attn_merge_kernel<float, 64>), grid, block, 0, stream, args, rows_per_group);
  }
  return hipGetLastError();
}

}  // namespace dflash

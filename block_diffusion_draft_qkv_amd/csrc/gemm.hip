// HK1: grouped projection GEMM on gfx950 matrix cores.
//
// C[m][n] = sum_k A[m][k] W[n][k], the nn.Linear product y = x W^T used by the
// layer's fused qkv_proj (block rows -> q|k|v, context rows -> k|v through the
// k/v rows of the same weight) and by o_proj (vLLM page "qwen3_dflash":
// DFlashQwen3Attention.__init__/forward; "DFlash源码导读（二）" section 2).
//
// One work-group computes a BM x BN tile: four consumer waves in 2 x 2, each
// (BM/2) x (BN/2) from 16x16 MFMA blocks, and two producer waves that only
// stream operand tiles of 64 bf16 (32 fp32) along k from HBM into an S-stage
// LDS ring (S = 4..8 stages) with the LDS-DMA load and wait
// for them, so a full load queue stalls only them. Consumers read each
// half-step of fragments while the MFMAs of the previous half-step run.
// Rows past m or n are fetched as a copy of the last valid row (in bounds,
// never stored). The MFMA
// computes C^T = W . A^T, which leaves four consecutive n of one m in each lane,
// so results store as 16-byte (fp32) or 8-byte (bf16) runs. An optional split
// of k over gridDim.y writes fp32 partial sums;
// their consumer adds the slices (slice s of a problem at C + s * slice_stride).
#include "kernels.h"
#include "lds_dma.h"

namespace dflash {

namespace {

template <typename OutT> struct Store4;
template <> struct Store4<float> {
  __device__ static inline void put(float* p, const f32x4& v) { *reinterpret_cast<f32x4*>(p) = v; }
};
template <> struct Store4<__bf16> {
  __device__ static inline void put(__bf16* p, const f32x4& v) {
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    bf16x4 o;
#pragma unroll
    for (int r = 0; r < 4; ++r) o[r] = (__bf16)v[r];
    *reinterpret_cast<bf16x4*>(p) = o;
  }
};

// Wave roles of the 384-thread work-group: waves 0-3 compute (2 x 2, each a
// (BM/2) x (BN/2) sub-tile), waves 4-5 only issue and await the LDS-DMA loads.
constexpr int kGemmConsumers = 4;
constexpr int kGemmProducers = 2;
constexpr int kGemmThreads = 64 * (kGemmConsumers + kGemmProducers);

template <int BM, int BN> struct GemmShape {
  static constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128, STAGE = A_BYTES + B_BYTES;
  static constexpr int APP = BM / 8 / kGemmProducers, BPP = BN / 8 / kGemmProducers;  // 1 KB blocks per producer
  static constexpr int PER = APP + BPP;
  // LDS ring stages: as many as fit in 160 KB, at most 8, and few enough that
  // a producer's outstanding blocks ((S - 1) * PER) fit the 6-bit vmcnt.
  static constexpr int S_LDS = (160 * 1024) / STAGE, S_VM = 1 + 63 / PER;
  static constexpr int S = S_LDS < S_VM ? (S_LDS < 8 ? S_LDS : 8) : (S_VM < 8 ? S_VM : 8);
  static constexpr int WM = BM / 2, WN = BN / 2;
  static constexpr int MI = WM / 16, NI = WN / 16;
  static_assert((S - 1) * PER <= 63, "outstanding DMA blocks must fit vmcnt");
};

// Wait until at most n of this wave's stages (of PER blocks each) are in flight.
template <int PER, int S> __device__ inline void stage_wait(int n) {
  if constexpr (S > 7) { if (n >= 6) { DFLASH_VMWAIT(6 * PER); return; } }
  if constexpr (S > 6) { if (n == 5) { DFLASH_VMWAIT(5 * PER); return; } }
  if constexpr (S > 5) { if (n == 4) { DFLASH_VMWAIT(4 * PER); return; } }
  if constexpr (S > 4) { if (n == 3) { DFLASH_VMWAIT(3 * PER); return; } }
  if constexpr (S > 3) { if (n == 2) { DFLASH_VMWAIT(2 * PER); return; } }
  if constexpr (S > 2) { if (n == 1) { DFLASH_VMWAIT(PER); return; } }
  DFLASH_VMWAIT(0);
}

template <typename T, typename OutT, int BM, int BN>
__global__ __launch_bounds__(kGemmThreads, 1) void gemm_kernel(GemmArgs args) {
  using Sh = GemmShape<BM, BN>;
  constexpr int S = Sh::S, STAGE = Sh::STAGE, A_BYTES = Sh::A_BYTES;
  constexpr int APP = Sh::APP, BPP = Sh::BPP, PER = Sh::PER;
  constexpr int WM = Sh::WM, WN = Sh::WN, MI = Sh::MI, NI = Sh::NI;
  __shared__ u32x4 lds[S * STAGE / 16];

  int tile = blockIdx.x;
  const bool second = args.nprob > 1 && tile >= args.p[1].tile_begin;
  const GemmProblem P = second ? args.p[1] : args.p[0];
  tile -= P.tile_begin;
  const int m0 = (tile / P.tiles_n) * BM;
  const int n0 = (tile % P.tiles_n) * BN;
  const int ksl = gridDim.y;                       // k slices
  const int nk_all = P.k / (8 * (16 / (int)sizeof(T)));  // 128-byte k steps
  const int k_first = (int)(((int64_t)nk_all * blockIdx.y) / ksl);
  const int nk = (int)(((int64_t)nk_all * (blockIdx.y + 1)) / ksl) - k_first;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t lds0 = lds_base(lds);

  // Step s lives in ring stage s % S. Barrier s is passed once stage s has
  // landed (the producers wait for it first) and the consumers have read every
  // fragment of step s - 1, whose stage the producers refill right after it.
  if (wave >= kGemmConsumers) {
    // ---------------------------------------------------------- producers
    const int pw = wave - kGemmConsumers;
    // Block i * kGemmProducers + pw of an operand covers 8 rows; each lane
    // fetches the chunk that belongs at its swizzled LDS position, from a
    // clamped row.
    uint32_t aoff[APP], boff[BPP];
#pragma unroll
    for (int i = 0; i < APP; ++i) {
      const int row = (i * kGemmProducers + pw) * 8 + lane / 8;
      const int c = (lane % 8) ^ rswz<8>(row);
      const int gr = m0 + row < P.m ? m0 + row : P.m - 1;
      aoff[i] = (uint32_t)((size_t)gr * P.lda * sizeof(T)) + (uint32_t)(c * 16);
    }
#pragma unroll
    for (int i = 0; i < BPP; ++i) {
      const int row = (i * kGemmProducers + pw) * 8 + lane / 8;
      const int c = (lane % 8) ^ rswz<8>(row);
      const int gr = n0 + row < P.n ? n0 + row : P.n - 1;
      boff[i] = (uint32_t)((size_t)gr * P.ldb * sizeof(T)) + (uint32_t)(c * 16);
    }
    const char* Ab = static_cast<const char*>(P.a);
    const char* Bb = static_cast<const char*>(P.b);
    auto issue = [&](int step) {
      const size_t kbyte = (size_t)(k_first + step) * 128;
      const uint32_t sl = lds0 + (uint32_t)(step % S) * STAGE;
      const void* ab = uniform_ptr(Ab + kbyte);
      const void* bb = uniform_ptr(Bb + kbyte);
#pragma unroll
      for (int i = 0; i < APP; ++i)
        lds_dma16(aoff[i], ab, sl + (uint32_t)(i * kGemmProducers + pw) * 1024u);
#pragma unroll
      for (int i = 0; i < BPP; ++i)
        lds_dma16(boff[i], bb, sl + A_BYTES + (uint32_t)(i * kGemmProducers + pw) * 1024u);
    };
#pragma unroll
    for (int s = 0; s < S - 1; ++s)
      if (s < nk) issue(s);
    for (int it = 0; it < nk; ++it) {
      // Stages issued after `it`: it+1 .. min(nk-1, it+S-2).
      const int after = nk - 1 - it < S - 2 ? nk - 1 - it : S - 2;
      stage_wait<PER, S>(after);
      block_barrier();
      if (it + S - 1 < nk) issue(it + S - 1);
    }
    return;
  }

  // ------------------------------------------------------------ consumers
  const int wm = wave >> 1, wn = wave & 1;
  const int q = lane >> 4, r16 = lane & 15;
  // LDS read offsets (lane part): operand rows wm*WM + mi*16 + r16 (A) and
  // wn*WN + ni*16 + r16 (W), logical chunk 4*kb + q.
  uint32_t ard[2], brd[2];
  {
    const int sw = rswz<8>(r16);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      ard[kb] = (uint32_t)((wm * WM + r16) * 8 + ((4 * kb + q) ^ sw)) * 16u;
      brd[kb] = (uint32_t)((wn * WN + r16) * 8 + ((4 * kb + q) ^ sw)) * 16u + A_BYTES;
    }
  }

  f32x4 acc[NI][MI];
#pragma unroll
  for (int ni = 0; ni < NI; ++ni)
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) acc[ni][mi] = f32x4{0.f, 0.f, 0.f, 0.f};

  // A step's 64 k split into halves kb = 0, 1. Right after barrier s the
  // consumer reads half 0 of step s while the products of half 1 of step s - 1
  // run, then reads half 1 of step s while the products of half 0 run, so the
  // LDS reads always overlap MFMAs; only two half-sets of fragments are live.
  // (The scheduling barriers keep the compiler from hoisting reads across
  // these phases.)
  struct Half {
    u32x4 a[MI], b[NI];
  };
  auto read = [&](Half& h, int step, int kb) {
    const uint32_t sl = lds0 + (uint32_t)(step % S) * STAGE;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) h.a[mi] = lds_read16(sl + ard[kb] + (uint32_t)(mi * 16 * 128));
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) h.b[ni] = lds_read16(sl + brd[kb] + (uint32_t)(ni * 16 * 128));
  };
  auto mma = [&](const Half& h) {
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) Mfma<T>::chunk(acc[ni][mi], h.b[ni], h.a[mi]);
  };
  Half h0, h1;
  for (int it = 0; it < nk; ++it) {
    block_barrier();
    read(h0, it, 0);
    __builtin_amdgcn_sched_barrier(0);
    if (it > 0) mma(h1);
    __builtin_amdgcn_sched_barrier(0);
    read(h1, it, 1);
    __builtin_amdgcn_sched_barrier(0);
    mma(h0);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (nk > 0) mma(h1);

  // acc[ni][mi]: lane holds m = r16 of block mi and n = 4q .. 4q+3 of block ni.
  OutT* C = static_cast<OutT*>(P.c) + (size_t)blockIdx.y * P.slice_stride;
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
    const int m = m0 + wm * WM + mi * 16 + r16;
    if (m >= P.m) continue;
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      const int n = n0 + wn * WN + ni * 16 + 4 * q;
      if (n < P.n) Store4<OutT>::put(C + (size_t)m * P.ldc + n, acc[ni][mi]);
    }
  }
}

template <typename T, typename OutT>
hipError_t launch_t(const GemmArgs& args, int total_tiles, int bm, int bn, int kslices, hipStream_t s) {
  const dim3 grid(total_tiles, kslices), block(kGemmThreads);
  if (bm == 128 && bn == 128)
    hipLaunchKernelGGL((gemm_kernel<T, OutT, 128, 128>), grid, block, 0, s, args);
  else if (bm == 128 && bn == 64)
    hipLaunchKernelGGL((gemm_kernel<T, OutT, 128, 64>), grid, block, 0, s, args);
  else if (bm == 64 && bn == 128)
    hipLaunchKernelGGL((gemm_kernel<T, OutT, 64, 128>), grid, block, 0, s, args);
  else
    hipLaunchKernelGGL((gemm_kernel<T, OutT, 64, 64>), grid, block, 0, s, args);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(int dtype, bool out_f32, const GemmArgs& args, int total_tiles, int bm, int bn,
                       int kslices, hipStream_t stream) {
  if (total_tiles <= 0) return hipSuccess;
  if (dtype == 1)
    return out_f32 ? launch_t<__bf16, float>(args, total_tiles, bm, bn, kslices, stream)
                   : launch_t<__bf16, __bf16>(args, total_tiles, bm, bn, kslices, stream);
  return launch_t<float, float>(args, total_tiles, bm, bn, kslices, stream);
}

}  // namespace dflash

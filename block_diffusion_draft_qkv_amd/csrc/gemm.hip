// HK1: grouped projection GEMM on gfx950 matrix cores.
//
// C[m][n] = sum_k A[m][k] W[n][k], the nn.Linear product y = x W^T used by the
// layer's fused qkv_proj (block rows -> q|k|v, context rows -> k|v through the
// k/v rows of the same weight) and by o_proj (vLLM page "qwen3_dflash":
// DFlashQwen3Attention.__init__/forward; "DFlash源码导读（二）" section 2).
//
// One 256-thread work-group computes a BM x BN tile (4 waves in 2 x 2, each
// (BM/2) x (BN/2) from 16x16 MFMA blocks). Operand tiles of 64 bf16 (32 fp32)
// along k stream from HBM into an S-stage LDS ring with the LDS-DMA load, so
// S-1 stages are in flight while one feeds the MFMAs; rows past m or n are
// fetched as a copy of the last valid row (in bounds, never stored). The MFMA
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

template <int BM, int BN> struct GemmShape {
  static constexpr int S = 3;                     // LDS ring stages
  static constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128, STAGE = A_BYTES + B_BYTES;
  static constexpr int APW = BM / 32, BPW = BN / 32;  // 1 KB DMA blocks per wave and stage
  static constexpr int WM = BM / 2, WN = BN / 2;
  static constexpr int MI = WM / 16, NI = WN / 16;
};

template <typename T, typename OutT, int BM, int BN>
__global__ __launch_bounds__(256, 1) void gemm_kernel(GemmArgs args) {
  using Sh = GemmShape<BM, BN>;
  constexpr int E = 16 / (int)sizeof(T);
  constexpr int S = Sh::S, STAGE = Sh::STAGE, A_BYTES = Sh::A_BYTES;
  constexpr int APW = Sh::APW, BPW = Sh::BPW, PER = APW + BPW;
  constexpr int WM = Sh::WM, WN = Sh::WN, MI = Sh::MI, NI = Sh::NI;
  __shared__ u32x4 lds[S * STAGE / 16];

  int tile = blockIdx.x;
  const bool second = args.nprob > 1 && tile >= args.p[1].tile_begin;
  const GemmProblem P = second ? args.p[1] : args.p[0];
  tile -= P.tile_begin;
  const int m0 = (tile / P.tiles_n) * BM;
  const int n0 = (tile % P.tiles_n) * BN;
  const int ksl = gridDim.y;                       // k slices
  const int nk_all = P.k / (8 * E);                // 128-byte k steps
  const int k_first = (int)(((int64_t)nk_all * blockIdx.y) / ksl);
  const int nk = (int)(((int64_t)nk_all * (blockIdx.y + 1)) / ksl) - k_first;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int wm = wave_u >> 1, wn = wave_u & 1;
  const int q = lane >> 4, r16 = lane & 15;
  const uint32_t lds0 = lds_base(lds);

  // DMA sources: block i of this wave covers 8 rows; each lane fetches the
  // chunk that belongs at its swizzled LDS position, from a clamped row.
  uint32_t aoff[APW], boff[BPW];
#pragma unroll
  for (int i = 0; i < APW; ++i) {
    const int row = (i * 4 + wave_u) * 8 + lane / 8;
    const int c = (lane % 8) ^ rswz<8>(row);
    const int gr = m0 + row < P.m ? m0 + row : P.m - 1;
    aoff[i] = (uint32_t)((size_t)gr * P.lda * sizeof(T)) + (uint32_t)(c * 16);
  }
#pragma unroll
  for (int i = 0; i < BPW; ++i) {
    const int row = (i * 4 + wave_u) * 8 + lane / 8;
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
    for (int i = 0; i < APW; ++i) lds_dma16(aoff[i], ab, sl + (uint32_t)(i * 4 + wave_u) * 1024u);
#pragma unroll
    for (int i = 0; i < BPW; ++i) lds_dma16(boff[i], bb, sl + A_BYTES + (uint32_t)(i * 4 + wave_u) * 1024u);
  };

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

#pragma unroll
  for (int s = 0; s < S - 1; ++s)
    if (s < nk) issue(s);
  for (int it = 0; it < nk; ++it) {
    // Stage it has landed once at most the blocks of later stages remain.
    const int after = nk - 1 - it < S - 2 ? nk - 1 - it : S - 2;
    if (after >= 1) DFLASH_VMWAIT(PER); else DFLASH_VMWAIT(0);
    block_barrier();
    if (it + S - 1 < nk) issue(it + S - 1);
    const uint32_t sl = lds0 + (uint32_t)(it % S) * STAGE;
    // All fragment reads of the stage go out before the first MFMA, so LDS
    // latency overlaps the products instead of stalling each of them.
    u32x4 af[2][MI], bf[2][NI];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) af[kb][mi] = lds_read16(sl + ard[kb] + (uint32_t)(mi * 16 * 128));
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) bf[kb][ni] = lds_read16(sl + brd[kb] + (uint32_t)(ni * 16 * 128));
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) Mfma<T>::chunk(acc[ni][mi], bf[kb][ni], af[kb][mi]);
  }

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
  const dim3 grid(total_tiles, kslices), block(256);
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

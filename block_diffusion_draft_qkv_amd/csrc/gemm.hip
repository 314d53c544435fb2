// HK1: grouped projection GEMM on gfx950 matrix cores.
//
// C[m][n] = sum_k A[m][k] B[n][k], the nn.Linear product y = x W^T used by the
// layer's fused qkv_proj (block rows -> q|k|v, context rows -> k|v through the
// k/v rows of the same weight) and by o_proj (vLLM page "qwen3_dflash":
// DFlashQwen3Attention.__init__/forward; "DFlash源码导读（二）" section 2).
//
// Tile BM x BN per 256-thread work-group (4 waves in 2 x 2), 128 bytes of k
// per stage (64 bf16 / 32 fp32), double-buffered through LDS with global loads
// of the next stage in flight during the MFMAs of the current one. LDS rows are
// 8 chunks of 16 bytes stored at chunk c ^ (row & 7), so the 8 lanes of a
// ds_read_b128 phase hit 8 different chunks. Rows past m or n load as zero and
// are not stored.
#include "kernels.h"

namespace dflash {

namespace {

template <typename OutT> struct Store;
template <> struct Store<float> {
  __device__ static inline void put(float* p, float v) { *p = v; }
};
template <> struct Store<__bf16> {
  __device__ static inline void put(__bf16* p, float v) { *p = (__bf16)v; }
};

template <typename T, typename OutT, int BM, int BN>
__global__ __launch_bounds__(256) void gemm_nt_kernel(GemmArgs args) {
  constexpr int E = Elem<T>::kPerChunk;
  constexpr int BKC = 8;  // chunks of k per stage
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int MI = WM / 16, NI = WN / 16;
  constexpr int A_CH = BM * BKC, B_CH = BN * BKC;
  constexpr int A_PT = A_CH / 256, B_PT = B_CH / 256;
  static_assert(A_CH % 256 == 0 && B_CH % 256 == 0, "tile must split over 256 threads");
  __shared__ u32x4 lds[2][A_CH + B_CH];

  int tile = blockIdx.x;
  const bool second = args.nprob > 1 && tile >= args.p[1].tile_begin;
  const GemmProblem P = second ? args.p[1] : args.p[0];
  tile -= P.tile_begin;
  const int m0 = (tile / P.tiles_n) * BM;
  const int n0 = (tile % P.tiles_n) * BN;
  const T* __restrict__ A = static_cast<const T*>(P.a);
  const T* __restrict__ B = static_cast<const T*>(P.b);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int q = lane >> 4, r16 = lane & 15;

  u32x4 ra[A_PT], rb[B_PT];
  auto load = [&](int kc0) {
#pragma unroll
    for (int i = 0; i < A_PT; ++i) {
      const int id = tid + 256 * i, row = id / BKC, c = id % BKC;
      const int gr = m0 + row;
      ra[i] = gr < P.m ? ldg16(A + (size_t)gr * P.lda + (size_t)(kc0 + c) * E) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < B_PT; ++i) {
      const int id = tid + 256 * i, row = id / BKC, c = id % BKC;
      const int gr = n0 + row;
      rb[i] = gr < P.n ? ldg16(B + (size_t)gr * P.ldb + (size_t)(kc0 + c) * E) : u32x4{0, 0, 0, 0};
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_PT; ++i) {
      const int id = tid + 256 * i, row = id / BKC, c = id % BKC;
      lds[buf][row * BKC + (c ^ (row & 7))] = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_PT; ++i) {
      const int id = tid + 256 * i, row = id / BKC, c = id % BKC;
      lds[buf][A_CH + row * BKC + (c ^ (row & 7))] = rb[i];
    }
  };

  f32x4 acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = P.k / (BKC * E);
  load(0);
  store(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load((kt + 1) * BKC);
#pragma unroll
    for (int kb = 0; kb < BKC / 4; ++kb) {
      u32x4 af[MI], bf[NI];
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        const int row = wm * WM + mi * 16 + r16;
        af[mi] = lds[cur][row * BKC + ((4 * kb + q) ^ (row & 7))];
      }
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        const int row = wn * WN + ni * 16 + r16;
        bf[ni] = lds[cur][A_CH + row * BKC + ((4 * kb + q) ^ (row & 7))];
      }
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) Mfma<T>::chunk(acc[mi][ni], af[mi], bf[ni]);
    }
    if (kt + 1 < nk) store(cur ^ 1);
    __syncthreads();
  }

  OutT* __restrict__ C = static_cast<OutT*>(P.c);
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      const int col = n0 + wn * WN + ni * 16 + r16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + wm * WM + mi * 16 + 4 * q + r;
        if (row < P.m && col < P.n) Store<OutT>::put(C + (size_t)row * P.ldc + col, acc[mi][ni][r]);
      }
    }
}

}  // namespace

hipError_t launch_gemm(int dtype, bool out_f32, const GemmArgs& args, int total_tiles,
                       hipStream_t stream) {
  if (total_tiles <= 0) return hipSuccess;
  const dim3 grid(total_tiles), block(256);
  if (dtype == 1) {
    if (out_f32)
      hipLaunchKernelGGL((gemm_nt_kernel<__bf16, float, kGemmBM, kGemmBN>), grid, block, 0, stream, args);
    else
      hipLaunchKernelGGL((gemm_nt_kernel<__bf16, __bf16, kGemmBM, kGemmBN>), grid, block, 0, stream, args);
  } else {
    hipLaunchKernelGGL((gemm_nt_kernel<float, float, kGemmBM, kGemmBN>), grid, block, 0, stream, args);
  }
  return hipGetLastError();
}

}  // namespace dflash

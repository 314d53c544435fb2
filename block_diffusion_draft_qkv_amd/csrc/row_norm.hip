// Row RMSNorm of the raw context states before the multi-layer context K/V
// projection (vLLM page "qwen3_dflash", DFlashQwen3Model
// _normalize_context_states: hidden_norm, an RMSNorm over the hidden size whose
// output is in the activation dtype).
//
// One 256-thread work-group per row, 16-byte loads: the sum of squares in fp32
// (wave butterflies, then the four waves' sums through LDS), then x *
// rsqrt(mean + eps) * gain rounded to the element type. A thread keeps up to
// kChunks of its row's 16-byte chunks in registers (hidden <= 8192 at bf16,
// 4096 at fp32); longer rows are read a second time (from L2).
#include "kernels.h"

namespace dflash {

namespace {

constexpr int kChunks = 4;

template <typename T>
__global__ __launch_bounds__(256) void rms_rows_kernel(const T* __restrict__ x, const T* __restrict__ g,
                                                       T* __restrict__ out, int h, float eps) {
  constexpr int V = 16 / (int)sizeof(T);  // elements per chunk
  __shared__ float part[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nchunk = h / V;
  const u32x4* row = reinterpret_cast<const u32x4*>(x + (size_t)blockIdx.x * h);
  u32x4 keep[kChunks];
  float ss = 0.f;
  auto sq = [&](const u32x4& c) {
    const T* e = reinterpret_cast<const T*>(&c);
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const float v = Elem<T>::to_f32(e[i]);
      ss += v * v;
    }
  };
#pragma unroll
  for (int k = 0; k < kChunks; ++k) {
    const int c = tid + k * 256;
    if (c < nchunk) keep[k] = row[c];
  }
#pragma unroll
  for (int k = 0; k < kChunks; ++k)
    if (tid + k * 256 < nchunk) sq(keep[k]);
  for (int c = tid + kChunks * 256; c < nchunk; c += 256) sq(row[c]);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) ss += shfl_xor(ss, m);
  if (lane == 0) part[wave] = ss;
  __syncthreads();
  const float inv = rsqrtf((part[0] + part[1] + part[2] + part[3]) / (float)h + eps);
  const u32x4* gv = reinterpret_cast<const u32x4*>(g);
  u32x4* o = reinterpret_cast<u32x4*>(out + (size_t)blockIdx.x * h);
  auto put = [&](int c, const u32x4& xc) {
    const u32x4 gc = gv[c];
    const T* xe = reinterpret_cast<const T*>(&xc);
    const T* ge = reinterpret_cast<const T*>(&gc);
    u32x4 r;
    T* re = reinterpret_cast<T*>(&r);
#pragma unroll
    for (int i = 0; i < V; ++i) re[i] = Elem<T>::from_f32(Elem<T>::to_f32(xe[i]) * inv * Elem<T>::to_f32(ge[i]));
    o[c] = r;
  };
#pragma unroll
  for (int k = 0; k < kChunks; ++k) {
    const int c = tid + k * 256;
    if (c < nchunk) put(c, keep[k]);
  }
  for (int c = tid + kChunks * 256; c < nchunk; c += 256) put(c, row[c]);
}

}  // namespace

hipError_t launch_rms_rows(int dtype, const void* x, const void* g, void* out, int rows, int h,
                           float eps, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  if (dtype == 1)
    hipLaunchKernelGGL(rms_rows_kernel<__bf16>, dim3(rows), dim3(256), 0, stream,
                       static_cast<const __bf16*>(x), static_cast<const __bf16*>(g),
                       static_cast<__bf16*>(out), h, eps);
  else
    hipLaunchKernelGGL(rms_rows_kernel<float>, dim3(rows), dim3(256), 0, stream, static_cast<const float*>(x),
                       static_cast<const float*>(g), static_cast<float*>(out), h, eps);
  return hipGetLastError();
}

}  // namespace dflash

// Row RMSNorm of the raw context states before the multi-layer context K/V
// projection (vLLM page "qwen3_dflash", DFlashQwen3Model
// _normalize_context_states: hidden_norm, an RMSNorm over the hidden size whose
// output is in the activation dtype).
//
// One 256-thread work-group per row: the sum of squares in fp32 (wave
// butterflies, then the four waves' sums through LDS), then x * rsqrt(mean +
// eps) * gain rounded to the element type. The row is read twice (the second
// time from L2); rows are at most a few hundred KB in all, so the kernel is a
// small share of the precompute next to its projection.
#include "kernels.h"

namespace dflash {

namespace {

template <typename T>
__global__ __launch_bounds__(256) void rms_rows_kernel(const T* __restrict__ x, const T* __restrict__ g,
                                                       T* __restrict__ out, int h, float eps) {
  __shared__ float part[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const T* row = x + (size_t)blockIdx.x * h;
  float ss = 0.f;
  for (int c = tid; c < h; c += 256) {
    const float v = Elem<T>::to_f32(row[c]);
    ss += v * v;
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) ss += shfl_xor(ss, m);
  if (lane == 0) part[wave] = ss;
  __syncthreads();
  const float inv = rsqrtf((part[0] + part[1] + part[2] + part[3]) / (float)h + eps);
  T* o = out + (size_t)blockIdx.x * h;
  for (int c = tid; c < h; c += 256)
    o[c] = Elem<T>::from_f32(Elem<T>::to_f32(row[c]) * inv * Elem<T>::to_f32(g[c]));
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

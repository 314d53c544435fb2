// Row RMSNorm kernels:
//  * rms_rows: out = x / sqrt(mean(x^2) + eps) * g. It serves the hidden_norm of
//    the raw context states before the multi-layer context K/V projection (vLLM
//    page "qwen3_dflash", DFlashQwen3Model._normalize_context_states, output in
//    the activation dtype), a decoder layer's input_layernorm and the draft
//    model's final norm (NeMo page "draft_qwen3": Qwen3DFlashDecoderLayer
//    input_layernorm; vLLM page: DFlashQwen3Model.forward, self.norm).
//  * add_rms_rows: h = x + y rounded to the element type (the residual
//    stream), and out = rmsnorm(h) * g: a decoder layer's residual add followed
//    by post_attention_layernorm (vLLM threads the residual through the norm the
//    same way).
//
// One 256-thread work-group per row, 16-byte loads: the sum of squares in fp32
// (wave butterflies, then the four waves' sums through LDS), then the scaled,
// gained values rounded to the element type. A thread keeps up to kChunks of
// its row's 16-byte chunks in registers (hidden <= 8192 at bf16, 4096 at
// fp32); longer rows are read a second time (from L2).
#include "kernels.h"

namespace dflash {

namespace {

constexpr int kChunks = 4;

template <typename T>
__global__ __launch_bounds__(256) void rms_rows_kernel(const T* __restrict__ x, const T* __restrict__ y,
                                                       const T* __restrict__ g, T* __restrict__ hout,
                                                       T* __restrict__ out, int h, float eps) {
  constexpr int V = 16 / (int)sizeof(T);  // elements per chunk
  __shared__ float part[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nchunk = h / V;
  const size_t roff = (size_t)blockIdx.x * h;
  const u32x4* row = reinterpret_cast<const u32x4*>(x + roff);
  const u32x4* add = y ? reinterpret_cast<const u32x4*>(y + roff) : nullptr;
  u32x4* hrow = hout ? reinterpret_cast<u32x4*>(hout + roff) : nullptr;
  // The row's chunk c (x + y rounded to T when y is given; stored to hout).
  auto load = [&](int c) -> u32x4 {
    u32x4 v = row[c];
    if (add) {
      const u32x4 w = add[c];
      T* ve = reinterpret_cast<T*>(&v);
      const T* we = reinterpret_cast<const T*>(&w);
#pragma unroll
      for (int i = 0; i < V; ++i) ve[i] = Elem<T>::from_f32(Elem<T>::to_f32(ve[i]) + Elem<T>::to_f32(we[i]));
    }
    return v;
  };
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
    if (c < nchunk) keep[k] = load(c);
  }
#pragma unroll
  for (int k = 0; k < kChunks; ++k) {
    const int c = tid + k * 256;
    if (c < nchunk) {
      sq(keep[k]);
      if (hrow) hrow[c] = keep[k];
    }
  }
  for (int c = tid + kChunks * 256; c < nchunk; c += 256) {
    const u32x4 v = load(c);
    sq(v);
    if (hrow) hrow[c] = v;
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) ss += shfl_xor(ss, m);
  if (lane == 0) part[wave] = ss;
  __syncthreads();
  const float inv = rsqrtf((part[0] + part[1] + part[2] + part[3]) / (float)h + eps);
  const u32x4* gv = reinterpret_cast<const u32x4*>(g);
  u32x4* o = reinterpret_cast<u32x4*>(out + roff);
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
  // rows longer than the registers hold: re-read (the residual sum from hout)
  for (int c = tid + kChunks * 256; c < nchunk; c += 256) put(c, hrow ? hrow[c] : row[c]);
}

}  // namespace

hipError_t launch_rms_rows(int dtype, const void* x, const void* y, const void* g, void* hout, void* out,
                           int rows, int h, float eps, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  if (dtype == 1)
    hipLaunchKernelGGL(rms_rows_kernel<__bf16>, dim3(rows), dim3(256), 0, stream, static_cast<const __bf16*>(x),
                       static_cast<const __bf16*>(y), static_cast<const __bf16*>(g), static_cast<__bf16*>(hout),
                       static_cast<__bf16*>(out), h, eps);
  else
    hipLaunchKernelGGL(rms_rows_kernel<float>, dim3(rows), dim3(256), 0, stream, static_cast<const float*>(x),
                       static_cast<const float*>(y), static_cast<const float*>(g), static_cast<float*>(hout),
                       static_cast<float*>(out), h, eps);
  return hipGetLastError();
}

}  // namespace dflash

// Row RMSNorm kernels:
//  * rms_rows: out = x / sqrt(mean(x^2) + eps) * g. It serves the hidden_norm of
//    the raw context states before the multi-layer context K/V projection (vLLM
//    page "qwen3_dflash", DFlashQwen3Model._normalize_context_states, output in
//    the activation dtype), a decoder layer's input_layernorm and the draft
//    model's final norm (NeMo page "draft_qwen3": Qwen3DFlashDecoderLayer
//    input_layernorm; vLLM page: DFlashQwen3Model.forward, self.norm).
//  * rms_rows_mx: the hidden_norm written as MXFP8 rows for the block-scaled
//    context K/V projection (or a plain MXFP8 quantisation of bf16 rows).
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

// MXFP8 quantisation of bf16 rows (OCP MX: one E8M0 scale per 32 consecutive
// elements, E4M3 elements), optionally after the hidden_norm: the input of the
// block-scaled context K/V projection (vLLM page "qwen3_dflash",
// _build_mxfp8_context_kv_proj; the states are hidden_norm-ed into the
// activation dtype first, _normalize_context_states). Per block: amax, shared
// exponent floor(log2 amax) - 8 clamped to [-127, 127] (scale byte =
// biased exponent of amax - 8, clamped to [0, 254]), elements x / 2^exponent
// (exact: a power of two) clamped to +-448 and converted by gfx950's packed
// FP8 conversion (OCP E4M3, round to nearest even, sign kept for zero; the
// clamp makes it saturate). The conversion does in one instruction per two
// elements what an integer encoding took some fifteen for: the kernel is
// bound by its vector ALU work otherwise.
//
// One 256-thread work-group per row (rows are few in a decode round, so each
// needs many lanes), the row kept in registers (hidden <= 8192); thread t
// holds chunks t + 256 k of 8 elements, and a 32-element block is the chunks
// of four consecutive threads, whose amax is reduced over those lanes. Scales
// go out row-major [rows][h / 32], or, with step_rows > 0, step-major
// [h / 128][step_rows][4] (a row's four blocks of a 128-wide k step together,
// the rows of one step contiguous), the layout the MXFP8 GEMM streams.
__device__ __forceinline__ void mx_row(const __bf16* __restrict__ x, const __bf16* __restrict__ g,
                                       uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, int r, int h,
                                       float eps, int step_rows) {
  constexpr int V = 8;
  __shared__ float part[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nchunk = h / V;  // a multiple of 16: a block's four chunks are in one pass
  const size_t roff = (size_t)r * h;
  const u32x4* row = reinterpret_cast<const u32x4*>(x + roff);
  const u32x4* gv = reinterpret_cast<const u32x4*>(g);
  uint2* out = reinterpret_cast<uint2*>(codes + roff);
  u32x4 keep[kChunks];
#pragma unroll
  for (int k = 0; k < kChunks; ++k) {
    const int c = tid + k * 256;
    if (c < nchunk) keep[k] = row[c];
  }
  float inv = 1.f;
  if (g != nullptr) {
    float ss = 0.f;
    auto sq = [&](const u32x4& v) {
      const __bf16* e = reinterpret_cast<const __bf16*>(&v);
#pragma unroll
      for (int i = 0; i < V; ++i) ss += (float)e[i] * (float)e[i];
    };
#pragma unroll
    for (int k = 0; k < kChunks; ++k)
      if (tid + k * 256 < nchunk) sq(keep[k]);
    for (int c = tid + kChunks * 256; c < nchunk; c += 256) sq(row[c]);
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) ss += shfl_xor(ss, m);
    if (lane == 0) part[wave] = ss;
    __syncthreads();
    inv = rsqrtf((part[0] + part[1] + part[2] + part[3]) / (float)h + eps);
  }
  auto put = [&](int c, const u32x4& v) {
    const __bf16* e = reinterpret_cast<const __bf16*>(&v);
    float y[V];
    if (g != nullptr) {
      const u32x4 gc = gv[c];
      const __bf16* ge = reinterpret_cast<const __bf16*>(&gc);
#pragma unroll
      for (int i = 0; i < V; ++i) y[i] = (float)(__bf16)((float)e[i] * inv * (float)ge[i]);
    } else {
#pragma unroll
      for (int i = 0; i < V; ++i) y[i] = (float)e[i];
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < V; ++i) amax = fmaxf(amax, fabsf(y[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
    const int ef = (int)((__float_as_uint(amax) >> 23) & 0xff);
    const int sbyte = min(max(ef - 8, 0), 254);
    const float mul = __uint_as_float((uint32_t)(254 - sbyte) << 23);  // 2^-(sbyte - 127), normal
    float t[V];
#pragma unroll
    for (int i = 0; i < V; ++i) t[i] = fminf(fmaxf(y[i] * mul, -448.f), 448.f);
    uint2 packed;
    packed.x = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(t[0], t[1], 0, false);
    packed.x = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(t[2], t[3], (int)packed.x, true);
    packed.y = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(t[4], t[5], 0, false);
    packed.y = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(t[6], t[7], (int)packed.y, true);
    out[c] = packed;
    if ((tid & 3) == 0) {
      const size_t at = step_rows > 0 ? ((size_t)(c / 16) * step_rows + r) * 4 + (c / 4) % 4
                                      : (size_t)r * (h / 32) + c / 4;
      scales[at] = (uint8_t)sbyte;
    }
  };
#pragma unroll
  for (int k = 0; k < kChunks; ++k) {
    const int c = tid + k * 256;
    if (c < nchunk) put(c, keep[k]);
  }
  for (int c = tid + kChunks * 256; c < nchunk; c += 256) put(c, row[c]);  // longer rows: from L2
}

__global__ __launch_bounds__(256) void rms_rows_mx_kernel(const __bf16* __restrict__ x,
                                                          const __bf16* __restrict__ g,
                                                          uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales, int h, float eps,
                                                          int step_rows) {
  mx_row(x, g, codes, scales, blockIdx.x, h, eps, step_rows);
}

// out[i] = sum over s of in[s * slice_stride + i] (+ res[i]), rounded once to
// T: the k-sliced fp32 partial sums of a projection folded into its output,
// with the residual of a projection that adds one. Four elements per thread
// (n % 4 == 0, 16-byte aligned rows).
template <typename T>
__global__ __launch_bounds__(256) void sum_slices_kernel(const float* __restrict__ in, int slices,
                                                         int64_t slice_stride, const T* __restrict__ res,
                                                         T* __restrict__ out, int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  f32x4 acc = reinterpret_cast<const f32x4*>(in)[i];
  for (int s = 1; s < slices; ++s) acc += reinterpret_cast<const f32x4*>(in + (size_t)s * slice_stride)[i];
  if (res != nullptr) {
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] += Elem<T>::to_f32(res[4 * i + r]);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) out[4 * i + r] = Elem<T>::from_f32(acc[r]);
}

__global__ __launch_bounds__(512) void table_patch_kernel(int32_t* __restrict__ table, TablePatch p, int count) {
  const int i = threadIdx.x;
  if (i < count) table[p.idx[i]] = p.val[i];
}

// Two row sets quantised (no norm) in one launch, each with step-major scale
// planes of its own rows: a layer step's draft block and new context rows.
__global__ __launch_bounds__(256) void rows_mx2_kernel(const __bf16* __restrict__ x1, uint8_t* __restrict__ c1,
                                                       uint8_t* __restrict__ s1, int rows1,
                                                       const __bf16* __restrict__ x2, uint8_t* __restrict__ c2,
                                                       uint8_t* __restrict__ s2, int rows2, int h) {
  const int r = blockIdx.x;
  if (r < rows1) mx_row(x1, nullptr, c1, s1, r, h, 0.f, rows1);
  else mx_row(x2, nullptr, c2, s2, r - rows1, h, 0.f, rows2);
}

// Row-major E8M0 scales [n][k / 32] -> step-major [k / 128][n][4]: one
// thread per (row, step) moves the step's four bytes.
__global__ __launch_bounds__(256) void scales_step_major_kernel(const uint32_t* __restrict__ src,
                                                                uint32_t* __restrict__ dst, int n, int steps) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // i = row * steps + step
  if (i >= (int64_t)n * steps) return;
  const int64_t row = i / steps, step = i % steps;
  dst[step * n + row] = src[i];
}

}  // namespace

hipError_t launch_rms_rows_mx(const void* x, const void* g, uint8_t* codes, uint8_t* scales, int rows, int h,
                              float eps, int step_rows, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(rms_rows_mx_kernel, dim3(rows), dim3(256), 0, stream, static_cast<const __bf16*>(x),
                     static_cast<const __bf16*>(g), codes, scales, h, eps, step_rows);
  return hipGetLastError();
}

hipError_t launch_sum_slices(int dtype, const float* in, int slices, int64_t slice_stride, void* out, int64_t n,
                             hipStream_t stream, const void* residual) {
  if (n <= 0) return hipSuccess;
  const int64_t n4 = n / 4;
  const dim3 grid((unsigned)((n4 + 255) / 256)), block(256);
  if (dtype == 1)
    hipLaunchKernelGGL(sum_slices_kernel<__bf16>, grid, block, 0, stream, in, slices, slice_stride,
                       static_cast<const __bf16*>(residual), static_cast<__bf16*>(out), n4);
  else
    hipLaunchKernelGGL(sum_slices_kernel<float>, grid, block, 0, stream, in, slices, slice_stride,
                       static_cast<const float*>(residual), static_cast<float*>(out), n4);
  return hipGetLastError();
}

hipError_t launch_table_patch(int32_t* table, const TablePatch& patch, int count, hipStream_t stream) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(table_patch_kernel, dim3(1), dim3(512), 0, stream, table, patch, count);
  return hipGetLastError();
}

hipError_t launch_rows_mx2(const void* x1, uint8_t* c1, uint8_t* s1, int rows1, const void* x2, uint8_t* c2,
                           uint8_t* s2, int rows2, int h, hipStream_t stream) {
  if (rows1 + rows2 <= 0) return hipSuccess;
  hipLaunchKernelGGL(rows_mx2_kernel, dim3(rows1 + rows2), dim3(256), 0, stream, static_cast<const __bf16*>(x1), c1,
                     s1, rows1, static_cast<const __bf16*>(x2), c2, s2, rows2, h);
  return hipGetLastError();
}

hipError_t launch_scales_step_major(const void* src, void* dst, int n, int k, hipStream_t stream) {
  const int steps = k / 128;
  const int64_t total = (int64_t)n * steps;
  if (total <= 0) return hipSuccess;
  hipLaunchKernelGGL(scales_step_major_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                     static_cast<const uint32_t*>(src), static_cast<uint32_t*>(dst), n, steps);
  return hipGetLastError();
}

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

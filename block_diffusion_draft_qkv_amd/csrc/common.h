// Shared device-side definitions of the draft-attention kernels (gfx950).
//
// Element types: activations, weights and the KV cache are either fp32 or
// bf16 (clang's __bf16, converted with the hardware round-to-nearest-even
// v_cvt_pk_bf16_f32). Accumulation is fp32 everywhere.
//
// MFMA operand convention used by every kernel here. A "chunk" is 16 bytes of
// one operand row along the reduction axis: 8 bf16 or 4 fp32 values. One
// "reduction block" c covers 4 chunks; lane group q = lane / 16 supplies chunk
// 4c + q of the row selected by lane % 16, for both operands. For bf16 this is
// exactly the A/B layout of v_mfma_f32_16x16x32_bf16 (8 consecutive k per
// lane); for fp32 the chunk feeds four v_mfma_f32_16x16x4f32, element e of
// every lane's chunk going to the e-th instruction. Both operands use the same
// rule, so the reduction is complete whatever order the hardware sums in.
// The 16x16 fp32 result holds column lane % 16 and rows 4q .. 4q+3 per lane.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dflash {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kMaxBatch = 256;
constexpr int kKeyTile = 64;       // cache capacity granule (attention key tiles)
constexpr int kMaxQueryRows = 64;  // block_size * (n_q / n_kv) rows per KV head
constexpr int kMaxGroups = 256;    // attention work-groups per launch
constexpr int kMaxKvHeads = 256;   // (sequence, KV head) pairs index in 16 bits
constexpr int kMaxCapacity = 1 << 21;  // cache rows; key tiles index in 16 bits
constexpr int kMaxLayers = 16;     // draft layers one context K/V precompute fills

// Per-sequence lengths of one step, passed to kernels by value.
struct SeqTable {
  int32_t batch;
  int32_t len[kMaxBatch];          // L_b: cache rows before the step
  int32_t ctx_off[kMaxBatch + 1];  // new context rows of b: [ctx_off[b], ctx_off[b+1])
};

template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kPerChunk = 4;
  __device__ static inline float to_f32(float x) { return x; }
  __device__ static inline float from_f32(float x) { return x; }
};
template <> struct Elem<__bf16> {
  static constexpr int kPerChunk = 8;
  __device__ static inline float to_f32(__bf16 x) { return (float)x; }
  __device__ static inline __bf16 from_f32(float x) { return (__bf16)x; }
};

// acc += A_chunk(16x?) * B_chunk, per the convention above.
template <typename T> struct Mfma;
template <> struct Mfma<__bf16> {
  __device__ static inline void chunk(f32x4& acc, const u32x4& a, const u32x4& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
  }
};
template <> struct Mfma<float> {
  __device__ static inline void chunk(f32x4& acc, const u32x4& a, const u32x4& b) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[e]), __uint_as_float(b[e]),
                                                 acc, 0, 0, 0);
  }
};

__device__ inline u32x4 ldg16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ inline void stg16(void* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }

// Wave-wide (64 lanes) butterfly over lanes xor `mask`.
__device__ inline float shfl_xor(float v, int mask) { return __shfl_xor(v, mask, 64); }

}  // namespace dflash

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
#include <type_traits>

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

// The tile of one work-group: which problem, where, and which k steps.
struct TileJob {
  GemmProblem P;
  bool second;
  int m0, n0, k_first, nk;
};
template <int BM, int BN> __device__ inline TileJob tile_job(const GemmArgs& args) {
  TileJob t;
  int tile = blockIdx.x;
  t.second = args.nprob > 1 && tile >= args.p[1].tile_begin;
  t.P = t.second ? args.p[1] : args.p[0];
  tile -= t.P.tile_begin;
  t.m0 = (tile / t.P.tiles_n) * BM;
  t.n0 = (tile % t.P.tiles_n) * BN;
  return t;
}

// Main loop shared by the plain and the appending GEMM. Producers return
// false after `extra` more barriers (those of the caller's epilogue);
// consumers return true with their sub-tile in acc.
template <typename T, int BM, int BN>
__device__ __forceinline__ bool gemm_core(const TileJob& J, uint32_t lds0, int extra,
                                          f32x4 (&acc)[GemmShape<BM, BN>::NI][GemmShape<BM, BN>::MI]) {
  using Sh = GemmShape<BM, BN>;
  constexpr int S = Sh::S, STAGE = Sh::STAGE, A_BYTES = Sh::A_BYTES;
  constexpr int APP = Sh::APP, BPP = Sh::BPP, PER = Sh::PER;
  constexpr int WM = Sh::WM, WN = Sh::WN, MI = Sh::MI, NI = Sh::NI;
  const GemmProblem& P = J.P;
  const int m0 = J.m0, n0 = J.n0, k_first = J.k_first, nk = J.nk;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

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
      int gr;
      if (P.b_pair == 0) {
        gr = n0 + row < P.n ? n0 + row : P.n - 1;
      } else {  // gate rows for the tile's first half, up rows for its second
        const int j = n0 / 2 + (row < BN / 2 ? row : row - BN / 2);
        gr = (j < P.b_pair ? j : P.b_pair - 1) + (row < BN / 2 ? 0 : P.b_pair);
      }
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
    for (int e = 0; e < extra; ++e) block_barrier();
    return false;
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
  return true;
}

// MXFP8 operands (OCP MX: E4M3 elements, one E8M0 scale byte per 32
// consecutive k). A k step is 128 elements: the same 128 bytes per row as a
// bf16 step, plus 4 scale bytes per row (the step's four blocks), which the
// producers stream into the stage behind the data with 256-byte LDS-DMA
// loads (64 rows each; the (BM + BN) / 64 of a step alternate between the two
// producers, so their per-step block counts may differ by one). The scales
// are stored step-major, so a load reads 256 contiguous bytes; row-major
// scales put every lane on a cache line of its own.
template <int BM, int BN> struct GemmShapeMX {
  static constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128;
  static constexpr int AS_OFF = A_BYTES + B_BYTES, BS_OFF = AS_OFF + BM * 4, STAGE = BS_OFF + BN * 4;
  static constexpr int APP = BM / 8 / kGemmProducers, BPP = BN / 8 / kGemmProducers;
  static constexpr int SCALE_LOADS = (BM + BN) / 64;
  static constexpr int PER0 = APP + BPP + (SCALE_LOADS + 1) / 2, PER1 = APP + BPP + SCALE_LOADS / 2;
  static constexpr int S_LDS = (160 * 1024) / STAGE, S_VM = 1 + 63 / PER0;
  static constexpr int S = S_LDS < S_VM ? (S_LDS < 8 ? S_LDS : 8) : (S_VM < 8 ? S_VM : 8);
  static constexpr int WM = BM / 2, WN = BN / 2;
  static constexpr int MI = WM / 16, NI = WN / 16;
  static_assert((S - 1) * PER0 <= 63, "outstanding DMA blocks must fit vmcnt");
  static_assert(STAGE % 16 == 0, "stages stay 16-byte aligned");
};

// The MXFP8 main loop, with gemm_core's protocol (producers return false after
// `extra` more barriers, consumers true with their sub-tile in acc). In a
// 16x16x128 scaled MFMA, lane (q, r) of an operand holds row r's k 16q ..
// 16q + 15 in its first 16 bytes and k 64 + 16q .. 64 + 16q + 15 in its last
// 16 (logical chunks q and q + 4 of the 128-byte step row), and supplies the
// scale of k block q (k 32q .. 32q + 31) of row r; measured on gfx950 with
// one-hot operands. Consumers read step s + 1's fragments while the MFMAs of
// step s run (two fragment sets).
template <int BM, int BN>
__device__ __forceinline__ bool gemm_core_mx(const TileJob& J, uint32_t lds0, int extra,
                                             f32x4 (&acc)[GemmShapeMX<BM, BN>::NI][GemmShapeMX<BM, BN>::MI]) {
  using Sh = GemmShapeMX<BM, BN>;
  constexpr int S = Sh::S, STAGE = Sh::STAGE, A_BYTES = Sh::A_BYTES, AS_OFF = Sh::AS_OFF, BS_OFF = Sh::BS_OFF;
  constexpr int APP = Sh::APP, BPP = Sh::BPP, WM = Sh::WM, WN = Sh::WN, MI = Sh::MI, NI = Sh::NI;
  constexpr int SL = Sh::SCALE_LOADS, ASL = BM / 64;
  const GemmProblem& P = J.P;
  const int m0 = J.m0, n0 = J.n0, nk = J.nk;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  if (wave >= kGemmConsumers) {
    // ---------------------------------------------------------- producers
    const int pw = wave - kGemmConsumers;
    uint32_t aoff[APP], boff[BPP], soff[(SL + 1) / 2];
#pragma unroll
    for (int i = 0; i < APP; ++i) {
      const int row = (i * kGemmProducers + pw) * 8 + lane / 8;
      const int c = (lane % 8) ^ rswz<8>(row);
      const int gr = m0 + row < P.m ? m0 + row : P.m - 1;
      aoff[i] = (uint32_t)((size_t)gr * P.lda) + (uint32_t)(c * 16);
    }
#pragma unroll
    for (int i = 0; i < BPP; ++i) {
      const int row = (i * kGemmProducers + pw) * 8 + lane / 8;
      const int c = (lane % 8) ^ rswz<8>(row);
      const int gr = n0 + row < P.n ? n0 + row : P.n - 1;
      boff[i] = (uint32_t)((size_t)gr * P.ldb) + (uint32_t)(c * 16);
    }
    // Scale load u = 2 i + pw: A rows 64 u .. 64 u + 63 when u < BM / 64,
    // else B rows 64 (u - BM / 64) ..; lane l fetches its row's 4 bytes.
#pragma unroll
    for (int i = 0; i < (SL + 1) / 2; ++i) {
      const int u = 2 * i + pw;
      int gr = 0;
      if (u < ASL) {
        gr = m0 + 64 * u + lane;
        gr = gr < P.m ? gr : P.m - 1;
      } else if (u < SL) {
        gr = n0 + 64 * (u - ASL) + lane;
        gr = gr < P.n ? gr : P.n - 1;
      }
      soff[i] = (uint32_t)gr * 4u;
    }
    const char* Ab = static_cast<const char*>(P.a);
    const char* Bb = static_cast<const char*>(P.b);
    auto issue = [&](int step) {
      const size_t kbyte = (size_t)step * 128;
      const uint32_t sl = lds0 + (uint32_t)(step % S) * STAGE;
      const void* ab = uniform_ptr(Ab + kbyte);
      const void* bb = uniform_ptr(Bb + kbyte);
#pragma unroll
      for (int i = 0; i < APP; ++i)
        lds_dma16(aoff[i], ab, sl + (uint32_t)(i * kGemmProducers + pw) * 1024u);
#pragma unroll
      for (int i = 0; i < BPP; ++i)
        lds_dma16(boff[i], bb, sl + A_BYTES + (uint32_t)(i * kGemmProducers + pw) * 1024u);
      const void* sab = uniform_ptr(P.sa + (size_t)step * (P.sa_plane ? P.sa_plane : (int64_t)P.m * 4));
      const void* sbb = uniform_ptr(P.sb + (size_t)step * (P.sb_plane ? P.sb_plane : (int64_t)P.n * 4));
#pragma unroll
      for (int i = 0; i < (SL + 1) / 2; ++i) {
        const int u = 2 * i + pw;
        if (u < ASL) lds_dma4(soff[i], sab, sl + AS_OFF + (uint32_t)u * 256u);
        else if (u < SL) lds_dma4(soff[i], sbb, sl + BS_OFF + (uint32_t)(u - ASL) * 256u);
      }
    };
#pragma unroll
    for (int s = 0; s < S - 1; ++s)
      if (s < nk) issue(s);
    for (int it = 0; it < nk; ++it) {
      const int after = nk - 1 - it < S - 2 ? nk - 1 - it : S - 2;
      if (pw == 0) stage_wait<Sh::PER0, S>(after);
      else stage_wait<Sh::PER1, S>(after);
      block_barrier();
      if (it + S - 1 < nk) issue(it + S - 1);
    }
    for (int e = 0; e < extra; ++e) block_barrier();
    return false;
  }

  // ------------------------------------------------------------ consumers
  const int wm = wave >> 1, wn = wave & 1;
  const int q = lane >> 4, r16 = lane & 15;
  uint32_t ard[2], brd[2];
  {
    const int sw = rswz<8>(r16);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      ard[j] = (uint32_t)((wm * WM + r16) * 8 + ((q + 4 * j) ^ sw)) * 16u;
      brd[j] = (uint32_t)((wn * WN + r16) * 8 + ((q + 4 * j) ^ sw)) * 16u + A_BYTES;
    }
  }
  const uint32_t asc = (uint32_t)(AS_OFF + (wm * WM + r16) * 4 + q);
  const uint32_t bsc = (uint32_t)(BS_OFF + (wn * WN + r16) * 4 + q);
#pragma unroll
  for (int ni = 0; ni < NI; ++ni)
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) acc[ni][mi] = f32x4{0.f, 0.f, 0.f, 0.f};

  struct Frag {
    u32x4 a[MI][2], b[NI][2];
    uint32_t sa[MI], sb[NI];
  };
  auto read = [&](Frag& f, int step) {
    const uint32_t sl = lds0 + (uint32_t)(step % S) * STAGE;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      f.a[mi][0] = lds_read16(sl + ard[0] + (uint32_t)(mi * 16 * 128));
      f.a[mi][1] = lds_read16(sl + ard[1] + (uint32_t)(mi * 16 * 128));
      f.sa[mi] = lds_read_u8(sl + asc + (uint32_t)(mi * 64));
    }
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      f.b[ni][0] = lds_read16(sl + brd[0] + (uint32_t)(ni * 16 * 128));
      f.b[ni][1] = lds_read16(sl + brd[1] + (uint32_t)(ni * 16 * 128));
      f.sb[ni] = lds_read_u8(sl + bsc + (uint32_t)(ni * 64));
    }
  };
  // C^T = W . A^T: the weight fragment is the MFMA's first operand, so a lane
  // ends with m = r16 and n = 4q .. 4q + 3, as in the bf16 loop.
  auto mma = [&](const Frag& f) {
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      const i32x8 wb = {(int)f.b[ni][0][0], (int)f.b[ni][0][1], (int)f.b[ni][0][2], (int)f.b[ni][0][3],
                        (int)f.b[ni][1][0], (int)f.b[ni][1][1], (int)f.b[ni][1][2], (int)f.b[ni][1][3]};
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        const i32x8 xa = {(int)f.a[mi][0][0], (int)f.a[mi][0][1], (int)f.a[mi][0][2], (int)f.a[mi][0][3],
                          (int)f.a[mi][1][0], (int)f.a[mi][1][1], (int)f.a[mi][1][2], (int)f.a[mi][1][3]};
        acc[ni][mi] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wb, xa, acc[ni][mi], 0, 0, 0,
                                                                      (int)f.sb[ni], 0, (int)f.sa[mi]);
      }
    }
  };
  Frag f0, f1;
  int it = 0;
  for (; it + 1 < nk; it += 2) {
    block_barrier();
    read(f0, it);
    __builtin_amdgcn_sched_barrier(0);
    if (it > 0) mma(f1);
    __builtin_amdgcn_sched_barrier(0);
    block_barrier();
    read(f1, it + 1);
    __builtin_amdgcn_sched_barrier(0);
    mma(f0);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (it < nk) {
    block_barrier();
    read(f0, it);
    __builtin_amdgcn_sched_barrier(0);
    if (it > 0) mma(f1);
    __builtin_amdgcn_sched_barrier(0);
    mma(f0);
  } else if (nk > 0) {
    mma(f1);
  }
  return true;
}

// With MX the operands are MXFP8 (gemm_core_mx, no k split): o_proj of the
// layer in its MXFP8 configuration.
template <typename T, typename OutT, int BM, int BN, bool MX = false>
__global__ __launch_bounds__(kGemmThreads, 1) void gemm_kernel(GemmArgs args) {
  using Sh = std::conditional_t<MX, GemmShapeMX<BM, BN>, GemmShape<BM, BN>>;
  constexpr int WM = Sh::WM, WN = Sh::WN, MI = Sh::MI, NI = Sh::NI;
  __shared__ u32x4 lds[Sh::S * Sh::STAGE / 16];
  TileJob J = tile_job<BM, BN>(args);
  const int ksl = gridDim.y;                                      // k slices
  const int nk_all = MX ? J.P.k / 128 : J.P.k / (8 * (16 / (int)sizeof(T)));  // 128-byte k steps
  J.k_first = (int)(((int64_t)nk_all * blockIdx.y) / ksl);
  J.nk = (int)(((int64_t)nk_all * (blockIdx.y + 1)) / ksl) - J.k_first;
  f32x4 acc[NI][MI];
  bool consumer;
  if constexpr (MX) consumer = gemm_core_mx<BM, BN>(J, lds_base(lds), 0, acc);
  else consumer = gemm_core<T, BM, BN>(J, lds_base(lds), 0, acc);
  if (!consumer) return;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1, q = lane >> 4, r16 = lane & 15;
  // acc[ni][mi]: lane holds m = r16 of block mi and n = 4q .. 4q+3 of block ni.
  OutT* C = static_cast<OutT*>(J.P.c) + (size_t)blockIdx.y * J.P.slice_stride;
  const OutT* Rs = static_cast<const OutT*>(J.P.r);
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
    const int m = J.m0 + wm * WM + mi * 16 + r16;
    if (m >= J.P.m) continue;
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      const int n = J.n0 + wn * WN + ni * 16 + 4 * q;
      if (n >= J.P.n) continue;
      f32x4 v = acc[ni][mi];
      if (Rs != nullptr) {
        const OutT* rr = Rs + (size_t)m * J.P.ldc + n;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] += Elem<OutT>::to_f32(rr[r]);
      }
      Store4<OutT>::put(C + (size_t)m * J.P.ldc + n, v);
    }
  }
}

// Qwen3MLP's gate/up projection with SiLU(gate) * up in the epilogue (NeMo
// page "draft_qwen3": Qwen3DFlashDecoderLayer, mlp = Qwen3MLP; vLLM page
// "qwen3_dflash": gate_proj and up_proj stacked as gate_up_proj). A tile is
// BM rows x 128 columns whose first 64 are gate rows j0 .. j0+63 of the weight
// and last 64 the up rows b_pair + j0 .. (b_pair set); consumer wave (wm, wn)
// holds the gate (wn = 0) or up (wn = 1) half, so every value's partner sits
// in the same lane and register of wave (wm, 1 - wn). The two waves trade half
// of their row blocks through the free LDS ring and each finishes the other
// half: silu(g) = g / (1 + e^-g), times u, rounded once to the output type.
template <typename T, int BM>
__global__ __launch_bounds__(kGemmThreads, 1) void gemm_swiglu_kernel(GemmArgs args) {
  constexpr int BN = 128;
  using Sh = GemmShape<BM, BN>;
  constexpr int MI = Sh::MI, NI = Sh::NI, WM = Sh::WM, MH = MI / 2, XR = MH * NI * 4;
  static_assert(4 * XR * 64 * 4 <= Sh::S * Sh::STAGE, "the exchange fits in the ring");
  __shared__ u32x4 lds[Sh::S * Sh::STAGE / 16];
  TileJob J = tile_job<BM, BN>(args);
  J.k_first = 0;
  J.nk = J.P.k / (8 * (16 / (int)sizeof(T)));
  f32x4 acc[NI][MI];
  if (!gemm_core<T, BM, BN>(J, lds_base(lds), 2, acc)) return;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1, q = lane >> 4, r16 = lane & 15;
  float* xch = reinterpret_cast<float*>(lds);
  const int partner = wm * 2 + (1 - wn);
  block_barrier();  // the last fragment reads of the main loop are done
  // hand over the row blocks the partner finishes: (1 - wn) * MH .. + MH - 1
#pragma unroll
  for (int ni = 0; ni < NI; ++ni)
#pragma unroll
    for (int u = 0; u < MH; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        xch[(wave * XR + (ni * MH + u) * 4 + r) * 64 + lane] =
            wn == 0 ? acc[ni][MH + u][r] : acc[ni][u][r];
  block_barrier();
  T* C = static_cast<T*>(J.P.c);
  const int j0 = J.n0 / 2;
#pragma unroll
  for (int u = 0; u < MH; ++u) {
    const int mi = wn * MH + u;
    const int m = J.m0 + wm * WM + mi * 16 + r16;
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      f32x4 o;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float own = wn == 0 ? acc[ni][u][r] : acc[ni][MH + u][r];
        const float oth = xch[(partner * XR + (ni * MH + u) * 4 + r) * 64 + lane];
        const float g = wn == 0 ? own : oth, up = wn == 0 ? oth : own;
        o[r] = g / (1.0f + __expf(-g)) * up;
      }
      const int j = j0 + ni * 16 + 4 * q;
      if (m < J.P.m && j < J.P.b_pair) Store4<T>::put(C + (size_t)m * J.P.ldc + j, o);
    }
  }
}

// The SwiGLU GEMM in 256 x 192 tiles (96 gate + 96 up columns), bf16 only.
// At 512 rows and a 12288-wide MLP that is 256 work-groups, one round of 256
// CUs, where 128-column tiles make 384 (a round and a half) and stream more
// bytes per output. Roles as in gemm_core (four consumer waves in 2 x 2, two
// producer waves), but a k step is 32 elements (64-byte rows): a 64-element
// step of this tile (56 KB) would leave LDS room for two stages only, while
// 28 KB steps give five, as many bytes in flight as the 128-column tiles
// keep. A consumer wave holds a 128 x 96 sub-tile (192 accumulator VGPRs), so
// it reads its A fragments four 16-row blocks at a time. k is summed in the
// same 32-element MFMA blocks and the same order as gemm_swiglu_kernel, so
// the outputs are the same bits.
struct WideShape {
  static constexpr int BM = 256, BN = 192;
  static constexpr int A_BYTES = BM * 64, B_BYTES = BN * 64, STAGE = A_BYTES + B_BYTES;
  static constexpr int APP = BM / 16 / kGemmProducers, BPP = BN / 16 / kGemmProducers;  // 1 KB blocks
  static constexpr int PER = APP + BPP;
  static constexpr int S = 5;
  static constexpr int WM = BM / 2, WN = BN / 2, MI = WM / 16, NI = WN / 16, MH = MI / 2;
  static_assert(S * STAGE <= 160 * 1024, "the ring fits in LDS");
  static_assert((S - 1) * PER <= 63, "outstanding DMA blocks must fit vmcnt");
  static_assert(MI % 4 == 0, "A fragments go four blocks at a time");
};

__global__ __launch_bounds__(kGemmThreads, 1) void gemm_swiglu_wide_kernel(GemmArgs args) {
  using Sh = WideShape;
  using T = __bf16;
  constexpr int S = Sh::S, STAGE = Sh::STAGE, A_BYTES = Sh::A_BYTES, APP = Sh::APP, BPP = Sh::BPP;
  constexpr int PER = Sh::PER, BN = Sh::BN, WM = Sh::WM, WN = Sh::WN, MI = Sh::MI, NI = Sh::NI, MH = Sh::MH;
  constexpr int XR = MH * NI * 4;
  static_assert(4 * XR * 64 * 4 <= S * STAGE, "the exchange fits in the ring");
  __shared__ u32x4 lds[S * STAGE / 16];
  const TileJob J = tile_job<Sh::BM, Sh::BN>(args);
  const GemmProblem& P = J.P;
  const int nk = P.k / 32;  // 64-byte k steps
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t lds0 = lds_base(lds);

  if (wave >= kGemmConsumers) {
    // ---------------------------------------------------------- producers
    // Block i * kGemmProducers + pw of an operand covers 16 rows of 64 bytes;
    // each lane fetches the chunk that belongs at its swizzled LDS position.
    const int pw = wave - kGemmConsumers;
    uint32_t aoff[APP], boff[BPP];
#pragma unroll
    for (int i = 0; i < APP; ++i) {
      const int row = (i * kGemmProducers + pw) * 16 + lane / 4;
      const int c = (lane % 4) ^ rswz<4>(row);
      const int gr = J.m0 + row < P.m ? J.m0 + row : P.m - 1;
      aoff[i] = (uint32_t)((size_t)gr * P.lda * sizeof(T)) + (uint32_t)(c * 16);
    }
#pragma unroll
    for (int i = 0; i < BPP; ++i) {
      const int row = (i * kGemmProducers + pw) * 16 + lane / 4;
      const int c = (lane % 4) ^ rswz<4>(row);
      // gate rows for the tile's first half, up rows for its second
      const int j = J.n0 / 2 + (row < BN / 2 ? row : row - BN / 2);
      const int gr = (j < P.b_pair ? j : P.b_pair - 1) + (row < BN / 2 ? 0 : P.b_pair);
      boff[i] = (uint32_t)((size_t)gr * P.ldb * sizeof(T)) + (uint32_t)(c * 16);
    }
    const char* Ab = static_cast<const char*>(P.a);
    const char* Bb = static_cast<const char*>(P.b);
    auto issue = [&](int step) {
      const size_t kbyte = (size_t)step * 64;
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
      const int after = nk - 1 - it < S - 2 ? nk - 1 - it : S - 2;
      stage_wait<PER, S>(after);
      block_barrier();
      if (it + S - 1 < nk) issue(it + S - 1);
    }
    block_barrier();  // the epilogue's two barriers
    block_barrier();
    return;
  }

  // ------------------------------------------------------------ consumers
  const int wm = wave >> 1, wn = wave & 1, q = lane >> 4, r16 = lane & 15;
  // operand rows wm*WM + mi*16 + r16 (A) and wn*WN + ni*16 + r16 (W), logical
  // chunk q (k 8q .. 8q + 7 of the step); the swizzle depends on r16 only
  const int sw = rswz<4>(r16);
  const uint32_t ard = (uint32_t)((wm * WM + r16) * 64 + ((q ^ sw) * 16));
  const uint32_t brd = (uint32_t)(A_BYTES + (wn * WN + r16) * 64 + ((q ^ sw) * 16));
  f32x4 acc[NI][MI];
#pragma unroll
  for (int ni = 0; ni < NI; ++ni)
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) acc[ni][mi] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < nk; ++it) {
    block_barrier();
    const uint32_t sl = lds0 + (uint32_t)(it % S) * STAGE;
    u32x4 b[NI], a[4];
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) b[ni] = lds_read16(sl + brd + (uint32_t)(ni * 1024));
#pragma unroll
    for (int g = 0; g < MI / 4; ++g) {
#pragma unroll
      for (int u = 0; u < 4; ++u) a[u] = lds_read16(sl + ard + (uint32_t)((4 * g + u) * 1024));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) Mfma<T>::chunk(acc[ni][4 * g + u], b[ni], a[u]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // Epilogue as in gemm_swiglu_kernel: wave (wm, 0) holds the gate and wave
  // (wm, 1) the up half of the same outputs; each hands the partner the row
  // blocks the partner finishes, then writes silu(g) * u for its own.
  float* xch = reinterpret_cast<float*>(lds);
  const int partner = wm * 2 + (1 - wn);
  block_barrier();  // the last fragment reads of the main loop are done
#pragma unroll
  for (int ni = 0; ni < NI; ++ni)
#pragma unroll
    for (int u = 0; u < MH; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        xch[(wave * XR + (ni * MH + u) * 4 + r) * 64 + lane] = wn == 0 ? acc[ni][MH + u][r] : acc[ni][u][r];
  block_barrier();
  T* C = static_cast<T*>(P.c);
  const int j0 = J.n0 / 2;
#pragma unroll
  for (int u = 0; u < MH; ++u) {
    const int mi = wn * MH + u;
    const int m = J.m0 + wm * WM + mi * 16 + r16;
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      f32x4 o;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float own = wn == 0 ? acc[ni][u][r] : acc[ni][MH + u][r];
        const float oth = xch[(partner * XR + (ni * MH + u) * 4 + r) * 64 + lane];
        const float g = wn == 0 ? own : oth, up = wn == 0 ? oth : own;
        o[r] = g / (1.0f + __expf(-g)) * up;
      }
      const int j = j0 + ni * 16 + 4 * q;
      if (m < P.m && j < P.b_pair) Store4<T>::put(C + (size_t)m * P.ldc + j, o);
    }
  }
}

// Sum over the four lanes l, l^16, l^32, l^48 that hold one row's columns.
__device__ inline float quad_sum(float v) {
  v += __shfl_xor(v, 16, 64);
  return v + __shfl_xor(v, 32, 64);
}

// The q|k|v + context k|v projection with the work of the norm/RoPE/append
// kernel in its epilogue (same definitions: NeMo page "draft_qwen3"
// Qwen3DFlashAttention.forward and apply_rotary_pos_emb; "DFlash源码导读（二）"
// sections 1-4). A tile is BM rows x one head (BN = D columns, no k split);
// consumer wave (wm, wn) holds columns wn*D/2 .. wn*D/2 + D/2 - 1, so the
// rotation partner of every value (t <-> t + D/2) sits in the same lane and
// register of wave (wm, 1 - wn). After the main loop the two waves trade
// halves through LDS (the ring is free by then) so that each finishes whole
// rows of half the row blocks: the row's sum of squares (summed over the four
// lanes of the row), RMSNorm with the head gain (and, for queries, the scale
// head_dim^-1/2 log2 e), neox rotation at the row's position from the fp64-
// built cos/sin table, and the stores: queries packed as rows i*g + hh of their
// KV head's tile, keys to cache K, values (raw) transposed to cache V.
// Positions outside the table are clamped and latched in the error flag.
// With MX the operands are MXFP8 (gemm_core_mx; T, the cache and gain type, is
// bf16): the multi-layer context precompute's block-scaled K/V projection
// (vLLM page "qwen3_dflash", _build_mxfp8_context_kv_proj).
template <typename T, int BM, int D, bool MX = false>
__global__ __launch_bounds__(kGemmThreads, 1) void gemm_append_kernel(GemmArgs args, NormRopeArgs a) {
  using Sh = std::conditional_t<MX, GemmShapeMX<BM, D>, GemmShape<BM, D>>;
  constexpr int WM = Sh::WM, MI = Sh::MI, NI = Sh::NI, HALF = D / 2, REGS = MI * NI * 4;
  static_assert(Sh::WN == HALF, "a tile holds one head");
  static_assert(4 * REGS / 2 * 64 * 4 <= Sh::S * Sh::STAGE, "the exchange fits in the ring");
  __shared__ u32x4 lds[Sh::S * Sh::STAGE / 16];
  TileJob J = tile_job<BM, D>(args);
  J.k_first = 0;
  J.nk = MX ? J.P.k / 128 : J.P.k / (8 * (16 / (int)sizeof(T)));
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1, q = lane >> 4, r16 = lane & 15;
  const int nq = a.nq, nkv = a.nkv, bs = a.bs, g = nq / nkv, R = bs * g;
  // The head of this tile: kind 0 query, 1 key, 2 value. Context columns
  // come in groups of 2 nkv heads per layer (one group in a layer step, one
  // per draft layer in the multi-layer context precompute).
  const int h = J.n0 / D;
  int kind, j, hh = 0, layer = 0;
  if (!J.second) {
    kind = h < nq ? 0 : (h < nq + nkv ? 1 : 2);
    j = kind == 0 ? h / g : (kind == 1 ? h - nq : h - nq - nkv);
    hh = kind == 0 ? h % g : 0;
  } else {
    layer = h / (2 * nkv);
    const int hl = h - layer * 2 * nkv;
    kind = hl < nkv ? 1 : 2;
    j = kind == 1 ? hl : hl - nkv;
  }
  T* const kc = static_cast<T*>(layer == 0 ? a.kc : a.layer_kc[layer]);
  T* const vc = static_cast<T*>(layer == 0 ? a.vc : a.layer_vc[layer]);
  const CacheMap map = a.map_of(layer);

  // Consumers: this lane's rows (sequence, window row: context rows first,
  // then block rows). After the swap below, wave (wm, wn) finishes whole rows
  // of the row blocks wn*MH .. wn*MH + MH - 1; their positions are loaded
  // before the main loop (nothing waits for them until the epilogue).
  constexpr int MH = MI / 2;
  int sb[MI], win[MI], crow[MI], pos[MH];  // sequence, window row, cache row; positions
  int blk[MI];                             // the row's 64-row cache block (CacheMap::block_of)
  bool ok[MI];
  if (wave < kGemmConsumers) {
    // The sequences a wave's rows touch are few and found with wave-uniform
    // loops (scalar loads of the sequence table); each lane keeps its rows'.
    const int r0 = J.m0 + wm * WM, rl = min(r0 + WM, J.P.m) - 1;
    int pb[MI];  // first position index of the row's window
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      ok[mi] = r0 + mi * 16 + r16 <= rl;
      sb[mi] = win[mi] = crow[mi] = pb[mi] = 0;
    }
    if (!J.second) {
      for (int b = r0 / bs; b <= rl / bs; ++b) {
        const int c0 = a.seq.ctx_off[b], c1 = a.seq.ctx_off[b + 1], L = a.seq.len[b];
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
          const int m = r0 + mi * 16 + r16;
          if (ok[mi] && m / bs == b) {
            sb[mi] = b;
            win[mi] = (c1 - c0) + m % bs;
            crow[mi] = L + win[mi];
            pb[mi] = c0 + b * bs;
          }
        }
      }
    } else {
      int lo = 0, hi = a.seq.batch;  // last b with ctx_off[b] <= r0
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (a.seq.ctx_off[mid] <= r0) lo = mid;
        else hi = mid;
      }
      for (int b = lo; b < a.seq.batch && a.seq.ctx_off[b] <= rl; ++b) {
        const int c0 = a.seq.ctx_off[b], L = a.seq.len[b];
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
          const int m = r0 + mi * 16 + r16;
          if (ok[mi] && c0 <= m) {  // the last such b owns row m
            sb[mi] = b;
            win[mi] = m - c0;
            crow[mi] = L + win[mi];
            pb[mi] = c0 + b * bs;
          }
        }
      }
    }
    if (kind != 2) {
#pragma unroll
      for (int u = 0; u < MH; ++u) {
        // row block wn * MH + u, selected without indexing by a runtime value
        const int pi = wn == 0 ? pb[u] + win[u] : pb[MH + u] + win[MH + u];
        // no position array: contiguous positions, the row's cache row
        pos[u] = a.positions ? a.positions[pi] : (wn == 0 ? crow[u] : crow[MH + u]);
      }
    }
    // The cache block of each row (a paged cache's from its table, loaded with the positions).
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) blk[mi] = ok[mi] ? (int)map.block_of(sb[mi], crow[mi]) : 0;
  }

  f32x4 acc[NI][MI];
  bool consumer;
  if constexpr (MX) consumer = gemm_core_mx<BM, D>(J, lds_base(lds), 2, acc);
  else consumer = gemm_core<T, BM, D>(J, lds_base(lds), 2, acc);
  if (!consumer) return;

  float* xch = reinterpret_cast<float*>(lds);
  constexpr int XR = MH * NI * 4;  // values one lane hands over
  const int partner = wm * 2 + (1 - wn);
  if (kind == 2) {
    block_barrier();  // the epilogue's two barriers (no swap for values)
    block_barrier();
    // Values: raw, transposed into cache V (key index contiguous); each wave
    // writes its own half of the columns for all its rows.
    T* vbase = vc;
    const size_t vs = (size_t)CacheMap::vstride();
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      if (!ok[mi]) continue;
      const size_t col = ((size_t)blk[mi] * nkv + j) * D * kKeyTile + crow[mi] % kKeyTile;
      const size_t col0 = col + (size_t)(wn * HALF) * vs;
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          vbase[col0 + (size_t)(ni * 16 + 4 * q + r) * vs] = Elem<T>::from_f32(acc[ni][mi][r]);
    }
    return;
  }

  // Queries and keys. WN is this wave's wn as a constant, so that the row
  // blocks it finishes (WN * MH + u) index the register arrays statically.
  auto finish = [&](auto wn_c) __attribute__((always_inline)) {
    constexpr int WN = decltype(wn_c)::value;
    // The head gains and cos/sin of this wave's rows go out now and arrive
    // during the swap.
    const T* gain = kind == 0 ? static_cast<const T*>(a.q_norm) : static_cast<const T*>(a.k_norm) + layer * D;
    T g1[NI][4], g2[NI][4];  // gains of columns t and t + D/2
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        g1[ni][r] = gain[ni * 16 + 4 * q + r];
        g2[ni][r] = gain[HALF + ni * 16 + 4 * q + r];
      }
    const float* cos_t = a.cos_sin;
    const float* sin_t = a.cos_sin + (size_t)a.max_pos * HALF;
    f32x4 cs[MH][NI], sn[MH][NI];
#pragma unroll
    for (int u = 0; u < MH; ++u) {
      const int mi = WN * MH + u;
      int p = pos[u];
      if (p < 0 || p >= a.max_pos) {
        if (ok[mi] && q == 0) atomicOr(a.err, 1);
        p = p < 0 ? 0 : a.max_pos - 1;
      }
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        cs[u][ni] = *reinterpret_cast<const f32x4*>(cos_t + (size_t)p * HALF + ni * 16 + 4 * q);
        sn[u][ni] = *reinterpret_cast<const f32x4*>(sin_t + (size_t)p * HALF + ni * 16 + 4 * q);
      }
    }
    // Swap: hand the partner (wm, 1 - WN) this wave's half of the rows it
    // finishes, then take the partner's half of this wave's rows.
    block_barrier();  // the last fragment reads of the main loop are done
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int u = 0; u < MH; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          xch[(wave * XR + (ni * MH + u) * 4 + r) * 64 + lane] = acc[ni][(1 - WN) * MH + u][r];
    block_barrier();

    // Whole rows: RMSNorm over the head, then the rotation
    // (t, t + D/2) -> (x1 cos - x2 sin, x2 cos + x1 sin).
    const float scale = kind == 0 ? a.qscale : 1.0f;
#pragma unroll
    for (int u = 0; u < MH; ++u) {
      const int mi = WN * MH + u;
      const int b = sb[mi];
      f32x4 x1[NI], x2[NI];
      float ss = 0.f;
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float own = acc[ni][mi][r];
          const float oth = xch[(partner * XR + (ni * MH + u) * 4 + r) * 64 + lane];
          x1[ni][r] = WN == 0 ? own : oth;
          x2[ni][r] = WN == 0 ? oth : own;
          ss += own * own + oth * oth;
        }
      ss = quad_sum(ss);
      const float inv = rsqrtf(ss * (1.0f / D) + a.eps) * scale;
      if (!ok[mi]) continue;
      T* dst;
      if (kind == 0) {
        const int i = (J.m0 + wm * WM + mi * 16 + r16) % bs;
        dst = static_cast<T*>(a.qpack) + ((size_t)(b * nkv + j) * R + i * g + hh) * D;
      } else {
        dst = kc + (((size_t)blk[mi] * nkv + j) * kKeyTile + crow[mi] % kKeyTile) * D;
      }
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        f32x4 o1, o2;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float y1 = x1[ni][r] * inv * Elem<T>::to_f32(g1[ni][r]);
          const float y2 = x2[ni][r] * inv * Elem<T>::to_f32(g2[ni][r]);
          o1[r] = y1 * cs[u][ni][r] - y2 * sn[u][ni][r];
          o2[r] = y2 * cs[u][ni][r] + y1 * sn[u][ni][r];
        }
        Store4<T>::put(dst + ni * 16 + 4 * q, o1);
        Store4<T>::put(dst + HALF + ni * 16 + 4 * q, o2);
      }
    }
  };
  if (wn == 0) finish(std::integral_constant<int, 0>{});
  else finish(std::integral_constant<int, 1>{});
}

template <typename T, typename OutT>
hipError_t launch_t(const GemmArgs& args, int total_tiles, int bm, int bn, int kslices, hipStream_t s) {
  const dim3 grid(total_tiles, kslices), block(kGemmThreads);
  if constexpr (sizeof(T) == 2) {
    // 256 x 128 (bf16 only): 1.5 x the flops per streamed byte of 128 x 128
    if (bm == 256 && bn == 128) {
      hipLaunchKernelGGL((gemm_kernel<T, OutT, 256, 128>), grid, block, 0, s, args);
      return hipGetLastError();
    }
  }
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

template <typename T>
hipError_t launch_append_t(const GemmArgs& args, const NormRopeArgs& nr, int total_tiles, int bm, int d,
                           hipStream_t s) {
  const dim3 grid(total_tiles), block(kGemmThreads);
  if (d == 128) {
    if (bm == 128) hipLaunchKernelGGL((gemm_append_kernel<T, 128, 128>), grid, block, 0, s, args, nr);
    else hipLaunchKernelGGL((gemm_append_kernel<T, 64, 128>), grid, block, 0, s, args, nr);
  } else {
    if (bm == 128) hipLaunchKernelGGL((gemm_append_kernel<T, 128, 64>), grid, block, 0, s, args, nr);
    else hipLaunchKernelGGL((gemm_append_kernel<T, 64, 64>), grid, block, 0, s, args, nr);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_mx(const GemmArgs& args, int total_tiles, int bm, int bn, hipStream_t s) {
  if (total_tiles <= 0) return hipSuccess;
  const dim3 grid(total_tiles), block(kGemmThreads);
  if (bm == 128 && bn == 128)
    hipLaunchKernelGGL((gemm_kernel<__bf16, __bf16, 128, 128, true>), grid, block, 0, s, args);
  else if (bm == 128 && bn == 64)
    hipLaunchKernelGGL((gemm_kernel<__bf16, __bf16, 128, 64, true>), grid, block, 0, s, args);
  else if (bm == 64 && bn == 128)
    hipLaunchKernelGGL((gemm_kernel<__bf16, __bf16, 64, 128, true>), grid, block, 0, s, args);
  else
    hipLaunchKernelGGL((gemm_kernel<__bf16, __bf16, 64, 64, true>), grid, block, 0, s, args);
  return hipGetLastError();
}

hipError_t launch_gemm_append_mx(int head_dim, const GemmArgs& args, const NormRopeArgs& nr, int total_tiles,
                                 int bm, hipStream_t s) {
  if (total_tiles <= 0) return hipSuccess;
  const dim3 grid(total_tiles), block(kGemmThreads);
  if (head_dim == 128) {
    if (bm == 128) hipLaunchKernelGGL((gemm_append_kernel<__bf16, 128, 128, true>), grid, block, 0, s, args, nr);
    else hipLaunchKernelGGL((gemm_append_kernel<__bf16, 64, 128, true>), grid, block, 0, s, args, nr);
  } else {
    if (bm == 128) hipLaunchKernelGGL((gemm_append_kernel<__bf16, 128, 64, true>), grid, block, 0, s, args, nr);
    else hipLaunchKernelGGL((gemm_append_kernel<__bf16, 64, 64, true>), grid, block, 0, s, args, nr);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_append(int dtype, int head_dim, const GemmArgs& args, const NormRopeArgs& nr,
                              int total_tiles, int bm, hipStream_t stream) {
  if (total_tiles <= 0) return hipSuccess;
  if (dtype == 1) return launch_append_t<__bf16>(args, nr, total_tiles, bm, head_dim, stream);
  return launch_append_t<float>(args, nr, total_tiles, bm, head_dim, stream);
}

hipError_t launch_gemm_swiglu_wide(const GemmArgs& args, int total_tiles, hipStream_t stream) {
  if (total_tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL(gemm_swiglu_wide_kernel, dim3(total_tiles), dim3(kGemmThreads), 0, stream, args);
  return hipGetLastError();
}

hipError_t launch_gemm_swiglu(int dtype, const GemmArgs& args, int total_tiles, int bm, hipStream_t stream) {
  if (total_tiles <= 0) return hipSuccess;
  const dim3 grid(total_tiles), block(kGemmThreads);
  if (dtype == 1) {
    if (bm == 256) hipLaunchKernelGGL((gemm_swiglu_kernel<__bf16, 256>), grid, block, 0, stream, args);
    else if (bm == 128) hipLaunchKernelGGL((gemm_swiglu_kernel<__bf16, 128>), grid, block, 0, stream, args);
    else hipLaunchKernelGGL((gemm_swiglu_kernel<__bf16, 64>), grid, block, 0, stream, args);
  } else {
    if (bm == 128) hipLaunchKernelGGL((gemm_swiglu_kernel<float, 128>), grid, block, 0, stream, args);
    else hipLaunchKernelGGL((gemm_swiglu_kernel<float, 64>), grid, block, 0, stream, args);
  }
  return hipGetLastError();
}

hipError_t launch_gemm(int dtype, bool out_f32, const GemmArgs& args, int total_tiles, int bm, int bn,
                       int kslices, hipStream_t stream) {
  if (total_tiles <= 0) return hipSuccess;
  if (dtype == 1)
    return out_f32 ? launch_t<__bf16, float>(args, total_tiles, bm, bn, kslices, stream)
                   : launch_t<__bf16, __bf16>(args, total_tiles, bm, bn, kslices, stream);
  return launch_t<float, float>(args, total_tiles, bm, bn, kslices, stream);
}

}  // namespace dflash

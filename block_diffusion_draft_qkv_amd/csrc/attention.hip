// HK3: split-KV non-causal grouped-query attention of the draft block over the
// draft KV cache, and HK4: log-sum-exp merge of the pairs it split.
//
// What is computed (NeMo page "draft_qwen3": Qwen3DFlashAttention, scaling,
// _sliding_window_mask; "DFlash源码导读（二）" section on non-causal block
// attention): for sequence b with T_b keys and query head h of KV head
// j = h / g, o = softmax_t(d^-1/2 <q, k_t>) over every cached key t (the block
// included, no causal mask), restricted under a window W to
// |(T_b - bs + i) - t| < W; then o . V.
//
// Work split. The bs*g query rows that share KV head j (row i*g + hh) form one
// tile of up to 64 rows; consumer wave w (0-3) of the work-group owns rows
// 16w .. 16w+15. Every (sequence b, KV head j) pair owns the key tiles
// [lo_b, hi_b) (lo_b > 0 only under a sliding window); all tiles of all pairs
// are flattened head-major (j, then b, then tile) and cut into G ranges, one
// per work-group, of about equal cost whatever the ragged lengths: a range's
// tiles plus about a tile for every pair that starts inside it (the host's
// attn_bounds; a pair start stalls the stream while the previous segment's
// output is stored and the next queries are loaded). With G a multiple of nkv every head's
// tiles split at the same places, and the host deals the ranges so that the
// nkv work-groups covering the same tiles of all heads run on one XCD: they
// read neighbouring pieces of the same cache blocks together (measured at C3:
// 95 us against 108 us for b-major ranges dealt in contiguous runs of w,
// whose concurrent reads scatter over the cache whenever lengths are ragged).
// A range crosses pair boundaries; the part of a pair inside a range
// is a segment. A segment that is a whole pair writes the output directly; a
// pair cut by a range boundary leaves partials (un-normalised O in the
// element type, the exponent offset and the sum in fp32) in slot 2w (the
// range's first segment) or 2w+1 (its last),
// which HK4 merges in a launch of its own. Merging inside HK3 (the last
// part of a pair to finish folds it) needs the partials coherent across
// XCDs before the part counts itself in. Each XCD has its own L2, so that
// takes an L2 write-back per part or write-through stores and re-fetching
// loads, and every form measured cost more than the separate launch: at
// 32 ragged sequences the attention went from 96 us (+ 7 us merge) to 171 us
// with device-scope fences and to 120-127 us with coherent stores.
//
// Pipeline. One continuous stream of LDS-DMA loads (gfx950
// global_load_lds_dwordx4) runs through the whole range, crossing segment
// boundaries without draining: each step brings one K tile, one V^T tile and,
// when the step starts a segment, that pair's Q tile into an S-stage LDS ring
// while the previous stage is used. Two producer waves do nothing but issue
// these loads and wait for them, so a load queue that is full (the normal
// state when HBM is the bottleneck) stalls only them; the four consumer waves
// compute:
//   S^T (keys x queries) = K . Q^T     on MFMA, K from LDS, Q in VGPRs
//   online softmax in the log2 domain  (Q was pre-scaled by d^-1/2 log2 e)
//   O^T (d x queries)   += V^T . P^T   on MFMA, V^T from LDS, P^T from VGPRs
// The S^T accumulator gives every lane one query column and 4 keys per 16-key
// block, which is exactly the P^T operand layout the second product needs, so P
// never leaves registers; V is stored transposed in the cache so V^T tiles are
// plain row reads. For bf16 the key order inside a 32-key step is permuted
// (block 2s row 4q+r <-> key 8q+r, block 2s+1 row 4q+r <-> key 8q+4+r) so a
// lane's 8 P values are 8 consecutive keys, i.e. one 16-byte chunk of V^T.
// The exponent offset of a row is raised only when the row maximum passes it
// by more than kRescaleSlack (log2 units), so O is rescaled rarely; the result
// is exact for any offset because O and the sum share it.
// Keys past T_b inside the last tile are masked out of the softmax, and their
// V elements are zeroed in registers, so those keys contribute exact zeros to
// P.V whatever the dead rows of the cache hold.
#include "kernels.h"
#include "lds_dma.h"

namespace dflash {

namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr float kRescaleSlack = 8.0f;

// Wave roles of the 384-thread attention work-group: waves 0-3 compute (16
// query rows each), waves 4-5 only issue and await the LDS-DMA loads.
constexpr int kConsumerWaves = 4;
constexpr int kProducerWaves = 2;
constexpr int kAttnThreads = 64 * (kConsumerWaves + kProducerWaves);

// Shapes of the attention kernel for element type T and head_dim D.
template <typename T, int D> struct AttnShape {
  static constexpr int KT = (sizeof(T) == 4 && D == 128) ? 32 : 64;  // keys per tile
  static constexpr int E = 16 / (int)sizeof(T);                      // elements per 16 B chunk
  static constexpr int CPR = D * (int)sizeof(T) / 16;                // chunks per K or Q row
  static constexpr int VCPR = KT * (int)sizeof(T) / 16;              // chunks per V^T row
  static constexpr int NC = CPR / 4;                                 // reduction blocks over d
  static constexpr int NKS = VCPR / 4;                               // reduction blocks over keys
  static constexpr int KB = KT / 16;                                 // 16-key S^T blocks per tile
  static constexpr int K_BYTES = KT * D * (int)sizeof(T);
  static constexpr int TILE = 2 * K_BYTES;                           // K + V^T
  static constexpr int Q_BYTES = kMaxQueryRows * D * (int)sizeof(T);
  // 1 KB DMA blocks per producer wave: of a K tile (and of a V^T tile), of a Q tile.
  static constexpr int KPP = K_BYTES / 1024 / kProducerWaves;
  static constexpr int QPP = Q_BYTES / 1024 / kProducerWaves;
  static constexpr int QSLOT = Q_BYTES;
  static constexpr int S = 3 * (TILE + QSLOT) <= 150 * 1024 ? 3 : 2; // ring depth
  static constexpr int LDS = S * (TILE + QSLOT);
  static constexpr int DB = D / 16;
  static_assert(K_BYTES % (1024 * kProducerWaves) == 0, "a K tile splits into 1 KB blocks per producer");
  static_assert(Q_BYTES % (1024 * kProducerWaves) == 0, "a Q tile splits into 1 KB blocks per producer");
  static_assert(sizeof(T) == 4 || KT % 32 == 0, "bf16 P packing pairs 16-key blocks");
  static_assert(2 * (S - 1) * KPP + (S - 1) * QPP <= 63, "outstanding DMA blocks must fit vmcnt");
};

// Per-sequence key tiles [lo, lo + cnt) of the attention (uniform per wave).
__device__ inline void seq_tiles(const AttnArgs& a, int b, int kt, int& lo, int& cnt) {
  const int T = a.seq.len[b] + (a.seq.ctx_off[b + 1] - a.seq.ctx_off[b]) + a.bs;
  int first = 0;
  if (a.window > 0) {
    first = T - a.bs - a.window + 1;
    if (first < 0) first = 0;
  }
  lo = first / kt;
  cnt = (T + kt - 1) / kt - lo;
}



// Which key each lane's S^T accumulator row stands for (see the file comment).
template <typename T> __device__ inline int key_of(int kb, int m);
template <> __device__ inline int key_of<__bf16>(int kb, int m) {
  return 32 * (kb >> 1) + 8 * (m >> 2) + 4 * (kb & 1) + (m & 3);
}
template <> __device__ inline int key_of<float>(int kb, int m) { return 16 * kb + m; }

// LDS chunk swizzles. A ds_read_b128 of an MFMA operand reads 16 rows (lane %
// 16) at logical chunks 4 c + lane / 16; the chunk is stored at logical ^
// swz(row). gfx950's LDS has 128 banks of 4 bytes and serves a ds_read_b128 as
// two 8-byte halves, 32 lanes a pass (fitted to SQ_LDS_BANK_CONFLICT: a
// contiguous 1 KB read stalls 0 cycles, 16 rows of 128 bytes at one chunk 12,
// a swizzle built for 8- or 16-lane passes 4). A pass is conflict-free when
// its 32 lanes' 8-byte pieces fall on distinct bank pairs, (address / 8) % 64:
//   * 128-byte rows (CPR 8: V^T tiles, and K and Q at head_dim 64 in bf16):
//     the bank pair is (r % 4) * 16 + 2 c + h, so the rows r, r + 4, r + 8,
//     r + 12 of one residue class, read at the chunk pair {x, x ^ 1} of a
//     pass, need distinct bits 1-2 of the chunk: ((r >> 2) & 3) << 1;
//   * 256-byte rows (CPR 16): the pair is (r % 2) * 32 + 2 c + h: r % 16;
//   * 512-byte rows (CPR 32, fp32 at head_dim 128): the pair is 2 c + h, so
//     the 16 rows need 16 distinct chunk pairs: (r % 16) << 1.
// V^T and Q reads take 16 consecutive rows and use aswz; for K the 16 rows are
// key_of(kb, 0..15) and kswz depends only on bits kb does not change. (Moving
// V^T off the 8/16-lane swizzle, which stalled 4 cycles a read, measured 0.1
// to 0.7 us faster at C3 in same-box comparisons: the kernel is bound by its
// stream, not by these reads.)
template <int CPR> __device__ inline int aswz(int row) {
  if constexpr (CPR >= 32) return (row & 15) << 1;
  else if constexpr (CPR == 16) return row & 15;
  else if constexpr (CPR == 8) return ((row >> 2) & 3) << 1;
  else return ((row >> 1) ^ (row >> 2)) & 3;
}
template <typename T, int CPR> __device__ inline int kswz(int row) {
  if constexpr (sizeof(T) == 4) return CPR >= 32 ? (row & 15) << 1 : row & 15;
  else if constexpr (CPR == 16) return (row & 3) | ((row >> 1) & 12);
  else return (((row >> 1) & 1) | ((row >> 2) & 6)) ^ ((row & 1) << 2);
}
// Wait until at most n DMA blocks are outstanding, n being one of the three
// group sizes a step can leave in flight.
template <int KVW, int QW> __device__ inline void vm_wait(int n) {
  if (n == KVW + QW) DFLASH_VMWAIT(KVW + QW);
  else if (n == KVW) DFLASH_VMWAIT(KVW);
  else DFLASH_VMWAIT(0);
}

// Max / sum over the four lanes that hold one query row (l, l^16, l^32, l^48).
__device__ inline float max4(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ inline float sum4(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Bit mask keeping the first n (< elements per chunk) elements of a 16-byte chunk.
template <typename T> __device__ inline u32x4 keep_mask(int n);
template <> __device__ inline u32x4 keep_mask<__bf16>(int n) {
  u32x4 m;
#pragma unroll
  for (int w = 0; w < 4; ++w) m[w] = (2 * w < n ? 0x0000ffffu : 0u) | (2 * w + 1 < n ? 0xffff0000u : 0u);
  return m;
}
template <> __device__ inline u32x4 keep_mask<float>(int n) {
  u32x4 m;
#pragma unroll
  for (int w = 0; w < 4; ++w) m[w] = w < n ? 0xffffffffu : 0u;
  return m;
}

__device__ inline u32x4 pack_p_bf16(const f32x4& p0, const f32x4& p1) {
  bf16x8 v;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    v[r] = (__bf16)p0[r];
    v[4 + r] = (__bf16)p1[r];
  }
  return __builtin_bit_cast(u32x4, v);
}

// Four consecutive outputs of one row as one 16-byte (fp32) or 8-byte (bf16) store.
// MXFP8 output helpers (the same rule as the activation quantiser: values
// rounded to bf16, shared exponent floor(log2 amax) - 8 clamped to
// [-127, 127], elements x / 2^exponent clamped to +-448 and converted by the
// packed FP8 instruction, round to nearest even).
__device__ inline f32x4 round_bf16x4(const f32x4& v) {
  f32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = (float)(__bf16)v[i];
  return r;
}
__device__ inline float absmax4(const f32x4& v) {
  return fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
}
// Scale byte of a block maximum and the power of two that maps the block.
__device__ inline int mx_scale_byte(float amax, float& mul) {
  const int sbyte = min(max((int)((__float_as_uint(amax) >> 23) & 0xff) - 8, 0), 254);
  mul = __uint_as_float((uint32_t)(254 - sbyte) << 23);
  return sbyte;
}
__device__ inline uint32_t mx_codes4(const f32x4& y, float mul) {
  f32x4 t;
#pragma unroll
  for (int i = 0; i < 4; ++i) t[i] = fminf(fmaxf(y[i] * mul, -448.f), 448.f);
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(t[0], t[1], 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(t[2], t[3], lo, true);
}
// Scale byte of 32-column block `cb` of row `m` in the step-major layout.
__device__ inline size_t mx_scale_at(const MxOut& mo, int m, int cb) {
  return ((size_t)(cb >> 2) * mo.rows + m) * 4 + (cb & 3);
}

template <typename T> __device__ inline void store4(T* p, const f32x4& v);
template <> __device__ inline void store4<float>(float* p, const f32x4& v) {
  *reinterpret_cast<f32x4*>(p) = v;
}
template <> __device__ inline void store4<__bf16>(__bf16* p, const f32x4& v) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  bf16x4 o;
#pragma unroll
  for (int r = 0; r < 4; ++r) o[r] = (__bf16)v[r];
  *reinterpret_cast<bf16x4*>(p) = o;
}
template <typename T> __device__ inline f32x4 load4(const T* p);
template <> __device__ inline f32x4 load4<float>(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
template <> __device__ inline f32x4 load4<__bf16>(const __bf16* p) {
  const u32x2 w = *reinterpret_cast<const u32x2*>(p);  // element 0 in the low half
  return f32x4{__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u), __uint_as_float(w[1] << 16),
               __uint_as_float(w[1] & 0xffff0000u)};
}

// Position in the flattened work: pair (b, j), key tile, the pair's tiles.
struct Cursor {
  int b, j, tile, lo, hi;
};



template <typename T, int D>
__global__ __launch_bounds__(kAttnThreads, 1) void attn_splitkv_kernel(AttnArgs a) {
  using Sh = AttnShape<T, D>;
  constexpr int KT = Sh::KT, E = Sh::E, CPR = Sh::CPR, VCPR = Sh::VCPR, NC = Sh::NC, NKS = Sh::NKS;
  constexpr int KB = Sh::KB, DB = Sh::DB, S = Sh::S, TILE = Sh::TILE, K_BYTES = Sh::K_BYTES;
  constexpr int KPP = Sh::KPP, QPP = Sh::QPP, QSLOT = Sh::QSLOT;
  __shared__ u32x4 lds[Sh::LDS / 16];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nkv = a.nkv, R = a.R;
  const int w = a.range_of[blockIdx.x];
  const int total = a.count[blockIdx.x];
  const uint32_t lds0 = lds_base(lds);
  const uint32_t qlds0 = lds0 + S * TILE;

  // Producers and consumers walk the same flattened tiles from flat tile f0,
  // whose pair and tile the host worked out.
  Cursor cur;
  {
    const uint32_t st = a.start[w];
    const int pair0 = (int)(st & 0xffffu);
    cur.b = pair0 / nkv;
    cur.j = pair0 % nkv;
    cur.tile = (int)(st >> 16);
    int lo, cnt;
    seq_tiles(a, cur.b, KT, lo, cnt);
    cur.lo = lo;
    cur.hi = lo + cnt;
  }
  auto advance = [&](Cursor& c) {
    if (++c.tile == c.hi) {
      if (++c.b == a.seq.batch) {  // past the last pair the cursor is never used
        c.b = 0;
        ++c.j;
      }
      int lo, cnt;
      seq_tiles(a, c.b, KT, lo, cnt);
      c.lo = lo;
      c.hi = lo + cnt;
      c.tile = c.lo;
    }
  };

  // Step n lives in ring stage n % S. Barrier n (one per step) is passed once
  // stage n has landed (the producers wait for it first) and the consumers
  // have finished step n - 1, whose stage the producers refill right after it.
  if (wave >= kConsumerWaves) {
    // ---------------------------------------------------------- producers
    const int pw = wave - kConsumerWaves;
    const char* Kc = static_cast<const char*>(a.kc);
    const char* Vc = static_cast<const char*>(a.vc);
    const char* Qp = static_cast<const char*>(a.q);
    // Source offsets (relative to the tile's first row) of this wave's 1 KB
    // blocks i * kProducerWaves + pw; each lane fetches the chunk that belongs
    // at its swizzled LDS position.
    uint32_t kdma[KPP], vdma[KPP], qdma[QPP];
#pragma unroll
    for (int i = 0; i < KPP; ++i) {
      const int blk = i * kProducerWaves + pw, row = blk * (64 / CPR) + lane / CPR;
      const int c = (lane % CPR) ^ kswz<T, CPR>(row);
      kdma[i] = (uint32_t)(row * D + c * E) * (uint32_t)sizeof(T);
    }
    const int vstride = a.map.vstride();  // elements between V^T rows of a 64-row block
#pragma unroll
    for (int i = 0; i < KPP; ++i) {
      const int blk = i * kProducerWaves + pw, row = blk * (64 / VCPR) + lane / VCPR;
      const int c = (lane % VCPR) ^ aswz<VCPR>(row);
      vdma[i] = (uint32_t)(row * vstride + c * E) * (uint32_t)sizeof(T);
    }
#pragma unroll
    for (int i = 0; i < QPP; ++i) {
      const int blk = i * kProducerWaves + pw, row = blk * (64 / CPR) + lane / CPR;
      const int c = (lane % CPR) ^ aswz<CPR>(row);
      qdma[i] = (uint32_t)(row * D + c * E) * (uint32_t)sizeof(T);
    }
    // A paged cache's physical block of the cursor's tile is loaded one step
    // ahead (right after the cursor moves), so the lookup's latency overlaps
    // the wait for the previous step instead of delaying the next issue. It
    // is a scalar load: a vector one would make the compiler wait for the
    // whole vector-memory counter, i.e. for every DMA block still in flight.
    const bool paged = a.map.bt != nullptr;
    int phys = 0;
    auto lookup = [&]() {
      if (paged && cur.b < a.seq.batch) phys = a.map.entry_uniform(cur.b, cur.tile * KT);
    };
    lookup();
    // Issue step n (its tile is at the cursor; the Q tile too if a segment
    // starts there) and return the number of DMA blocks this wave issued.
    int iseg = 0;
    auto issue = [&](int n) -> int {
      const size_t pair = (size_t)cur.b * nkv + cur.j;
      int blocks = 2 * KPP;
      if (n == 0 || cur.tile == cur.lo) {
        const uint32_t qs = qlds0 + (uint32_t)(iseg % S) * QSLOT;
        const void* qsrc = uniform_ptr(Qp + pair * R * D * sizeof(T));
#pragma unroll
        for (int i = 0; i < QPP; ++i)
          lds_dma16<true>(qdma[i], qsrc, qs + (uint32_t)(i * kProducerWaves + pw) * 1024u);
        ++iseg;
        blocks += QPP;
      }
      const uint32_t sl = lds0 + (uint32_t)(n % S) * TILE;
      const void* kt;
      const void* vt;
      {
        // the tile's 64-row block (CacheMap::block_of; the table entry was loaded ahead)
        const size_t pb = paged ? (size_t)a.map.clamp_block(phys)
                                : (size_t)cur.b * (a.cap / kKeyTile) + (size_t)(cur.tile * KT) / kKeyTile;
        const size_t blk = pb * nkv + cur.j, off = (size_t)(cur.tile * KT) % kKeyTile;
        kt = uniform_ptr(Kc + (blk * kKeyTile + off) * D * sizeof(T));
        vt = uniform_ptr(Vc + (blk * D * kKeyTile + off) * sizeof(T));
      }
#pragma unroll
      for (int i = 0; i < KPP; ++i)
        lds_dma16<true>(kdma[i], kt, sl + (uint32_t)(i * kProducerWaves + pw) * 1024u);
#pragma unroll
      for (int i = 0; i < KPP; ++i)
        lds_dma16<true>(vdma[i], vt, sl + K_BYTES + (uint32_t)(i * kProducerWaves + pw) * 1024u);
      advance(cur);
      lookup();
      return blocks;
    };
    // Steps 0 .. S-2 go out before the first barrier; `pending` is the number
    // of blocks issued after the step the next wait is for.
    int sizes[S - 1];
#pragma unroll
    for (int n = 0; n < S - 1; ++n) sizes[n] = n < total ? issue(n) : 0;
    int pending = S >= 3 ? sizes[S - 2] : 0;
    for (int it = 0; it < total; ++it) {
      vm_wait<2 * KPP, QPP>(pending);
      block_barrier();
      int next = 0;
      if (it + S - 1 < total) next = issue(it + S - 1);
      pending = S >= 3 ? next : 0;
    }
    return;
  }

  // ------------------------------------------------------------ consumers
  const int q = lane >> 4, r16 = lane & 15;
  const int g = a.nq / nkv;
  const bool active = wave * 16 < R;
  const int qrow = wave * 16 + r16;
  const bool qvalid = qrow < R;

  // Per-lane LDS byte offsets, fixed for the whole kernel: K operand of block
  // kb, chunk c = koff[c] + kb_off(kb); V^T operand of d-block db, key chunk
  // ks = voff[ks] + db_off(db); Q row chunks.
  uint32_t koff[NC], voff[NKS], qoff[NC];
  {
    const int krow = key_of<T>(0, r16), ksw = kswz<T, CPR>(krow);
#pragma unroll
    for (int c = 0; c < NC; ++c) koff[c] = (uint32_t)(krow * CPR + ((4 * c + q) ^ ksw)) * 16u;
    const int vsw = aswz<VCPR>(r16);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) voff[ks] = (uint32_t)(r16 * VCPR + ((4 * ks + q) ^ vsw)) * 16u + K_BYTES;
    const int qsw = aswz<CPR>(qrow);
#pragma unroll
    for (int c = 0; c < NC; ++c) qoff[c] = (uint32_t)(qrow * CPR + ((4 * c + q) ^ qsw)) * 16u;
  }

  float m_run = kNegInf, l_run = 0.f;
  f32x4 acc[DB];
  u32x4 qf[NC];
  int cseg = 0;
  int seg_start_flat = 0;       // step index where the current segment began
  bool seg_from_lo = false;     // the segment starts at the pair's first tile
  int tb = 0, qpos = 0;

  for (int it = 0; it < total; ++it) {
    block_barrier();
    const bool seg_begin = it == 0 || cur.tile == cur.lo;
    const bool seg_end = it + 1 == total || cur.tile + 1 == cur.hi;
    if (seg_begin) {
      seg_start_flat = it;
      seg_from_lo = cur.tile == cur.lo;
      tb = a.seq.len[cur.b] + (a.seq.ctx_off[cur.b + 1] - a.seq.ctx_off[cur.b]) + a.bs;
      qpos = tb - a.bs + (qvalid ? qrow / g : 0);
      if (active) {
        const uint32_t qs = qlds0 + (uint32_t)(cseg % S) * QSLOT;
#pragma unroll
        for (int c = 0; c < NC; ++c) qf[c] = qvalid ? lds_read16(qs + qoff[c]) : u32x4{0, 0, 0, 0};
      }
      ++cseg;
      m_run = kNegInf;
      l_run = 0.f;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    if (active) {
      const uint32_t sl = lds0 + (uint32_t)(it % S) * TILE;
      const int t0 = cur.tile * KT;
      // Every K fragment of the tile is read before the first MFMA, and the
      // MFMAs cycle over the KB independent accumulators, so LDS latency is
      // paid once per tile rather than once per MFMA.
      u32x4 kf[KB][NC];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int c = 0; c < NC; ++c)
          kf[kb][c] = lds_read16(sl + koff[c] + (uint32_t)(key_of<T>(kb, 0) * CPR * 16));
      f32x4 s[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) Mfma<T>::chunk(s[kb], kf[kb][c], qf[c]);
      // The V^T fragments are read now and land while the softmax runs.
      u32x4 vf[DB][NKS];
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
          vf[db][ks] = lds_read16(sl + voff[ks] + (uint32_t)(db * 16 * VCPR * 16));
      if (t0 + KT > tb) {
        // Keys at or past T_b get zero weight, but the cache there may hold
        // anything (not even a number): zero those V elements so that 0 * V
        // stays 0. Chunk 4ks + q of a V^T row holds keys (4ks + q) * E ...
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const int nvalid = tb - (t0 + (4 * ks + q) * E);
          if (nvalid < E) {
            const u32x4 keep = keep_mask<T>(nvalid);
#pragma unroll
            for (int db = 0; db < DB; ++db) vf[db][ks] &= keep;
          }
        }
      }
      // Under a window W the band cuts into a tile only where the tile starts
      // before T_b - W (the query at T_b - 1 loses its oldest keys there) or
      // where W < bs (queries lose keys of the block ahead of them): for
      // t0 >= T_b - W and W >= bs every query q in [T_b - bs, T_b) and key t
      // in [t0, T_b) have q - t <= W - 1 and t - q <= bs - 1 <= W - 1.
      const bool band = a.window > 0 && (t0 < tb - a.window || a.window < a.bs);
      if (t0 + KT > tb || band) {
        // Key t survives if t < T_b and, under a window W, -W < qpos - t < W,
        // i.e. 0 <= qpos - t + W - 1 <= 2W - 2 as one unsigned compare (the
        // host passes W < capacity, so nothing wraps; without a window the
        // limit admits every key).
        const uint32_t wlim = a.window > 0 ? (uint32_t)(2 * a.window - 2) : 0xffffffffu;
        const uint32_t wbias = a.window > 0 ? (uint32_t)(a.window - 1) : 0u;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = t0 + key_of<T>(kb, 4 * q + r);
            const bool ok = (key < tb) & ((uint32_t)(qpos - key) + wbias <= wlim);
            s[kb][r] = ok ? s[kb][r] : kNegInf;
          }
      }
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        mx = fmaxf(fmaxf(fmaxf(mx, s[kb][0]), fmaxf(s[kb][1], s[kb][2])), s[kb][3]);
      mx = max4(mx);
      // Raise the exponent offset only when this row's maximum passed it by
      // more than the slack; the (rare) rescale is wave-uniform.
      const bool raise = mx > m_run + kRescaleSlack;
      if (__builtin_amdgcn_ballot_w64(raise) != 0) {
        const float m_new = raise ? mx : m_run;
        const float alpha = raise ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db] *= alpha;
        m_run = m_new;
      }
      const float m_use = m_run == kNegInf ? 0.f : m_run;
      f32x4 p[KB];
      float psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          p[kb][r] = __builtin_amdgcn_exp2f(s[kb][r] - m_use);
          psum += p[kb][r];
        }
      l_run += psum;
      if constexpr (sizeof(T) == 2) {
        u32x4 pf[NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) pf[ks] = pack_p_bf16(p[2 * ks], p[2 * ks + 1]);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
          for (int db = 0; db < DB; ++db) Mfma<T>::chunk(acc[db], vf[db][ks], pf[ks]);
      } else {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
          for (int db = 0; db < DB; ++db)
            Mfma<T>::chunk(acc[db], vf[db][ks], __builtin_bit_cast(u32x4, p[ks]));
      }

      if (seg_end) {
        const float lt = sum4(l_run);
        const bool full = seg_from_lo && cur.tile + 1 == cur.hi;
        if (qvalid) {
          if (full) {
            const float inv = 1.0f / lt;
            const int i = qrow / g, hh = qrow % g;
            if (a.mxo.codes != nullptr) {
              // MXFP8 o_proj input: a 32-column block is slices 2k, 2k+1 of the
              // four lanes (q = 0..3) that hold this row.
              const int m = cur.b * a.bs + i, col0 = (cur.j * g + hh) * D;
              uint8_t* crow = a.mxo.codes + (size_t)m * a.mxo.ld + col0;
#pragma unroll
              for (int k = 0; k < D / 32; ++k) {
                const f32x4 y0 = round_bf16x4(acc[2 * k] * inv), y1 = round_bf16x4(acc[2 * k + 1] * inv);
                float am = fmaxf(absmax4(y0), absmax4(y1));
                am = fmaxf(am, __shfl_xor(am, 16, 64));
                am = fmaxf(am, __shfl_xor(am, 32, 64));
                float mul;
                const int sb = mx_scale_byte(am, mul);
                *reinterpret_cast<uint32_t*>(crow + (2 * k) * 16 + 4 * q) = mx_codes4(y0, mul);
                *reinterpret_cast<uint32_t*>(crow + (2 * k + 1) * 16 + 4 * q) = mx_codes4(y1, mul);
                if (q == 0) a.mxo.scales[mx_scale_at(a.mxo, m, col0 / 32 + k)] = (uint8_t)sb;
              }
            } else {
              T* orow = static_cast<T*>(a.o) +
                        ((size_t)(cur.b * a.bs + i) * a.nq + (size_t)(cur.j * g + hh)) * D;
#pragma unroll
              for (int db = 0; db < DB; ++db) store4<T>(orow + db * 16 + 4 * q, acc[db] * inv);
            }
          } else {
            const int slot = 2 * (int)w + (seg_start_flat == 0 ? 0 : 1);
            T* po = static_cast<T*>(a.part_o) + ((size_t)slot * kMaxQueryRows + qrow) * D;
#pragma unroll
            for (int db = 0; db < DB; ++db) store4<T>(po + db * 16 + 4 * q, acc[db]);
            if (q == 0) {
              float* pm = a.part_ml + ((size_t)slot * kMaxQueryRows + qrow) * 2;
              pm[0] = m_run;
              pm[1] = lt;
            }
          }
        }
      }
    }
    advance(cur);
  }
}

// HK4: one work-group column per split pair (host list), one thread per four
// outputs of a row. o = sum_p 2^(m_p - M) O_p / sum_p 2^(m_p - M) l_p with
// M = max_p m_p, folded over the parts four at a time so that each group of
// loads goes out together. Part 0 sits in slot first_slot, part p > 0 (the
// work-group first + p, whose range starts inside the pair) in slot
// 2 (first + p).
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(MergeArgs a) {
  constexpr int TPR = D / 4, RPG = 256 / TPR;
  const int e = blockIdx.x;
  const int pair = a.pair[e], s0 = a.first_slot[e], np = a.nparts[e];
  const int row = blockIdx.y * RPG + (int)threadIdx.x / TPR;
  if (row >= a.R) return;
  const int d4 = ((int)threadIdx.x % TPR) * 4;
  auto slot = [&](int p) { return p == 0 ? s0 : (s0 & ~1) + 2 * p; };

  float M = kNegInf, den = 0.f;
  f32x4 num = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int p0 = 0; p0 < np; p0 += 4) {
    float m[4], l[4];
    f32x4 o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      m[k] = kNegInf;
      l[k] = 0.f;
      o[k] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (p0 + k < np) {
        const size_t sr = (size_t)slot(p0 + k) * kMaxQueryRows + row;
        m[k] = a.part_ml[sr * 2];
        l[k] = a.part_ml[sr * 2 + 1];
        o[k] = load4<T>(static_cast<const T*>(a.part_o) + sr * D + d4);
      }
    }
    const float Mn = fmaxf(fmaxf(M, fmaxf(m[0], m[1])), fmaxf(m[2], m[3]));
    const float Mu = Mn == kNegInf ? 0.f : Mn;  // rows no key reached yet
    const float sc = __builtin_amdgcn_exp2f(M - Mu);
    den *= sc;
    num *= sc;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float wk = __builtin_amdgcn_exp2f(m[k] - Mu);
      den += wk * l[k];
      num += wk * o[k];
    }
    M = Mn;
  }
  const int g = a.nq / a.nkv, b = pair / a.nkv, j = pair % a.nkv;
  const int i = row / g, hh = row % g;
  if (a.mxo.codes != nullptr) {
    // MXFP8 o_proj input: a 32-column block is 8 neighbouring threads of the row
    const int m = b * a.bs + i, col0 = (j * g + hh) * D;
    const f32x4 y = round_bf16x4(num * (1.0f / den));
    float am = absmax4(y);
    am = fmaxf(am, __shfl_xor(am, 1, 64));
    am = fmaxf(am, __shfl_xor(am, 2, 64));
    am = fmaxf(am, __shfl_xor(am, 4, 64));
    float mul;
    const int sb = mx_scale_byte(am, mul);
    *reinterpret_cast<uint32_t*>(a.mxo.codes + (size_t)m * a.mxo.ld + col0 + d4) = mx_codes4(y, mul);
    if (d4 % 32 == 0) a.mxo.scales[mx_scale_at(a.mxo, m, (col0 + d4) / 32)] = (uint8_t)sb;
    return;
  }
  T* orow = static_cast<T*>(a.o) + ((size_t)(b * a.bs + i) * a.nq + (size_t)(j * g + hh)) * D;
  store4<T>(orow + d4, num * (1.0f / den));
}

template <typename T, int D> int wgs_per_cu() { return (160 * 1024) / AttnShape<T, D>::LDS; }

}  // namespace

int attn_wgs_per_cu(int dtype, int head_dim) {
  if (dtype == 1) return head_dim == 128 ? wgs_per_cu<__bf16, 128>() : wgs_per_cu<__bf16, 64>();
  return head_dim == 128 ? wgs_per_cu<float, 128>() : wgs_per_cu<float, 64>();
}

int attn_kv_in_flight(int dtype, int head_dim) {
  if (dtype == 1)
    return head_dim == 128 ? (AttnShape<__bf16, 128>::S - 1) * AttnShape<__bf16, 128>::TILE
                           : (AttnShape<__bf16, 64>::S - 1) * AttnShape<__bf16, 64>::TILE;
  return head_dim == 128 ? (AttnShape<float, 128>::S - 1) * AttnShape<float, 128>::TILE
                         : (AttnShape<float, 64>::S - 1) * AttnShape<float, 64>::TILE;
}

int attn_key_tile(int dtype, int head_dim) {
  if (dtype == 1) return head_dim == 128 ? AttnShape<__bf16, 128>::KT : AttnShape<__bf16, 64>::KT;
  return head_dim == 128 ? AttnShape<float, 128>::KT : AttnShape<float, 64>::KT;
}

hipError_t launch_attn(int dtype, int head_dim, const AttnArgs& args, hipStream_t stream) {
  if (args.G <= 0) return hipSuccess;
  const dim3 grid(args.G), block(kAttnThreads);
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

hipError_t launch_merge(int dtype, int head_dim, const MergeArgs& args, hipStream_t stream) {
  if (args.n_split <= 0) return hipSuccess;
  const int rows_per_group = 256 / (head_dim / 4);
  const dim3 grid(args.n_split, (args.R + rows_per_group - 1) / rows_per_group), block(256);
  if (dtype == 1) {
    if (head_dim == 128)
      hipLaunchKernelGGL((attn_merge_kernel<__bf16, 128>), grid, block, 0, stream, args);
    else
      hipLaunchKernelGGL((attn_merge_kernel<__bf16, 64>), grid, block, 0, stream, args);
  } else {
    if (head_dim == 128)
      hipLaunchKernelGGL((attn_merge_kernel<float, 128>), grid, block, 0, stream, args);
    else
      hipLaunchKernelGGL((attn_merge_kernel<float, 64>), grid, block, 0, stream, args);
  }
  return hipGetLastError();
}

}  // namespace dflash

/*
 * dflash.h -- C ABI of the DFlash draft-model attention layer step on AMD
 * Instinct MI355X (gfx950).
 *
 * One call runs the layer that the pages call Qwen3DFlashAttention for a batch
 * of sequences: the draft block (one anchor plus block_size-1 mask tokens) is
 * projected to Q, K and V, the new target-context rows to K and V with the same
 * weights; q and k are RMS-normalised per head, rotated with neox RoPE (keys at
 * every position of the window [new context | block], queries at its trailing
 * block_size positions), appended to the draft KV cache, and the block's
 * queries attend non-causally (optionally inside a sliding-window band) over
 * every cached key; o_proj maps the heads back to the hidden size.
 *   - NeMo AutoModel page "draft_qwen3": Qwen3DFlashAttention, forward,
 *     apply_rotary_pos_emb, _sliding_window_mask.
 *   - vLLM page "qwen3_dflash": DFlashQwen3Attention.__init__ and forward
 *     (fused qkv_proj with rows q|k|v, per-head q_norm/k_norm, neox RoPE,
 *     o_proj, no bias).
 *   - "DFlash源码导读（二）" (cf-1.com), sections 1-5: QK-RMSNorm, dual-stream
 *     K/V concat, full-window RoPE, cache update and crop(start), non-causal
 *     block attention.
 *
 * Conventions shared by every entry point:
 *   - Every function returns a dflash_status (0 = DFLASH_OK). Nothing throws
 *     across the ABI.
 *   - All arguments are validated on the host before any work is enqueued; on
 *     an error nothing is launched and no state (cache lengths, outputs)
 *     changes.
 *   - Device pointers are borrowed: the caller allocates and frees every buffer
 *     passed in and keeps weights alive for the layer's lifetime. The library
 *     allocates only each handle's own cos/sin table and error flag (at
 *     create), and an MXFP8 layer or precompute handle its repacked weight
 *     scales; it also holds one static scratch array per device for
 *     dflash_attn_step_noalloc.
 *   - Work is enqueued on the caller's stream (a hipStream_t passed as void*;
 *     NULL is the default stream) and the calls return without synchronising,
 *     except dflash_layer_poll_error, dflash_layer_kernel_times and
 *     dflash_ctxkv_poll_error.
 *   - Element type of every activation, weight and cache buffer is the
 *     config's dtype (fp32 or bf16), except the MXFP8 weights of
 *     dflash_layer_create_mxfp8 and dflash_ctxkv_create_mxfp8; accumulation
 *     is fp32.
 */
#ifndef DFLASH_H
#define DFLASH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DFLASH_OK = 0,
    DFLASH_ERR_ARG = 1,          /* null pointer, bad index, bad flag value           */
    DFLASH_ERR_SHAPE = 2,        /* sizes inconsistent or not divisible as required   */
    DFLASH_ERR_CAPACITY = 3,     /* a step would write past the cache capacity        */
    DFLASH_ERR_RANGE = 4,        /* crop past the length; position outside the table  */
    DFLASH_ERR_UNSUPPORTED = 5,  /* valid but not built (head_dim, batch, query rows) */
    DFLASH_ERR_HIP = 6,          /* a HIP runtime call failed                         */
    DFLASH_ERR_WORKSPACE = 7     /* workspace missing or smaller than required        */
} dflash_status;

typedef enum { DFLASH_F32 = 0, DFLASH_BF16 = 1 } dflash_dtype;

/* Largest batch one step (or precompute append) accepts. Per-sequence lengths
 * ride in the kernel arguments of one launch for at most DFLASH_LAUNCH_BATCH
 * sequences; a larger batch runs as consecutive launches over runs of at most
 * DFLASH_LAUNCH_BATCH sequences (they are independent), each run checked
 * before the first is enqueued, sharing one workspace sized for one run. */
#define DFLASH_MAX_BATCH 65536
#define DFLASH_LAUNCH_BATCH 256

/* Layer shape and numerics. Limits checked by dflash_layer_create:
 *   head_dim in {64, 128}; n_q_heads % n_kv_heads == 0; n_kv_heads <= 256;
 *   block_size * (n_q_heads / n_kv_heads) <= 64 (the query rows that share one
 *   KV head, packed into MFMA tiles); hidden % 64 == 0;
 *   rope_theta > 0; rms_eps >= 0; sliding_window >= 0; max_position >= 1. */
typedef struct {
    int32_t hidden;          /* H                                                 */
    int32_t n_q_heads;       /* nq                                                */
    int32_t n_kv_heads;      /* nkv                                               */
    int32_t head_dim;        /* d                                                 */
    int32_t block_size;      /* bs: draft tokens per block (queries per sequence) */
    int32_t sliding_window;  /* 0: full attention; W > 0: key t visible to block
                                query i iff |(T - bs + i) - t| < W (strict band)  */
    int32_t max_position;    /* positions must lie in [0, max_position)           */
    int32_t dtype;           /* dflash_dtype                                      */
    double rope_theta;       /* RoPE base; inv_freq[t] = theta^(-2t/d)            */
    double rms_eps;          /* RMSNorm eps, added to the mean square             */
} dflash_config;

/* Weights, device memory, row-major in the config dtype (nn.Linear [out, in]). */
typedef struct {
    const void* w_qkv;   /* [(nq + 2*nkv) * d, H]: rows of all q heads, then all k
                            heads, then all v heads (head h = rows h*d .. h*d+d-1) */
    const void* w_o;     /* [H, nq * d]                                           */
    const void* q_norm;  /* [d] RMSNorm gain of q                                 */
    const void* k_norm;  /* [d] RMSNorm gain of k                                 */
} dflash_weights;

/* Draft KV cache of `batch` sequences, device memory owned by the caller.
 * Rows come in blocks of 64 (capacity / 64 blocks per sequence); block i of
 * sequence b holds rows 64 i .. 64 i + 63 of every KV head:
 *   k: [batch][capacity / 64][n_kv][64][head_dim]   K rows, key-major
 *   v: [batch][capacity / 64][n_kv][head_dim][64]   V transposed within the
 *                                          block (key index contiguous), so
 *                                          that the P*V contraction streams
 *                                          it directly
 * Every 64-key tile of one head is one contiguous piece of K and one of V, at
 * the same offsets whatever the capacity. (Row-major [batch][n_kv][capacity]
 * slabs put every sequence and head a capacity-dependent stride apart, and
 * some strides made the streams of concurrent work-groups collide in HBM.)
 *   len: HOST array [batch], the valid rows of each sequence; it is the
 *        authoritative length (kernels receive it by value).
 * K holds post-norm, post-RoPE keys; V holds raw values. Rows at or past len
 * are dead: they never contribute to a result.
 * capacity must be a positive multiple of 64, at most 2^21 rows.
 *
 * Paged layout (block_table != NULL; the serving cache of the vLLM page
 * "qwen3_dflash", whose cache update writes each row to the slot its
 * slot_mapping names): rows come in blocks of 64; logical block i of sequence
 * b (rows 64 i .. 64 i + 63) is physical block block_table[b * max_blocks + i]
 * of the pools (the contiguous layout with the blocks taken from a table)
 *   k: [num_blocks][n_kv][64][head_dim]
 *   v: [num_blocks][n_kv][head_dim][64]    (transposed within the block)
 * and capacity must equal 64 * max_blocks. block_table (device) is what the
 * kernels read; block_table_host is its host mirror, which the library checks
 * (every block a step touches must name a physical block in [0, num_blocks))
 * and the caller keeps equal to the device table. Sequences must not share a
 * block that a step writes. The kernels clamp entries into [0, num_blocks). */
typedef struct {
    void* k;
    void* v;
    int32_t* len;
    int32_t batch;
    int32_t capacity;
    const int32_t* block_table;       /* device [batch][max_blocks], or NULL     */
    const int32_t* block_table_host;  /* host mirror (required when paged)       */
    int32_t max_blocks;               /* table row length                         */
    int32_t num_blocks;               /* blocks in each pool                      */
} dflash_kv_cache;

typedef struct dflash_layer dflash_layer; /* opaque */

/* Create a layer handle for `cfg` over borrowed `weights` (device pointers that
 * must outlive the handle). Builds the RoPE cos/sin table on the host in
 * float64 and uploads it as fp32 [max_position][d/2] cos then sin (the pages
 * keep inv_freq in fp32 so that long positions do not dephase; the table keeps
 * the angle exact before rounding). The current HIP device at create time is
 * the layer's device.
 * Errors: DFLASH_ERR_ARG (null), DFLASH_ERR_SHAPE / DFLASH_ERR_UNSUPPORTED
 * (limits above), DFLASH_ERR_HIP (allocation or copy failed). */
int dflash_layer_create(const dflash_config* cfg, const dflash_weights* weights,
                        dflash_layer** out);

/* MXFP8 weights of a layer (the configuration in which the vLLM page
 * "qwen3_dflash" builds its MXFP8 context K/V projection: every layer's
 * qkv_proj is an MXFP8 linear; o_proj is taken to be one as well). Format as
 * for dflash_ctxkv_mxfp8_weights: E4M3 codes and one E8M0 scale per 32
 * consecutive elements of a row. */
typedef struct {
    const void* w_qkv;        /* [(nq + 2 nkv) d, H] E4M3, rows q | k | v; 16-byte aligned */
    const void* w_qkv_scale;  /* [(nq + 2 nkv) d, H / 32] E8M0; 4-byte aligned          */
    const void* w_o;          /* [H, nq d] E4M3; 16-byte aligned                         */
    const void* w_o_scale;    /* [H, nq d / 32] E8M0; 4-byte aligned                     */
    const void* q_norm;       /* [d] bf16                                                */
    const void* k_norm;       /* [d] bf16                                                */
} dflash_mxfp8_weights;

/* A layer handle whose projections are MXFP8. Each step quantises the draft
 * block rows and the new context rows once (dflash_mxfp8_quantize's rule) for
 * the block-scaled q|k|v + context k|v projection (16x16x128 scaled FP8
 * MFMA, fp32 sums, the same norm / RoPE / append epilogue), runs the attention
 * as in bf16 with the attention output (rounded to bf16, then quantised by
 * the same rule) written as MXFP8 by the attention and merge kernels, and
 * feeds that to the block-scaled o_proj. Everything else (arguments, workspace query, crop, errors) is as for
 * dflash_layer_create; hidden_states and target_hidden must be 16-byte
 * aligned, and DFLASH_APPEND_SEPARATE is not supported (the step then returns
 * DFLASH_ERR_UNSUPPORTED). create reads the scale arrays once and repacks them
 * into buffers of its own ([k / 128][rows][4]), freed by destroy.
 * Errors: those of dflash_layer_create; DFLASH_ERR_UNSUPPORTED (dtype not
 * bf16); DFLASH_ERR_SHAPE (hidden or nq d not a multiple of 128);
 * DFLASH_ERR_ARG (a missing or misaligned scale pointer). */
int dflash_layer_create_mxfp8(const dflash_config* cfg, const dflash_mxfp8_weights* weights,
                              dflash_layer** out);

/* Release the handle's own table and flag. Waits for the device to finish
 * work that may still read them. NULL is a no-op. */
void dflash_layer_destroy(dflash_layer* layer);

/* Bytes of device workspace a step needs for `batch` sequences with
 * `total_ctx` = sum of new context rows and `total_keys` = sum over sequences
 * of the keys each attends over (T_b = len_b + n_b + block_size). A bound: any
 * step with no larger batch, total_ctx and total_keys fits. 0 on bad input. */
size_t dflash_workspace_bytes(const dflash_layer* layer, int32_t batch,
                              int64_t total_ctx, int64_t total_keys);

/* Where a step leaves its intermediate results in the workspace (for tests
 * and inspection): the byte offset of `region` in the workspace of a step of
 * `batch` sequences and `total_ctx` new context rows (the layout that
 * dflash_workspace_bytes sizes). Once a dflash_attn_step with that workspace
 * has run, the region holds that step's values:
 *   DFLASH_WS_ATTN_OUT           [B * bs][nq * d] the attention output, o_proj's
 *                                input, in the dtype (not written by an MXFP8
 *                                layer)
 *   DFLASH_WS_ATTN_OUT_MX        [B * bs][nq * d] an MXFP8 layer's attention
 *                                output as E4M3 codes (o_proj's input)
 *   DFLASH_WS_ATTN_OUT_MX_SCALES its E8M0 scale bytes, step-major:
 *                                [nq * d / 128][B * bs][4], byte (c, m, j) scaling
 *                                columns 128 c + 32 j .. + 31 of row m
 * The scratch of dflash_attn_step_noalloc has another layout.
 * Errors: DFLASH_ERR_ARG (null layer or offset, batch outside [1,
 * DFLASH_LAUNCH_BATCH] (a larger step reuses the workspace run by run),
 * total_ctx < 0, unknown region, an MXFP8 region of a bf16 or fp32 layer). */
enum { DFLASH_WS_ATTN_OUT = 0, DFLASH_WS_ATTN_OUT_MX = 1, DFLASH_WS_ATTN_OUT_MX_SCALES = 2 };
int dflash_workspace_offset(const dflash_layer* layer, int32_t batch, int64_t total_ctx, int32_t region,
                            size_t* offset);

/* One layer step for every sequence of `cache` (B = cache->batch).
 *   hidden_states  device [B * bs, H]: the draft block of sequence b is rows
 *                  b*bs .. b*bs+bs-1 (one anchor plus bs-1 mask embeddings).
 *   target_hidden  device [sum n_b, H]: new context rows, sequence b owning
 *                  rows ctx_offsets[b] .. ctx_offsets[b+1]-1; may be NULL when
 *                  every n_b is 0.
 *   ctx_offsets    HOST [B + 1], ctx_offsets[0] == 0, non-decreasing.
 *   positions      device int32 [sum n_b + B * bs]: sequence b's window
 *                  [new context | block] (n_b + bs entries) starts at
 *                  ctx_offsets[b] + b*bs. Keys are rotated at their own
 *                  position, queries at the block's positions (the window's
 *                  suffix). Values outside [0, max_position) are clamped and
 *                  latch DFLASH_ERR_RANGE for dflash_layer_poll_error.
 *                  NULL: the contiguous positions len_b, len_b + 1, ...,
 *                  len_b + n_b + bs - 1 of every window (a draft that
 *                  continues its sequence), computed by the kernels; a window
 *                  reaching past max_position is then refused with
 *                  DFLASH_ERR_RANGE before anything is enqueued.
 *   cache          rows [len_b, len_b + n_b + bs) of each sequence receive the
 *                  new context rows then the block rows; len_b then becomes
 *                  T_b = len_b + n_b + bs. Nothing else in the cache is
 *                  written, and rows at or past a length are never used
 *                  (they may hold anything, NaN included).
 *   out            device [B * bs, H]: o_proj of the attention output.
 *   workspace      device scratch of at least dflash_workspace_bytes(...)
 *                  bytes, 256-byte aligned; contents need no initialisation.
 * Errors (nothing launched, nothing changed): DFLASH_ERR_ARG (null pointer,
 * batch outside [1, DFLASH_MAX_BATCH]), DFLASH_ERR_SHAPE (bad offsets,
 * negative len, capacity not a multiple of 64 or above 2^21), DFLASH_ERR_CAPACITY (some
 * T_b > capacity), DFLASH_ERR_WORKSPACE, DFLASH_ERR_UNSUPPORTED (one attention
 * work-group would get more than 65535 key tiles: more keys per step than an
 * MI355X can hold at 208 work-groups), DFLASH_ERR_HIP (launch failure;
 * lengths are then left unchanged). */
int dflash_attn_step(dflash_layer* layer, const void* hidden_states,
                     const void* target_hidden, const int32_t* ctx_offsets,
                     const int32_t* positions, dflash_kv_cache* cache, void* out,
                     void* workspace, size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the layer
 * step of dflash_attn_step without a workspace argument. Its scratch (packed
 * queries, the attention output, the split-KV partials and, where the step
 * uses them, fp32 projection slices) is a buffer the library keeps on every
 * device it runs on: a device array of DFLASH_NOALLOC_SCRATCH_BYTES, whose
 * address is resolved when a layer is created on that device and which lives
 * until the process ends. The call allocates nothing (no hipMalloc, no
 * allocating library routine) and needs no zeroed memory: each step writes
 * every scratch byte it reads. All calls on one device share that buffer, and
 * it keeps the last call's contents, so calls that overlap on one GPU (other
 * streams, other threads, other layers) race: the caller must order them.
 * The step carves exactly what it needs: for batch B and head_dim d about
 * 2 * B * block_size * n_q_heads * d elements of the dtype (queries and
 * attention output) plus at most 2 * 256 * 64 * (d * es + 8) bytes of partials
 * (es: the dtype's size; 8.6 MB for bf16 at d = 128), and fp32 slices when
 * o_proj splits k for few rows or the step appends in the separate kernel
 * (DFLASH_APPEND_SEPARATE, or DFLASH_APPEND_AUTO with few rows).
 * Arguments, effects and errors are those of dflash_attn_step, plus:
 * DFLASH_ERR_WORKSPACE (nothing launched, nothing changed) when the step needs
 * more than DFLASH_NOALLOC_SCRATCH_BYTES; DFLASH_ERR_HIP when the buffer's
 * address could not be resolved on the layer's device. */
#define DFLASH_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int dflash_attn_step_noalloc(dflash_layer* layer, const void* hidden_states,
                             const void* target_hidden, const int32_t* ctx_offsets,
                             const int32_t* positions, dflash_kv_cache* cache, void* out,
                             void* stream);

/* Rewind sequence `seq` to its first `new_len` rows (the accepted prefix after
 * verification; "DFlash源码导读（二）" section 4, crop(start)). Only the host
 * length changes: no data moves, rows below new_len stay bit-identical.
 * Host-only; safe to call while earlier steps are still in flight on a stream,
 * because later steps read the length when they are enqueued.
 * Errors: DFLASH_ERR_ARG (null cache or seq outside [0, batch)),
 * DFLASH_ERR_RANGE (new_len outside [0, len[seq]]: crop never grows). */
int dflash_cache_crop(dflash_kv_cache* cache, int32_t seq, int32_t new_len);

/* dflash_cache_crop for every sequence at once (one draft round's accepted
 * prefixes): new_len is a HOST array of cache->batch lengths. Every entry is
 * checked before any length changes, so an error leaves them all as they were.
 * Errors: DFLASH_ERR_ARG (null pointer), DFLASH_ERR_RANGE (an entry outside
 * [0, len[b]]). */
int dflash_cache_crop_all(dflash_kv_cache* cache, const int32_t* new_len);

/* ------------------------------------------------------------------------
 * Block pool of a paged cache: the host-side allocator behind the block table
 * (the vLLM page "qwen3_dflash" leaves block management to vLLM's cache
 * manager; this is the draft's own, so that a draft round needs no host work
 * outside the library). A pool owns the free physical blocks of one cache's
 * pools (or of a stack of caches that share one table) as a stack whose last
 * entry is taken next, and records every table entry it changes until they
 * are pushed to the device table. The table entries themselves live in the
 * cache descriptor's host mirror (block_table_host), which the calls below
 * write; they require a paged cache whose num_blocks equals the pool's.
 * ------------------------------------------------------------------------ */
typedef struct dflash_block_pool dflash_block_pool; /* opaque */

/* A pool of blocks 0 .. num_blocks - 1, all free, block 0 taken first.
 * Errors: DFLASH_ERR_ARG (null out), DFLASH_ERR_SHAPE (num_blocks <= 0). */
int dflash_block_pool_create(int32_t num_blocks, dflash_block_pool** out);
void dflash_block_pool_destroy(dflash_block_pool* pool);  /* NULL is a no-op */
/* Free blocks (-1 for a NULL pool). */
int32_t dflash_block_pool_free_count(const dflash_block_pool* pool);
/* Copy the free stack (bottom first; the last entry is taken next) into
 * blocks[capacity]. Errors: DFLASH_ERR_ARG, DFLASH_ERR_SHAPE (too small). */
int dflash_block_pool_get_free(const dflash_block_pool* pool, int32_t* blocks, int32_t capacity);
/* Replace the free stack by blocks[0 .. n-1] (distinct, in [0, num_blocks)),
 * e.g. a shuffled order. Errors: DFLASH_ERR_ARG, DFLASH_ERR_SHAPE (n too
 * large), DFLASH_ERR_RANGE (an entry out of range or repeated; nothing
 * changed). */
int dflash_block_pool_set_free(dflash_block_pool* pool, const int32_t* blocks, int32_t n);

/* Back rows [0, rows) of sequence `seq` (reserve) or of every sequence b with
 * rows[b] >= 0 (reserve_all; b ascending) with blocks: each logical block
 * past the sequence's blocks in use (its non-negative table entries) takes
 * the pool's next block. All or nothing: DFLASH_ERR_SHAPE when a sequence
 * would need more than max_blocks, DFLASH_ERR_CAPACITY when the pool holds too
 * few free blocks; DFLASH_ERR_ARG for a null or unpaged cache, a pool of
 * another size or a bad seq. Host-only. */
int dflash_cache_reserve(dflash_kv_cache* cache, dflash_block_pool* pool, int32_t seq, int64_t rows);
int dflash_cache_reserve_all(dflash_kv_cache* cache, dflash_block_pool* pool, const int64_t* rows);

/* Return to the pool every block of sequence `seq` (release) or of every
 * sequence b with rows[b] >= 0 (release_all) past the first ceil(rows / 64)
 * logical blocks (a crop's dropped blocks): sequence by sequence, last block
 * first; their entries become -1. The lengths are not changed (see
 * dflash_cache_crop / _crop_all). Errors: as for reserve. Host-only. */
int dflash_cache_release(dflash_kv_cache* cache, dflash_block_pool* pool, int32_t seq, int64_t rows);
int dflash_cache_release_all(dflash_kv_cache* cache, dflash_block_pool* pool, const int64_t* rows);

/* Write the table entries the pool changed since the last push into the
 * cache's device table (each index once, with its latest value): small patch
 * kernels on `stream` (448 entries each), so that steps enqueued after it see
 * them; then forget them. The device
 * table must be device memory. Errors: DFLASH_ERR_ARG, DFLASH_ERR_HIP. */
int dflash_cache_push_table(dflash_kv_cache* cache, dflash_block_pool* pool, void* stream);
/* Table entries changed since the last push (-1 for a NULL pool), and a way
 * to forget them (after the caller copied the whole table itself). */
int32_t dflash_block_pool_pending(const dflash_block_pool* pool);
int dflash_block_pool_drop_pending(dflash_block_pool* pool);

/* Synchronise `stream`, then return and clear the layer's sticky device-side
 * error (DFLASH_ERR_RANGE if a position fell outside the table since the last
 * poll), or DFLASH_OK. */
int dflash_layer_poll_error(dflash_layer* layer, void* stream);

/* Where a step normalises and rotates q and k, packs the queries and appends
 * the new rows to the cache (NeMo page "draft_qwen3": q_norm/k_norm and
 * apply_rotary_pos_emb; "DFlash源码导读（二）" sections 1-4: cache update):
 *   DFLASH_APPEND_AUTO      (default) as FUSED, except with few rows and a
 *                           deep k (the fused launch, one tile per head of
 *                           64 or 128 rows, would fill at most half the
 *                           CUs, and hidden >= 2048): then as SEPARATE,
 *                           whose projection splits k over the CUs;
 *   DFLASH_APPEND_FUSED     always in the projection's epilogue (never split k);
 *   DFLASH_APPEND_SEPARATE  always in the separate kernel.
 * The results agree up to the order of the fp32 sums of the projection. With
 * the fused form the step's DFLASH_K_NORM_ROPE time is part of
 * DFLASH_K_GEMM_QKV. Errors: DFLASH_ERR_ARG (null layer or unknown mode). */
enum { DFLASH_APPEND_AUTO = 0, DFLASH_APPEND_FUSED = 1, DFLASH_APPEND_SEPARATE = 2 };
int dflash_layer_set_append_mode(dflash_layer* layer, int32_t mode);

/* Timing with HIP events recorded on the launch stream. enable:
 *   DFLASH_PROFILE_OFF        no events (the default)
 *   DFLASH_PROFILE_KERNELS    an event pair around each kernel of a step
 *   DFLASH_PROFILE_ATTN_SPAN  one pair around the attention and its merge
 *                             together (DFLASH_K_ATTN_MERGE), nothing between
 *                             them: every event packet on the stream adds its
 *                             own time, so per-kernel pairs overstate a span
 *                             of consecutive kernels.
 * Setting a mode synchronises the device and clears the totals.
 * Errors: DFLASH_ERR_ARG (null layer, unknown mode), DFLASH_ERR_HIP. */
enum { DFLASH_PROFILE_OFF = 0, DFLASH_PROFILE_KERNELS = 1, DFLASH_PROFILE_ATTN_SPAN = 2 };
int dflash_layer_set_profiling(dflash_layer* layer, int32_t enable);

/* Synchronise on the recorded events and return, for each kernel of the step
 * (indices DFLASH_K_*), the summed milliseconds and the number of launches
 * (spans) since the profiling mode was set. `ms` and `count` hold DFLASH_K_COUNT entries. */
enum {
    DFLASH_K_GEMM_QKV = 0,   /* grouped projection: block QKV and context KV     */
    DFLASH_K_NORM_ROPE = 1,  /* per-head RMSNorm + RoPE + Q pack + cache append   */
    DFLASH_K_ATTN = 2,       /* split-KV non-causal GQA attention                 */
    DFLASH_K_MERGE = 3,      /* log-sum-exp merge of split partials               */
    DFLASH_K_GEMM_O = 4,     /* o_proj                                            */
    DFLASH_K_ATTN_MERGE = 5, /* attention + merge as one span (ATTN_SPAN mode)   */
    DFLASH_K_COUNT = 6
};
int dflash_layer_kernel_times(dflash_layer* layer, double* ms, int64_t* count);

/* ------------------------------------------------------------------------
 * Multi-layer context K/V precompute (vLLM page "qwen3_dflash",
 * DFlashQwen3Model: _build_context_kv_buffers, precompute_and_store_context_kv
 * and the helpers it calls). Instead of each layer projecting its new context
 * rows inside its step, the rows of every draft layer are made at once: the
 * raw context states (the fc output) are RMS-normalised with the model's
 * hidden_norm gain, one projection with the K/V rows of every layer's fused
 * q|k|v weight gives each layer's K and V, each K head is RMS-normalised with
 * its layer's k_norm gain and rotated (neox) at its context position, and each
 * layer's rows are appended to that layer's cache. A layer step that follows
 * is then called with no new context rows (ctx_offsets all 0).
 * ------------------------------------------------------------------------ */

/* Limits checked at create: 1 <= n_layers <= 16, head_dim in {64, 128},
 * n_kv_heads <= 256, hidden % 64 == 0, rope_theta > 0, rms_eps >= 0,
 * max_position >= 1. rms_eps is used by hidden_norm and by k_norm. */
typedef struct {
    int32_t hidden;
    int32_t n_layers;        /* L draft layers                                     */
    int32_t n_kv_heads;
    int32_t head_dim;
    int32_t max_position;
    int32_t dtype;           /* dflash_dtype                                       */
    double rope_theta;
    double rms_eps;
} dflash_ctxkv_config;

/* Device weights in the config dtype, borrowed (they must outlive the handle);
 * hidden_norm and w_kv 16-byte aligned. */
typedef struct {
    const void* hidden_norm;  /* [H] gain of the RMSNorm over the context states  */
    const void* w_kv;         /* [L * 2 * nkv * d, H]: layer l's K rows (its
                                 nkv heads), then its V rows, i.e. the rows of its
                                 fused q|k|v weight after the q rows; layers in
                                 order                                            */
    const void* k_norm;       /* [L, d] each layer's K RMSNorm gain               */
} dflash_ctxkv_weights;

/* MXFP8 weights of the precompute (vLLM page "qwen3_dflash",
 * _build_mxfp8_context_kv_proj: when every layer's qkv_proj is an MXFP8
 * linear, the context K/V projection is one block-scaled GEMM over the K/V
 * rows of all layers, rows and block scales copied as they are because the
 * scales belong to output rows). The format is OCP Microscaling MXFP8: FP8
 * E4M3 elements (bias 7, 3 mantissa bits, largest 448, S.1111.111 NaN) and
 * one E8M0 scale byte (2^(s - 127)) per 32 consecutive elements along hidden.
 * Borrowed device pointers, except w_kv_scale, which create only reads: it
 * repacks the scales into a buffer of its own ([H / 128][rows][4], so that
 * the GEMM reads a k step's scales of consecutive rows contiguously;
 * L * 2 * nkv * d * H / 32 bytes, freed by destroy). The config dtype must be
 * DFLASH_BF16 (states, gains and caches) and hidden a multiple of 128. */
typedef struct {
    const void* hidden_norm;  /* [H] bf16, 16-byte aligned                        */
    const void* w_kv;         /* [L * 2 * nkv * d, H] E4M3 bytes, rows ordered as
                                 dflash_ctxkv_weights.w_kv; 16-byte aligned       */
    const void* w_kv_scale;   /* [L * 2 * nkv * d, H / 32] E8M0 bytes: row r's
                                 block j scales w_kv[r][32 j .. 32 j + 31];
                                 4-byte aligned                                   */
    const void* k_norm;       /* [L, d] bf16                                      */
} dflash_ctxkv_mxfp8_weights;

typedef struct dflash_ctxkv dflash_ctxkv; /* opaque */

/* Create a precompute handle on the current device; it builds its own RoPE
 * cos/sin table exactly as dflash_layer_create does and an error flag.
 * Errors: DFLASH_ERR_ARG, DFLASH_ERR_SHAPE / DFLASH_ERR_UNSUPPORTED (limits),
 * DFLASH_ERR_HIP. */
int dflash_ctxkv_create(const dflash_ctxkv_config* cfg, const dflash_ctxkv_weights* weights,
                        dflash_ctxkv** out);

/* The same handle over MXFP8 weights. Each append then writes the
 * hidden_norm-ed rows (rounded to bf16) as MXFP8 rows (dflash_mxfp8_quantize's
 * rule) and runs the block-scaled projection (scaled 16x16x128 FP8 MFMA, fp32
 * sums) with the k_norm / RoPE / append epilogue; the other calls are
 * unchanged, except that DFLASH_APPEND_SEPARATE is not supported (append then
 * returns DFLASH_ERR_UNSUPPORTED).
 * Errors: those of dflash_ctxkv_create; DFLASH_ERR_UNSUPPORTED if the dtype is
 * not bf16; DFLASH_ERR_SHAPE if hidden % 128; DFLASH_ERR_ARG for a missing or
 * misaligned scale pointer. */
int dflash_ctxkv_create_mxfp8(const dflash_ctxkv_config* cfg, const dflash_ctxkv_mxfp8_weights* weights,
                              dflash_ctxkv** out);

/* Release the handle (waits for the device). NULL is a no-op. */
void dflash_ctxkv_destroy(dflash_ctxkv* h);

/* The optional fc projection before the precompute (vLLM page
 * "qwen3_dflash": the model's fc, a ReplicatedLinear with no bias, and
 * combine_hidden_states): the features of the selected target layers,
 * concatenated per row, projected to the draft's hidden size. The result is
 * the context_states that dflash_ctxkv_append takes.
 * set_fc registers the weight w_fc: device [hidden, fc_in] in the config
 * dtype, 16-byte aligned, borrowed (it must outlive the handle or the next
 * set_fc); fc_in > 0 and a multiple of 64. NULL w_fc removes it.
 * Errors: DFLASH_ERR_ARG (null handle, misaligned weight), DFLASH_ERR_SHAPE
 * (fc_in). */
int dflash_ctxkv_set_fc(dflash_ctxkv* h, const void* w_fc, int32_t fc_in);

/* Device workspace bytes dflash_ctxkv_combine may need for `rows` rows (fp32
 * partial sums of a k split); 0 on bad input. */
size_t dflash_ctxkv_combine_workspace_bytes(const dflash_ctxkv* h, int64_t rows);

/* context_states [rows, hidden] = aux_states [rows, fc_in] . w_fc^T, with fp32
 * sums rounded once to the dtype (for few rows the k axis is split over fp32
 * slices in the workspace and summed afterwards). Both device buffers are
 * 16-byte aligned and in the config dtype; the workspace (256-byte aligned,
 * at least dflash_ctxkv_combine_workspace_bytes) is scratch for the call;
 * enqueued on `stream`. rows == 0 is a no-op.
 * Errors: DFLASH_ERR_ARG (null handle or pointers, misaligned buffers, no fc
 * weight set), DFLASH_ERR_SHAPE (rows < 0 or > 2^31 - 1),
 * DFLASH_ERR_WORKSPACE, DFLASH_ERR_HIP. */
int dflash_ctxkv_combine(dflash_ctxkv* h, const void* aux_states, int64_t rows, void* context_states,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Device workspace bytes for up to `total_ctx` context rows; 0 on bad input. */
size_t dflash_ctxkv_workspace_bytes(const dflash_ctxkv* h, int64_t total_ctx);

/* Where an append leaves the hidden_norm-ed context rows in its workspace (for
 * tests and inspection): the byte offset of `region` in the workspace of an
 * append of `total_ctx` rows. After the append they hold:
 *   DFLASH_CTX_WS_NORMED            [total_ctx][H]: the rows in the dtype, or as
 *                                   E4M3 codes with MXFP8 weights
 *   DFLASH_CTX_WS_NORMED_MX_SCALES  their E8M0 scale bytes (MXFP8 weights only),
 *                                   step-major [H / 128][total_ctx][4]
 * Errors: DFLASH_ERR_ARG (null handle or offset, total_ctx < 0, unknown
 * region, the scales of a handle without MXFP8 weights). */
enum { DFLASH_CTX_WS_NORMED = 0, DFLASH_CTX_WS_NORMED_MX_SCALES = 1 };
int dflash_ctxkv_workspace_offset(const dflash_ctxkv* h, int64_t total_ctx, int32_t region, size_t* offset);

/* Append the new context rows of `caches[0 .. L-1]->batch` sequences to every
 * layer's cache.
 *   context_states  device [sum n_b, H] raw context rows (before hidden_norm),
 *                   16-byte aligned, sequence b owning rows
 *                   ctx_offsets[b] .. ctx_offsets[b+1]-1.
 *   ctx_offsets     HOST [B + 1], ctx_offsets[0] == 0, non-decreasing.
 *   positions       device int32 [sum n_b]: the position of every context row
 *                   (normally len_b, len_b + 1, ...); each must lie in
 *                   [0, max_position): a violation is clamped and latched as
 *                   for a layer step (dflash_ctxkv_poll_error). NULL: those
 *                   contiguous positions, computed by the kernels (rows past
 *                   max_position refused with DFLASH_ERR_RANGE up front).
 *   caches          HOST array of L cache descriptors, one per layer, with the
 *                   same batch, capacity and lengths; all contiguous or all
 *                   paged. Paged layers may share one block table or each
 *                   have their own table and pools (the vLLM page
 *                   "qwen3_dflash", precompute_and_store_context_kv, takes
 *                   one slot mapping for all layers or one per layer).
 * Effects: rows [len_b, len_b + n_b) of every layer's K and V for every b,
 * nothing else in the caches; then every layer's len[b] += n_b. Validation
 * (shapes, equal lengths across layers, capacity, every layer's table entries
 * for the rows written, workspace) happens before anything is enqueued; on an
 * error nothing runs and no length changes.
 * Errors: DFLASH_ERR_ARG, DFLASH_ERR_SHAPE (also a mix of paged and
 * contiguous layers), DFLASH_ERR_CAPACITY, DFLASH_ERR_RANGE (a needed table
 * entry of some layer outside its pools), DFLASH_ERR_WORKSPACE,
 * DFLASH_ERR_HIP. */
int dflash_ctxkv_append(dflash_ctxkv* h, const void* context_states, const int32_t* ctx_offsets,
                        const int32_t* positions, dflash_kv_cache* const* caches, void* workspace,
                        size_t workspace_bytes, void* stream);

/* Where the precompute normalises, rotates and appends its K/V rows, as for
 * dflash_layer_set_append_mode: DFLASH_APPEND_AUTO (default: in the
 * projection's epilogue when it has about a tile per CU without splitting k,
 * else in HK2 after an fp32 projection), DFLASH_APPEND_FUSED,
 * DFLASH_APPEND_SEPARATE. Errors: DFLASH_ERR_ARG. */
int dflash_ctxkv_set_append_mode(dflash_ctxkv* h, int32_t mode);

/* Synchronise `stream` and report the sticky device error (DFLASH_ERR_RANGE
 * if a position fell outside the table since the last poll, which clears it),
 * or DFLASH_OK. */
int dflash_ctxkv_poll_error(dflash_ctxkv* h, void* stream);

/* MXFP8 quantisation of bf16 rows, the rule the precompute applies to its
 * activations (the pages do not define the format; this is the OCP MX
 * conversion): per block of 32 consecutive elements of a row, the shared
 * exponent is floor(log2(amax)) - 8 clamped to [-127, 127] (scale byte 0 for
 * an all-zero block), and each element x / 2^exponent is rounded to the
 * nearest E4M3 value (ties to even), saturating at +-448 and keeping the sign
 * of a zero. NaN inputs are outside the contract.
 *   x       device bf16 [rows, cols], 16-byte aligned, cols % 128 == 0
 *   codes   device [rows, cols] E4M3 bytes, 16-byte aligned (output)
 *   scales  device [rows, cols / 32] E8M0 bytes (output)
 * Enqueued on `stream`. Errors: DFLASH_ERR_SHAPE (rows < 0 or > 2^31 - 1,
 * cols not a positive multiple of 128), DFLASH_ERR_ARG (null or misaligned
 * pointer), DFLASH_ERR_HIP. rows == 0 is a no-op. */
int dflash_mxfp8_quantize(const void* x, int64_t rows, int32_t cols, void* codes, void* scales, void* stream);

/* ------------------------------------------------------------------------
 * Draft decoder layer: the attention layer step inside its block (NeMo page
 * "draft_qwen3": Qwen3DFlashDecoderLayer with input_layernorm, self_attn,
 * post_attention_layernorm and mlp = Qwen3MLP; vLLM page "qwen3_dflash":
 * gate_proj/up_proj stacked as gate_up_proj, DFlashQwen3Model.forward threading
 * the residual stream and ending with the final norm). For the noise stream x
 * of the block's rows:
 *   a   = RMSNorm(x) * input_norm
 *   h   = x + attention_step(a, target_hidden, ...)     (o_proj included)
 *   m   = RMSNorm(h) * post_norm
 *   out = h + (silu(m Wg^T) * (m Wu^T)) Wd^T            silu(g) = g / (1 + e^-g)
 * The context rows (target_hidden) enter only the attention, as in a layer
 * step (they are already hidden_norm-ed upstream). Rounding: a, the
 * attention output, h, m and the MLP activation are stored in the dtype; h is
 * rounded after the add; out is rounded once after its add.
 * ------------------------------------------------------------------------ */

/* Limits: those of dflash_layer_create for `attn`, intermediate % 64 == 0. */
typedef struct {
    dflash_config attn;      /* the attention layer (its hidden is the block's)  */
    int32_t intermediate;    /* I: the MLP width                                  */
} dflash_decoder_config;

/* Device weights in the dtype, borrowed; norms 16-byte aligned. */
typedef struct {
    dflash_weights attn;     /* as for dflash_layer_create                        */
    const void* input_norm;  /* [H] input_layernorm gain                          */
    const void* post_norm;   /* [H] post_attention_layernorm gain                 */
    const void* w_gate_up;   /* [2I, H]: the gate_proj rows, then the up_proj rows */
    const void* w_down;      /* [H, I] down_proj                                  */
} dflash_decoder_weights;

typedef struct dflash_decoder dflash_decoder; /* opaque: owns its attention layer */

/* Create a decoder layer (and its attention layer handle). Errors as for
 * dflash_layer_create, and DFLASH_ERR_SHAPE for intermediate. */
int dflash_decoder_create(const dflash_decoder_config* cfg, const dflash_decoder_weights* weights,
                          dflash_decoder** out);

/* Release the decoder and its attention layer. NULL is a no-op. */
void dflash_decoder_destroy(dflash_decoder* decoder);

/* The decoder's attention layer (owned by the decoder, valid until it is
 * destroyed), for dflash_layer_set_append_mode / _set_profiling /
 * _kernel_times (the latter cover the attention kernels only). */
dflash_layer* dflash_decoder_attention(dflash_decoder* decoder);

/* Device workspace bytes of a decoder step for `batch` sequences with
 * `total_ctx` new context rows in all; 0 on bad input. */
size_t dflash_decoder_workspace_bytes(const dflash_decoder* decoder, int32_t batch, int64_t total_ctx);

/* The decoder step's intermediates in its workspace (for tests and
 * inspection), as for dflash_workspace_offset: the byte offset of `region` in
 * the workspace of a step of `batch` sequences and `total_ctx` context rows.
 * After the step they hold, in the dtype:
 *   DFLASH_DEC_WS_A    [B * bs][H] input_layernorm output a
 *   DFLASH_DEC_WS_ATT  [B * bs][H] the attention layer step's output (o_proj)
 *   DFLASH_DEC_WS_H    [B * bs][H] the residual h = x + att (rounded once)
 *   DFLASH_DEC_WS_M    [B * bs][H] post_attention_layernorm output m
 *   DFLASH_DEC_WS_ACT  [B * bs][I] the MLP activation silu(m Wg^T) * (m Wu^T)
 * Errors: DFLASH_ERR_ARG (null decoder or offset, bad batch, total_ctx < 0,
 * unknown region). */
enum { DFLASH_DEC_WS_A = 0, DFLASH_DEC_WS_ATT = 1, DFLASH_DEC_WS_H = 2, DFLASH_DEC_WS_M = 3, DFLASH_DEC_WS_ACT = 4 };
int dflash_decoder_workspace_offset(const dflash_decoder* decoder, int32_t batch, int64_t total_ctx,
                                    int32_t region, size_t* offset);

/* One decoder layer step. x and out: device [B * bs, H] (16-byte aligned; out
 * must not overlap x); the other arguments, the cache effects and the errors
 * are those of dflash_attn_step, whose checks all run before anything is
 * enqueued. */
int dflash_decoder_step(dflash_decoder* decoder, const void* x, const void* target_hidden,
                        const int32_t* ctx_offsets, const int32_t* positions, dflash_kv_cache* cache,
                        void* out, void* workspace, size_t workspace_bytes, void* stream);

/* RMSNorm of `rows` rows of `hidden` elements (the draft model's final norm):
 * out = x / sqrt(mean(x^2) + eps) * gain, fp32 math, one rounding. Device
 * pointers 16-byte aligned, hidden % 64 == 0. Errors: DFLASH_ERR_ARG,
 * DFLASH_ERR_HIP. */
int dflash_rms_norm(const void* x, const void* gain, void* out, int32_t rows, int32_t hidden, double eps,
                    int32_t dtype, void* stream);

/* Static description of a status code. */
const char* dflash_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* DFLASH_H */

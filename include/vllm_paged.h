/*
 * vllm_paged.h -- C ABI of the paged KV-cache hot path for AMD Instinct
 * MI355X (gfx950): the cache-write scatter that fills a block-paged KV pool,
 * attention decode over that pool (work split evenly over the GPU's waves,
 * pieces of cut sequences merged with the log-sum-exp rule), FP8 pools (E4M3
 * and E5M2, per-tensor or per-kv-head scales), an MFMA chunked-prefill
 * variant, a decode that reads a batch's shared prefix once, chunked-local
 * attention and page recycling for local attention, and a device-side
 * prefix-caching block manager that fills block tables and slot mappings.
 *
 * What is computed follows the pages' problem statement:
 *   - a block-paged KV cache held in FP16 or FP8 pages ("Building and
 *     Deploying vllm.cpp", architecture overview box and Step 3 CLI table:
 *     --kv-cache-dtype fp16|fp8, where fp8 stores one byte per element);
 *   - per-sequence block tables that may point at shared physical pages
 *     (same page, Step 3: zero-copy cache hits bind a new sequence's block
 *     table to existing physical pages);
 *   - 16-token pages (same page, the --block-size 16 launch commands);
 *   - paged attention over the block-paged cache in the model forward
 *     (vllm.cpp repository listing, "What's implemented", model forward),
 *     with the sliding window of its local-attention section.
 * ABI conventions follow the engine's own C ABI (vllm.cpp README, "Use it as
 * a library (C API)" and the note on the C ABI under the title): flat and
 * exception-free, every call returns a status with VLLM_OK on success and a
 * message from vllm_last_error(), the version is checkable at run time, and
 * option structs only grow by appending fields whose zero value keeps the
 * existing behaviour.
 *
 * Conventions for every call below
 *   - All tensor data pointers are DEVICE pointers (hipMalloc / torch CUDA
 *     tensors).  Host pointers are rejected with VLLM_ERR_DEVICE_PTR.
 *   - The caller owns every buffer (inputs, pools, outputs, workspace, the
 *     block manager's state).  The library keeps no device memory between
 *     calls; it keeps one extra stream and two events per device, created on
 *     first use by the shared-prefix decode.
 *   - Calls are asynchronous on `hip_stream` (a hipStream_t; NULL = the null
 *     stream) and never synchronize the host.  A VLLM_OK return means the
 *     work was enqueued; device-side faults surface on the stream.
 *   - Arguments are validated on the host before anything is launched; on
 *     error nothing is launched and no output is touched.
 *   - Values that only the device sees are not validated (that would need a
 *     host sync): slots, block ids and context lengths.  The kernels never
 *     read or write outside the pools and tables for any such value: a slot
 *     >= num_blocks*16 is skipped like a negative one, a block id outside
 *     [0, num_blocks) reads page 0, a context length above
 *     16*max_blocks_per_seq is clipped to it, and a context length <= 0
 *     yields an all-zero output row.  The results of such inputs are
 *     otherwise meaningless.  Duplicate slots in one cache write leave one of
 *     the written values in the slot.
 */
#ifndef VLLM_PAGED_H
#define VLLM_PAGED_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Version 2 appended k_scales / v_scales to vllm_attn_opts; version 3 added
 * FP8 pools in vllm_paged_attn_prefill and the local-attention and block
 * manager entry points; version 4 added vllm_paged_attn_decode_noalloc (no
 * struct changed); version 5 added vllm_paged_attn_prefill_workspace_size
 * (vllm_paged_attn_prefill now takes opts->workspace; no struct changed). */
#define VLLM_PAGED_ABI_VERSION 5
#define VLLM_PAGED_BLOCK_SIZE 16

typedef enum vllm_status {
  VLLM_OK = 0,
  VLLM_ERR_INVALID_ARG = 1,   /* null pointer, rank/shape/stride mismatch, Hq % Hkv != 0, window < 0 */
  VLLM_ERR_UNSUPPORTED = 2,   /* dtype combination, head_dim or block size outside the supported set */
  VLLM_ERR_DEVICE_PTR = 3,    /* a pointer that is not device memory */
  VLLM_ERR_WORKSPACE = 4,     /* caller workspace too small or misaligned */
  VLLM_ERR_HIP = 5            /* a HIP runtime call failed; message from hipGetErrorString */
} vllm_status;

typedef enum vllm_dtype {
  VLLM_DTYPE_F16 = 1,
  VLLM_DTYPE_BF16 = 2,
  VLLM_DTYPE_FP8_E4M3 = 3,    /* OCP FP8 E4M3 (bias 7, max 448, NaN 0x7F/0xFF, no infinities) */
  VLLM_DTYPE_I32 = 4,
  VLLM_DTYPE_I64 = 5,
  VLLM_DTYPE_F32 = 6,
  VLLM_DTYPE_FP8_E5M2 = 7     /* OCP FP8 E5M2 (bias 15, max 57344, infinities 0x7C/0xFC,
                                 NaN S.11111.xx with xx != 0) */
} vllm_dtype;

/* A dense tensor view: `data` is a device pointer, `shape` and `stride`
 * (in elements, row-major) give the first `ndim` dimensions.  Every tensor
 * passed to this library must be contiguous (stride of the last dimension
 * 1, each other stride the product of the later extents; dimensions of
 * extent 1, and tensors with no elements, may carry any strides). */
typedef struct vllm_tensor {
  void* data;
  int32_t dtype;     /* vllm_dtype */
  int32_t ndim;
  int64_t shape[4];
  int64_t stride[4];
} vllm_tensor;

/* Options shared by the calls; zero-initialised means defaults.  Fields are
 * only ever appended. */
typedef struct vllm_attn_opts {
  float k_scale;            /* FP8 pools only: K value = code * k_scale; 0 means 1.0 */
  float v_scale;            /* FP8 pools only: V value = code * v_scale; 0 means 1.0 */
  int32_t partition_size;   /* decode work split: 0 = automatic (the kept pages of the whole
                               batch are cut into one equal chunk per wave the GPU holds at
                               once); else a fixed chunk of this many tokens, a positive
                               multiple of 16.  Pieces of a sequence cut by chunk boundaries
                               are merged with the log-sum-exp rule by a second kernel */
  int32_t flags;            /* reserved, must be 0 */
  void* workspace;          /* device scratch, 256-byte aligned; needs no initialisation;
                               calls that share a workspace must not overlap.  Decode:
                               piece records, page prefix, partial results of cut
                               sequences, a spare page read by prefetches past the end.
                               Chunked prefill: the order of its tiles.  NULL = the library
                               allocates one stream-ordered (hipMallocAsync / hipFreeAsync
                               on hip_stream) for the call */
  size_t workspace_bytes;   /* size of `workspace`; see vllm_paged_attn_workspace_size,
                               vllm_paged_attn_shared_prefix_workspace_size and
                               vllm_paged_attn_prefill_workspace_size */
  /* appended in ABI version 2 (callers must be built against this header;
     check vllm_abi_version() >= 2): */
  const float* k_scales;    /* FP8 pools only: device pointer to Hkv fp32 scales, one per
                               kv-head (K value of head h = code * k_scales[h]), read on the
                               device, must be finite and > 0; NULL = k_scale for every head */
  const float* v_scales;    /* the same for V; NULL = v_scale for every head */
} vllm_attn_opts;

/* The ABI version this library was built with (VLLM_PAGED_ABI_VERSION). */
int32_t vllm_abi_version(void);

/* Message of the last failing call on this thread ("" if none).  The
 * pointer stays valid until the next call into this library on the same
 * thread. */
const char* vllm_last_error(void);

/*
 * Cache write (scatter).  For every token i with s = slot_mapping[i] >= 0:
 *   k_cache[s / 16, h, s % 16, :] = enc(k[i, h, :])   for every kv-head h,
 *   v_cache[s / 16, h, s % 16, :] = enc(v[i, h, :]).
 * Negative slots mark padding tokens and are skipped.  enc is the identity
 * (bit copy) when the pool has the input's dtype; for an FP8 pool it is the
 * OCP E4M3 (E5M2) code of (x / scale) with x converted exactly to fp32, one
 * correctly-rounded fp32 division by the scale of the token's kv-head from
 * opts, saturation to +-448 (+-57344; infinities included),
 * round-to-nearest-even, NaN -> 0x7F with the input's sign.  Bit-exact.
 * (FP8 E4M3/E5M2 KV: "Building and Deploying vllm.cpp", Step 6 table.)
 *   k, v         [T, Hkv, D]  F16 or BF16 (both the same dtype)
 *   slot_mapping [T]          I64
 *   k_cache, v_cache [num_blocks, Hkv, 16, D]  the input's dtype, FP8_E4M3 or FP8_E5M2
 *   opts         nullable; k_scale / v_scale (or per-head k_scales / v_scales)
 *                used for FP8 pools only
 * Supported: D a multiple of 8, D <= 512, T * Hkv * D / 8 below 2^31.
 * T = 0 is a no-op.
 */
vllm_status vllm_paged_cache_write(const vllm_tensor* k, const vllm_tensor* v,
                                   const vllm_tensor* slot_mapping,
                                   vllm_tensor* k_cache, vllm_tensor* v_cache,
                                   const vllm_attn_opts* opts, void* hip_stream);

/*
 * Paged attention decode: one query token per sequence, at position n - 1
 * where n = context_lens[s] counts every cached token including the query's
 * own (its K/V are written by vllm_paged_cache_write first).  This is the
 * paged attention over the block-paged KV cache of the model forward (vllm.cpp
 * repository listing, "What's implemented (CPU, behaviorally tested)", model
 * forward), over 16-token FP16/FP8 pages reached through per-sequence block
 * tables that may share physical pages ("Building and Deploying vllm.cpp",
 * Step 3), with the sliding window of the listing's local-attention entry.
 *   out[s, h, :] = sum_t softmax_t(scale * <q[s, h, :], K_s[t, h / g, :]>) V_s[t, h / g, :]
 * over t in [max(0, n - window), n) (window = 0: all n tokens), where token t
 * of sequence s is row t % 16 of physical page block_tables[s, t / 16] and
 * g = Hq / Hkv (consecutive grouping of query heads).  fp32 accumulation,
 * output rounded to nearest-even in q's dtype.  Entries of block_tables past
 * ceil(n / 16) are never read; pool rows outside the kept range are never
 * used (they may hold NaN).
 *   out          [B, Hq, D]  dtype of q (written; 16-byte aligned)
 *   q            [B, Hq, D]  F16 or BF16
 *   k_cache, v_cache [num_blocks, Hkv, 16, D]  q's dtype, FP8_E4M3 or FP8_E5M2
 *                (FP8 values: code * the scale of the kv-head, from opts)
 *   block_tables [B, max_blocks_per_seq]  I32
 *   context_lens [B]  I32
 *   scale        softmax scale applied to q.k (e.g. 1/sqrt(D))
 *   window       sliding window in tokens, 0 = off, must be >= 0
 *   opts         nullable; fp8 scales, split-K partition size, workspace
 * Work split: by default the kept pages of the whole batch are cut into one
 * equal chunk per wave the GPU holds at once.  A nonzero partition_size fixes
 * the chunk at that many tokens instead, but the chunks still tile the
 * batch's page stream (sequence by sequence, kv-head by kv-head), not each
 * sequence from its token 0.  So a chunk boundary inside a sequence falls
 * where the pages before it put it, and the log-sum-exp merge combines pieces
 * of that sequence cut there.  Either way the result is the same softmax;
 * only the rounding order differs.
 * Supported: D in {64, 128}; Hq % Hkv == 0 (any g >= 1); at most 131072
 * work units B * Hkv * (g / head chunk), where the head chunk is g for
 * g <= 8, else the largest divisor of g not above 8; the work bound
 * units * max_blocks_per_seq below 2^31 pages.  B = 0 is a no-op.
 */
vllm_status vllm_paged_attn_decode(vllm_tensor* out, const vllm_tensor* q,
                                   const vllm_tensor* k_cache, const vllm_tensor* v_cache,
                                   const vllm_tensor* block_tables,
                                   const vllm_tensor* context_lens, float scale,
                                   int32_t window, const vllm_attn_opts* opts,
                                   void* hip_stream);

/*
 * Cache write of each sequence's newest token fused into the decode (the two
 * calls of a decode step in one launch sequence): the same result, bit for
 * bit, as vllm_paged_cache_write(k_new, v_new, slot_mapping, ...) followed
 * by vllm_paged_attn_decode(...) with the same pools and options.
 *   k_new, v_new   [B, Hkv, D]  q's dtype: K/V of token context_lens[s] - 1
 *   slot_mapping   [B] I64      its slot (page * 16 + row); negative = none.
 *                  It must be the slot that sequence s's table gives for
 *                  that token: the wave that reads the sequence's last page
 *                  writes the token there first (a slot elsewhere is
 *                  written too, but unordered with the reads of that page).
 *   other arguments as vllm_paged_attn_decode (k_cache, v_cache are written).
 * FP8 pools quantize as vllm_paged_cache_write does (opts scales).
 */
vllm_status vllm_paged_attn_decode_append(vllm_tensor* out, const vllm_tensor* q,
                                          const vllm_tensor* k_new, const vllm_tensor* v_new,
                                          const vllm_tensor* slot_mapping,
                                          vllm_tensor* k_cache, vllm_tensor* v_cache,
                                          const vllm_tensor* block_tables,
                                          const vllm_tensor* context_lens, float scale,
                                          int32_t window, const vllm_attn_opts* opts,
                                          void* hip_stream);

/*
 * Bytes of workspace vllm_paged_attn_decode needs for these sizes (it
 * depends on the sizes and partition_size only, not on the device or the
 * dtypes).  partition_size as in vllm_attn_opts.  Returns 0 for invalid
 * arguments.
 */
size_t vllm_paged_attn_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t head_dim,
                                      int32_t max_blocks_per_seq,
                                      int32_t partition_size);

/*
 * Decode that allocates nothing, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, and harnesses
 * that forbid hipMalloc.  The same computation and result, bit for bit, as
 * vllm_paged_attn_decode with the same arguments; instead of a caller's
 * workspace or a stream-ordered allocation it uses a scratch array of
 * VLLM_PAGED_NOALLOC_SCRATCH_BYTES bytes that the library's code object
 * holds on each GPU it runs on until the process ends (its address is looked
 * up once per device, on the first call there).
 *   arguments  as vllm_paged_attn_decode; opts->workspace must be NULL.
 * Errors: VLLM_ERR_WORKSPACE when the sizes need more scratch than that
 * (compare vllm_paged_attn_workspace_size with the limit: e.g. 32 sequences
 * of up to 4096 tokens at Hq = 32, Hkv = 8, D = 128 need about 16 MiB).
 * Every call on one GPU shares that GPU's array and leaves its contents
 * behind; the kernels rewrite whatever they read, so nothing needs clearing,
 * but calls that overlap on one GPU (other streams, other host threads)
 * race and must be serialised by the caller.
 */
#define VLLM_PAGED_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
vllm_status vllm_paged_attn_decode_noalloc(vllm_tensor* out, const vllm_tensor* q,
                                           const vllm_tensor* k_cache, const vllm_tensor* v_cache,
                                           const vllm_tensor* block_tables,
                                           const vllm_tensor* context_lens, float scale,
                                           int32_t window, const vllm_attn_opts* opts,
                                           void* hip_stream);

/*
 * Decode with a prefix shared by the whole batch read once ("cascade"): the
 * same result as vllm_paged_attn_decode, for batches whose sequences all map
 * their first `shared_pages` logical pages to the same physical pages (a
 * prefix hit binds a new sequence's block table to existing pages:
 * "Building and Deploying vllm.cpp", Step 3).  Those pages are read from
 * sequence 0's table (the other sequences' first shared_pages entries are not
 * read) once per kv-head for the whole batch: every sequence's query is
 * scored against them together on the matrix cores, in splits of 64 pages,
 * by workgroups of the same launch as the decode of the rest of each
 * sequence (so the call is two kernels on hip_stream and uses no other
 * stream), and the parts are merged with the log-sum-exp rule.  Keys of the shared pages are kept per sequence as in
 * decode: t < n (a sequence shorter than the prefix uses its first n tokens)
 * and t >= n - window.  The probabilities of the shared part are rounded to
 * q's 16-bit format before the product with V, as in decode.
 *   shared_pages  0 .. max_blocks_per_seq (0: same as vllm_paged_attn_decode)
 *   scale         > 0 when shared_pages > 0
 *   other arguments as vllm_paged_attn_decode; the workspace must hold
 *   vllm_paged_attn_shared_prefix_workspace_size bytes.
 * Supported: as vllm_paged_attn_decode.
 */
vllm_status vllm_paged_attn_decode_shared_prefix(vllm_tensor* out, const vllm_tensor* q,
                                                 const vllm_tensor* k_cache,
                                                 const vllm_tensor* v_cache,
                                                 const vllm_tensor* block_tables,
                                                 const vllm_tensor* context_lens,
                                                 int32_t shared_pages, float scale, int32_t window,
                                                 const vllm_attn_opts* opts, void* hip_stream);

/*
 * Bytes of workspace vllm_paged_attn_decode_shared_prefix needs for these
 * sizes (sizes and partition_size only).  Returns 0 for invalid arguments
 * (including head_dim other than 64 or 128, or shared_pages outside
 * [0, max_blocks_per_seq]).
 */
size_t vllm_paged_attn_shared_prefix_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                                    int32_t num_kv_heads, int32_t head_dim,
                                                    int32_t max_blocks_per_seq, int32_t shared_pages,
                                                    int32_t partition_size);

/*
 * Chunked-prefill attention on matrix cores, for the multi-token query
 * chunks that a token-budget scheduler with chunked prefill produces (vllm.cpp
 * repository listing, "What's implemented (CPU, behaviorally tested)", engine
 * core: the unified token-budget scheduler with chunked prefill; its CUDA path
 * runs a vendored FlashAttention-2 prefill, listed under the optimized paths
 * of the same listing).  Prefix hits skip the prefill of the cached part
 * ("Building and Deploying vllm.cpp", Step 3), so a chunk attends to cached
 * pages plus its own.  Sequence s has Q_s =
 * query_start_loc[s+1] - query_start_loc[s] query tokens (rows
 * query_start_loc[s] .. query_start_loc[s+1]-1 of q) at positions
 * n - Q_s .. n - 1, where n = context_lens[s] includes them (their K/V are
 * already in the pool).  Query row at position p attends to keys t <= p with
 * t > p - window (window = 0: no lower bound).  Scores use bf16/f16 matrix
 * products with fp32 accumulation; the softmax probabilities are rounded to
 * q's dtype before the product with V; output rounded to q's dtype.  FP8
 * pools: every E4M3 / E5M2 value is exact in fp16 and bf16, so codes enter
 * the products unchanged; the K scale multiplies the scores and the V scale
 * the output (per tensor, or per kv-head through opts->k_scales / v_scales,
 * as for decode).
 *   out          [sumQ, Hq, D]  dtype of q (written)
 *   q            [sumQ, Hq, D]  F16 or BF16
 *   k_cache, v_cache [num_blocks, Hkv, 16, D]  q's dtype, FP8_E4M3 or FP8_E5M2
 *   block_tables [B, max_blocks_per_seq]  I32
 *   query_start_loc [B + 1]  I32, non-decreasing, query_start_loc[0] = 0,
 *                    query_start_loc[B] = sumQ
 *   context_lens [B]  I32, n >= Q_s
 *   max_query_len    an upper bound of max_s Q_s (rows of longer chunks past
 *                    it are not computed)
 *   scale        softmax scale applied to q.k, finite and > 0
 * Supported: D in {64, 128}; g = Hq / Hkv <= 128.  sumQ = 0 is a no-op.  Values of
 * query_start_loc are clamped to [0, sumQ], so no value leads outside q/out.
 * Work order: a first kernel on hip_stream sorts the sequences by the keys of
 * their longest tile and lays out the tiles of every (sequence, kv-head) pair
 * together, longest sequences first, with no empty tiles in between; the tile
 * kernel follows that order (the workgroup scheduler serves workgroups in
 * launch order).  The order lives in opts->workspace
 * (vllm_paged_attn_prefill_workspace_size bytes; VLLM_ERR_WORKSPACE if
 * smaller) or in memory allocated stream-ordered for the call.  Calls of
 * fewer than 2048 workgroups (ceil(B Hkv / 8) * 8 * ceil(max_query_len /
 * (128 / g))) or more than 4096 sequences run in launch order and need no
 * workspace.  The order changes no result: every tile computes the same
 * values in any order.
 */
vllm_status vllm_paged_attn_prefill(vllm_tensor* out, const vllm_tensor* q,
                                    const vllm_tensor* k_cache, const vllm_tensor* v_cache,
                                    const vllm_tensor* block_tables,
                                    const vllm_tensor* query_start_loc,
                                    const vllm_tensor* context_lens,
                                    int32_t max_query_len, float scale, int32_t window,
                                    const vllm_attn_opts* opts, void* hip_stream);

/*
 * Bytes of workspace vllm_paged_attn_prefill needs for these sizes (0: none,
 * also for invalid arguments).  The same sizes as the call: B sequences,
 * Hq and Hkv heads, max_query_len.
 */
size_t vllm_paged_attn_prefill_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                              int32_t num_kv_heads, int32_t max_query_len);

/*
 * Chunked-local attention as a virtual batch (the local-attention section of
 * the vllm.cpp repository listing, "What's implemented": exact virtual Q/K
 * batches and a reusable block-table gather/update plan).  Chunked-local
 * attention of chunk L keeps, for the query at position p, the keys
 * floor(p / L) * L .. p.  The plan turns every (sequence, chunk) holding query
 * tokens into one ordinary causal sequence, in (sequence, chunk) order:
 *   v_query_start_loc[v]  first row of q of virtual sequence v (the rows stay
 *                         in place, so q and out are used as they are)
 *   v_context_lens[v]     keys from the chunk start to its last query token
 *   v_block_tables[v, :]  the pages of the original table from the chunk
 *                         start, -1 past the virtual context
 * Entries past the batch's virtual sequences have no rows (start = sumQ),
 * context 0 and -1 tables.  The plan depends only on the metadata, so one
 * plan serves every layer.  Running vllm_paged_attn_prefill (max_query_len
 * min(max_query_len, chunk_size), window 0) or, when every sequence has one
 * query token, vllm_paged_attn_decode (first B entries) on the virtual batch
 * gives chunked-local attention.
 *   query_start_loc [B + 1] I32, context_lens [B] I32 (n >= Q_s),
 *   block_tables [B, max_blocks_per_seq] I32   (as vllm_paged_attn_prefill)
 *   chunk_size        tokens per chunk, a positive multiple of 16
 *   v_query_start_loc [V + 1] I32, v_context_lens [V] I32,
 *   v_block_tables [V, chunk_size / 16] I32   written; V from
 *                     vllm_paged_chunked_local_virtual_count
 * Device values are clamped so that nothing is read or written out of
 * bounds; inconsistent metadata gives unspecified plans.
 */
vllm_status vllm_paged_chunked_local_plan(const vllm_tensor* query_start_loc,
                                          const vllm_tensor* context_lens,
                                          const vllm_tensor* block_tables, int32_t chunk_size,
                                          vllm_tensor* v_query_start_loc,
                                          vllm_tensor* v_context_lens,
                                          vllm_tensor* v_block_tables, void* hip_stream);

/* Upper bound V of the virtual sequences of a plan: floor(sumQ / chunk) +
 * 2 * num_seqs (each sequence's Q_s tokens span at most Q_s / chunk + 2
 * chunks).  0 for invalid arguments. */
int64_t vllm_paged_chunked_local_virtual_count(int32_t num_seqs, int32_t num_tokens,
                                               int32_t chunk_size);

/*
 * Page recycling for local attention: the leading pages of each sequence that
 * no query at position >= n (n = context_lens[s], the next token's position)
 * can attend to -- keys t <= n - window with a sliding window, keys below
 * floor(n / chunk_size) * chunk_size with chunked-local attention, the larger
 * of the two -- are reported and their block_tables entries set to -1
 * (entries already -1 are skipped, so repeated calls report each page once).
 * Reported ids of sequence s are freed_pages[freed_offsets[s] ..
 * freed_offsets[s + 1]).  Pages shared with other sequences are reported by
 * each sequence that drops them: reference counting belongs to the caller's
 * allocator.  Decode and prefill never read table entries below the kept
 * range, so recycled entries are never read.
 *   context_lens [B] I32; block_tables [B, max_blocks_per_seq] I32 (updated)
 *   window, chunk_size  0 = off; chunk_size a multiple of 16
 *   freed_offsets [B + 1] I32, freed_pages [B * max_blocks_per_seq] I32 written
 */
vllm_status vllm_paged_recycle_pages(const vllm_tensor* context_lens, vllm_tensor* block_tables,
                                     int32_t window, int32_t chunk_size,
                                     vllm_tensor* freed_offsets, vllm_tensor* freed_pages,
                                     void* hip_stream);

/*
 * Measurement aid: a plain read of a list of pages, the practical ceiling of
 * the decode's memory access pattern on this GPU.  Page page_ids[j] (bytes
 * page_bytes * id .. of `buffer`; ids outside the buffer read page 0) is
 * read once for every j, with 16-byte non-temporal loads, 64 lanes per page
 * and 16 KiB in flight per wave, the list cut into one equal contiguous
 * chunk per wave; nothing is computed but an XOR of the bytes each wave read,
 * stored to sink[wave].  Timing it over the pages of a decode's K and V, in a
 * random order, gives the bandwidth the decode could reach if it did nothing
 * but read.
 *   buffer     any dtype, rank 1 to 4, contiguous, at least one page
 *   page_ids   [P] I32
 *   page_bytes 1024, 2048 or 4096
 *   sink       [W] I32 written: W waves (a multiple of 4, at most 2^20)
 */
vllm_status vllm_paged_read_pages(const vllm_tensor* buffer, const vllm_tensor* page_ids,
                                  int32_t page_bytes, vllm_tensor* sink, void* hip_stream);

/*
 * Prefix-caching KV block manager on the device: the step before the path,
 * which fills block tables and slot mappings ("Building and Deploying
 * vllm.cpp", Step 3, RadixTree prefix caching: radix matching over runs of
 * physical blocks, zero-copy hits that bind a new sequence's table to
 * existing pages, LRU eviction of the oldest leaves returning their blocks
 * to the pool; the vllm.cpp repository listing, "What's implemented":
 * hash-based prefix caching in the KV cache manager).
 *
 * The manager's whole state lives in one caller-owned device buffer of
 * vllm_block_manager_state_size(num_blocks) bytes, set up by
 * vllm_block_manager_init.  Cached prefixes form a trie with one node per
 * full 16-token block, keyed by (parent block, its 16 token ids), behind a
 * chain-hash index (Karp-Rabin polynomial hash of the whole prefix modulo
 * 2^64; cached blocks carry distinct hashes, and a block whose hash is taken
 * stays uncached).  Every call is stream-ordered and runs on the device;
 * calls on one state must not overlap.
 */
size_t vllm_block_manager_state_size(int32_t num_blocks);   /* 0 if num_blocks is not in [1, 2^24] */

/* Byte offsets inside the state of its regions, for inspection: [0] the
 * int32 header (free-stack height, cached blocks, index tombstones,
 * num_blocks, index slots), then free stack (int32, bottom first), ref
 * (int32), last-access step (uint32), depth (int32), parent (int32), flags
 * (int32, bit 0 = cached), chain hash (uint64), tokens (int32 x 16), index
 * slots (int32: -1 empty, -2 tombstone, else a block), two per-call scratch
 * arrays (int32); [12] the total size.  Returns the number written (<= n). */
int32_t vllm_block_manager_state_layout(int32_t num_blocks, int64_t* offsets, int32_t n);

/* Empty pool: all blocks free (the first allocations take 0, 1, 2, ...),
 * nothing cached. */
vllm_status vllm_block_manager_init(void* state, size_t state_bytes, int32_t num_blocks,
                                    void* hip_stream);

/* Scratch bytes of a schedule call (chain hashes and candidates per
 * (request, block)). */
size_t vllm_block_manager_workspace_size(int32_t num_seqs, int32_t max_blocks_per_seq);

/*
 * Admit or extend a batch of requests, in request order.  Request r holds
 * old = num_computed[r] tokens in the cache (0: a new request) and adds
 * q = query_start_loc[r+1] - query_start_loc[r] tokens; its token ids, all
 * old + q of them, are token_ids[token_start[r] .. token_start[r+1]).
 *  - A new request reuses the longest cached prefix of whole blocks, at most
 *    floor((old + q - 1) / 16) blocks so that one token is computed; lookups
 *    see the index as it stood before the call.  Reused blocks gain a
 *    reference.
 *  - Missing blocks are popped from the free stack (request order, block
 *    order).  When too few are free, unreferenced cached blocks are evicted
 *    in (last access, deeper first, lower id) order -- only leaves -- and
 *    pushed in increasing id order first.
 *  - Blocks that become full are cached, request by request; a request
 *    stops caching at the first block whose hash is already taken.
 *  - block_tables[r, ceil(old/16) ..) is written; entries before are read.
 *  - slot_mapping[query_start_loc[r] + i] = slot of token old + i (block *
 *    16 + offset), or -1 for tokens served by the cache (the cache write
 *    skips negative slots); num_cached_tokens[r] = max(old, 16 * reused).
 *  - Blocks touched (reused or allocated) get last access = now.
 * status[0] (device) = 0 done, 1 not enough free plus evictable blocks, 2
 * metadata that do not fit (old < 0, q < 0, a token count that is not
 * old + q, a row too short, an existing entry outside [0, num_blocks),
 * offsets outside the arrays); with 1 or 2 nothing changes.
 *   token_ids [T] I32; token_start, query_start_loc [B + 1] I32;
 *   num_computed [B] I32; block_tables [B, max_blocks_per_seq] I32;
 *   slot_mapping [sum q] I64; num_cached_tokens [B] I32; status [1] I32.
 *   B <= 2048.  workspace: null (allocated on the stream) or at least
 *   vllm_block_manager_workspace_size(B, max_blocks_per_seq) bytes.
 */
vllm_status vllm_block_manager_schedule(void* state, int32_t num_blocks,
                                        const vllm_tensor* token_ids,
                                        const vllm_tensor* token_start,
                                        const vllm_tensor* num_computed,
                                        const vllm_tensor* query_start_loc,
                                        vllm_tensor* block_tables, vllm_tensor* slot_mapping,
                                        vllm_tensor* num_cached_tokens, vllm_tensor* status,
                                        uint32_t now, void* workspace, size_t workspace_bytes,
                                        void* hip_stream);

/*
 * Sequences end: each block of row r's first ceil(num_tokens[r] / 16)
 * entries loses one reference and gets last access = now; blocks that are
 * not cached go back on the free stack (request order, block order), cached
 * ones stay in the index, evictable once unreferenced.  Entries outside
 * [0, num_blocks) are skipped.  B <= 2048.
 *   block_tables [B, max_blocks_per_seq] I32; num_tokens [B] I32.
 */
vllm_status vllm_block_manager_release(void* state, int32_t num_blocks,
                                       const vllm_tensor* block_tables,
                                       const vllm_tensor* num_tokens, uint32_t now,
                                       void* hip_stream);

#ifdef __cplusplus
}  /* extern "C" */
#endif

#endif  /* VLLM_PAGED_H */

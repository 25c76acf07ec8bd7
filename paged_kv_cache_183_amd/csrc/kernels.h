// Parameter blocks and host-side launchers of the gfx950 kernels.  The C ABI
// layer (abi.cpp) validates everything before filling these.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vp {

// Storage formats handled by the kernels.
enum Fmt : int { kF16 = 0, kBF16 = 1, kE4M3 = 2, kE5M2 = 3 };

constexpr bool is_fp8(int f) { return f == kE4M3 || f == kE5M2; }

struct CacheWriteParams {
  const void* k;               // [T, Hkv, D] 16-bit
  const void* v;
  const int64_t* slot_mapping; // [T]
  void* k_cache;               // [num_blocks, Hkv, 16, D]
  void* v_cache;
  int64_t num_slots;           // num_blocks * 16
  int64_t src_tok_stride;      // elements between tokens of k / v (Hkv * D)
  uint32_t num_items;          // T * Hkv * D / 8
  uint32_t items_per_token;    // Hkv * D / 8
  uint32_t items_per_head;     // D / 8
  int32_t num_kv_heads;
  int32_t head_dim;
  float k_scale;               // FP8 pools: stored code = fp8(x / k_scale)
  float v_scale;
  const float* k_scales;       // FP8 pools: [Hkv] per-head scales, or null for k_scale
  const float* v_scales;
};

// dst_fmt: src_fmt (bit copy), kE4M3 or kE5M2.
hipError_t launch_cache_write(const CacheWriteParams& p, int src_fmt, int dst_fmt,
                              hipStream_t stream);

struct DecodeParams {
  const void* q;               // [B, Hq, D]
  void* out;                   // [B, Hq, D]
  const void* k_cache;         // [num_blocks, Hkv, 16, D]
  const void* v_cache;
  const int32_t* block_tables; // [B, bt_stride]
  const int32_t* context_lens; // [B]
  int32_t* ws_prefix;          // [B + 3]: pages before each sequence, then T, C
  float* ws_o;                 // [2 * max_chunks, G, D] normalized partial outputs
  float* ws_m;                 // [2 * max_chunks, G]    running max, log2 units
  float* ws_l;                 // [2 * max_chunks, G]    sum of exp2(s - m)
  int32_t* ws_unit;            // [B * units][2]: slot of the first piece, number of pieces
  const void* ws_spare;        // one page (16 x D 16-bit) read by prefetches past the end
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;               // g = Hq / Hkv
  int32_t head_chunk;          // query heads per work unit (G of the kernel)
  int32_t bt_stride;           // max_blocks_per_seq
  int32_t num_blocks;
  int32_t window;              // 0 = off
  int32_t num_workers;         // waves in the grid
  int32_t chunk_pages;         // pages per chunk; 0 = ceil(T / num_workers)
  int32_t max_chunks;          // capacity of the partial arrays (chunks)
  float score_scale;           // scale * log2(e) * k_scale
  float out_scale;             // v_scale (1 for 16-bit pools)
  float score_base;            // scale * log2(e)
  const float* k_scales;       // FP8 pools: [Hkv] per-head scales (null: k_scale)
  const float* v_scales;       // FP8 pools: [Hkv] per-head scales (null: v_scale)
  // Shared prefix (0 = none): keys below skip_tokens are left to the
  // shared-prefix pass; every unit then goes through the merge, which also
  // takes the num_splits prefix partials of each row.
  int32_t skip_tokens;
  int32_t num_splits;
  float* ws_uo;                // [units, G, D] partials of whole units (shared prefix only)
  float* ws_um;                // [units, G]
  float* ws_ul;                // [units, G]
  const float* pfx_o;
  const float* pfx_m;
  const float* pfx_l;
  // Fused cache write of each sequence's newest token (null: none): k_new /
  // v_new [B, Hkv, D] in q's format, written to new_slots[s] as the cache
  // write would, by the wave that reads the unit's last page, before it reads it.
  const void* k_new;
  const void* v_new;
  const int64_t* new_slots;
  int64_t num_slots;
  float k_scale, v_scale;      // FP8 pools: the per-tensor scales of the write
};

// kv_fmt: kF16 / kBF16 / kE4M3 / kE5M2; q_fmt: kF16 / kBF16.  Launches the
// decode kernel, then the merge.
hipError_t launch_decode(const DecodeParams& p, int head_dim, int kv_fmt, int q_fmt,
                         hipStream_t stream);
hipError_t launch_decode_merge(const DecodeParams& p, int head_dim, int q_fmt, hipStream_t stream);

struct PrefillParams {
  const void* q;               // [sumQ, Hq, D]
  void* out;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* query_start_loc;  // [B + 1]
  const int32_t* context_lens;     // [B]
  int32_t num_tokens;          // sumQ (rows of q)
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;
  int32_t bt_stride;
  int32_t num_blocks;
  int32_t max_query_len;
  int32_t window;
  int32_t num_tiles;           // row tiles (set by the launchers)
  float score_scale;           // scale * log2(e) (* k_scale for FP8 pools)
  float score_base;            // scale * log2(e)
  const float* k_scales;       // FP8 pools: [Hkv] per-head K scales (null: folded in score_scale)
  float out_scale;             // chunked prefill: V scale of FP8 pools, else 1
  const float* v_scales;       // chunked prefill, FP8 pools: [Hkv] per-head V scales (or null)
  // shared-prefix partials (launch_decode_shared only): the first
  // shared_pages pages of every sequence, in splits of split_pages pages
  int32_t shared_pages;
  int32_t split_pages;
  int32_t num_splits;
  float* pfx_o;                // [num_splits, B, Hq, D] normalized partial outputs
  float* pfx_m;                // [num_splits, B, Hq] running max, log2 units (-inf: empty)
  float* pfx_l;                // [num_splits, B, Hq] sum of exp2(s - m)
  // chunked prefill: tile order built on the device ahead of the tiles (null:
  // the grid order).  List x (of plan_stride entries) holds the tiles run by
  // the workgroups b with b % 8 == x, in dispatch order: (s Hkv + kv-head,
  // tile), or x = -1 past the list's tiles.
  int2* plan;
  int32_t plan_stride;
};

// Chunked-prefill grid: ceil(B Hkv / 8) * 8 pair slots times the row tiles of
// the longest chunk (kRows = 128 rows per tile, 128 / g tokens).
inline int64_t prefill_grid(int64_t num_seqs, int64_t num_kv_heads, int64_t group,
                            int64_t max_query_len) {
  const int64_t tq = 128 / group;
  if (tq < 1 || num_seqs <= 0 || max_query_len <= 0) return 0;
  return (num_seqs * num_kv_heads + 7) / 8 * 8 * ((max_query_len + tq - 1) / tq);
}
// The tile order is built for grids of kPlanMinGrid to kPlanMaxGrid
// workgroups (one int2 each) of at most kPlanMaxSeqs sequences; other calls
// run in the grid order.  Below kPlanMinGrid (under three rounds of the 768
// tiles the GPU holds at once) most tiles start together anyway, and the
// order's own kernel would cost more than it saves.
constexpr int kPlanMaxSeqs = 4096;
constexpr int64_t kPlanMinGrid = 2048;
constexpr int64_t kPlanMaxGrid = int64_t(1) << 22;
inline size_t prefill_plan_bytes(int64_t num_seqs, int64_t num_kv_heads, int64_t group,
                                 int64_t max_query_len) {
  const int64_t grid = prefill_grid(num_seqs, num_kv_heads, group, max_query_len);
  if (grid < kPlanMinGrid || num_seqs > kPlanMaxSeqs || grid > kPlanMaxGrid) return 0;
  return (size_t)grid * sizeof(int2);
}

// Chunked prefill: kv_fmt = q_fmt, kE4M3 or kE5M2.  With p.plan set
// (prefill_plan_bytes of memory) the tile order is built first, on the same
// stream.
hipError_t launch_prefill(const PrefillParams& p, int head_dim, int kv_fmt, int q_fmt,
                          hipStream_t stream);
// Shared-prefix partials: kv_fmt = q_fmt, kE4M3 or kE5M2.
// Shared-prefix decode: the prefix tiles (p.shared_pages, split_pages,
// num_splits and the partial arrays of sp) and the decode of every
// sequence's own pages (p.skip_tokens = 16 shared_pages) in one grid, then
// the merge, all on one stream.
hipError_t launch_decode_shared(const DecodeParams& p, const PrefillParams& sp, int head_dim,
                                int kv_fmt, int q_fmt, hipStream_t stream);
// Pages per split of the shared-prefix pass.  (A 4096-token prefix in 4
// splits: 8 splits of 32 pages made the prefix-shared FP8 decode 3% slower
// through the merge's reads of the partials, 2 splits 19% slower through the
// tiles' longer walk.)
constexpr int kPrefixSplitPages = 64;

struct LocalPlanParams {
  const int32_t* query_start_loc;  // [B + 1]
  const int32_t* context_lens;     // [B]
  const int32_t* block_tables;     // [B, bt_stride]
  int32_t* v_query_start_loc;      // [num_virtual + 1]
  int32_t* v_context_lens;         // [num_virtual]
  int32_t* v_block_tables;         // [num_virtual, chunk / 16]
  int32_t num_seqs;
  int32_t num_tokens;              // sumQ, or -1: query_start_loc[B]
  int32_t bt_stride;
  int32_t chunk;                   // tokens per local chunk, a multiple of 16
  int64_t num_virtual;
};

hipError_t launch_chunked_local_plan(const LocalPlanParams& p, hipStream_t stream);

struct RecycleParams {
  const int32_t* context_lens;     // [B] tokens cached (the next token's position)
  int32_t* block_tables;           // [B, bt_stride]: dead entries set to -1
  int32_t* freed_offsets;          // [B + 1]
  int32_t* freed_pages;            // [B * bt_stride]
  int32_t num_seqs;
  int32_t bt_stride;
  int32_t window;                  // 0 = off
  int32_t chunk;                   // 0 = off
};

hipError_t launch_recycle_pages(const RecycleParams& p, hipStream_t stream);

// Plain random-page read (the ceiling of the decode's access pattern).
struct ReadPagesParams {
  const uint8_t* base;         // pages of page_bytes bytes
  const int32_t* page_ids;     // [num_pages] pages to read (outside the buffer: page 0)
  uint32_t* sink;              // [num_waves] XOR of the bytes each wave read
  int64_t num_pages;
  int64_t num_base_pages;      // pages in the buffer
  int32_t page_bytes;          // 1024, 2048 or 4096
  int32_t num_waves;           // a multiple of 4
};
hipError_t launch_read_pages(const ReadPagesParams& p, hipStream_t stream);

// ---- prefix-caching block manager -------------------------------------------
// State of a pool of N blocks, one device buffer (regions 256-byte aligned, in
// this order after a 256-byte header of int32: free count, cached count,
// tombstones, N, table capacity).
enum BmRegion { kBmFree, kBmRef, kBmTs, kBmDepth, kBmParent, kBmFlags, kBmHash, kBmTokens,
                kBmTable, kBmMark, kBmOwner, kBmRegions };
struct BmLayout {
  int64_t off[kBmRegions];
  int64_t bytes;
  int32_t cap;                      // table slots (a power of two >= 2N)
};
BmLayout bm_layout(int32_t num_blocks);

struct BmState {
  int32_t* hdr;
  int32_t* free_stack;   // [N], top at hdr[0] - 1
  int32_t* ref;          // [N]
  uint32_t* ts;          // [N]
  int32_t* depth;        // [N]
  int32_t* parent;       // [N]
  int32_t* flags;        // [N] bit 0: cached
  uint64_t* chash;       // [N] chain hash of a cached block's whole prefix
  int32_t* tokens;       // [N, 16]
  int32_t* table;        // [cap] -1 empty, -2 tombstone, else a cached block
  int32_t* mark;         // [N] per-call scratch
  int32_t* owner;        // [N] per-call scratch
  int32_t num_blocks;
  int32_t cap;
};
BmState bm_state(void* base, int32_t num_blocks);

struct BmScheduleParams {
  BmState st;
  const int32_t* token_ids;
  const int32_t* token_start;    // [B + 1]
  const int32_t* num_computed;   // [B]
  const int32_t* query_start_loc;  // [B + 1]
  int32_t* block_tables;         // [B, mb]
  int64_t* slot_mapping;         // [sum_q]
  int32_t* num_cached;           // [B]
  int32_t* status;               // [1]
  uint64_t* ws_hash;             // [B * mb] chain hashes
  int32_t* ws_cand;              // [B * mb] lookup candidates, then claimed slots
  int64_t num_token_ids;
  int32_t num_seqs;
  int32_t mb;
  int32_t sum_q;
  uint32_t now;
};
constexpr int kBmMaxSeqs = 2048;
size_t bm_workspace_bytes(int32_t num_seqs, int32_t mb);
hipError_t launch_bm_init(const BmState& st, hipStream_t stream);
hipError_t launch_bm_schedule(const BmScheduleParams& p, hipStream_t stream);

struct BmReleaseParams {
  BmState st;
  const int32_t* block_tables;   // [B, mb]
  const int32_t* num_tokens;     // [B]
  int32_t num_seqs;
  int32_t mb;
  uint32_t now;
};
hipError_t launch_bm_release(const BmReleaseParams& p, hipStream_t stream);

// Decode work split: at most this many waves, each taking at least
// kMinChunkPages pages when the chunk size is automatic.
constexpr int kMaxWorkers = 4096;
constexpr int kMinChunkPages = 4;
// Bytes at the start of a decode workspace for the per-unit piece records
// (two int32 per unit).
constexpr size_t kUnitBytes = size_t(1) << 20;
// Waves per workgroup of the decode kernel.
constexpr int kDecodeWaves = 4;

// Query heads handled per decode work unit: the whole group when g <= 8,
// else the largest divisor of g that is at most 8.
inline int decode_head_chunk(int g) {
  if (g <= 8) return g;
  for (int c = 8; c > 1; --c)
    if (g % c == 0) return c;
  return 1;
}

// Largest wave count decode_workers returns for an upper bound of the page
// count: at least one workgroup, at most kMaxWorkers, about kMinChunkPages
// pages per wave, a whole number of workgroups.
constexpr int64_t decode_workers_bound(int64_t pages_bound) {
  int64_t w = (pages_bound + kMinChunkPages - 1) / kMinChunkPages;
  w = w < kDecodeWaves ? kDecodeWaves : w;
  w = w > kMaxWorkers ? kMaxWorkers : w;
  return (w + kDecodeWaves - 1) / kDecodeWaves * kDecodeWaves;
}

// Workers (waves) the decode grid uses for an upper bound of the page count
// (never more than decode_workers_bound(pages_bound)).
int decode_workers(int64_t pages_bound, int head_dim, int kv_fmt, int q_fmt, int head_chunk,
                   bool append = false);

}  // namespace vp

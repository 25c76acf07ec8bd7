// Prefix-caching KV block manager on the device: the step before paged
// attention, which fills each sequence's block table and the cache write's
// slot mapping ("Building and Deploying vllm.cpp", Step 3: radix prefix
// matching over runs of physical blocks, zero-copy hits that bind a new
// sequence's table to existing pages, LRU eviction of the oldest leaves; the
// vllm.cpp repository listing, "What's implemented": hash-based prefix
// caching in the KV cache manager).
//
// The trie has one node per full 16-token block, keyed by (parent, tokens).
// Its index is an open-addressing table over the chain hash of the block's
// whole token prefix: h_j = h_{j-1} * R^16 + sum_k (t_k + 1) R^(15-k) mod
// 2^64 (Karp and Rabin's polynomial hash, h_{-1} = 1), slots picked by the
// splitmix64 finalizer.  A hit is exact: the block found must hold the same
// tokens and hang under the block matched one level up.  Cached blocks
// carry distinct chain hashes (a block whose hash is taken stays uncached).
//
// One call runs as one workgroup of 1024 threads; every step is parallel
// over (request, block) items, with per-request values in LDS:
//   1. chain hashes of every full block;
//   2. lookups of a new request's blocks (at most (len - 1) / 16 of them,
//      so one token is computed) against the index as it stood, then a
//      parallel check of tokens and parent links; the hit length is the
//      first failing block;
//   3. the blocks needed are prefix-summed; if fewer are free, the oldest
//      unreferenced cached blocks are evicted: a radix select over
//      (timestamp, -depth) finds the cut, an ordered compaction takes them
//      in block-id order (ties at the cut by id), their index slots become
//      tombstones and they go on the free stack;
//   4. hits are bound (reference +1), fresh blocks popped in (request,
//      block) order;
//   5. blocks that became full are inserted: each claims a slot with
//      compare-and-swap; an equal hash already cached wins, between two
//      requests of the call the lower one wins, and a request stops at its
//      first loss (its later blocks are withdrawn again);
//   6. slots of the computed tokens (-1 for reused ones).
// The index is rebuilt in place when entries and tombstones would pass 3/4
// of its slots.  Calls that cannot be served leave everything unchanged.
#include <algorithm>
#include <climits>

#include "common.h"
#include "kernels.h"

namespace vp {

namespace {

constexpr int kBT = 1024;                 // threads of the manager's workgroup
constexpr int kBlk = 16;
constexpr int32_t kEmpty = -1, kTomb = -2;
constexpr int32_t kCached = 1;
constexpr int32_t kMarkHit = 1, kMarkCand = 2;
constexpr uint64_t kBase = 0x9E3779B97F4A7C15ull;   // odd
constexpr uint64_t kSeed = 1;

constexpr uint64_t pow_base(int e) {
  uint64_t r = 1;
  for (int i = 0; i < e; ++i) r *= kBase;
  return r;
}
constexpr uint64_t kBase16 = pow_base(kBlk);

__device__ __forceinline__ uint64_t mix64(uint64_t z) {     // splitmix64 finalizer
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Every call runs as one workgroup, so the threads that race on the index
// (claims of a slot) synchronize at workgroup scope; all other data is
// handed between phases by the workgroup barriers.
template <class T>
__device__ __forceinline__ T ld_acq(const T* p) {
  return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ int32_t cas(int32_t* p, int32_t expected, int32_t desired) {
  __hip_atomic_compare_exchange_strong(p, &expected, desired, __ATOMIC_ACQ_REL, __ATOMIC_ACQUIRE,
                                       __HIP_MEMORY_SCOPE_WORKGROUP);
  return expected;                         // the value found (== expected on success)
}

// Exclusive prefix of a[0 .. n) in place (n <= kBmMaxSeqs); a[n] = total.
// Thread t owns entries 2t and 2t + 1: a wave-wide scan of the pair sums,
// then one scan of the 16 wave totals.
__device__ void excl_scan(int* a, int n) {
  __shared__ int s_w[kBT / 64];
  __shared__ int s_total;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  __syncthreads();                                   // the callers' writes of a[]
  const int i0 = 2 * t, i1 = 2 * t + 1;
  const int x0 = i0 < n ? a[i0] : 0, x1 = i1 < n ? a[i1] : 0;
  int v = x0 + x1;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int u = __shfl_up(v, off);
    if (lane >= off) v += u;
  }
  if (lane == 63) s_w[w] = v;
  __syncthreads();
  if (w == 0) {
    const int tw = lane < kBT / 64 ? s_w[lane] : 0;
    int c = tw;
#pragma unroll
    for (int off = 1; off < kBT / 64; off <<= 1) {
      const int u = __shfl_up(c, off);
      if (lane >= off) c += u;
    }
    if (lane < kBT / 64) s_w[lane] = c - tw;
    if (lane == kBT / 64 - 1) s_total = c;
  }
  __syncthreads();
  const int base = s_w[w] + v - (x0 + x1);
  a[i0] = base;                                      // (entries past n end up = total)
  a[i1] = base + x0;
  if (t == 0) a[kBmMaxSeqs] = s_total;
  __syncthreads();
}

// Request holding item i of an exclusive prefix pre[0 .. B] (last r with
// pre[r] <= i).
__device__ __forceinline__ int find_req(const int* pre, int B, int i) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pre[mid] <= i) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ uint64_t evict_key(const BmState& S, int b) {
  const uint32_t d = (uint32_t)min(max(S.depth[b], 0), 0xFFFF);
  return ((uint64_t)S.ts[b] << 16) | (0xFFFFu - d);
}

__device__ __forceinline__ bool evictable(const BmState& S, int b) {
  return (S.flags[b] & kCached) && S.ref[b] == 0 && !(S.mark[b] & kMarkHit);
}

// Slot of cached block b in the index (the table holds it).
__device__ __forceinline__ int find_slot(const BmState& S, int b) {
  int slot = (int)(mix64(S.chash[b]) & (uint64_t)(S.cap - 1));
  for (int it = 0; it < S.cap; ++it) {
    const int v = S.table[slot];
    if (v == b) return slot;
    if (v == kEmpty) return -1;
    slot = (slot + 1) & (S.cap - 1);
  }
  return -1;
}

// Insert a cached block whose hash is unique in the table (rebuild).
__device__ __forceinline__ void insert_unique(const BmState& S, int b) {
  int slot = (int)(mix64(S.chash[b]) & (uint64_t)(S.cap - 1));
  for (int it = 0; it < S.cap; ++it) {
    if (S.table[slot] == kEmpty && cas(&S.table[slot], kEmpty, b) == kEmpty) return;
    slot = (slot + 1) & (S.cap - 1);
  }
}

}  // namespace

__global__ __launch_bounds__(kBT) void bm_init_kernel(BmState S) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int N = S.num_blocks;
  for (int64_t i = i0; i < N; i += stride) {
    S.free_stack[i] = N - 1 - (int32_t)i;
    S.ref[i] = 0;
    S.ts[i] = 0;
    S.depth[i] = 0;
    S.parent[i] = -1;
    S.flags[i] = 0;
    S.chash[i] = 0;
    S.mark[i] = 0;
    S.owner[i] = 0;
  }
  for (int64_t i = i0; i < (int64_t)N * kBlk; i += stride) S.tokens[i] = 0;
  for (int64_t i = i0; i < S.cap; i += stride) S.table[i] = kEmpty;
  if (i0 == 0) {
    S.hdr[0] = N;          // free blocks
    S.hdr[1] = 0;          // cached blocks
    S.hdr[2] = 0;          // tombstones
    S.hdr[3] = N;
    S.hdr[4] = S.cap;
  }
}

// First block of request r whose chain hash the call needs: all of a new
// request's full blocks (lookups, then insertions); for a running request the
// blocks that became full, when the block before them is cached (else it
// caches nothing and needs none).
__device__ __forceinline__ int hash_lo(const BmScheduleParams& p, const int* s_old,
                                       const int* s_new, int r) {
  const int old = s_old[r], last = s_new[r] / kBlk;
  if (old == 0) return 0;
  const int first = old / kBlk;
  if (first >= last) return last;
  if (first == 0) return 0;
  const int b = p.block_tables[(int64_t)r * p.mb + first - 1];
  return (p.st.flags[b] & kCached) ? first : last;
}

__global__ __launch_bounds__(kBT) void bm_schedule_kernel(BmScheduleParams p) {
  __shared__ int s_old[kBmMaxSeqs], s_new[kBmMaxSeqs], s_hits[kBmMaxSeqs], s_lost[kBmMaxSeqs];
  __shared__ int s_pre[kBmMaxSeqs + 1], s_off[kBmMaxSeqs + 1], s_tmp[kBmMaxSeqs + 1];
  __shared__ uint32_t s_hist[256];
  __shared__ int s_bad, s_evictable, s_free, s_live, s_tomb, s_rem;
  __shared__ uint64_t s_prefix;
  const BmState& S = p.st;
  const int t = threadIdx.x;
  const int B = p.num_seqs, mb = p.mb, N = S.num_blocks, cap = S.cap;
  const int64_t MB = mb;
  int32_t* const rows = p.block_tables;
  if (t == 0) {
    s_bad = S.hdr[3] != N;                 // a state set up for another pool size
    s_evictable = 0;
    s_free = S.hdr[0];
    s_live = S.hdr[1];
    s_tomb = S.hdr[2];
  }
  __syncthreads();

  // ---- per-request values; metadata that do not fit change nothing
  for (int r = t; r < B; r += kBT) {
    {
      const int64_t old = p.num_computed[r];
      const int64_t qa = p.query_start_loc[r], qb = p.query_start_loc[r + 1];
      const int64_t ta = p.token_start[r], tb = p.token_start[r + 1];
      const int64_t nw = old + (qb - qa);
      const bool bad = old < 0 || qb < qa || qa < 0 || qb > p.sum_q || ta < 0 ||
                       tb > p.num_token_ids || tb - ta != nw || (nw + kBlk - 1) / kBlk > mb;
      if (bad) atomicOr(&s_bad, 1);
      s_old[r] = bad ? 0 : (int)old;
      s_new[r] = bad ? 0 : (int)nw;
      s_hits[r] = (!bad && old == 0 && nw > 0) ? (int)((nw - 1) / kBlk) : 0;   // at most
      s_lost[r] = INT_MAX;
    }
  }
  // existing entries in range, 16 per item
  for (int r = t; r < kBmMaxSeqs; r += kBT)
    s_pre[r] = r < B ? ((s_old[r] + kBlk - 1) / kBlk + 15) / 16 : 0;
  excl_scan(s_pre, B);
  for (int i = t; i < s_pre[B]; i += kBT) {
    const int r = find_req(s_pre, B, i), j0 = 16 * (i - s_pre[r]);
    const int j1 = min(j0 + 16, (s_old[r] + kBlk - 1) / kBlk);
    bool out = false;
    for (int j = j0; j < j1; ++j) out |= (uint32_t)rows[r * MB + j] >= (uint32_t)N;
    if (out) atomicOr(&s_bad, 1);
  }
  __syncthreads();
  if (s_bad) {
    if (t == 0) *p.status = 2;
    return;
  }

  // ---- 1. chain hashes of the blocks the call needs
  for (int r = t; r < kBmMaxSeqs; r += kBT)
    s_pre[r] = r < B ? s_new[r] / kBlk - hash_lo(p, s_old, s_new, r) : 0;
  excl_scan(s_pre, B);
  for (int i = t; i < s_pre[B]; i += kBT) {
    const int r = find_req(s_pre, B, i);
    const int j = hash_lo(p, s_old, s_new, r) + i - s_pre[r];
    const int32_t* tk = p.token_ids + p.token_start[r] + (int64_t)kBlk * j;
    uint64_t h = 0;
#pragma unroll
    for (int k = 0; k < kBlk; ++k) h = h * kBase + (uint64_t)(uint32_t)tk[k] + 1;
    p.ws_hash[r * MB + j] = h;
  }
  __syncthreads();
  for (int r = t; r < B; r += kBT) {
    const int lo = hash_lo(p, s_old, s_new, r), nf = s_new[r] / kBlk;
    if (lo >= nf) continue;
    uint64_t h = lo == 0 ? kSeed : S.chash[rows[r * MB + lo - 1]];
    uint64_t* w = p.ws_hash + r * MB;
    // (eight blocks' hashes read before any is chained: one memory round
    // trip per eight blocks of a long prompt, not one per block)
    for (int j0 = lo; j0 < nf; j0 += 8) {
      uint64_t x[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) x[k] = j0 + k < nf ? w[j0 + k] : 0;
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (j0 + k < nf) {
          h = h * kBase16 + x[k];
          w[j0 + k] = h;
        }
    }
  }
  __syncthreads();

  // ---- 2. lookups, then the exact check (tokens, parent link)
  for (int r = t; r < kBmMaxSeqs; r += kBT) s_pre[r] = r < B ? s_hits[r] : 0;
  excl_scan(s_pre, B);
  for (int i = t; i < s_pre[B]; i += kBT) {
    const int r = find_req(s_pre, B, i), j = i - s_pre[r];
    const uint64_t c = p.ws_hash[r * MB + j];
    int slot = (int)(mix64(c) & (uint64_t)(cap - 1)), cand = -1;
    for (int it = 0; it < cap; ++it) {
      const int v = S.table[slot];
      if (v == kEmpty) break;
      if (v >= 0 && S.chash[v] == c) { cand = v; break; }
      slot = (slot + 1) & (cap - 1);
    }
    p.ws_cand[r * MB + j] = cand;
  }
  __syncthreads();
  for (int i = t; i < s_pre[B]; i += kBT) {
    const int r = find_req(s_pre, B, i), j = i - s_pre[r];
    const int b = p.ws_cand[r * MB + j];
    bool ok = b >= 0 && (S.flags[b] & kCached) &&
              S.parent[b] == (j > 0 ? p.ws_cand[r * MB + j - 1] : -1);
    if (ok) {
      const int32_t* tk = p.token_ids + p.token_start[r] + (int64_t)kBlk * j;
      for (int k = 0; k < kBlk; ++k) ok = ok && S.tokens[(int64_t)b * kBlk + k] == tk[k];
    }
    if (!ok) atomicMin(&s_hits[r], j);
  }
  __syncthreads();

  // ---- 3. blocks needed; eviction when the free stack is short
  for (int r = t; r < kBmMaxSeqs; r += kBT) {
    s_off[r] = r < B ? (s_new[r] + kBlk - 1) / kBlk - (s_old[r] + kBlk - 1) / kBlk - s_hits[r] : 0;
    s_pre[r] = r < B ? s_hits[r] : 0;
  }
  __syncthreads();
  excl_scan(s_off, B);
  excl_scan(s_pre, B);
  const int total = s_off[B];
  for (int i = t; i < s_pre[B]; i += kBT) {
    const int r = find_req(s_pre, B, i), j = i - s_pre[r];
    atomicOr(&S.mark[p.ws_cand[r * MB + j]], kMarkHit);
  }
  __syncthreads();
  const int E = total - s_free;
  if (E > 0) {
    int cnt = 0;
    for (int b = t; b < N; b += kBT) cnt += evictable(S, b);
    atomicAdd(&s_evictable, cnt);
    __syncthreads();
    if (E > s_evictable) {
      for (int i = t; i < s_pre[B]; i += kBT) {            // leave the marks clear
        const int r = find_req(s_pre, B, i), j = i - s_pre[r];
        S.mark[p.ws_cand[r * MB + j]] = 0;
      }
      if (t == 0) *p.status = 1;
      return;
    }
    // radix select of the E-th smallest key (8-bit digits, most significant first)
    if (t == 0) { s_prefix = 0; s_rem = E; }
    for (int shift = 40; shift >= 0; shift -= 8) {
      for (int d = t; d < 256; d += kBT) s_hist[d] = 0;
      __syncthreads();
      const uint64_t pre = s_prefix;
      for (int b = t; b < N; b += kBT) {
        if (!evictable(S, b)) continue;
        const uint64_t k = evict_key(S, b);
        if ((k >> (shift + 8)) == (pre >> (shift + 8))) atomicAdd(&s_hist[(k >> shift) & 255], 1u);
      }
      __syncthreads();
      if (t == 0) {
        int cum = 0;
        for (int d = 0; d < 256; ++d) {
          if (cum + (int)s_hist[d] >= s_rem) {
            s_prefix = pre | ((uint64_t)d << shift);
            s_rem -= cum;
            break;
          }
          cum += (int)s_hist[d];
        }
      }
      __syncthreads();
    }
    const uint64_t K = s_prefix;
    const int take_eq = s_rem;             // blocks with key K taken, lowest ids first
    // ordered compaction: thread t owns ids [lo, hi)
    const int per = (N + kBT - 1) / kBT;
    const int lo = min(N, t * per), hi = min(N, lo + per);
    int eq = 0;
    for (int b = lo; b < hi; ++b) eq += evictable(S, b) && evict_key(S, b) == K;
    s_tmp[t] = eq;
    excl_scan(s_tmp, kBT);
    const int eq_before = s_tmp[t];
    __syncthreads();
    int take = 0;
    for (int b = lo, e = eq_before; b < hi; ++b) {
      if (!evictable(S, b)) continue;
      const uint64_t k = evict_key(S, b);
      if (k < K) ++take;
      else if (k == K) take += (e++ < take_eq);
    }
    s_tmp[t] = take;
    excl_scan(s_tmp, kBT);
    int pos = s_free + s_tmp[t];
    for (int b = lo, e = eq_before; b < hi; ++b) {
      if (!evictable(S, b)) continue;
      const uint64_t k = evict_key(S, b);
      const bool v = k < K || (k == K && e++ < take_eq);
      if (!v) continue;
      const int slot = find_slot(S, b);
      if (slot >= 0) S.table[slot] = kTomb;
      S.flags[b] = 0;
      S.free_stack[pos++] = b;
    }
    __syncthreads();
    if (t == 0) {
      s_free += E;
      s_live -= E;
      s_tomb += E;
    }
    __syncthreads();
  }

  // ---- 4. bind hits, pop fresh blocks
  const int fc = s_free;                   // free stack height before the pops
  for (int i = t; i < s_pre[B]; i += kBT) {
    const int r = find_req(s_pre, B, i), j = i - s_pre[r];
    const int b = p.ws_cand[r * MB + j];
    rows[r * MB + j] = b;
    atomicAdd(&S.ref[b], 1);
    S.ts[b] = p.now;
    S.mark[b] = 0;
  }
  for (int i = t; i < total; i += kBT) {
    const int r = find_req(s_off, B, i), k = i - s_off[r];
    const int base = (s_old[r] + kBlk - 1) / kBlk + s_hits[r];   // first fresh entry
    const int j = base + k;
    const int b = S.free_stack[fc - 1 - i];
    int par = -1;                          // the block one level up
    if (j > 0) {
      if (k > 0) par = S.free_stack[fc - i];
      else if (s_hits[r] > 0) par = p.ws_cand[r * MB + j - 1];
      else par = rows[r * MB + j - 1];
    }
    rows[r * MB + j] = b;
    S.ref[b] = 1;
    S.ts[b] = p.now;
    S.depth[b] = j;
    S.parent[b] = par;
    S.flags[b] = 0;
  }
  __syncthreads();
  if (t == 0) s_free = fc - total;

  // ---- 5. cache the blocks that became full
  for (int r = t; r < kBmMaxSeqs; r += kBT) {
    int cnt = 0;
    if (r < B) {
      const int first = s_old[r] == 0 ? s_hits[r] : s_old[r] / kBlk, last = s_new[r] / kBlk;
      const bool base_ok = first == 0 || (S.flags[rows[r * MB + first - 1]] & kCached);
      cnt = (first < last && base_ok) ? last - first : 0;
    }
    s_tmp[r] = cnt;
  }
  excl_scan(s_tmp, B);
  const int ncand = s_tmp[B];
  if (s_live + s_tomb + ncand > cap / 4 * 3) {            // rebuild the index in place
    for (int i = t; i < cap; i += kBT) S.table[i] = kEmpty;
    __syncthreads();
    for (int b = t; b < N; b += kBT)
      if (S.flags[b] & kCached) insert_unique(S, b);
    __syncthreads();
    if (t == 0) s_tomb = 0;
  }
  __syncthreads();
  for (int i = t; i < ncand; i += kBT) {                   // claims
    const int r = find_req(s_tmp, B, i);
    const int first = s_old[r] == 0 ? s_hits[r] : s_old[r] / kBlk;
    const int j = first + i - s_tmp[r];
    const int b = rows[r * MB + j];
    const uint64_t c = p.ws_hash[r * MB + j];
    const int32_t* tk = p.token_ids + p.token_start[r] + (int64_t)kBlk * j;
    for (int k = 0; k < kBlk; ++k) S.tokens[(int64_t)b * kBlk + k] = tk[k];
    S.chash[b] = c;
    S.parent[b] = j > 0 ? rows[r * MB + j - 1] : -1;
    S.depth[b] = j;
    S.owner[b] = r;
    S.mark[b] = kMarkCand;
    // (the compare-and-swap below releases these writes to the readers of the slot)
    int slot = (int)(mix64(c) & (uint64_t)(cap - 1)), got = -1;
    for (int it = 0; it < 4 * cap + 64; ++it) {            // each retry follows another claim
      int v = ld_acq(&S.table[slot]);
      if (v == kEmpty) {
        v = cas(&S.table[slot], kEmpty, b);
        if (v == kEmpty) { got = slot; break; }
      }
      if (v == kTomb || (v >= 0 && S.chash[v] != c)) {
        slot = (slot + 1) & (cap - 1);
        continue;
      }
      if (v < 0) continue;                 // (the slot changed under us: look again)
      // equal hash: an entry cached before the call, or the lower request, keeps it
      if (!(S.mark[v] & kMarkCand) || S.owner[v] <= r) break;
      if (cas(&S.table[slot], v, b) == v) { got = slot; break; }
    }
    p.ws_cand[r * MB + j] = got;
  }
  __syncthreads();
  for (int i = t; i < ncand; i += kBT) {                   // losses
    const int r = find_req(s_tmp, B, i);
    const int first = s_old[r] == 0 ? s_hits[r] : s_old[r] / kBlk;
    const int j = first + i - s_tmp[r];
    const int b = rows[r * MB + j];
    const int got = p.ws_cand[r * MB + j];
    if (got < 0 || ld_acq(&S.table[got]) != b) atomicMin(&s_lost[r], j);
  }
  __syncthreads();
  for (int i = t; i < ncand; i += kBT) {                   // keep or withdraw
    const int r = find_req(s_tmp, B, i);
    const int first = s_old[r] == 0 ? s_hits[r] : s_old[r] / kBlk;
    const int j = first + i - s_tmp[r];
    const int b = rows[r * MB + j];
    const int got = p.ws_cand[r * MB + j];
    S.mark[b] = 0;
    if (got < 0 || S.table[got] != b) continue;
    if (j < s_lost[r]) {
      S.flags[b] = kCached;
      atomicAdd(&s_live, 1);
    } else {
      S.table[got] = kTomb;
      atomicAdd(&s_tomb, 1);
    }
  }
  __syncthreads();

  // ---- 6. slots of the computed tokens
  for (int r = t; r < B; r += kBT) p.num_cached[r] = max(s_old[r], kBlk * s_hits[r]);
  // 16 query rows per item
  for (int r = t; r < kBmMaxSeqs; r += kBT)
    s_pre[r] = r < B ? (s_new[r] - s_old[r] + 15) / 16 : 0;
  excl_scan(s_pre, B);
  for (int i = t; i < s_pre[B]; i += kBT) {
    const int r = find_req(s_pre, B, i), c = i - s_pre[r];
    const int q0 = p.query_start_loc[r];
    const int start = max(s_old[r], kBlk * s_hits[r]);
    const int i1 = min(16 * c + 16, s_new[r] - s_old[r]);
    for (int k = 16 * c; k < i1; ++k) {
      const int tok = s_old[r] + k;
      p.slot_mapping[q0 + k] = tok >= start ? (int64_t)rows[r * MB + tok / kBlk] * kBlk + tok % kBlk
                                            : (int64_t)-1;
    }
  }
  {
    // rows of no request (before the first or past the last offset)
    const int q0 = B > 0 ? p.query_start_loc[0] : p.sum_q, qe = B > 0 ? p.query_start_loc[B] : p.sum_q;
    for (int i = t; i < q0; i += kBT) p.slot_mapping[i] = -1;
    for (int i = qe + t; i < p.sum_q; i += kBT) p.slot_mapping[i] = -1;
  }
  if (t == 0) {
    S.hdr[0] = s_free;
    S.hdr[1] = s_live;
    S.hdr[2] = s_tomb;
    *p.status = 0;
  }
}

__global__ __launch_bounds__(kBT) void bm_release_kernel(BmReleaseParams p) {
  __shared__ int s_pre[kBmMaxSeqs + 1];
  __shared__ int s_free;
  const BmState& S = p.st;
  const int t = threadIdx.x;
  const int B = p.num_seqs, N = S.num_blocks;
  const int64_t MB = p.mb;
  if (S.hdr[3] != N) return;               // a state set up for another pool size
  if (t == 0) s_free = S.hdr[0];
  for (int r = t; r < kBmMaxSeqs; r += kBT) {
    int cnt = 0;
    if (r < B) {
      const int nb = min(max((p.num_tokens[r] + kBlk - 1) / kBlk, 0), p.mb);
      for (int j = 0; j < nb; ++j) {
        const int b = p.block_tables[r * MB + j];
        cnt += b >= 0 && b < N && !(S.flags[b] & kCached);
      }
    }
    s_pre[r] = cnt;
  }
  excl_scan(s_pre, B);
  for (int r = t; r < B; r += kBT) {
    const int nb = min(max((p.num_tokens[r] + kBlk - 1) / kBlk, 0), p.mb);
    int pos = s_free + s_pre[r];
    for (int j = 0; j < nb; ++j) {
      const int b = p.block_tables[r * MB + j];
      if (b < 0 || b >= N) continue;
      int cur = ld_acq(&S.ref[b]);             // one reference less, never below 0
      while (cur > 0) {
        const int seen = cas(&S.ref[b], cur, cur - 1);
        if (seen == cur) break;
        cur = seen;
      }
      S.ts[b] = p.now;
      if (!(S.flags[b] & kCached)) {
        if (pos < N) S.free_stack[pos] = b;
        ++pos;
      }
    }
  }
  __syncthreads();
  if (t == 0) S.hdr[0] = min(N, s_free + s_pre[B]);
}

hipError_t launch_bm_init(const BmState& st, hipStream_t stream) {
  const int64_t work = std::max<int64_t>((int64_t)st.num_blocks * kBlk, st.cap);
  const int grid = (int)std::min<int64_t>(1024, (work + kBT - 1) / kBT);
  hipLaunchKernelGGL(bm_init_kernel, dim3(std::max(grid, 1)), dim3(kBT), 0, stream, st);
  return hipGetLastError();
}

hipError_t launch_bm_schedule(const BmScheduleParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(bm_schedule_kernel, dim3(1), dim3(kBT), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_bm_release(const BmReleaseParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(bm_release_kernel, dim3(1), dim3(kBT), 0, stream, p);
  return hipGetLastError();
}

}  // namespace vp

// Metadata kernels of local attention (the local-attention section of the
// vllm.cpp repository listing, "What's implemented": chunked-local attention
// through exact virtual Q/K batches and a reusable block-table gather/update
// plan; sliding-window and fixed-chunk page recycling).
//
// chunked_local_plan_kernel.  Chunked-local attention of chunk L keeps, for
// the query at position p, the keys floor(p / L) * L .. p.  Every (sequence,
// chunk) holding query tokens becomes one ordinary causal sequence of a
// virtual batch, in (sequence, chunk) order: its query rows are the chunk's
// rows of q (in place), its context runs from the chunk start to its last
// query token, and its block table is the slice of the sequence's table from
// the chunk start (-1 past its context).  The plan depends only on the batch
// metadata, so one plan serves every layer.
//
// recycle_pages_kernel.  Leading pages that no query at position >= n (the
// next token's) can attend to are reported (compactly, with per-sequence
// offsets) and their table entries set to -1: keys t <= n - W with a sliding
// window W, keys below floor(n / L) * L with chunked-local attention of L.
//
// Both prefix-sum per-sequence counts with a block scan over the threads of
// a workgroup.  The recycling runs as one workgroup: a wave per sequence
// counts the live entries of its dead pages (coalesced reads), the scan turns
// the counts into offsets, and a wave per sequence writes its entries in
// table order (a ballot and a bit count per 64 entries).  The plan's tables are most of its output
// (V rows of L / 16 entries), so it runs on several workgroups: each one
// repeats the scan (a few loads per thread), describes its share of the
// virtual rows in LDS and then writes their table entries, consecutive
// threads on consecutive entries with several reads in flight per thread.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace vp {

namespace {

constexpr int kLT = 1024;     // threads of a metadata workgroup
constexpr int kRowBatch = 1024;    // virtual rows a plan workgroup describes in LDS at once
constexpr int kCopyUnroll = 8;     // table entries in flight per thread
constexpr int kPlanMaxGroups = 64;

// Exclusive prefix of per-thread totals over the workgroup; returns this
// thread's offset and writes the grand total to *total.  Each wave scans its
// 64 values with lane shifts, then every thread adds the totals of the waves
// before its own (two barriers).
__device__ int64_t block_exclusive_scan(int64_t v, int64_t* total) {
  constexpr int kW = kLT / 64;
  __shared__ int64_t s_w[kW];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int64_t x = v;                                 // inclusive scan within the wave
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) s_w[w] = x;
  __syncthreads();
  int64_t before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < kW; ++i) {
    const int64_t t = s_w[i];
    before += i < w ? t : 0;
    all += t;
  }
  *total = all;
  __syncthreads();                               // (s_w is reused by the next call)
  return before + x - v;
}

}  // namespace

__global__ __launch_bounds__(kLT) void chunked_local_plan_kernel(LocalPlanParams p) {
  const int B = p.num_seqs;
  const int L = p.chunk;
  const int P = L / 16;                         // table entries per virtual sequence
  const int per = (B + kLT - 1) / kLT;
  const int s0 = threadIdx.x * per;
  // rows of q: given, or query_start_loc[B]
  const int sumq = p.num_tokens >= 0 ? p.num_tokens : max(p.query_start_loc[B], 0);
  // (clamped so that no value of the metadata leads outside the tables: a
  // context shorter than its chunk keeps only its last n query rows)
  auto seq = [&](int s, int& qa, int& qb, int& n) __attribute__((always_inline)) {
    qa = min(max(p.query_start_loc[s], 0), sumq);
    qb = min(max(p.query_start_loc[s + 1], qa), sumq);
    n = min(max(p.context_lens[s], 0), p.bt_stride * 16);
    if (qb - qa > n) qa = qb - n;
  };
  int64_t cnt = 0;
  for (int i = 0; i < per; ++i) {
    const int s = s0 + i;
    if (s >= B) break;
    int qa, qb, n;
    seq(s, qa, qb, n);
    if (qb > qa) cnt += (n - 1) / L - (n - (qb - qa)) / L + 1;
  }
  int64_t total = 0;
  const int64_t v0 = block_exclusive_scan(cnt, &total);   // this thread's first row
  const int64_t V = p.num_virtual;
  const int64_t used = min(total, V);
  // this workgroup's rows [r0, r1), in batches of nb rows (nb P < 2^31)
  const int64_t span = (V + gridDim.x - 1) / gridDim.x;
  const int64_t r0 = min(V, (int64_t)blockIdx.x * span), r1 = min(V, r0 + span);
  const int nb = max(1, min(kRowBatch, (1 << 30) / P));
  __shared__ int64_t s_src[kRowBatch];          // block_tables offset of a row's first entry
  __shared__ int s_npg[kRowBatch];              // the row's pages (0: an unused row)
  for (int64_t b0 = r0; b0 < r1; b0 += nb) {
    const int64_t b1 = min(r1, b0 + nb);
    // unused virtual sequences: no rows, no keys
    for (int64_t w = max(used, b0) + threadIdx.x; w < b1; w += kLT) {
      p.v_query_start_loc[w] = sumq;
      p.v_context_lens[w] = 0;
      s_src[w - b0] = 0;
      s_npg[w - b0] = 0;
    }
    // the rows of this thread's sequences that fall in the batch
    int64_t v = v0;
    for (int i = 0; i < per && v < b1; ++i) {
      const int s = s0 + i;
      if (s >= B) break;
      int qa, qb, n;
      seq(s, qa, qb, n);
      if (qb <= qa) continue;
      const int first = n - (qb - qa);          // position of the first query token
      const int c_first = first / L, c_last = (n - 1) / L;
      if (v + (c_last - c_first + 1) <= b0) {   // all before the batch
        v += c_last - c_first + 1;
        continue;
      }
      for (int c = c_first; c <= c_last && v < b1; ++c, ++v) {
        if (v < b0) continue;
        const int lo = max(first, c * L), hi = min(n - 1, c * L + L - 1);
        const int vlen = hi + 1 - c * L;
        p.v_query_start_loc[v] = qa + (lo - first);
        p.v_context_lens[v] = vlen;
        s_src[v - b0] = (int64_t)s * p.bt_stride + (int64_t)c * P;
        s_npg[v - b0] = (vlen + 15) / 16;
      }
    }
    __syncthreads();
    // their table entries: the slice of the sequence's table, -1 past the
    // context (and for unused rows)
    int32_t* dst = p.v_block_tables + b0 * P;
    const uint32_t ne = (uint32_t)((b1 - b0) * P);
    for (uint32_t e = threadIdx.x; e < ne; e += kCopyUnroll * kLT) {
      int32_t x[kCopyUnroll];
#pragma unroll
      for (int k = 0; k < kCopyUnroll; ++k) {
        const uint32_t ek = e + k * kLT;
        x[k] = -1;
        if (ek < ne) {
          const uint32_t r = ek / (uint32_t)P, j = ek - r * (uint32_t)P;
          if ((int)j < s_npg[r]) x[k] = p.block_tables[s_src[r] + j];
        }
      }
#pragma unroll
      for (int k = 0; k < kCopyUnroll; ++k) {
        const uint32_t ek = e + k * kLT;
        if (ek < ne) dst[ek] = x[k];
      }
    }
    __syncthreads();
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) p.v_query_start_loc[V] = sumq;
}

__global__ __launch_bounds__(kLT) void recycle_pages_kernel(RecycleParams p) {
  constexpr int kWaves = kLT / 64;
  constexpr int kU = 4;                         // 64-entry pieces read at once per wave
  const int B = p.num_seqs;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  auto dead_of = [&](int s) __attribute__((always_inline)) {
    const int n = max(p.context_lens[s], 0);
    int dead = 0;
    if (p.window > 0) dead = max(dead, n + 1 - p.window);
    if (p.chunk > 0) dead = max(dead, (n / p.chunk) * p.chunk);
    return min(max(dead, 0) / 16, p.bt_stride);
  };
  // live entries among each sequence's dead pages, into freed_offsets[s]
  for (int s = wave; s < B; s += kWaves) {
    const int32_t* bt = p.block_tables + (int64_t)s * p.bt_stride;
    const int d = dead_of(s);
    int c = 0;
    for (int j0 = 0; j0 < d; j0 += 64 * kU) {
      int32_t x[kU];
#pragma unroll
      for (int k = 0; k < kU; ++k) {
        const int j = j0 + 64 * k + lane;
        x[k] = j < d ? bt[j] : -1;
      }
#pragma unroll
      for (int k = 0; k < kU; ++k) c += x[k] >= 0;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o);
    if (lane == 0) p.freed_offsets[s] = c;
  }
  __syncthreads();
  // the counts become offsets (each thread a run of consecutive sequences)
  const int per = (B + kLT - 1) / kLT;
  const int s0 = threadIdx.x * per;
  int64_t cnt = 0;
  for (int i = 0; i < per; ++i) {
    const int s = s0 + i;
    if (s >= B) break;
    cnt += p.freed_offsets[s];
  }
  int64_t total = 0;
  int64_t off = block_exclusive_scan(cnt, &total);
  for (int i = 0; i < per; ++i) {
    const int s = s0 + i;
    if (s >= B) break;
    const int c = p.freed_offsets[s];
    p.freed_offsets[s] = (int32_t)off;
    off += c;
  }
  if (threadIdx.x == 0) p.freed_offsets[B] = (int32_t)total;
  __syncthreads();
  // the entries: reported in table order, then set to -1 (entries already
  // -1 were recycled before)
  for (int s = wave; s < B; s += kWaves) {
    int32_t* bt = p.block_tables + (int64_t)s * p.bt_stride;
    const int d = dead_of(s);
    int o = p.freed_offsets[s];
    for (int j0 = 0; j0 < d; j0 += 64 * kU) {
      int32_t x[kU];
#pragma unroll
      for (int k = 0; k < kU; ++k) {
        const int j = j0 + 64 * k + lane;
        x[k] = j < d ? bt[j] : -1;
      }
#pragma unroll
      for (int k = 0; k < kU; ++k) {
        const bool keep = x[k] >= 0;
        const uint64_t m = __ballot(keep);
        if (keep) {
          p.freed_pages[o + __popcll(m & ((1ull << lane) - 1))] = x[k];
          bt[j0 + 64 * k + lane] = -1;
        }
        o += __popcll(m);
      }
    }
  }
}

hipError_t launch_chunked_local_plan(const LocalPlanParams& p, hipStream_t stream) {
  // about kCopyUnroll table entries per thread, at most one workgroup per row
  const int64_t entries = p.num_virtual * (int64_t)(p.chunk / 16);
  int64_t groups = (entries + (int64_t)kCopyUnroll * kLT - 1) / ((int64_t)kCopyUnroll * kLT);
  groups = std::max<int64_t>(1, std::min<int64_t>({groups, (int64_t)kPlanMaxGroups, p.num_virtual}));
  hipLaunchKernelGGL(chunked_local_plan_kernel, dim3((unsigned)groups), dim3(kLT), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_recycle_pages(const RecycleParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(recycle_pages_kernel, dim3(1), dim3(kLT), 0, stream, p);
  return hipGetLastError();
}

}  // namespace vp

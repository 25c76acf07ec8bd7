// Chunked-prefill and shared-prefix attention tiles on the matrix cores
// (the tile itself: attn_tile.h): the kernels and their launchers.
#include "attn_tile.h"

namespace vp {

// PFX = false: chunked prefill, normalized output rows.  PFX = true: shared
// prefix, (max, sum, normalized output) partials per row and split.
template <int D, int QF, int KF, bool PFX>
__global__ __launch_bounds__(tile::kPW * 64) void attn_tile_kernel(PrefillParams p) {
  tile::attn_tile_body<D, QF, KF, PFX>(p, blockIdx.x);
}

// Tile order of a chunked-prefill call, one workgroup.  Workgroups are handed
// out in grid order, and the hardware deals consecutive ones to the XCDs and,
// inside an XCD, to its shader engines in a fixed rotation: a workgroup waits
// until the engine it is dealt to has room, and every later one waits behind
// it.  Tiles of very different lengths in a row therefore leave slots idle
// while work is still queued, and so do the empty tiles of short chunks.  The
// order built here removes both:
//  * sequences sorted by the key blocks of their last tile (their longest),
//    longest first, ties by index; the (sequence, kv-head) pairs of sorted
//    sequence r are v = r Hkv + h, run on XCD v % 8, all tiles of a pair
//    together (they read the same K/V, which then stays in that XCD's L2),
//    last tile first;
//  * per XCD, the tiles packed in that order with no empty ones, and every
//    entry past them marked empty (those workgroups exit at once).
// The cost of a tile is the kernel's own block count, from the same clamped
// metadata.  Sort keys are (~cost << 16 | s), so they are distinct.  Up to
// kPlanThreads sequences a key's rank is the count of smaller keys (one pass
// over LDS, no barriers); larger batches sort bitonically in LDS.  The list of
// XCD x is written by the 32 lanes of half-wave x, which carry its running
// length in registers: no barrier in that loop either.  The kernel is all
// latency, so it runs as one workgroup of 4 waves.
constexpr int kPlanThreads = 256;

__global__ __launch_bounds__(kPlanThreads) void prefill_plan_kernel(PrefillParams p) {
  __shared__ __attribute__((aligned(16))) uint32_t s_key[kPlanMaxSeqs];   // sort keys
  __shared__ uint32_t s_ord[kPlanMaxSeqs];     // rank -> key (rank sort)
  __shared__ int32_t s_nt[kPlanMaxSeqs];       // tiles of sequence s
  const int tid = threadIdx.x;
  const int B = p.num_seqs, H = p.num_kv_heads;
  const int tq = tile::kRows / p.group;
  int N = 4;
  while (N < B) N <<= 1;
  for (int s = tid; s < N; s += kPlanThreads) {
    uint32_t key = 0xFFFFFFFFu;                // padding: after every sequence
    if (s < B) {
      const int q_begin = min(max(p.query_start_loc[s], 0), p.num_tokens);
      const int Qs = min(max(p.query_start_loc[s + 1], q_begin), p.num_tokens) - q_begin;
      const int nt = min((Qs + tq - 1) / tq, p.num_tiles);
      int cost = 0;
      if (nt > 0) {
        const int q0 = (nt - 1) * tq;
        const int n = min(p.context_lens[s], p.bt_stride * 16);
        const int pos0 = n - Qs + q0;
        const int kend = pos0 + min(tq, Qs - q0);
        const int kbeg = p.window > 0 ? max(0, pos0 - p.window + 1) : 0;
        cost = kend > kbeg ? (kend - 1) / 32 - kbeg / 32 + 1 : 0;
      }
      s_nt[s] = nt;
      key = ((uint32_t)(0xFFFF - min(cost, 0xFFFF)) << 16) | (uint32_t)s;
    }
    s_key[s] = key;
  }
  __syncthreads();
  const uint32_t* ord = s_key;                 // rank -> key
  if (N <= kPlanThreads) {
    if (tid < N) {
      const uint32_t mine = s_key[tid];
      int r = 0;
      for (int i = 0; i < N; i += 4) {
        const uint4 k4 = *reinterpret_cast<const uint4*>(&s_key[i]);
        r += (k4.x < mine) + (k4.y < mine) + (k4.z < mine) + (k4.w < mine);
      }
      s_ord[r] = mine;                         // (padding keys share a rank >= B)
    }
    ord = s_ord;
  } else {
    for (int k = 2; k <= N; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < N; i += kPlanThreads) {
          const int l = i ^ j;
          if (l > i) {
            const uint32_t a = s_key[i], c = s_key[l];
            if ((a > c) == ((i & k) == 0)) {   // ascending where (i & k) == 0
              s_key[i] = c;
              s_key[l] = a;
            }
          }
        }
        __syncthreads();
      }
    }
  }
  __syncthreads();
  // Pairs in chunks of kPlanThreads: lane k of half-wave x takes
  // v = base + 8 k + x (on XCD x); its place in list x is the list's length
  // so far plus the tiles of the half-wave's earlier lanes.
  const int x = tid >> 5, k = tid & 31;
  int2* list = p.plan + (int64_t)x * p.plan_stride;
  int run = 0;
  const int64_t npairs = (int64_t)B * H;
  for (int64_t base = 0; base < npairs; base += kPlanThreads) {
    const int64_t v = base + 8 * k + x;
    int u = 0, cnt = 0;
    if (v < npairs) {
      const int r = (int)(v / H);
      const int h = (int)(v - (int64_t)r * H);
      const int s = (int)(ord[r] & 0xFFFFu);
      u = s * H + h;
      cnt = s_nt[s];
    }
    int inc = cnt;
#pragma unroll
    for (int d = 1; d < 32; d <<= 1) {
      const int y = __shfl_up(inc, d, 32);
      if (k >= d) inc += y;
    }
    const int pos = run + inc - cnt;
    for (int i = 0; i < cnt; ++i) list[pos + i] = make_int2(u, cnt - 1 - i);
    run += __shfl(inc, 31, 32);
  }
  for (int i = run + k; i < p.plan_stride; i += 32) list[i] = make_int2(-1, 0);
}

template <int QF, int KF, bool PFX>
static hipError_t launch_tiles(const PrefillParams& x, int head_dim, int64_t grid, hipStream_t stream) {
  if (head_dim == 128)
    hipLaunchKernelGGL((attn_tile_kernel<128, QF, KF, PFX>), dim3((unsigned)grid), dim3(tile::kPW * 64), 0,
                       stream, x);
  else if (head_dim == 64)
    hipLaunchKernelGGL((attn_tile_kernel<64, QF, KF, PFX>), dim3((unsigned)grid), dim3(tile::kPW * 64), 0,
                       stream, x);
  else
    return hipErrorNotSupported;
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillParams& p, int head_dim, int kv_fmt, int q_fmt,
                          hipStream_t stream) {
  if (head_dim != 128 && head_dim != 64) return hipErrorNotSupported;
  const int tq = tile::kRows / p.group;
  if (tq < 1) return hipErrorNotSupported;
  PrefillParams x = p;
  x.num_tiles = (p.max_query_len + tq - 1) / tq;
  const int64_t pairs = (int64_t)p.num_seqs * p.num_kv_heads;
  const int64_t grid = (pairs + 7) / 8 * 8 * x.num_tiles;
  if (grid == 0) return hipSuccess;
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  if (x.plan) {
    if (p.num_seqs > kPlanMaxSeqs || grid < kPlanMinGrid || grid > kPlanMaxGrid) return hipErrorInvalidValue;
    x.plan_stride = (int32_t)(grid / 8);
    hipLaunchKernelGGL(prefill_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, x);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (kv_fmt == kE4M3)
    return q_fmt == kBF16 ? launch_tiles<kBF16, kE4M3, false>(x, head_dim, grid, stream)
                          : launch_tiles<kF16, kE4M3, false>(x, head_dim, grid, stream);
  if (kv_fmt == kE5M2)
    return q_fmt == kBF16 ? launch_tiles<kBF16, kE5M2, false>(x, head_dim, grid, stream)
                          : launch_tiles<kF16, kE5M2, false>(x, head_dim, grid, stream);
  if (kv_fmt != q_fmt) return hipErrorNotSupported;
  return q_fmt == kBF16 ? launch_tiles<kBF16, kBF16, false>(x, head_dim, grid, stream)
                        : launch_tiles<kF16, kF16, false>(x, head_dim, grid, stream);
}

}  // namespace vp

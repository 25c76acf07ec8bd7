// Paged attention decode for gfx950: one query token per sequence attends to
// its K/V, read page by page through the sequence's block table (paged
// attention over the block-paged KV cache of the vllm.cpp model forward,
// repository listing "What's implemented"; 16-token FP16/FP8 pages and block
// tables bound to shared physical pages, "Building and Deploying vllm.cpp",
// Step 3).  The pages give no kernel design; this one is built for CDNA4.
//
// Work split (equal work per wave).  A work unit is (sequence, kv-head,
// up to 8 query heads of its group); unit u holds the np(s) pages of its
// sequence's kept range.  All pages of all units are laid end to end in
// (sequence, unit, page) order, T pages in total, and cut into chunks of C
// pages; each wave takes one chunk (C = ceil(T / waves)), so every wave
// streams the same number of pages whatever the context lengths are.  A
// chunk covers the tail of one unit, whole units, and the head of another;
// a unit finished inside one chunk writes its output directly; each piece
// of a unit cut by chunk boundaries writes a (max, sum, normalized output)
// triple to the workspace, and decode_merge_kernel (launched right after)
// merges them with the log-sum-exp rule.  The per-sequence page prefix is
// computed by every workgroup with a block-wide scan.
//
// Inside a wave the products run on the matrix cores (v_mfma_f32_16x16x32,
// f16 or bf16 by q's format, fp32 accumulate).  Lane l is (n, kg) =
// (l % 16, l / 16); the MFMA's operands are A[i][k] at lane (i, k / 8),
// B[k][c] at lane (c, k / 8) and C[i][c] at lane (c, i / 4).  The query heads
// of a unit (up to 16) are the MFMA columns; columns past the unit's G have
// q = 0 and are never stored.  Pages go in pairs of 32 keys:
//  * S^T = K Q^T per page in D / 32 k-steps: lane (n, kg) loads 16-byte
//    pieces of K row n (load i covers bytes 64 i + 16 kg .. of the row, so
//    every load instruction reads 64 contiguous bytes of each of 16 rows);
//    FP8 codes are converted exactly to q's format.  Q^T, the B operand,
//    takes the same element order.  Lane (n, kg) then holds the scores of
//    head n for keys 4 kg + r of the page (r < 4).
//  * Online softmax in fp32, log2 domain, with a running max per head that
//    only moves when a score exceeds it by more than 2^8 (one wave vote per
//    page pair; the head's maximum is reduced over its four lanes).  Keys
//    outside [max(0, n - window), n) get score -inf and their V rows are
//    replaced by zeros: NaN garbage in unused rows never reaches a product.
//  * The probabilities are rounded to q's 16-bit format (the row sums use the
//    rounded values).  Keys 4 kg + r of page A then of page B are exactly the
//    A operand (head n, 8 keys) of O = P V, so the probabilities stay in
//    place.
//  * V: lane (n, kg) loads, for those 8 keys, the D / 16 elements
//    (D / 16) n .. of each row (16 lanes cover a row, 4 rows per load
//    instruction).  The B operand of output tile mt is element mt of the 8
//    rows, paired by byte or half-word permutes (and converted exactly from
//    FP8), so the accumulator of tile mt holds O[head 4 kg + r][(D/16) n + mt]
//    and a lane finally stores D / 16 consecutive outputs of each of its heads.
//  * PP page pairs of K and V are in flight per wave (2 for FP8 pages, 1 for
//    16-bit: 16 KiB at D = 128).  The next pair's K is loaded as soon as
//    S^T has consumed the registers and its V as soon as O has; past the end
//    of the stretch the loads read a spare page of the workspace (kept hot in
//    L2), so no buffer goes through a control-flow merge.
#include <atomic>
#include <cstdlib>
#include <type_traits>
#include <utility>

#include "attn_tile.h"
#include "common.h"
#include "kernels.h"

namespace vp {

constexpr int kNW = kDecodeWaves;
constexpr float kTau = 8.0f;       // rescale headroom, log2 units
constexpr int kScanMax = 2048;     // sequences whose page prefix fits in LDS

// Streaming (non-temporal) loads: every KV byte is read once per call.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
template <typename T>
__device__ __forceinline__ T ld_stream(const uint8_t* ptr);
template <>
__device__ __forceinline__ uint4 ld_stream<uint4>(const uint8_t* ptr) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(ptr));
  return make_uint4(v.x, v.y, v.z, v.w);
}
template <>
__device__ __forceinline__ uint2 ld_stream<uint2>(const uint8_t* ptr) {
  const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(ptr));
  return make_uint2(v.x, v.y);
}

// Two 16-bit values (low, high) of q's format from two floats, round to
// nearest even (hardware conversions of gfx950).
template <int QF>
__device__ __forceinline__ uint32_t pack16(float lo, float hi) {
  if constexpr (QF == kBF16) {
    bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return bitcast<uint32_t>(v);
  } else {
    half2_t v = {(_Float16)lo, (_Float16)hi};
    return bitcast<uint32_t>(v);
  }
}

template <int QF>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  if constexpr (QF == kF16)
    return __builtin_amdgcn_fdot2(bitcast<half2_t>(a), bitcast<half2_t>(b), c, false);
  else
    return __builtin_amdgcn_fdot2_f32_bf16(bitcast<bf16x2_t>(a), bitcast<bf16x2_t>(b), c, false);
}

// Kept key range of a decode query and its page range.
struct SeqRange {
  int n, lo, lo_page, np;   // np = pages of the kept range (0 if n <= 0)
};

// (ctx: the sequence's context length as stored in context_lens)
__device__ __forceinline__ SeqRange seq_range_of(const DecodeParams& p, int ctx) {
  SeqRange r;
  r.n = min(ctx, p.bt_stride * 16);
  if (r.n <= 0) {
    r.n = 0; r.lo = 0; r.lo_page = 0; r.np = 0;
    return r;
  }
  r.lo = p.window > 0 ? max(0, r.n - p.window) : 0;
  r.lo = max(r.lo, p.skip_tokens);             // shared prefix: decoded by its own pass
  if (r.lo >= r.n) {
    r.lo = 0; r.lo_page = 0; r.np = 0;
    return r;
  }
  r.lo_page = r.lo >> 4;
  r.np = ((r.n + 15) >> 4) - r.lo_page;
  return r;
}

// Exclusive prefix of np(s) over the batch, computed by one workgroup of
// kNW * 64 threads into pre[0 .. B] (pre[B] = total): each thread sums a
// run of sequences, the runs are scanned within each wave with lane
// shuffles, then across the kNW wave totals.
// ctx (null: not kept): also receives each sequence's context length, so
// that the waves take it from LDS instead of reading it again.
__device__ void page_prefix(const DecodeParams& p, int* pre, int* ctx = nullptr) {
  __shared__ int s_wave[kNW];
  __shared__ int s_total;
  const int B = p.num_seqs;
  const int nt = kNW * 64;
  const int per = (B + nt - 1) / nt;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  int sum = 0;
  for (int i = 0; i < per; ++i) {
    const int s = t * per + i;
    if (s < B) {
      const int c = p.context_lens[s];
      if (ctx) ctx[s] = c;
      sum += seq_range_of(p, c).np;
    }
  }
  int incl = sum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int u = __shfl_up(incl, off);
    if (lane >= off) incl += u;
  }
  if (lane == 63) s_wave[w] = incl;
  __syncthreads();
  if (t == 0) {
    int run = 0;
    for (int i = 0; i < kNW; ++i) {
      const int x = s_wave[i];
      s_wave[i] = run;
      run += x;
    }
    s_total = run;
  }
  __syncthreads();
  int run = s_wave[w] + incl - sum;
  for (int i = 0; i < per; ++i) {
    const int s = t * per + i;
    if (s < B) {
      pre[s] = run;
      run += seq_range_of(p, ctx ? ctx[s] : p.context_lens[s]).np;
    }
  }
  if (t == 0) pre[B] = s_total;
  __syncthreads();
}

// Fused cache write: the new token of sequence s, kv-head hk, written to its
// slot exactly as the cache-write kernel writes it (bit copy for 16-bit
// pools; for FP8 pools one correctly rounded fp32 division by the scale, then
// the saturating nearest-even encoder).  Lanes 0..D/8-1 write K chunks, the
// next D/8 lanes V chunks.  The stores complete before the wave goes on, so
// its own reads of that page see them.
template <int D, int KF, int QF>
__device__ __forceinline__ void append_row(const DecodeParams& p, int s, int hk, int lane) {
  constexpr int CH = D / 8;
  // (an opaque copy of the lane index: nothing lane-dependent of this write
  // is hoisted out of the segment loop, where it would hold registers
  // through the whole page stream)
  asm volatile("" : "+v"(lane));
  const int64_t slot = p.new_slots[s];
  if (slot >= 0 && slot < p.num_slots && lane < 2 * CH) {
    const bool is_v = lane >= CH;
    const int c = is_v ? lane - CH : lane;
    const int64_t src = ((int64_t)s * p.num_kv_heads + hk) * D + c * 8;
    const int64_t dst = (((slot >> 4) * p.num_kv_heads + hk) * 16 + (slot & 15)) * D + c * 8;
    const uint4 x = *reinterpret_cast<const uint4*>(
        static_cast<const uint16_t*>(is_v ? p.v_new : p.k_new) + src);
    void* pool = is_v ? const_cast<void*>(p.v_cache) : const_cast<void*>(p.k_cache);
    if constexpr (!is_fp8(KF)) {
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(pool) + dst) = x;
    } else {
      const float sc = is_v ? (p.v_scales ? p.v_scales[hk] : p.v_scale)
                            : (p.k_scales ? p.k_scales[hk] : p.k_scale);
      const uint32_t w[4] = {x.x, x.y, x.z, x.w};
      uint32_t o[2] = {0, 0};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float a, b;
        x2_to_f32<QF>(w[i], a, b);
        const uint32_t ca = fp8_from_f32<KF>(a / sc), cb = fp8_from_f32<KF>(b / sc);
        o[i >> 1] |= (ca | (cb << 8)) << ((i & 1) * 16);
      }
      *reinterpret_cast<uint2*>(static_cast<uint8_t*>(pool) + dst) = make_uint2(o[0], o[1]);
    }
  }
  // the stores are done before any lane of the wave reads the page back:
  // release for the writing lanes, acquire for the reading ones
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
}

// ---- the decode kernel (matrix cores; see the top of this file) -------------
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

template <int QF>
__device__ __forceinline__ f32x4_t mfma16(uint4 a, uint4 b, f32x4_t c) {
  if constexpr (QF == kBF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8_t>(a), bitcast<bf16x8_t>(b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(bitcast<f16x8_t>(a), bitcast<f16x8_t>(b), c, 0, 0, 0);
}

template <int D, int KF>
struct MmaShape {
  static constexpr int EB = is_fp8(KF) ? 1 : 2;     // bytes per pool element
  static constexpr int RB = D * EB;                  // bytes per K / V row
  static constexpr int STEPS = D / 32;               // k-steps of S^T per page
  static constexpr int NL = RB / 64;                 // 16-byte K loads per lane per page
  static constexpr int TILES = D / 16;               // output tiles of 16 d
  static constexpr int VW = TILES * EB / 4;          // 32-bit words of V per lane per row
};

template <int NW> struct Words { uint32_t w[NW]; };

template <int NW>
__device__ __forceinline__ Words<NW> ld_words(const uint8_t* ptr) {
  Words<NW> r;
  if constexpr (NW == 4) {
    const uint4 x = ld_stream<uint4>(ptr);
    r.w[0] = x.x; r.w[1] = x.y; r.w[2] = x.z; r.w[3] = x.w;
  } else if constexpr (NW == 2) {
    const uint2 x = ld_stream<uint2>(ptr);
    r.w[0] = x.x; r.w[1] = x.y;
  } else {
    r.w[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(ptr));
  }
  return r;
}

// bid, nbid: this workgroup's index among the decode workgroups and their
// number (the whole grid, or its part after the shared-prefix tiles).
template <int D, int KF, int QF, int PP, bool AP>
__device__ __forceinline__ void decode_body(const DecodeParams& p, const int bid, const int nbid) {
  using S = MmaShape<D, KF>;
  constexpr int EB = S::EB, RB = S::RB, STEPS = S::STEPS, NL = S::NL, TILES = S::TILES, VW = S::VW;
  constexpr int64_t kPageBytes = 16 * RB;

  __shared__ int s_pre[kScanMax + 1];
  __shared__ int s_ctx[kScanMax];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int B = p.num_seqs;
  const int G = p.head_chunk;
  const int ngc = p.group / G;
  const int NY = p.num_kv_heads * ngc;                 // units per sequence

  const int* pre;
  if (B <= kScanMax) {
    page_prefix(p, s_pre, s_ctx);
    pre = s_pre;
  } else {
    pre = p.ws_prefix;
  }
  const int64_t T = (int64_t)NY * __builtin_amdgcn_readfirstlane(pre[B]);
  const int64_t C = p.chunk_pages > 0 ? p.chunk_pages
                                      : max((int64_t)1, (T + p.num_workers - 1) / p.num_workers);
  const int64_t num_chunks = (T + C - 1) / C;

  for (int sq = bid; sq < B; sq += nbid) {
    if (pre[sq + 1] == pre[sq]) {
      if (p.skip_tokens == 0) {
        uint16_t* o = static_cast<uint16_t*>(p.out) + (int64_t)sq * p.num_q_heads * D;
        for (int i = threadIdx.x; i < p.num_q_heads * D; i += kNW * 64) o[i] = 0;
      }
      for (int i = threadIdx.x; i < NY; i += kNW * 64) p.ws_unit[((int64_t)sq * NY + i) * 2 + 1] = 0;
    }
  }

  const int64_t blk_stride = (int64_t)p.num_kv_heads * kPageBytes;
  constexpr uint32_t kOnes = QF == kBF16 ? 0x3F803F80u : 0x3C003C00u;   // (1, 1)

  for (int64_t chunk = (int64_t)bid * kNW + wave; chunk < num_chunks;
       chunk += p.num_workers) {
    int64_t g = chunk * C;
    const int64_t g_end = min(g + C, T);
    int s = 0;
    {
      int lo_s = 0, hi_s = B - 1;
      while (lo_s < hi_s) {
        const int mid = (lo_s + hi_s + 1) >> 1;
        if ((int64_t)NY * __builtin_amdgcn_readfirstlane(pre[mid]) <= g) lo_s = mid; else hi_s = mid - 1;
      }
      s = lo_s;
    }
    bool first_seg = true;
    while (g < g_end) {
      while ((int64_t)NY * __builtin_amdgcn_readfirstlane(pre[s + 1]) <= g) ++s;
      const SeqRange sr = seq_range_of(
          p, B <= kScanMax ? __builtin_amdgcn_readfirstlane(s_ctx[s]) : p.context_lens[s]);
      const int64_t off = g - (int64_t)NY * __builtin_amdgcn_readfirstlane(pre[s]);
      const int y = (int)(off / sr.np);
      const int i0 = (int)(off - (int64_t)y * sr.np);
      const int i1 = (int)min((int64_t)sr.np, i0 + (g_end - g));
      const int slot = first_seg ? 0 : 1;
      const bool whole = (i0 == 0) && (i1 == sr.np);
      const bool complete = whole && p.skip_tokens == 0;
      const int hk = y / ngc;
      const int h0 = hk * p.group + (y - hk * ngc) * G;
      const float sscale = p.k_scales ? p.score_base * p.k_scales[hk] : p.score_scale;
      const float oscale = p.v_scales ? p.v_scales[hk] : p.out_scale;
      // (the lane roles as opaque values: nothing lane-dependent is hoisted
      // out of the segment loop to hold registers through the page stream)
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int n = ln & 15, kg = ln >> 4;
      const int k_lane = n * RB + 16 * kg;               // this lane's K bytes in a page (+ 64 i)
      const int v_lane = n * (TILES * EB);               // this lane's V bytes in a row
      const bool head_ok = n < G;

      if constexpr (AP) {
        if (i1 == sr.np) append_row<D, KF, QF>(p, s, hk, lane);
      }
      // Q^T operand: head n, the k-step's 8 elements in the K loads' order
      uint4 qv[STEPS];
      {
        const uint16_t* qp =
            static_cast<const uint16_t*>(p.q) + ((int64_t)s * p.num_q_heads + h0 + min(n, G - 1)) * D;
#pragma unroll
        for (int t = 0; t < STEPS; ++t) {
          const int e = is_fp8(KF) ? 64 * (t / 2) + 16 * kg + 8 * (t % 2) : 32 * t + 8 * kg;
          const uint4 x = *reinterpret_cast<const uint4*>(qp + e);
          qv[t] = head_ok ? x : make_uint4(0, 0, 0, 0);
        }
      }
      const int32_t* bt = p.block_tables + (int64_t)s * p.bt_stride + sr.lo_page;
      const uint8_t* kbase = static_cast<const uint8_t*>(p.k_cache) + (int64_t)hk * kPageBytes;
      const uint8_t* vbase = static_cast<const uint8_t*>(p.v_cache) + (int64_t)hk * kPageBytes;
      const uint8_t* spare = static_cast<const uint8_t*>(p.ws_spare);
      const int count = i1 - i0;
      const int npairs = (count + 1) >> 1;
      int bt_base = 0;
      auto bt_fetch = [&](int base) __attribute__((always_inline)) {
        const int q = i0 + base + lane;
        int b = q < i1 ? bt[q] : 0;
        return (unsigned)b < (unsigned)p.num_blocks ? b : 0;
      };
      int bt_cur = bt_fetch(0), bt_nxt = count > 64 ? bt_fetch(64) : 0;
      auto blk_of = [&](int jj) __attribute__((always_inline)) {
        if (jj >= bt_base + 64) {
          bt_base += 64;
          bt_cur = bt_nxt;
          if (bt_base + 64 < count) bt_nxt = bt_fetch(bt_base + 64);
        }
        return __builtin_amdgcn_readlane(bt_cur, jj - bt_base);
      };
      // page of pair jp, half h (0: A, 1: B); past the segment: the spare page
      auto page_ptr = [&](const uint8_t* base, int jp, int h) __attribute__((always_inline)) {
        const int jj = 2 * jp + h;
        return jj < count ? base + blk_of(min(jj, count - 1)) * blk_stride : spare;
      };
      auto load_k = [&](int jp, uint4 (&kd)[2][NL]) __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint8_t* pg = page_ptr(kbase, jp, h) + k_lane;
#pragma unroll
          for (int i = 0; i < NL; ++i) kd[h][i] = ld_stream<uint4>(pg + 64 * i);
        }
      };
      auto load_v = [&](int jp, Words<VW> (&vd)[8]) __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint8_t* pg = page_ptr(vbase, jp, h) + v_lane;
#pragma unroll
          for (int r = 0; r < 4; ++r) vd[4 * h + r] = ld_words<VW>(pg + (4 * kg + r) * RB);
        }
      };

      float m = -INFINITY, l = 0.0f;
      f32x4_t o[TILES];
#pragma unroll
      for (int t = 0; t < TILES; ++t) o[t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

      uint4 kd[PP][2][NL];
      Words<VW> vd[PP][8];
#pragma unroll
      for (int u = 0; u < PP; ++u) {
        load_k(u, kd[u]);
        load_v(u, vd[u]);
      }
      for (int jb = 0; jb < npairs; jb += PP) {
#pragma unroll
        for (int u = 0; u < PP; ++u) {
          const int jp = jb + u;
          const bool valid = jp < npairs;
          const int t0 = (sr.lo_page + i0 + 2 * min(jp, npairs - 1)) * 16;   // first key of page A
          const bool has_b = 2 * jp + 1 < count;
          const bool full = has_b && (t0 >= sr.lo) && (t0 + 32 <= sr.n);
          float sc[8];
          if (valid) {
            // ---- S^T = K Q^T, page A then page B ----
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              f32x4_t acc = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
              for (int t = 0; t < STEPS; ++t) {
                uint4 ka;
                if constexpr (!is_fp8(KF)) {
                  ka = kd[u][h][t];
                } else {
                  const uint4 x = kd[u][h][t / 2];
                  const uint32_t lo = (t % 2) ? x.z : x.x, hi = (t % 2) ? x.w : x.y;
                  ka = make_uint4(fp8x2_to_q16<KF, QF, false>(lo), fp8x2_to_q16<KF, QF, true>(lo),
                                  fp8x2_to_q16<KF, QF, false>(hi), fp8x2_to_q16<KF, QF, true>(hi));
                }
                acc = mfma16<QF>(ka, qv[t], acc);
              }
#pragma unroll
              for (int r = 0; r < 4; ++r) sc[4 * h + r] = acc[r] * sscale;
            }
          }
          __builtin_amdgcn_sched_barrier(0);
          load_k(jp + PP, kd[u]);
          __builtin_amdgcn_sched_barrier(0);
          if (valid) {
            // keys outside [lo, n) and page B past the segment: -inf.  (Heads
            // past G have q = 0, so finite scores; they only reach output rows
            // that are never stored.)
            if (!full) {
#pragma unroll
              for (int j = 0; j < 8; ++j) {
                const int t = t0 + 16 * (j >> 2) + 4 * kg + (j & 3);
                const bool keep = t >= sr.lo && t < sr.n && (j < 4 || has_b);
                if (!keep) sc[j] = -INFINITY;
              }
            }
            // ---- online softmax (head n; its four lanes agree on m) ----
            bool need = false;
#pragma unroll
            for (int j = 0; j < 8; ++j) need |= sc[j] > m + kTau;
            if (__any(need)) {
              float pm = sc[0];
#pragma unroll
              for (int j = 1; j < 8; ++j) pm = fmaxf(pm, sc[j]);
              pm = fmaxf(pm, __shfl_xor(pm, 16));
              pm = fmaxf(pm, __shfl_xor(pm, 32));
              const float mn = fmaxf(m, pm);
              const float alpha = (m == -INFINITY) ? 0.0f : fast_exp2(m - mn);
              m = mn;
              l *= alpha;
              // accumulator rows are heads 4 kg + r: their factors from lanes 4 kg + r
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const float ar = __shfl(alpha, 4 * kg + r);
#pragma unroll
                for (int t = 0; t < TILES; ++t) o[t][r] *= ar;
              }
            }
            const float mu = (m == -INFINITY) ? 0.0f : m;
            uint32_t pw[4];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              pw[w] = pack16<QF>(fast_exp2(sc[2 * w] - mu), fast_exp2(sc[2 * w + 1] - mu));
              l = dot2<QF>(pw[w], kOnes, l);              // row sum of the rounded weights
            }
            const uint4 pa = make_uint4(pw[0], pw[1], pw[2], pw[3]);
            // ---- O += P V ----
            Words<VW> vv[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              vv[j] = vd[u][j];
              if (!full) {
                const int t = t0 + 16 * (j >> 2) + 4 * kg + (j & 3);
                const bool keep = t >= sr.lo && t < sr.n && (j < 4 || has_b);
#pragma unroll
                for (int w = 0; w < VW; ++w) vv[j].w[w] = keep ? vv[j].w[w] : 0u;
              }
            }
            if constexpr (!is_fp8(KF)) {
#pragma unroll
              for (int t = 0; t < TILES; ++t) {
                const uint32_t sel = (t & 1) ? 0x07060302u : 0x05040100u;
                uint32_t b[4];
#pragma unroll
                for (int w = 0; w < 4; ++w)
                  b[w] = __builtin_amdgcn_perm(vv[2 * w + 1].w[t >> 1], vv[2 * w].w[t >> 1], sel);
                o[t] = mfma16<QF>(pa, make_uint4(b[0], b[1], b[2], b[3]), o[t]);
              }
            } else {
#pragma unroll
              for (int t = 0; t < TILES; t += 2) {
                const int q = t & 3;                      // byte of the word (0 or 2)
                const uint32_t sel = (uint32_t)q | ((uint32_t)(4 + q) << 8) |
                                     ((uint32_t)(q + 1) << 16) | ((uint32_t)(5 + q) << 24);
                uint32_t b0[4], b1[4];
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                  const uint32_t x =
                      __builtin_amdgcn_perm(vv[2 * w + 1].w[t >> 2], vv[2 * w].w[t >> 2], sel);
                  b0[w] = fp8x2_to_q16<KF, QF, false>(x);
                  b1[w] = fp8x2_to_q16<KF, QF, true>(x);
                }
                o[t] = mfma16<QF>(pa, make_uint4(b0[0], b0[1], b0[2], b0[3]), o[t]);
                o[t + 1] = mfma16<QF>(pa, make_uint4(b1[0], b1[1], b1[2], b1[3]), o[t + 1]);
              }
            }
          }
          __builtin_amdgcn_sched_barrier(0);
          load_v(jp + PP, vd[u]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }

      // Sums of head n over its four lanes; accumulator rows 4 kg + r take
      // theirs (and m) from lanes 4 kg + r.
      float lt = l + __shfl_xor(l, 16);
      lt += __shfl_xor(lt, 32);
      if (complete) {
        const float inv = oscale / lt;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float ir = __shfl(inv, 4 * kg + r);
          const int h = 4 * kg + r;
          if (h < G) {
            uint32_t w[TILES / 2];
#pragma unroll
            for (int t = 0; t < TILES / 2; ++t)
              w[t] = (uint32_t)f32_to_16<QF>(o[2 * t][r] * ir) |
                     ((uint32_t)f32_to_16<QF>(o[2 * t + 1][r] * ir) << 16);
            uint16_t* op = static_cast<uint16_t*>(p.out) +
                           ((int64_t)s * p.num_q_heads + h0 + h) * D + n * TILES;
            if constexpr (TILES == 8)
              *reinterpret_cast<uint4*>(op) = make_uint4(w[0], w[1], w[2], w[3]);
            else
              *reinterpret_cast<uint2*>(op) = make_uint2(w[0], w[1]);
          }
        }
      } else {
        const int64_t unit = (int64_t)s * NY + y;
        const int64_t sl = chunk * 2 + slot;
        float* wo = whole ? p.ws_uo + unit * G * D : p.ws_o + sl * G * D;
        float* wm = whole ? p.ws_um + unit * G : p.ws_m + sl * G;
        float* wl = whole ? p.ws_ul + unit * G : p.ws_l + sl * G;
        const float inv = 1.0f / lt;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float ir = __shfl(inv, 4 * kg + r);
          const int h = 4 * kg + r;
          if (h < G) {
            float* op = wo + h * D + n * TILES;
#pragma unroll
            for (int t = 0; t < TILES; t += 4)
              *reinterpret_cast<float4*>(op + t) =
                  make_float4(o[t][r] * ir, o[t + 1][r] * ir, o[t + 2][r] * ir, o[t + 3][r] * ir);
          }
        }
        if (kg == 0 && head_ok) {
          wm[n] = m;
          wl[n] = lt;
        }
      }
      if (i0 == 0 && lane == 0) {
        int npieces = 0;
        if (!complete) {
          const int64_t base = g;
          npieces = (int)((base + sr.np - 1) / C - base / C + 1);
        }
        p.ws_unit[((int64_t)s * NY + y) * 2] = whole ? -1 : (int32_t)(chunk * 2 + slot);
        p.ws_unit[((int64_t)s * NY + y) * 2 + 1] = npieces;
      }
      g += i1 - i0;
      first_seg = false;
    }
  }
}

template <int D, int KF, int QF, int PP, bool AP>
__global__ __launch_bounds__(kNW * 64) void decode_mma_kernel(DecodeParams p) {
  decode_body<D, KF, QF, PP, AP>(p, blockIdx.x, gridDim.x);
}

// Decode with a shared prefix, in one grid: the decode of the sequences' own
// pages first, then the npfx shared-prefix tiles, which fill the slot each CU
// has left beside its two decode workgroups (dispatched in this order, the
// decode waves have the memory system first: tiles first made the call
// about 7% slower).  Both write partials that the merge kernel, launched next
// on the same stream, combines.  (Three waves per SIMD: the two decode
// workgroups and the tile share each CU, so the kernel keeps to 168 VGPRs.)
static_assert(kNW == tile::kPW, "decode and tile workgroups have the same size");
template <int D, int KF, int QF, int PP>
__global__ __launch_bounds__(kNW * 64) __attribute__((amdgpu_waves_per_eu(3)))
void decode_shared_kernel(DecodeParams p, PrefillParams sp, int npfx) {
  const int ndec = (int)gridDim.x - npfx;
  if ((int)blockIdx.x < ndec)
    decode_body<D, KF, QF, PP, false>(p, blockIdx.x, ndec);
  else
    tile::attn_tile_body<D, QF, KF, true>(sp, blockIdx.x - ndec);
}

// Log-sum-exp merge of the pieces of units cut by chunk boundaries (and, with
// a shared prefix, of every unit with its prefix splits).  One workgroup per
// unit, one thread per 4 consecutive outputs of its G x D block; the unit's
// record (first slot, piece count) comes from the decode kernel.  Pieces are
// read in rounds of kMergeBatch (units of more decode pieces: twice that)
// straight into registers, every load of a round independent (padding pieces
// past the count re-read the last piece and get weight 0), so a round costs
// one memory latency; the prefix splits, whose rows need nothing from the
// record, go first, so their loads overlap the record's:
// M = max m, w = l 2^(m - M), out = sum w o / sum w.
constexpr int kMergeBatch = 8;

template <int D, int G, int QF>
__global__ __launch_bounds__(G * D / 4) void decode_merge_kernel(DecodeParams p) {
  const int64_t u = blockIdx.x;
  const int ns = p.num_splits;
  const int ngc = p.group / G;
  const int NY = p.num_kv_heads * ngc;
  const int s = (int)(u / NY);
  const int y = (int)(u - (int64_t)s * NY);
  const int hk = y / ngc;
  const int h0 = hk * p.group + (y - hk * ngc) * G;
  const int64_t prow = (int64_t)s * p.num_q_heads + h0;    // row of head h0 in the prefix partials
  const int64_t split_rows = (int64_t)p.num_seqs * p.num_q_heads;
  const int e = threadIdx.x * 4;
  const int h = e / D;
  float M = -INFINITY, den = 0.0f;
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  // One round: NB pieces (rows given by row_of(k), k < n; padding re-reads
  // piece n - 1 with weight 0), all loads independent.
  auto round = [&](auto nb, int k0, int n, auto row_of) __attribute__((always_inline)) {
    constexpr int NB = decltype(nb)::value;
    float mk[NB], lk[NB];
    float4 ok[NB];
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const float *op, *mp, *lp;
      const int64_t r = row_of(min(k0 + k, n - 1), op, mp, lp) + h;
      mk[k] = mp[r];
      lk[k] = lp[r];
      ok[k] = *reinterpret_cast<const float4*>(op + r * D + (e - h * D));
    }
    float Mn = M;
#pragma unroll
    for (int k = 0; k < NB; ++k)
      if (k0 + k < n) Mn = fmaxf(Mn, mk[k]);
    const float a = (M == -INFINITY) ? 0.0f : fast_exp2(M - Mn);
    den *= a;
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] *= a;
    M = Mn;
    const float Mu = (M == -INFINITY) ? 0.0f : M;   // (every piece so far empty)
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const float w = (k0 + k < n) ? lk[k] * fast_exp2(mk[k] - Mu) : 0.0f;  // 0: padding, empty
      den += w;
      acc[0] = fmaf(w, ok[k].x, acc[0]);
      acc[1] = fmaf(w, ok[k].y, acc[1]);
      acc[2] = fmaf(w, ok[k].z, acc[2]);
      acc[3] = fmaf(w, ok[k].w, acc[3]);
    }
  };
  // The shared-prefix splits first: their rows need nothing from the decode
  // kernel's record of the unit, so their loads overlap the record's.
  auto split_row = [&](int k, const float*& op, const float*& mp, const float*& lp)
      __attribute__((always_inline)) {
    op = p.pfx_o;
    mp = p.pfx_m;
    lp = p.pfx_l;
    return (int64_t)k * split_rows + prow;
  };
  for (int k0 = 0; k0 < ns; k0 += kMergeBatch) round(std::integral_constant<int, kMergeBatch>{}, k0, ns, split_row);
  const int nsuf = p.ws_unit[u * 2 + 1];
  if (nsuf == 0 && ns == 0) return;           // finished inside one chunk, or empty
  if (nsuf > 0) {
    const int64_t sl0 = p.ws_unit[u * 2];
    const int64_t fk = sl0 >> 1;
    // piece k of the decode: the first in the slot its wave recorded (or the
    // unit's own slot when that is -1), the later ones open the following
    // chunks, slot 0 of each
    auto piece_row = [&](int k, const float*& op, const float*& mp, const float*& lp)
        __attribute__((always_inline)) {
      if (sl0 < 0) {
        op = p.ws_uo;
        mp = p.ws_um;
        lp = p.ws_ul;
        return u * G;
      }
      op = p.ws_o;
      mp = p.ws_m;
      lp = p.ws_l;
      return (k == 0 ? sl0 : (fk + k) * 2) * G;
    };
    // (nsuf is uniform over the workgroup)
    if (nsuf <= kMergeBatch) round(std::integral_constant<int, kMergeBatch>{}, 0, nsuf, piece_row);
    else
      for (int k0 = 0; k0 < nsuf; k0 += 2 * kMergeBatch)
        round(std::integral_constant<int, 2 * kMergeBatch>{}, k0, nsuf, piece_row);
  }
  const float oscale = p.v_scales ? p.v_scales[hk] : p.out_scale;
  const float f = den > 0.0f ? oscale / den : 0.0f;
  uint16_t* out = static_cast<uint16_t*>(p.out) + prow * D + e;
  const uint32_t lo = (uint32_t)f32_to_16<QF>(acc[0] * f) | ((uint32_t)f32_to_16<QF>(acc[1] * f) << 16);
  const uint32_t hi = (uint32_t)f32_to_16<QF>(acc[2] * f) | ((uint32_t)f32_to_16<QF>(acc[3] * f) << 16);
  *reinterpret_cast<uint2*>(out) = make_uint2(lo, hi);
}

// Page prefix for batches too large for the LDS scan of decode_mma_kernel.
__global__ __launch_bounds__(kNW * 64) void decode_prefix_kernel(DecodeParams p) {
  page_prefix(p, p.ws_prefix);
}

// Decode kernels: 2 page pairs in flight for FP8 pages, 1 for 16-bit.
template <int D, int KF, int QF>
static const void* mma_ptr(bool ap) {
  constexpr int PP = is_fp8(KF) ? 2 : 1;
  return ap ? reinterpret_cast<const void*>(&decode_mma_kernel<D, KF, QF, PP, true>)
            : reinterpret_cast<const void*>(&decode_mma_kernel<D, KF, QF, PP, false>);
}

static const void* decode_mma_kernel_for(int D, int kv_fmt, int q_fmt, bool ap) {
#define VP_MMA(DD)                                                                    \
  if (kv_fmt == kF16 && q_fmt == kF16) return mma_ptr<DD, kF16, kF16>(ap);            \
  if (kv_fmt == kBF16 && q_fmt == kBF16) return mma_ptr<DD, kBF16, kBF16>(ap);        \
  if (kv_fmt == kE4M3 && q_fmt == kF16) return mma_ptr<DD, kE4M3, kF16>(ap);          \
  if (kv_fmt == kE4M3 && q_fmt == kBF16) return mma_ptr<DD, kE4M3, kBF16>(ap);        \
  if (kv_fmt == kE5M2 && q_fmt == kF16) return mma_ptr<DD, kE5M2, kF16>(ap);          \
  if (kv_fmt == kE5M2 && q_fmt == kBF16) return mma_ptr<DD, kE5M2, kBF16>(ap);
  if (D == 128) { VP_MMA(128) }
  if (D == 64) { VP_MMA(64) }
#undef VP_MMA
  return nullptr;
}

static const void* decode_kernel_for(int D, int kv_fmt, int q_fmt, bool ap) {
  return decode_mma_kernel_for(D, kv_fmt, q_fmt, ap);
}

static const void* decode_shared_kernel_for(int D, int kv_fmt, int q_fmt) {
#define VP_SHARED(DD, KK, QQ)                                                         \
  if (kv_fmt == KK && q_fmt == QQ)                                                    \
    return reinterpret_cast<const void*>(&decode_shared_kernel<DD, KK, QQ, is_fp8(KK) ? 2 : 1>);
#define VP_SHARED_D(DD)                                                               \
  VP_SHARED(DD, kF16, kF16) VP_SHARED(DD, kBF16, kBF16) VP_SHARED(DD, kE4M3, kF16)     \
  VP_SHARED(DD, kE4M3, kBF16) VP_SHARED(DD, kE5M2, kF16) VP_SHARED(DD, kE5M2, kBF16)
  if (D == 128) { VP_SHARED_D(128) }
  if (D == 64) { VP_SHARED_D(64) }
#undef VP_SHARED_D
#undef VP_SHARED
  return nullptr;
}

template <int D, int QF>
static const void* merge_for(int gc) {
  switch (gc) {
    case 1: return reinterpret_cast<const void*>(&decode_merge_kernel<D, 1, QF>);
    case 2: return reinterpret_cast<const void*>(&decode_merge_kernel<D, 2, QF>);
    case 3: return reinterpret_cast<const void*>(&decode_merge_kernel<D, 3, QF>);
    case 4: return reinterpret_cast<const void*>(&decode_merge_kernel<D, 4, QF>);
    case 5: return reinterpret_cast<const void*>(&decode_merge_kernel<D, 5, QF>);
    case 6: return reinterpret_cast<const void*>(&decode_merge_kernel<D, 6, QF>);
    case 7: return reinterpret_cast<const void*>(&decode_merge_kernel<D, 7, QF>);
    case 8: return reinterpret_cast<const void*>(&decode_merge_kernel<D, 8, QF>);
    default: return nullptr;
  }
}

static const void* merge_kernel_for(int D, int q_fmt, int gc) {
  if (D == 128) return q_fmt == kBF16 ? merge_for<128, kBF16>(gc) : merge_for<128, kF16>(gc);
  if (D == 64) return q_fmt == kBF16 ? merge_for<64, kBF16>(gc) : merge_for<64, kF16>(gc);
  return nullptr;
}

// Per-device caches of the CU count and of each kernel variant's resident
// workgroups per CU: filled on first use, read without locks (a racing first
// use computes the same value twice).
constexpr int kMaxDevices = 64;
constexpr int kVariants = 2 * 2 * 4 * 2;      // (append, D = 128, kv format, q format)
static std::atomic<int> g_cus[kMaxDevices];
static std::atomic<int> g_occ[kMaxDevices][kVariants];

int decode_workers(int64_t pages_bound, int head_dim, int kv_fmt, int q_fmt, int, bool append) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    dev = 0;
  }
  const bool cached = dev >= 0 && dev < kMaxDevices;
  int cus = cached ? g_cus[dev].load(std::memory_order_relaxed) : 0;
  if (cus <= 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0) {
      (void)hipGetLastError();
      cus = 256;
    }
    if (cached) g_cus[dev].store(cus, std::memory_order_relaxed);
  }
  int per_cu = 2;
  const int vi = (((int)append * 2 + (head_dim == 128)) * 4 + kv_fmt) * 2 + (q_fmt == kBF16);
  const bool vcached = cached && vi >= 0 && vi < kVariants;
  const int occ_seen = vcached ? g_occ[dev][vi].load(std::memory_order_relaxed) : 0;
  if (occ_seen > 0) {
    per_cu = occ_seen;
  } else if (const void* k = decode_kernel_for(head_dim, kv_fmt, q_fmt, append)) {
    int occ = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, k, kNW * 64, 0) == hipSuccess && occ > 0) {
      per_cu = occ;
      if (vcached) g_occ[dev][vi].store(occ, std::memory_order_relaxed);
    } else {
      (void)hipGetLastError();
    }
  }
  // The kernel fits three workgroups per CU at head_dim 128 (more at 64), but
  // two are faster: a third makes the chunks a third shorter (more pieces to
  // merge) and leaves no room beside the decode for the shared-prefix pass.
  per_cu = min(per_cu, 2);
  if (const char* e = getenv("VLLM_PAGED_WG_PER_CU")) {
    const int v = atoi(e);
    if (v > 0) per_cu = v;
  }
  const int64_t w = (int64_t)cus * per_cu * kNW;
  return (int)min(decode_workers_bound(pages_bound), (w + kNW - 1) / kNW * kNW);
}

hipError_t launch_decode(const DecodeParams& p, int head_dim, int kv_fmt, int q_fmt, hipStream_t stream) {
  if (p.num_seqs == 0) return hipSuccess;
  const void* k = decode_kernel_for(head_dim, kv_fmt, q_fmt, p.new_slots != nullptr);
  const void* mk = merge_kernel_for(head_dim, q_fmt, p.head_chunk);
  if (!k || !mk) return hipErrorInvalidValue;
  DecodeParams a = p;
  void* args[] = {&a};
  if (p.num_seqs > kScanMax) {
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&decode_prefix_kernel), dim3(1),
                                   dim3(kNW * 64), args, 0, stream);
    if (e != hipSuccess) return e;
  }
  hipError_t e = hipLaunchKernel(k, dim3(p.num_workers / kNW), dim3(kNW * 64), args, 0, stream);
  if (e != hipSuccess) return e;
  return launch_decode_merge(p, head_dim, q_fmt, stream);
}

hipError_t launch_decode_shared(const DecodeParams& p, const PrefillParams& sp, int head_dim,
                                int kv_fmt, int q_fmt, hipStream_t stream) {
  if (p.num_seqs == 0) return hipSuccess;
  const void* k = decode_shared_kernel_for(head_dim, kv_fmt, q_fmt);
  if (!k || sp.num_splits < 1) return hipErrorInvalidValue;
  DecodeParams a = p;
  PrefillParams x = sp;
  // the tile grid of the prefix pass: (kv-head, split) pairs over the 8 XCDs,
  // times the tiles of 128 (sequence, query head) rows
  x.num_tiles = (int)(((int64_t)sp.num_seqs * sp.group + tile::kRows - 1) / tile::kRows);
  const int64_t pairs = (int64_t)sp.num_kv_heads * sp.num_splits;
  const int64_t npfx = (pairs + 7) / 8 * 8 * x.num_tiles;
  const int64_t grid = npfx + p.num_workers / kNW;
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  int n = (int)npfx;
  if (p.num_seqs > kScanMax) {
    void* pargs[] = {&a};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&decode_prefix_kernel), dim3(1),
                                   dim3(kNW * 64), pargs, 0, stream);
    if (e != hipSuccess) return e;
  }
  void* args[] = {&a, &x, &n};
  hipError_t e = hipLaunchKernel(k, dim3((unsigned)grid), dim3(kNW * 64), args, 0, stream);
  if (e != hipSuccess) return e;
  return launch_decode_merge(p, head_dim, q_fmt, stream);
}

hipError_t launch_decode_merge(const DecodeParams& p, int head_dim, int q_fmt, hipStream_t stream) {
  if (p.num_seqs == 0) return hipSuccess;
  const void* mk = merge_kernel_for(head_dim, q_fmt, p.head_chunk);
  if (!mk) return hipErrorInvalidValue;
  DecodeParams a = p;
  void* args[] = {&a};
  const int64_t units = (int64_t)p.num_seqs * p.num_kv_heads * (p.group / p.head_chunk);
  return hipLaunchKernel(mk, dim3((unsigned)units), dim3(p.head_chunk * head_dim / 4), args, 0, stream);
}

}  // namespace vp

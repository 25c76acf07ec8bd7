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
// Inside a wave, per 16-token page of one kv-head (CH = D/8 chunks of 8
// elements per token row):
//  * K role: LPR lanes share a token row; load instruction k gives lane
//    (rho, c) chunk (k % CPL) * LPR + c of row (k / CPL) * RPI + rho, so the
//    LPR lanes of a row read LPR adjacent chunks.  Packed dot2 (fp16 or bf16
//    pairs; FP8 codes are first converted exactly to q's format) gives
//    partial dot products, summed over the LPR lanes with DPP.
//  * Online softmax in fp32, log2 domain, with a running max that is uniform
//    over the wave and only moves when a score exceeds it by more than 2^8
//    (one wave vote per page).  Keys outside [max(0, n - window), n) get
//    score -inf and their V rows are replaced by zeros: NaN garbage in the
//    unused rows of a page never reaches the output.
//  * The probabilities, rounded to q's 16-bit format, go through a small
//    per-wave LDS buffer to the V role: CH lanes share a V row, one chunk
//    each, so every wave load reads 64 contiguous chunks.  Rows of two
//    consecutive load instructions are paired so that P.V runs on packed
//    dot2 (v[t1][e], v[t2][e]) . (p[t1][h], p[t2][h]) with fp32
//    accumulation; the row sums use the same rounded probabilities.
//  * The next page's K is loaded as soon as Q.K has consumed the registers,
//    and the next V as soon as P.V has; these loads are unconditional (past
//    the end of the stretch they read a spare page of the workspace, which
//    stays in L2) so that the compiler can keep the buffers in flight across
//    iterations.
#include <atomic>
#include <cstdlib>
#include <type_traits>
#include <utility>

#include "common.h"
#include "kernels.h"

namespace vp {

constexpr int kNW = kDecodeWaves;
constexpr float kTau = 8.0f;       // rescale headroom, log2 units
constexpr int kScanMax = 2048;     // sequences whose page prefix fits in LDS

template <int KF> struct KvChunk { using T = uint4; };      // 8 x 16-bit
template <> struct KvChunk<kE4M3> { using T = uint2; };     // 8 x fp8
template <> struct KvChunk<kE5M2> { using T = uint2; };

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

// 8 K elements -> 4 packed pairs in q's format.
template <int KF, int QF>
__device__ __forceinline__ void k_pairs(const typename KvChunk<KF>::T& x, uint32_t (&w)[4]) {
  if constexpr (!is_fp8(KF)) {
    w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
  } else {
    w[0] = fp8x2_to_q16<KF, QF, false>(x.x);
    w[1] = fp8x2_to_q16<KF, QF, true>(x.x);
    w[2] = fp8x2_to_q16<KF, QF, false>(x.y);
    w[3] = fp8x2_to_q16<KF, QF, true>(x.y);
  }
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

// V elements of two tokens, paired per element for dot2: o[e] holds
// (element e of token A, element e of token B) in q's 16-bit format.
template <int KF, int QF>
__device__ __forceinline__ void v_pairs(const typename KvChunk<KF>::T& a,
                                        const typename KvChunk<KF>::T& b, uint32_t (&o)[8]) {
  if constexpr (!is_fp8(KF)) {
    const uint32_t aw[4] = {a.x, a.y, a.z, a.w};
    const uint32_t bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = __builtin_amdgcn_perm(bw[i], aw[i], 0x05040100u);       // (a.lo, b.lo)
      o[2 * i + 1] = __builtin_amdgcn_perm(bw[i], aw[i], 0x07060302u);   // (a.hi, b.hi)
    }
  } else {
    const uint32_t aw[2] = {a.x, a.y};
    const uint32_t bw[2] = {b.x, b.y};
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      // byte interleave (a0, b0, a1, b1) and (a2, b2, a3, b3), then convert
      // each byte pair exactly to two 16-bit values.
      const uint32_t w01 = __builtin_amdgcn_perm(bw[i], aw[i], 0x05010400u);
      const uint32_t w23 = __builtin_amdgcn_perm(bw[i], aw[i], 0x07030602u);
      o[4 * i + 0] = fp8x2_to_q16<KF, QF, false>(w01);
      o[4 * i + 1] = fp8x2_to_q16<KF, QF, true>(w01);
      o[4 * i + 2] = fp8x2_to_q16<KF, QF, false>(w23);
      o[4 * i + 3] = fp8x2_to_q16<KF, QF, true>(w23);
    }
  }
}

template <int QF>
__device__ __forceinline__ float lo16_to_f32(uint32_t w) {
  if constexpr (QF == kBF16) return bitcast<float>(w << 16);
  else return (float)bitcast<half2_t>(w).x;
}
template <int QF>
__device__ __forceinline__ float hi16_to_f32(uint32_t w) {
  if constexpr (QF == kBF16) return bitcast<float>(w & 0xFFFF0000u);
  else return (float)bitcast<half2_t>(w).y;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) x += __shfl_xor(x, off);
  return x;
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

__device__ __forceinline__ SeqRange seq_range(const DecodeParams& p, int s) {
  return seq_range_of(p, p.context_lens[s]);
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

// AP: with the fused cache write of each sequence's newest token (a variant
// of its own, so that the plain decode keeps its registers).
template <int D, int G, int KF, int QF, int LPR, int PD, bool AP>
__global__ __launch_bounds__(kNW * 64) void decode_kernel(DecodeParams p) {
  constexpr int CH = D / 8;
  static_assert(LPR >= 4 && LPR <= CH, "lanes per K row");
  constexpr int CPL = CH / LPR;          // chunks per lane per K row
  constexpr int RPI = 64 / LPR;          // K rows per load instruction
  constexpr int NKI = CH / 4;            // load instructions per page (K or V)
  constexpr int TPL = 16 / RPI;          // K rows per lane per page
  constexpr int RPIV = 64 / CH;          // V rows per load instruction
  static_assert(NKI % 2 == 0, "V rows are paired");
  constexpr int GW = (G + 1) / 2;        // dwords of packed probabilities per token
  using LT = typename KvChunk<KF>::T;
  constexpr int CB = (int)sizeof(LT);    // bytes per 8-element chunk
  constexpr int ROWB = CH * CB;
  constexpr int64_t kPageBytes = 16 * ROWB;

  __shared__ int s_pre[kScanMax + 1];
  __shared__ int s_ctx[kScanMax];      // context lengths (batches of up to kScanMax)
  __shared__ uint32_t s_p[kNW][16][GW];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rho = lane / LPR, c = lane % LPR;          // K role
  const int rv = lane / CH, cv = lane % CH;            // V role
  const int B = p.num_seqs;
  const int ngc = p.group / G;
  const int NY = p.num_kv_heads * ngc;                 // units per sequence

  // Page prefix over the batch: in LDS for small batches (workgroup 0 also
  // stores it for the merge), else precomputed in the workspace.
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

  // Sequences with no key to attend to get all-zero output rows (with a
  // shared prefix the merge writes their rows from the prefix partials).
  for (int sq = blockIdx.x; sq < B; sq += gridDim.x) {
    if (pre[sq + 1] == pre[sq]) {
      if (p.skip_tokens == 0) {
        uint16_t* o = static_cast<uint16_t*>(p.out) + (int64_t)sq * p.num_q_heads * D;
        for (int i = threadIdx.x; i < p.num_q_heads * D; i += kNW * 64) o[i] = 0;
      }
      for (int i = threadIdx.x; i < NY; i += kNW * 64) p.ws_unit[((int64_t)sq * NY + i) * 2 + 1] = 0;
    }
  }

  const int64_t blk_stride = (int64_t)p.num_kv_heads * kPageBytes;
  int koff[NKI];
#pragma unroll
  for (int k = 0; k < NKI; ++k)
    koff[k] = ((k / CPL) * RPI + rho) * ROWB + ((k % CPL) * LPR + c) * CB;

  for (int64_t chunk = (int64_t)blockIdx.x * kNW + wave; chunk < num_chunks;
       chunk += p.num_workers) {
    int64_t g = chunk * C;
    const int64_t g_end = min(g + C, T);
    // sequence holding global page g: last s with NY * pre[s] <= g
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
      // (values read from LDS are wave-uniform: keep them in scalar registers)
      while ((int64_t)NY * __builtin_amdgcn_readfirstlane(pre[s + 1]) <= g) ++s;   // skip empty seqs
      const SeqRange sr = seq_range_of(
          p, B <= kScanMax ? __builtin_amdgcn_readfirstlane(s_ctx[s]) : p.context_lens[s]);
      const int64_t off = g - (int64_t)NY * __builtin_amdgcn_readfirstlane(pre[s]);
      const int y = (int)(off / sr.np);
      const int i0 = (int)(off - (int64_t)y * sr.np);
      const int i1 = (int)min((int64_t)sr.np, i0 + (g_end - g));
      const int slot = first_seg ? 0 : 1;
      // A unit finished inside this chunk writes its output directly, or,
      // when shared-prefix partials still have to be merged in, its partial
      // to a slot of its own (a chunk may hold several whole units).
      const bool whole = (i0 == 0) && (i1 == sr.np);
      const bool complete = whole && p.skip_tokens == 0;
      const int hk = y / ngc;
      const int h0 = hk * p.group + (y - hk * ngc) * G;
      // FP8 scales of this kv-head (per-head arrays, else the per-tensor ones)
      const float sscale = p.k_scales ? p.score_base * p.k_scales[hk] : p.score_scale;
      const float oscale = p.v_scales ? p.v_scales[hk] : p.out_scale;

      // ---- one segment: pages [i0, i1) of unit (s, y) ----
      if constexpr (AP) {
        if (i1 == sr.np) append_row<D, KF, QF>(p, s, hk, lane);
      }
      uint4 qv[G][CPL];
      {
        const uint16_t* qp =
            static_cast<const uint16_t*>(p.q) + ((int64_t)s * p.num_q_heads + h0) * D;
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
          for (int sub = 0; sub < CPL; ++sub)
            qv[h][sub] = *reinterpret_cast<const uint4*>(qp + h * D + (sub * LPR + c) * 8);
      }
      const int32_t* bt = p.block_tables + (int64_t)s * p.bt_stride + sr.lo_page;
      const uint8_t* kbase = static_cast<const uint8_t*>(p.k_cache) + (int64_t)hk * kPageBytes;
      const uint8_t* vbase = static_cast<const uint8_t*>(p.v_cache) + (int64_t)hk * kPageBytes +
                             rv * ROWB + cv * CB;
      const uint8_t* spare = static_cast<const uint8_t*>(p.ws_spare);
      const uint8_t* spare_v = spare + rv * ROWB + cv * CB;
      const int count = i1 - i0;
      // Block ids, 64 pages per lane vector; the next 64 are fetched one
      // batch ahead so that reading them never waits on the page loads.
      int bt_base = 0;
      auto bt_fetch = [&](int base) __attribute__((always_inline)) {
        const int q = i0 + base + lane;
        int b = q < i1 ? bt[q] : 0;
        return (unsigned)b < (unsigned)p.num_blocks ? b : 0;
      };
      int bt_cur = bt_fetch(0), bt_nxt = count > 64 ? bt_fetch(64) : 0;
      auto blk_of = [&](int jj) __attribute__((always_inline)) {
        if (jj >= bt_base + 64) {          // pages are requested in increasing order
          bt_base += 64;
          bt_cur = bt_nxt;
          if (bt_base + 64 < count) bt_nxt = bt_fetch(bt_base + 64);
        }
        return __builtin_amdgcn_readlane(bt_cur, jj - bt_base);
      };
      // kp: the page's K base (this kv-head); vp: its V base plus this lane's offset
      auto load_k = [&](const uint8_t* kp, LT (&kd)[NKI]) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < NKI; ++k) kd[k] = ld_stream<LT>(kp + koff[k]);
      };
      auto load_v = [&](const uint8_t* vp, LT (&vd)[NKI]) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < NKI; ++k) vd[k] = ld_stream<LT>(vp + k * RPIV * ROWB);
      };

      float m[G], l[G], acc[G][8];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.0f;
      }
      // PD pages of K and V in flight: buffer u holds page jb + u.  Loads are
      // unconditional (past the end they re-read the last page) so that no
      // buffer goes through a control-flow merge.
      LT kd[PD][NKI], vd[PD][NKI];
#pragma unroll
      for (int u = 0; u < PD; ++u) {
        const int b0 = blk_of(min(u, count - 1));
        load_k(u < count ? kbase + b0 * blk_stride : spare, kd[u]);
        load_v(u < count ? vbase + b0 * blk_stride : spare_v, vd[u]);
      }
      for (int jb = 0; jb < count; jb += PD) {
#pragma unroll
        for (int u = 0; u < PD; ++u) {
          const int jj = jb + u;
          const bool valid = jj < count;
          const int t0 = (sr.lo_page + i0 + min(jj, count - 1)) * 16;
          const bool full = (t0 >= sr.lo) && (t0 + 16 <= sr.n);
          // page loaded into this buffer next; past the end of the stretch
          // the loads read the spare page instead (kept hot in L2, its
          // values are never used)
          const bool past = jj + PD >= count;
          const int bn = blk_of(min(jj + PD, count - 1));
          const uint8_t* knext = past ? spare : kbase + bn * blk_stride;
          const uint8_t* vnext = past ? spare_v : vbase + bn * blk_stride;
          float sc[TPL][G];
          if (valid) {
            // ---- Q.K (K role) ----
#pragma unroll
            for (int rg = 0; rg < TPL; ++rg)
#pragma unroll
              for (int h = 0; h < G; ++h) sc[rg][h] = 0.0f;
#pragma unroll
            for (int k = 0; k < NKI; ++k) {
              uint32_t kw[4];
              k_pairs<KF, QF>(kd[u][k], kw);
#pragma unroll
              for (int h = 0; h < G; ++h) {
                const uint4 qq = qv[h][k % CPL];
                float a = sc[k / CPL][h];
                a = dot2<QF>(qq.x, kw[0], a);
                a = dot2<QF>(qq.y, kw[1], a);
                a = dot2<QF>(qq.z, kw[2], a);
                a = dot2<QF>(qq.w, kw[3], a);
                sc[k / CPL][h] = a;
              }
            }
          }
          __builtin_amdgcn_sched_barrier(0);
          load_k(knext, kd[u]);
          __builtin_amdgcn_sched_barrier(0);
          if (valid) {
#pragma unroll
            for (int rg = 0; rg < TPL; ++rg)
#pragma unroll
              for (int h = 0; h < G; ++h) sc[rg][h] = group_sum<LPR>(sc[rg][h]) * sscale;
            if (!full) {
#pragma unroll
              for (int rg = 0; rg < TPL; ++rg) {
                const int t = t0 + rg * RPI + rho;
                if (t < sr.lo || t >= sr.n) {
#pragma unroll
                  for (int h = 0; h < G; ++h) sc[rg][h] = -INFINITY;
                }
              }
            }

            // ---- online softmax ----
            bool need = false;
#pragma unroll
            for (int rg = 0; rg < TPL; ++rg)
#pragma unroll
              for (int h = 0; h < G; ++h) need |= sc[rg][h] > m[h] + kTau;
            if (__any(need)) {
#pragma unroll
              for (int h = 0; h < G; ++h) {
                float pm = sc[0][h];
#pragma unroll
                for (int rg = 1; rg < TPL; ++rg) pm = fmaxf(pm, sc[rg][h]);
                pm = wave_max(pm);
                const float mn = fmaxf(m[h], pm);
                const float alpha = (m[h] == -INFINITY) ? 0.0f : fast_exp2(m[h] - mn);
                m[h] = mn;
                l[h] *= alpha;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[h][e] *= alpha;
              }
            }
#pragma unroll
            for (int rg = 0; rg < TPL; ++rg) {
              uint32_t pw[GW];
#pragma unroll
              for (int i = 0; i < GW; ++i) {
                const int ha = 2 * i, hb = 2 * i + 1;
                const float ma = (m[ha] == -INFINITY) ? 0.0f : m[ha];
                const float pa = fast_exp2(sc[rg][ha] - ma);
                float pb = 0.0f;
                if (hb < G) {
                  const float mb = (m[hb] == -INFINITY) ? 0.0f : m[hb];
                  pb = fast_exp2(sc[rg][hb] - mb);
                }
                pw[i] = pack16<QF>(pa, pb);
                l[ha] += lo16_to_f32<QF>(pw[i]);
                if (hb < G) l[hb] += hi16_to_f32<QF>(pw[i]);
              }
              if (c == 0) {
#pragma unroll
                for (int i = 0; i < GW; ++i) s_p[wave][rg * RPI + rho][i] = pw[i];
              }
            }

            // ---- P.V (V role) ----
            auto pv = [&](const LT (&vx)[NKI]) __attribute__((always_inline)) {
#pragma unroll
              for (int pr = 0; pr < NKI / 2; ++pr) {
                const int ta = (2 * pr) * RPIV + rv, tb = (2 * pr + 1) * RPIV + rv;
                uint32_t vp2[8];
                v_pairs<KF, QF>(vx[2 * pr], vx[2 * pr + 1], vp2);
                uint32_t pp[G];
#pragma unroll
                for (int i = 0; i < GW; ++i) {
                  const uint32_t A = s_p[wave][ta][i], B2 = s_p[wave][tb][i];
                  pp[2 * i] = __builtin_amdgcn_perm(B2, A, 0x05040100u);
                  if (2 * i + 1 < G) pp[2 * i + 1] = __builtin_amdgcn_perm(B2, A, 0x07060302u);
                }
#pragma unroll
                for (int h = 0; h < G; ++h)
#pragma unroll
                  for (int e = 0; e < 8; ++e) acc[h][e] = dot2<QF>(pp[h], vp2[e], acc[h][e]);
              }
            };
            if (full) {
              pv(vd[u]);
            } else {
              // rows outside the kept range may hold NaN: replace them by zeros
              LT vv[NKI];
#pragma unroll
              for (int k = 0; k < NKI; ++k) {
                const int t = t0 + k * RPIV + rv;
                vv[k] = (t < sr.lo || t >= sr.n) ? LT{} : vd[u][k];
              }
              pv(vv);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
          load_v(vnext, vd[u]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }

      // Sum the V rows (lanes cv, cv + CH, ...) and the K-role row sums (one
      // lane per row: c == 0).  m is uniform over the wave.
#pragma unroll
      for (int off = CH; off < 64; off <<= 1)
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[h][e] += __shfl_xor(acc[h][e], off);
#pragma unroll
      for (int h = 0; h < G; ++h) l[h] = wave_sum(c == 0 ? l[h] : 0.0f);

      if (complete) {
        if (rv == 0) {
#pragma unroll
          for (int h = 0; h < G; ++h) {
            const float inv = oscale / l[h];
            uint32_t w[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
              w[i] = (uint32_t)f32_to_16<QF>(acc[h][2 * i] * inv) |
                     ((uint32_t)f32_to_16<QF>(acc[h][2 * i + 1] * inv) << 16);
            uint16_t* o = static_cast<uint16_t*>(p.out) +
                          ((int64_t)s * p.num_q_heads + h0 + h) * D + cv * 8;
            *reinterpret_cast<uint4*>(o) = make_uint4(w[0], w[1], w[2], w[3]);
          }
        }
      } else {
        const int64_t unit = (int64_t)s * NY + y;
        const int64_t sl = chunk * 2 + slot;
        float* wo = whole ? p.ws_uo + unit * G * D : p.ws_o + sl * G * D;
        float* wm = whole ? p.ws_um + unit * G : p.ws_m + sl * G;
        float* wl = whole ? p.ws_ul + unit * G : p.ws_l + sl * G;
        if (rv == 0) {
#pragma unroll
          for (int h = 0; h < G; ++h) {
            const float inv = 1.0f / l[h];
            float* o = wo + h * D + cv * 8;
            *reinterpret_cast<float4*>(o) =
                make_float4(acc[h][0] * inv, acc[h][1] * inv, acc[h][2] * inv, acc[h][3] * inv);
            *reinterpret_cast<float4*>(o + 4) =
                make_float4(acc[h][4] * inv, acc[h][5] * inv, acc[h][6] * inv, acc[h][7] * inv);
          }
        }
        if (lane == 0) {
#pragma unroll
          for (int h = 0; h < G; ++h) {
            wm[h] = m[h];
            wl[h] = l[h];
          }
        }
      }
      // The wave holding page 0 of the unit records where its pieces are:
      // (slot of the first piece, number of pieces), or 0 pieces if done
      // (a unit inside one chunk with a shared prefix has 1 piece).
      if (i0 == 0 && lane == 0) {
        int npieces = 0;
        if (!complete) {
          const int64_t base = g;                 // = NY * pre[s] + y * np
          npieces = (int)((base + sr.np - 1) / C - base / C + 1);
        }
        // (first slot -1: the single piece sits in the unit's own slot)
        p.ws_unit[((int64_t)s * NY + y) * 2] = whole ? -1 : (int32_t)(chunk * 2 + slot);
        p.ws_unit[((int64_t)s * NY + y) * 2 + 1] = npieces;
      }
      g += i1 - i0;
      first_seg = false;
    }
  }
}

// Log-sum-exp merge of the pieces of units cut by chunk boundaries (and, with
// a shared prefix, of every unit with its prefix splits).  One workgroup per
// unit, one thread per 4 consecutive outputs of its G x D block; the unit's
// record (first slot, piece count) comes from the decode kernel.  Pieces are
// read in rounds of kMergeBatch (units of more pieces: twice that) straight
// into registers, every load of a round independent (padding pieces past the
// count re-read the last piece and get weight 0), so a round costs one
// memory latency:
// M = max m, w = l 2^(m - M), out = sum w o / sum w.
constexpr int kMergeBatch = 8;

template <int D, int G, int QF>
__global__ __launch_bounds__(G * D / 4) void decode_merge_kernel(DecodeParams p) {
  const int ngc = p.group / G;
  const int NY = p.num_kv_heads * ngc;
  const int64_t u = blockIdx.x;
  const int nsuf = p.ws_unit[u * 2 + 1];
  const int npieces = nsuf + p.num_splits;
  if (npieces == 0) return;                   // finished inside one chunk, or empty
  const int64_t sl0 = p.ws_unit[u * 2];
  const int s = (int)(u / NY);
  const int y = (int)(u - (int64_t)s * NY);
  const int hk = y / ngc;
  const int h0 = hk * p.group + (y - hk * ngc) * G;
  const int64_t prow = (int64_t)s * p.num_q_heads + h0;    // row of head h0 in the prefix partials
  const int64_t fk = sl0 >> 1;
  const int64_t split_rows = (int64_t)p.num_seqs * p.num_q_heads;
  const int e = threadIdx.x * 4;
  const int h = e / D;
  // Piece k < nsuf: a piece of the decode (the first sits in the slot its
  // wave recorded, or in the unit's own slot when that is -1; the later ones
  // open the following chunks, slot 0 of each); piece nsuf + i: split i of
  // the shared-prefix partials.  Gives the row of head 0 of the unit in the
  // piece's (o, m, l) arrays.
  auto ml_row = [&](int k, const float*& op, const float*& mp, const float*& lp)
      __attribute__((always_inline)) {
    if (k < nsuf) {
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
    }
    op = p.pfx_o;
    mp = p.pfx_m;
    lp = p.pfx_l;
    return (int64_t)(k - nsuf) * split_rows + prow;
  };
  float M = -INFINITY, den = 0.0f;
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  auto rounds = [&](auto nb) __attribute__((always_inline)) {
    constexpr int NB = decltype(nb)::value;
    for (int k0 = 0; k0 < npieces; k0 += NB) {
      float mk[NB], lk[NB];
      float4 ok[NB];
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        const float *op, *mp, *lp;
        const int64_t r = ml_row(min(k0 + k, npieces - 1), op, mp, lp) + h;
        mk[k] = mp[r];
        lk[k] = lp[r];
        ok[k] = *reinterpret_cast<const float4*>(op + r * D + (e - h * D));
      }
      float Mn = M;
#pragma unroll
      for (int k = 0; k < NB; ++k)
        if (k0 + k < npieces) Mn = fmaxf(Mn, mk[k]);
      const float a = (M == -INFINITY) ? 0.0f : fast_exp2(M - Mn);
      den *= a;
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] *= a;
      M = Mn;
      const float Mu = (M == -INFINITY) ? 0.0f : M;   // (every piece so far empty)
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        const float w = (k0 + k < npieces) ? lk[k] * fast_exp2(mk[k] - Mu) : 0.0f;  // 0: padding, empty
        den += w;
        acc[0] = fmaf(w, ok[k].x, acc[0]);
        acc[1] = fmaf(w, ok[k].y, acc[1]);
        acc[2] = fmaf(w, ok[k].z, acc[2]);
        acc[3] = fmaf(w, ok[k].w, acc[3]);
      }
    }
  };
  // (npieces is uniform over the workgroup)
  if (npieces <= kMergeBatch) rounds(std::integral_constant<int, kMergeBatch>{});
  else rounds(std::integral_constant<int, 2 * kMergeBatch>{});
  const float oscale = p.v_scales ? p.v_scales[hk] : p.out_scale;
  const float f = den > 0.0f ? oscale / den : 0.0f;
  uint16_t* out = static_cast<uint16_t*>(p.out) + prow * D + e;
  const uint32_t lo = (uint32_t)f32_to_16<QF>(acc[0] * f) | ((uint32_t)f32_to_16<QF>(acc[1] * f) << 16);
  const uint32_t hi = (uint32_t)f32_to_16<QF>(acc[2] * f) | ((uint32_t)f32_to_16<QF>(acc[3] * f) << 16);
  *reinterpret_cast<uint2*>(out) = make_uint2(lo, hi);
}

// Page prefix for batches too large for the LDS scan of decode_kernel.
__global__ __launch_bounds__(kNW * 64) void decode_prefix_kernel(DecodeParams p) {
  page_prefix(p, p.ws_prefix);
}

// Lanes per K row: fewer lanes -> fewer cross-lane sums but more query
// registers per lane (CH / LPR chunks per head).
template <int D, int G>
constexpr int kLpr = (D == 64) ? (G <= 4 ? 4 : 8) : (G <= 2 ? 4 : (G <= 5 ? 8 : 16));

// Pages of K and V in flight per wave.
template <int D, int G>
constexpr int kPd = 2;

template <int D, int G, int KF, int QF>
static const void* kernel_ptr(bool ap) {
  return ap ? reinterpret_cast<const void*>(&decode_kernel<D, G, KF, QF, kLpr<D, G>, kPd<D, G>, true>)
            : reinterpret_cast<const void*>(&decode_kernel<D, G, KF, QF, kLpr<D, G>, kPd<D, G>, false>);
}

template <int D, int KF, int QF>
static const void* pick(int gc, bool ap) {
  switch (gc) {
    case 1: return kernel_ptr<D, 1, KF, QF>(ap);
    case 2: return kernel_ptr<D, 2, KF, QF>(ap);
    case 3: return kernel_ptr<D, 3, KF, QF>(ap);
    case 4: return kernel_ptr<D, 4, KF, QF>(ap);
    case 5: return kernel_ptr<D, 5, KF, QF>(ap);
    case 6: return kernel_ptr<D, 6, KF, QF>(ap);
    case 7: return kernel_ptr<D, 7, KF, QF>(ap);
    case 8: return kernel_ptr<D, 8, KF, QF>(ap);
    default: return nullptr;
  }
}

static const void* decode_kernel_for(int D, int kv_fmt, int q_fmt, int gc, bool ap) {
  if (D == 128) {
    if (kv_fmt == kF16 && q_fmt == kF16) return pick<128, kF16, kF16>(gc, ap);
    if (kv_fmt == kBF16 && q_fmt == kBF16) return pick<128, kBF16, kBF16>(gc, ap);
    if (kv_fmt == kE4M3 && q_fmt == kF16) return pick<128, kE4M3, kF16>(gc, ap);
    if (kv_fmt == kE4M3 && q_fmt == kBF16) return pick<128, kE4M3, kBF16>(gc, ap);
    if (kv_fmt == kE5M2 && q_fmt == kF16) return pick<128, kE5M2, kF16>(gc, ap);
    if (kv_fmt == kE5M2 && q_fmt == kBF16) return pick<128, kE5M2, kBF16>(gc, ap);
  } else if (D == 64) {
    if (kv_fmt == kF16 && q_fmt == kF16) return pick<64, kF16, kF16>(gc, ap);
    if (kv_fmt == kBF16 && q_fmt == kBF16) return pick<64, kBF16, kBF16>(gc, ap);
    if (kv_fmt == kE4M3 && q_fmt == kF16) return pick<64, kE4M3, kF16>(gc, ap);
    if (kv_fmt == kE4M3 && q_fmt == kBF16) return pick<64, kE4M3, kBF16>(gc, ap);
    if (kv_fmt == kE5M2 && q_fmt == kF16) return pick<64, kE5M2, kF16>(gc, ap);
    if (kv_fmt == kE5M2 && q_fmt == kBF16) return pick<64, kE5M2, kBF16>(gc, ap);
  }
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
constexpr int kVariants = 2 * 2 * 4 * 16;     // (append, D = 128, kv format, q format, G)
static std::atomic<int> g_cus[kMaxDevices];
static std::atomic<int> g_occ[kMaxDevices][kVariants];

int decode_workers(int64_t pages_bound, int head_dim, int kv_fmt, int q_fmt, int head_chunk,
                   bool append) {
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
  int per_cu = 4;
  const int vi = (((int)append * 2 + (head_dim == 128)) * 4 + kv_fmt) * 16 + q_fmt * 8 + (head_chunk - 1);
  const bool vcached = cached && vi >= 0 && vi < kVariants;
  const int occ_seen = vcached ? g_occ[dev][vi].load(std::memory_order_relaxed) : 0;
  if (occ_seen > 0) {
    per_cu = occ_seen;
  } else if (const void* k = decode_kernel_for(head_dim, kv_fmt, q_fmt, head_chunk, append)) {
    int occ = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, k, kNW * 64, 0) == hipSuccess && occ > 0) {
      per_cu = occ;
      if (vcached) g_occ[dev][vi].store(occ, std::memory_order_relaxed);
    } else {
      (void)hipGetLastError();
    }
  }
  if (const char* e = getenv("VLLM_PAGED_WG_PER_CU")) {
    const int v = atoi(e);
    if (v > 0) per_cu = v;
  }
  const int64_t w = (int64_t)cus * per_cu * kNW;
  return (int)min(decode_workers_bound(pages_bound), (w + kNW - 1) / kNW * kNW);
}

hipError_t launch_decode(const DecodeParams& p, int head_dim, int kv_fmt, int q_fmt, hipStream_t stream,
                         bool split) {
  if (p.num_seqs == 0) return hipSuccess;
  const void* k = decode_kernel_for(head_dim, kv_fmt, q_fmt, p.head_chunk, p.new_slots != nullptr);
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
  if (e != hipSuccess || split) return e;
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

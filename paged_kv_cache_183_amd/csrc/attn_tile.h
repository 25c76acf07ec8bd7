// Attention tiles on the matrix cores of gfx950, in two uses:
//
// Chunked prefill.  Sequence s has Q_s new query tokens at positions
// n - Q_s .. n - 1 of its n cached tokens (their K/V are already in the
// block-paged pool); the query row at position p attends to keys t <= p with
// t > p - window (window 0: no lower bound).  This is the paged attention of
// the vllm.cpp model forward (repository listing, "What's implemented") for a
// chunk of several query tokens, with the sliding window of its
// local-attention section.
//
// Shared prefix.  Every sequence of a decode batch maps its first P logical
// pages to the same physical pages (a prefix hit binds a new sequence's block
// table to existing pages, "Building and Deploying vllm.cpp", Step 3).  The
// decode queries of all sequences (one row per sequence and query head) are
// scored against those pages together, so each shared page is read once per
// kv-head instead of once per sequence; the result is a (max, sum, output)
// partial per row and split of the prefix, merged later with the rest of the
// sequence by the log-sum-exp rule.
//
// The pages give no kernel design; this one is built for CDNA4.
//
// Work: a workgroup takes 128 query rows, 32 per wave, and one kv-head: in
// prefill TQ = 128 / g consecutive tokens of one sequence times the g query
// heads; for the shared prefix 128 consecutive (sequence, query head) rows
// and one split of the prefix pages.  Every row has its own kept key range
// [lo, hi); the workgroup walks the union of its rows' ranges in blocks of 32
// keys (two 16-token pages), staged through LDS once for its four waves.
// 16-bit pages at D = 128 in prefill go from HBM straight into LDS (buffer
// loads that write LDS, no registers on the way), two blocks ahead of the
// block being computed, in three LDS stages; the layouts are given where that
// loop is.  The other tiles (FP8 pages, D = 64, the shared prefix, which runs
// beside the decode in one grid and shares its LDS budget) stage through
// registers, one block ahead:
//  * K block row-major ([key][D], rows padded by 16 bytes);
//  * V block row-major as well (rows padded by 32 bytes), staged exactly like
//    K; the P.V operand of a lane is two transposing 8-byte reads
//    (ds_read_b64_tr_b16), each giving 4 consecutive keys at the lane's own d.
//    The padding puts the four rows one read touches in distinct banks.
//  FP8 pages (E4M3 or E5M2) are converted exactly to q's 16-bit format when
//  staged.
// Per block and wave, on v_mfma_f32_32x32x16 (bf16 or f16, fp32 accumulate):
//  * S^T = K Q^T: the output column of a lane is its query row, so each lane
//    holds 16 scores of one row (keys 8j + 4h + i, h = lane / 32);
//  * online softmax per row in fp32 (log2 domain), the two half-waves of a
//    row combined with one lane exchange; the running max only moves when a
//    score exceeds it by more than 2^8;
//  * P is rounded to q's 16-bit format (the row sums, on v_dot2 against
//    ones, use the rounded values) and used in place as the B operand of
//    O^T += V^T P^T: the contraction over keys follows the same key order in
//    both operands, so no transpose of P is needed and O^T keeps each query
//    row in one lane as well.
// Keys past every row's range (page tails, padding pages) are staged as zeros
// and masked, and their block-table entries are never read.
#pragma once

#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace vp {
namespace tile {

constexpr int kPW = 4;                 // waves per workgroup
constexpr int kRows = 32 * kPW;        // query rows per workgroup
constexpr int kBK = 32;                // keys per block
constexpr float kTauP = 8.0f;          // rescale headroom, log2 units
// Word 3 of a raw buffer resource on gfx9-family GPUs: 32-bit data format,
// no swizzle, no thread-id offset.
constexpr int kBufferFlags = 0x00020000;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

template <int QF>
__device__ __forceinline__ f32x16_t mfma32(uint4 a, uint4 b, f32x16_t c) {
  if constexpr (QF == kBF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(bitcast<bf16x8_t>(a), bitcast<bf16x8_t>(b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(bitcast<f16x8_t>(a), bitcast<f16x8_t>(b), c, 0, 0, 0);
}

template <int QF>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  if constexpr (QF == kBF16) {
    bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return bitcast<uint32_t>(v);
  } else {
    half2_t v = {(_Float16)lo, (_Float16)hi};
    return bitcast<uint32_t>(v);
  }
}

// a.lo * b.lo + a.hi * b.hi + c with fp32 accumulation.
template <int QF>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  if constexpr (QF == kF16)
    return __builtin_amdgcn_fdot2(bitcast<half2_t>(a), bitcast<half2_t>(b), c, false);
  else
    return __builtin_amdgcn_fdot2_f32_bf16(bitcast<bf16x2_t>(a), bitcast<bf16x2_t>(b), c, false);
}

// Max of x over lanes l and l ^ 32 (v_permlane32_swap exchanges the halves).
__device__ __forceinline__ float half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(bitcast<uint32_t>(x), bitcast<uint32_t>(x), false, false);
  return __builtin_elementwise_maximum(bitcast<float>((uint32_t)r[0]), bitcast<float>((uint32_t)r[1]));
}

// Raw pool data of one 8-element chunk: 16 bytes for 16-bit pools, 8 for FP8.
template <int KF> struct Raw { using T = uint4; };
template <> struct Raw<kE4M3> { using T = uint2; };
template <> struct Raw<kE5M2> { using T = uint2; };

// The chunk as 8 values of q's 16-bit format (FP8 codes converted exactly).
template <int KF, int QF>
__device__ __forceinline__ uint4 to_q16(const typename Raw<KF>::T& x) {
  if constexpr (!is_fp8(KF)) {
    return x;
  } else {
    return make_uint4(fp8x2_to_q16<KF, QF, false>(x.x), fp8x2_to_q16<KF, QF, true>(x.x),
                      fp8x2_to_q16<KF, QF, false>(x.y), fp8x2_to_q16<KF, QF, true>(x.y));
  }
}

// PFX = false: chunked prefill, normalized output rows.  PFX = true: shared
// prefix, (max, sum, normalized output) partials per row and split.
// b: the workgroup's index in the grid of tiles (the kernels pass blockIdx.x,
// or its offset in a grid shared with the decode).
template <int D, int QF, int KF, bool PFX>
__device__ __forceinline__ void attn_tile_body(const PrefillParams& p, const int b) {
  static_assert(D == 64 || D == 128, "head_dim 64 or 128");
  constexpr int CH = D / 8;                    // 8-element chunks per K/V row
  constexpr int KS = D / 16;                   // k-steps of S^T = K Q^T (16 values of d each)
  constexpr int KPT = CH / 8;                  // K chunks a thread stages per block (2 or 1)
  constexpr int EB = is_fp8(KF) ? 1 : 2;       // bytes per pool element
  constexpr int KROW = D * 2 + 16;             // bytes per LDS K row
  constexpr int VROW = D * 2 + 32;             // bytes per LDS V row (bank offset 8 per row)
  constexpr int KBUF = kBK * KROW;             // bytes per K buffer
  constexpr int VBUF = kBK * VROW;             // bytes per V buffer
  constexpr int64_t kPageBytes = 16 * D * EB;
  using RawT = typename Raw<KF>::T;
  static_assert(kPW * 64 * KPT == 32 * CH, "staging map: K chunks of a block over the threads");
  // Direct path (HBM -> LDS) for 16-bit pages at D = 128 in prefill; the
  // register-staged buffers shrink to placeholders there.
  constexpr bool DMA = !PFX && !is_fp8(KF) && D == 128;
  __shared__ __attribute__((aligned(16))) uint8_t s_k[DMA ? 1 : 2][DMA ? 16 : KBUF];
  __shared__ __attribute__((aligned(16))) uint8_t s_v[DMA ? 1 : 2][DMA ? 16 : VBUF];
  // direct path: three stages of 16 KiB (K at +0, V at +8 KiB)
  __shared__ __attribute__((aligned(16))) uint8_t d_s0[DMA ? 16384 : 16], d_s1[DMA ? 16384 : 16],
      d_s2[DMA ? 16384 : 16];
  __shared__ int s_red[PFX ? 3 * kPW : 1];    // per-wave row bounds (shared prefix)

  const int g = p.group;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 31, hf = lane >> 5;
  const int row = wave * 32 + col;             // this lane's query row in the workgroup

  // Workgroup -> (pair u, tile).  Workgroups go to the 8 XCDs round-robin;
  // pair u runs on XCD u % 8 with all its tiles, which read the same K/V
  // (they share it in that XCD's L2), and the XCDs get even work.  Later
  // tiles attend to more keys (prefill) and are dispatched first.
  //   prefill: u = (sequence, kv-head), tiles of TQ tokens;
  //   shared prefix: u = (kv-head, split), tiles of 128 (sequence, head) rows.
  // A prefill with a tile order takes entry b / 8 of list b % 8 instead
  // (sorted pairs, still one XCD per pair, no empty tiles in between).
  const int ntiles = p.num_tiles;
  const int npairs = PFX ? p.num_kv_heads * p.num_splits : p.num_seqs * p.num_kv_heads;
  const int xcd = b % 8, kk = b / 8;
  int u = (kk / ntiles) * 8 + xcd;
  int tile = ntiles - 1 - (kk % ntiles);
  if constexpr (!PFX) {
    if (p.plan) {
      if (kk >= p.plan_stride) return;
      const int2 e = p.plan[(int64_t)xcd * p.plan_stride + kk];
      if (e.x < 0) return;
      u = e.x;
      tile = e.y;
    }
  }
  if (u >= npairs) return;

  int hk, seq_tbl;                             // kv-head, sequence whose table is read
  int key_begin, key_end;                      // keys of this workgroup, before row ranges
  int r_lo, r_hi;                              // this row's kept keys [r_lo, r_hi)
  int max_lo = 0, min_hi = 0;                  // over the workgroup's rows (see below)
  bool row_ok;
  bool wave_on;                                // some row of this wave is valid (uniform)
  int64_t q_off;                               // element offset of this row in q (and out)
  int split = 0;
  if constexpr (!PFX) {
    const int s = u / p.num_kv_heads;
    hk = u - s * p.num_kv_heads;
    seq_tbl = s;
    const int tq = kRows / g;                  // query tokens per workgroup
    // (clamped to the rows of q, so that no value of query_start_loc leads
    // outside q / out)
    const int q_begin = min(max(p.query_start_loc[s], 0), p.num_tokens);
    const int Qs = min(max(p.query_start_loc[s + 1], q_begin), p.num_tokens) - q_begin;
    const int q0 = tile * tq;
    if (q0 >= Qs) return;
    const int nt = min(tq, Qs - q0);           // tokens of this tile
    const int n = min(p.context_lens[s], p.bt_stride * 16);
    const int pos0 = n - Qs + q0;              // position of the tile's first token
    row_ok = row < nt * g;
    wave_on = __builtin_amdgcn_readfirstlane(wave * 32 < nt * g);
    const int tok = min(row, nt * g - 1) / g;
    const int head = min(row, nt * g - 1) - tok * g;
    const int ppos = pos0 + tok;               // query position of the row
    r_hi = ppos + 1;
    r_lo = p.window > 0 ? max(0, ppos - p.window + 1) : 0;
    key_begin = p.window > 0 ? max(0, pos0 - p.window + 1) : 0;
    key_end = pos0 + nt;
    // the rows are the positions pos0 .. pos0 + nt - 1 (each for g heads): the
    // largest lower bound is the last token's, the smallest upper the first's
    max_lo = p.window > 0 ? max(0, pos0 + nt - p.window) : 0;
    min_hi = pos0 + 1;
    q_off = ((int64_t)(q_begin + q0 + tok) * p.num_q_heads + hk * g + head) * D;
  } else {
    hk = u / p.num_splits;
    split = u - hk * p.num_splits;
    seq_tbl = 0;                               // the shared pages, as sequence 0 maps them
    key_begin = split * p.split_pages * 16;
    key_end = min(p.shared_pages, (split + 1) * p.split_pages) * 16;
    const int rows_total = p.num_seqs * g;
    if (tile * kRows >= rows_total) return;
    const int rg = tile * kRows + row;
    row_ok = rg < rows_total;
    wave_on = __builtin_amdgcn_readfirstlane(tile * kRows + wave * 32 < rows_total);
    const int rgc = min(rg, rows_total - 1);
    const int s = rgc / g;
    const int head = rgc - s * g;
    const int n = min(p.context_lens[s], p.bt_stride * 16);
    const int lo = p.window > 0 ? max(0, n - p.window) : 0;
    r_lo = max(lo, key_begin);
    r_hi = min(n, key_end);
    q_off = ((int64_t)s * p.num_q_heads + hk * g + head) * D;
  }

  // Q operand: lane (row, hf) holds d = D/2 hf + 8 t + i for k-step t.  The
  // loads are in flight during the setup below (block ids, the first loads,
  // the shared prefix's row bounds) and waited for at its end: once that wait has been seen, the block loop need not wait for them (the
  // memory counter cannot tell them from the next block's loads, so an
  // in-loop wait for Q would wait for those every block).
  uint4 qr[KS];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(p.q) + q_off + (D / 2) * hf;
#pragma unroll
    for (int t = 0; t < KS; ++t) qr[t] = *reinterpret_cast<const uint4*>(qp + 8 * t);
  }

  const int32_t* bt = p.block_tables + (int64_t)seq_tbl * p.bt_stride;
  const uint8_t* kpool = static_cast<const uint8_t*>(p.k_cache) + (int64_t)hk * kPageBytes;
  const uint8_t* vpool = static_cast<const uint8_t*>(p.v_cache) + (int64_t)hk * kPageBytes;
  const int64_t blk_stride = (int64_t)p.num_kv_heads * kPageBytes;
  // Keys of the block walk.  In prefill every row's range ends at or below
  // key_end and the tile's last row reaches it, so n_valid = key_end; the
  // shared prefix takes it from the reduction of its rows' bounds below.
  int n_valid = key_end;
  int kb0 = (key_begin / kBK) * kBK;
  int nblk = n_valid > key_begin ? ((n_valid - 1) / kBK - kb0 / kBK + 1) : 0;
  // Staging map (256 threads, one block = pages A and B of 16 rows), the same
  // for K and V: thread i stages chunk i % CH of block row i / CH and, for
  // D = 128, of the same row of page B as well (block row + 16); for D = 64
  // the waves 2 and 3 take page B.
  const int k_r = threadIdx.x / CH, k_c = threadIdx.x % CH;     // k_r: block row (D = 64) or page row
  const uint32_t k_off = (uint32_t)((k_r & 15) * (D * EB) + k_c * 8 * EB);
  const bool k_pgB = wave >= 2;                // (D = 64) rows 16..31: page B, uniform per wave
  // Block ids: uniform over the workgroup, read through the constant address
  // space (scalar loads, counted apart from the K/V loads) and clamped where
  // they are used, so that no wait for them also waits for later K/V loads.
  typedef const int32_t __attribute__((address_space(4)))* const_i32p;
  const const_i32p bt_s = (const_i32p)bt;
  auto page_blk = [&](int j) __attribute__((always_inline)) {
    int blk = 0;
    if (j * 16 < n_valid) blk = bt_s[j];
    return blk;
  };
  auto clamp_blk = [&](int blk) __attribute__((always_inline)) {
    return (unsigned)blk < (unsigned)p.num_blocks ? blk : 0;
  };
  // Direct path: the loads of one block into a stage (see the block loop)
  typedef __attribute__((address_space(3))) void* lds_ptr;
  const int l16 = lane & 15, lq = lane >> 4;
  const int dpage = wave >> 1;                 // the page this wave loads (uniform)
  const int dhalf = wave & 1;
  const int k_dma = l16 * 256 + lq * 16;       // + 16 c0
  const int v_dma = lq * 256 + ((l16 ^ (4 * lq)) * 16);   // + 256 R0
  auto dma = [&](uint8_t* dk, uint8_t* dv, int ida, int idb, int kb) __attribute__((always_inline)) {
    const int id = __builtin_amdgcn_readfirstlane(clamp_blk(dpage ? idb : ida));
    const uint64_t pg = (uint64_t)(uint32_t)id * (uint64_t)blk_stride;
    // (clamped in two steps: as one min-max the compiler forms a vector med3)
    const int rows = __builtin_amdgcn_readfirstlane(max(n_valid - (kb + 16 * dpage), 0));
    const int bytes = min(rows, 16) * 256;
    __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(kpool + pg), (short)0, bytes, kBufferFlags);
    __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(vpool + pg), (short)0, bytes, kBufferFlags);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c0 = 8 * dhalf + 4 * i;        // K chunks of this load
      const int r0 = 8 * dhalf + 4 * i;        // V rows of this load
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_ptr)(dk + dpage * 4096 + c0 * 256), 16,
                                               k_dma, c0 * 16, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_ptr)(dv + (16 * dpage + r0) * 256), 16,
                                               v_dma, r0 * 256, 0, 0);
    }
  };
  // the block ids of a block, read a block before its loads
  auto ids_of = [&](int (&ids)[2], int kb) __attribute__((always_inline)) {
    ids[0] = page_blk(kb >> 4);
    ids[1] = page_blk((kb >> 4) + 1);
  };
  auto kb_of = [&](int bi) __attribute__((always_inline)) {
    return kb0 + max(min(bi, nblk - 1), 0) * kBK;
  };
  int ids[2] = {0, 0};

  // Over the workgroup's rows: the largest lower and the smallest and largest
  // upper bounds.  A block inside every row's range needs no per-key mask;
  // keys at or past every row's range are staged as zeros.  Prefill takes
  // them from its first and last token (above).  Shared-prefix rows belong to
  // different sequences: each wave reduces its rows by lane exchanges (both
  // half-waves hold the same rows), then the waves' bounds meet in LDS.
  if constexpr (PFX) {
    int a = row_ok ? r_lo : INT32_MIN, m = row_ok ? r_hi : INT32_MAX, x = row_ok ? r_hi : INT32_MIN;
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) {
      a = max(a, __shfl_xor(a, o));
      m = min(m, __shfl_xor(m, o));
      x = max(x, __shfl_xor(x, o));
    }
    if (lane == 0) {
      s_red[3 * wave] = a;
      s_red[3 * wave + 1] = m;
      s_red[3 * wave + 2] = x;
    }
    __syncthreads();
    int max_hi = INT32_MIN;
    max_lo = INT32_MIN;
    min_hi = INT32_MAX;
#pragma unroll
    for (int w = 0; w < kPW; ++w) {
      max_lo = max(max_lo, s_red[3 * w]);
      min_hi = min(min_hi, s_red[3 * w + 1]);
      max_hi = max(max_hi, s_red[3 * w + 2]);
    }
    max_lo = __builtin_amdgcn_readfirstlane(max_lo);
    min_hi = __builtin_amdgcn_readfirstlane(min_hi);
    n_valid = min(key_end, __builtin_amdgcn_readfirstlane(max_hi));
    nblk = n_valid > key_begin ? ((n_valid - 1) / kBK - kb0 / kBK + 1) : 0;
  }
  if constexpr (DMA) {
    // blocks 0 and 1, unconditionally (with no block the loads have size 0)
    int i0[2], i1[2];
    ids_of(i0, kb_of(0));
    ids_of(i1, kb_of(1));
    dma(d_s0, d_s0 + 8192, i0[0], i0[1], kb_of(0));
    dma(d_s1, d_s1 + 8192, i1[0], i1[1], kb_of(1));
    ids_of(ids, kb_of(2));
    __builtin_amdgcn_s_waitcnt(0x0F78);        // vmcnt(8): the Q loads (blocks 0 and 1 may fly)
  } else {
    __builtin_amdgcn_s_waitcnt(0);             // (the Q loads)
  }

  // Loads are unconditional (rows at or past n_valid are replaced by zeros
  // when written to LDS) so that nothing waits on them before the LDS write.
  // (the two block ids of a block are read one block ahead of its K/V)
  // K and V rows take the same map: each page is read through a buffer
  // resource of its own (base and size in scalar registers, the size one
  // page, so the hardware bounds every access to it) with the lane offset
  // k_off: no 64-bit vector arithmetic per load.
  auto page_load = [&](const uint8_t* page) __attribute__((always_inline)) {
    __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(page), (short)0, (int)kPageBytes, kBufferFlags);
    if constexpr (sizeof(RawT) == 16) {
      return bitcast<RawT>(__builtin_amdgcn_raw_buffer_load_b128(r, (int)k_off, 0, 0));
    } else {
      return bitcast<RawT>(__builtin_amdgcn_raw_buffer_load_b64(r, (int)k_off, 0, 0));
    }
  };
  auto fetch = [&](RawT (&kr)[KPT], RawT (&vr)[KPT], int ida, int idb) __attribute__((always_inline)) {
    const int64_t pa = (int64_t)__builtin_amdgcn_readfirstlane(clamp_blk(ida)) * blk_stride;
    const int64_t pb = (int64_t)__builtin_amdgcn_readfirstlane(clamp_blk(idb)) * blk_stride;
    if constexpr (KPT == 2) {
      kr[0] = page_load(kpool + pa);
      kr[1] = page_load(kpool + pb);
      vr[0] = page_load(vpool + pa);
      vr[1] = page_load(vpool + pb);
    } else {
      const int64_t pg = k_pgB ? pb : pa;
      kr[0] = page_load(kpool + pg);
      vr[0] = page_load(vpool + pg);
    }
  };
  auto masked = [](uint4 x, bool keep) __attribute__((always_inline)) {
    const uint32_t m = keep ? 0xFFFFFFFFu : 0u;    // value-level select (no pointer select)
    return make_uint4(x.x & m, x.y & m, x.z & m, x.w & m);
  };
  auto stage = [&](int buf, const RawT (&kr)[KPT], const RawT (&vr)[KPT], int kb)
      __attribute__((always_inline)) {
    const bool crossing = kb + kBK > n_valid;  // block crossing n_valid: zero the rows past it
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int r = k_r + 16 * j;              // block row
      uint4 kx = to_q16<KF, QF>(kr[j]), vx = to_q16<KF, QF>(vr[j]);
      if (crossing) {
        kx = masked(kx, kb + r < n_valid);
        vx = masked(vx, kb + r < n_valid);
      }
      *reinterpret_cast<uint4*>(&s_k[buf][r * KROW + k_c * 16]) = kx;
      *reinterpret_cast<uint4*>(&s_v[buf][r * VROW + k_c * 16]) = vx;
    }
  };

  constexpr uint32_t kOnes = QF == kBF16 ? 0x3F803F80u : 0x3C003C00u;   // (1, 1)
  f32x16_t o[D / 32];
#pragma unroll
  for (int m = 0; m < D / 32; ++m) o[m] = f32x16_t{};
  float mrow = -INFINITY, lsum = 0.0f;
  // scale * log2(e), times the K scale of this kv-head for FP8 pools
  const float c = p.k_scales ? p.score_base * p.k_scales[hk] : p.score_scale;
  const float inv_c = 1.0f / c;
  float thr = -INFINITY;                       // (mrow + kTauP) / c: compared with raw scores
  float nmu = 0.0f;                            // -mrow (0 while mrow is -inf)

  // One block: S^T, online softmax, O^T update.  buf holds the block's K and
  // V^T.  Lane reads: K rows col (16 bytes at d = D/2 hf + 8 t), V^T rows
  // d = 32 m + col (8 bytes at key pairs 8 kap + 2 hf and + 4).
  const uint8_t* k_rd = &s_k[0][col * KROW + D * hf];
  // V operand of O^T += V^T P^T by transposing LDS reads: in each 16-lane
  // group (d = 16 (g % 2) + i, key half kh = g / 2) lane i addresses row
  // 4 kh + i / 4, columns 16 (g % 2) + 4 (i % 4) .. + 3, and receives the
  // 4 keys of that half at its own d.
  const int vg = lane >> 4, vi = lane & 15;
  const uint8_t* v_rd = &s_v[0][(4 * (vg >> 1) + (vi >> 2)) * VROW + (16 * (vg & 1) + 4 * (vi & 3)) * 2];
  // Online softmax of one block's scores (row = col; this lane holds keys
  // 8j + 4hf + i): masks, running maximum, rescale, weights pw, row sum.
  auto softmax = [&](const f32x16_t& sacc, int kb, uint32_t (&pw)[8]) __attribute__((always_inline)) {
    // Scores stay unscaled up to the exponent (scale > 0: max(c s) = c max(s)),
    // which is then one fma per score: exp2(c s - m).
    float sc[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) sc[k] = sacc[k];
    const bool edge = kb < max_lo || kb + kBK > min_hi;
    if (edge) {
      asm volatile("");                        // keep this a branch (rarely taken)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = kb + 8 * j + 4 * hf + i;
          if (t < r_lo || t >= r_hi) sc[4 * j + i] = -INFINITY;
        }
    }
    // (the NaN-propagating maximum is v_maximum3_f32 with no canonicalising
    // of its operands; the raw maximum is compared with the threshold
    // (mrow + tau) / c, which only changes with mrow.  A row's two half-waves
    // each test their own 16 scores: the row needs a new maximum exactly when
    // one of them does, so the exchange of the halves' maxima waits for that.)
    float mx = sc[0];
#pragma unroll
    for (int k = 1; k < 16; ++k) mx = __builtin_elementwise_maximum(mx, sc[k]);
    if (__any(mx > thr)) {
      mx = half_max(mx);                       // the row's 32 scores
      const bool need = mx > thr;
      const float mn = need ? fmaxf(mrow, mx * c) : mrow;
      const float alpha = (mrow == -INFINITY) ? 0.0f : fast_exp2(mrow - mn);
      mrow = mn;
      thr = (mrow + kTauP) * inv_c;
      nmu = (mrow == -INFINITY) ? 0.0f : -mrow;
      lsum *= alpha;
#pragma unroll
      for (int m = 0; m < D / 32; ++m)
#pragma unroll
        for (int k = 0; k < 16; ++k) o[m][k] *= alpha;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      pw[k] = pack2<QF>(fast_exp2(fmaf(sc[2 * k], c, nmu)), fast_exp2(fmaf(sc[2 * k + 1], c, nmu)));
      lsum = dot2<QF>(pw[k], kOnes, lsum);       // row sum of the rounded weights
    }

  };

  auto block = [&](int buf, int kb) __attribute__((always_inline)) {
    // ---- S^T = K Q^T ----
    uint4 ka[KS];
#pragma unroll
    for (int t = 0; t < KS; ++t) ka[t] = *reinterpret_cast<const uint4*>(k_rd + buf * KBUF + 16 * t);
    f32x16_t sacc = f32x16_t{};
#pragma unroll
    for (int t = 0; t < KS; ++t) sacc = mfma32<QF>(ka[t], qr[t], sacc);

    uint32_t pw[8];
    softmax(sacc, kb, pw);

    // ---- O^T += V^T P^T ----
    typedef short v4i16_t __attribute__((ext_vector_type(4)));
    typedef v4i16_t __attribute__((address_space(3)))* lds_v4p;
    const uint8_t* vb = v_rd + buf * VBUF;
#pragma unroll
    for (int kap = 0; kap < 2; ++kap) {
      const uint4 pb = make_uint4(pw[4 * kap], pw[4 * kap + 1], pw[4 * kap + 2], pw[4 * kap + 3]);
#pragma unroll
      for (int m = 0; m < D / 32; ++m) {
        // keys 16 kap + 4 kh .. + 3 and 16 kap + 8 + 4 kh .. + 3 at d = 32 m + col
        const uint8_t* vr = vb + 16 * kap * VROW + 64 * m;
        const v4i16_t a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4p)(vr));
        const v4i16_t a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4p)(vr + 8 * VROW));
        const uint2 u0 = bitcast<uint2>(a0), u1 = bitcast<uint2>(a1);
        o[m] = mfma32<QF>(make_uint4(u0.x, u0.y, u1.x, u1.y), pb, o[m]);
      }
    }
  };

  if constexpr (!DMA) {
  // ---- register staging (FP8 pools, D = 64, shared-prefix tiles) ----
  // The barriers order the LDS buffers only, so the K/V loads of the next
  // block stay in flight across them.
  auto lds_barrier = []() __attribute__((always_inline)) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  };
  // Block bi + 1 is fetched into registers while block bi is computed, then
  // written to the other LDS buffer.  (A single-block loop body keeps the
  // accumulators in place; unrolling by two made the compiler copy them.)
  RawT kr[KPT], vr[KPT];
  int ida = 0, idb = 0;                        // block ids of the block fetched next
  if (nblk > 0) {
    fetch(kr, vr, page_blk(kb_of(0) >> 4), page_blk((kb_of(0) >> 4) + 1));
    ida = page_blk(kb_of(1) >> 4);
    idb = page_blk((kb_of(1) >> 4) + 1);
    stage(0, kr, vr, kb_of(0));
  }
  lds_barrier();
  for (int bi = 0; bi < nblk; ++bi) {
    const int buf = bi & 1;
    const int na = page_blk(kb_of(bi + 2) >> 4);
    const int nb = page_blk((kb_of(bi + 2) >> 4) + 1);
    fetch(kr, vr, ida, idb);                   // (past the end: re-reads the last block)
    ida = na;
    idb = nb;
    __builtin_amdgcn_sched_barrier(0);
    if (wave_on) block(buf, kb0 + bi * kBK);   // (a wave of padding rows only stages)
    __builtin_amdgcn_sched_barrier(0);
    stage(buf ^ 1, kr, vr, kb_of(bi + 1));
    lds_barrier();
  }

  } else {
    // ---- direct loads into LDS (16-bit pools, D = 128, prefill) ----
    // Each wave issues four buffer loads into LDS per block (K
    // and V, two 1 KiB pieces each), two blocks ahead of the one computed, into
    // three stages of 16 KiB (K at +0, V at +8 KiB).  Every page's resource is
    // sized to its valid rows, so rows at or past n_valid arrive as zeros.
    //  K stage: [page][chunk (16 B)][row] -- load i of wave w covers chunks
    //    8 (w & 1) + 4 i .. + 3 of page w >> 1, lane l chunk + l / 16, row l % 16;
    //    the score operand of lane (col, hf) at k-step t is then at a fixed
    //    lane offset + 256 t, and 16 lanes read 256 contiguous bytes.
    //  V stage: row-major [32 rows][16 chunks], chunk c of row r at position
    //    c ^ 4 (r % 4) -- load i of wave w covers rows 8 (w & 1) + 4 i .. + 3
    //    of page w >> 1; the transposing reads of two 16-lane groups then hit
    //    64 distinct banks.
    const int kbase = (col >> 4) * 4096 + 8 * hf * 256 + (col & 15) * 16;
    const int vgq = lane >> 4, vj = (lane & 15) >> 2;
    const int vrow = (4 * (vgq >> 1) + vj) * 256 + 32 * (vgq & 1) + 8 * (lane & 3);
    int vb[D / 32];
#pragma unroll
    for (int m = 0; m < D / 32; ++m) vb[m] = vrow + 64 * (m ^ vj);
    typedef short v4i16_t __attribute__((ext_vector_type(4)));
    typedef v4i16_t __attribute__((address_space(3)))* lds_v4p;
    auto block_dma = [&](const uint8_t* dk, const uint8_t* dv, int kb) __attribute__((always_inline)) {
      uint4 ka[KS];
#pragma unroll
      for (int t = 0; t < KS; ++t) ka[t] = *reinterpret_cast<const uint4*>(dk + kbase + 256 * t);
      f32x16_t sacc = f32x16_t{};
#pragma unroll
      for (int t = 0; t < KS; ++t) sacc = mfma32<QF>(ka[t], qr[t], sacc);
      uint32_t pw[8];
      softmax(sacc, kb, pw);
#pragma unroll
      for (int kap = 0; kap < 2; ++kap) {
        const uint4 pb = make_uint4(pw[4 * kap], pw[4 * kap + 1], pw[4 * kap + 2], pw[4 * kap + 3]);
#pragma unroll
        for (int m = 0; m < D / 32; ++m) {
          const uint8_t* vr = dv + vb[m] + 16 * kap * 256;
          const v4i16_t a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4p)(vr));
          const v4i16_t a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4p)(vr + 8 * 256));
          const uint2 u0 = bitcast<uint2>(a0), u1 = bitcast<uint2>(a1);
          o[m] = mfma32<QF>(make_uint4(u0.x, u0.y, u1.x, u1.y), pb, o[m]);
        }
      }
    };
    // A barrier that the compiler keeps in place for memory operations but
    // that waits for nothing by itself: the waits are explicit.
    auto raw_barrier = []() __attribute__((always_inline)) {
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    };
    // step of block bi in stage S: its loads done (the next block's four may
    // still fly), this wave's reads of the stage loaded next done; barrier;
    // the loads of block bi + 2 into the stage block bi - 1 used; compute.
    // Every step issues exactly four loads, which keeps the vmcnt(4) exact,
    // and the loop runs whole rounds of three: the steps past the last block
    // only load (the last block again) and wait.  Skipping whole steps
    // instead puts branches between the loads and the reads of a stage, and
    // at those joins the compiler's wait insertion no longer tells the three
    // stages apart: it then waits for the next block's loads as well before
    // the K reads, which leaves a single block in flight.
    auto step = [&](auto S, int bi) __attribute__((always_inline)) {
      constexpr int s = decltype(S)::value;
      uint8_t* dk = s == 0 ? d_s0 : s == 1 ? d_s1 : d_s2;
      uint8_t* dv = dk + 8192;
      uint8_t* nk = s == 0 ? d_s2 : s == 1 ? d_s0 : d_s1;
      uint8_t* nv = nk + 8192;
      __builtin_amdgcn_s_waitcnt(0x0074);       // vmcnt(4) lgkmcnt(0)
      raw_barrier();
      dma(nk, nv, ids[0], ids[1], kb_of(bi + 2));
      ids_of(ids, kb_of(bi + 3));
      if (bi < nblk && wave_on) block_dma(dk, dv, kb0 + bi * kBK);   // (padding waves: loads only)
    };
    for (int bo = 0; bo < nblk; bo += 3) {
      step(std::integral_constant<int, 0>{}, bo);
      step(std::integral_constant<int, 1>{}, bo + 1);
      step(std::integral_constant<int, 2>{}, bo + 2);
    }
    __builtin_amdgcn_s_waitcnt(0x0070);         // vmcnt(0): no load into LDS outlives the workgroup
  }

  // ---- finalize: row values at d = 32 m + 8 j + 4 hf + i ----
  const float lt = lsum + __shfl_xor(lsum, 32);
  const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
  if (!row_ok) return;
  if constexpr (!PFX) {
    // FP8 pools: the V scale (per tensor or per kv-head) applies once here
    const float w = inv * (p.v_scales ? p.v_scales[hk] : p.out_scale);
    uint16_t* op = static_cast<uint16_t*>(p.out) + q_off + 4 * hf;
#pragma unroll
    for (int m = 0; m < D / 32; ++m)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int k = 4 * j;
        const uint32_t w0 = (uint32_t)f32_to_16<QF>(o[m][k] * w) |
                            ((uint32_t)f32_to_16<QF>(o[m][k + 1] * w) << 16);
        const uint32_t w1 = (uint32_t)f32_to_16<QF>(o[m][k + 2] * w) |
                            ((uint32_t)f32_to_16<QF>(o[m][k + 3] * w) << 16);
        *reinterpret_cast<uint2*>(op + 32 * m + 8 * j) = make_uint2(w0, w1);
      }
  } else {
    // partial rows [split][sequence][query head]; an empty row stores
    // (-inf, 0, 0), which the merge weighs 0
    const int64_t pr = (int64_t)split * p.num_seqs * p.num_q_heads + q_off / D;
    float* op = p.pfx_o + pr * D + 4 * hf;
#pragma unroll
    for (int m = 0; m < D / 32; ++m)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int k = 4 * j;
        *reinterpret_cast<float4*>(op + 32 * m + 8 * j) =
            make_float4(o[m][k] * inv, o[m][k + 1] * inv, o[m][k + 2] * inv, o[m][k + 3] * inv);
      }
    if (hf == 0) {
      p.pfx_m[pr] = lt > 0.0f ? mrow : -INFINITY;
      p.pfx_l[pr] = lt;
    }
  }
}

}  // namespace tile
}  // namespace vp

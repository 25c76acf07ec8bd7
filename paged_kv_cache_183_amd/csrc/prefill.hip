// Chunked-prefill attention on the matrix cores of gfx950.  Sequence s has
// Q_s new query tokens at positions n - Q_s .. n - 1 of its n cached tokens
// (their K/V are already in the block-paged pool); the query row at position
// p attends to keys t <= p with t > p - window (window 0: no lower bound).
// This is the paged attention of the vllm.cpp model forward (repository
// listing, "What's implemented") for a chunk of several query tokens, with
// the sliding window of its local-attention section; the pages give no kernel
// design, this one is built for CDNA4.
//
// Work: a workgroup takes TQ = 128 / g consecutive query tokens of one
// sequence and the g query heads of one kv-head: 128 rows, 32 per wave.  It
// walks the kept keys in blocks of 32 (two 16-token pages), staged through
// LDS once for its four waves:
//  * K block row-major ([key][D], rows padded by 16 bytes);
//  * V block transposed ([D][key pair], rows padded to 18 dwords), so that
//    the P.V operand of a lane is two 8-byte reads; the staging writes and
//    these reads hit distinct banks.
// Global loads run two blocks ahead of the matrix cores.
// Per block and wave, on v_mfma_f32_32x32x16 (bf16 or f16, fp32 accumulate):
//  * S^T = K Q^T: the output column of a lane is its query row, so each lane
//    holds 16 scores of one row (keys 8j + 4h + i, h = lane / 32);
//  * online softmax per row in fp32 (log2 domain), the two half-waves of a
//    row combined with one lane exchange; the running max only moves when a
//    score exceeds it by more than 2^8;
//  * P is rounded to q's 16-bit format (the row sums, on v_dot2 against
//    ones, use the rounded values)
//    and used in place as the B operand of O^T += V^T P^T: the contraction
//    over keys follows the same key order in both operands, so no transpose
//    of P is needed and O^T keeps each query row in one lane as well.
// Keys at or past n (page tails, padding pages) are staged as zeros and
// masked, and their block-table entries are never read.
#include "common.h"
#include "kernels.h"

namespace vp {

namespace {

constexpr int kPW = 4;                 // waves per workgroup
constexpr int kRows = 32 * kPW;        // query rows (token, head) per workgroup
constexpr int kBK = 32;                // keys per block
constexpr float kTauP = 8.0f;          // rescale headroom, log2 units

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
  return fmaxf(bitcast<float>((uint32_t)r[0]), bitcast<float>((uint32_t)r[1]));
}

}  // namespace

template <int D, int QF>
__global__ __launch_bounds__(kPW * 64) void prefill_kernel(PrefillParams p) {
  static_assert(D == 128, "head_dim 128");
  constexpr int CH = D / 8;                    // 16-byte chunks per K/V row
  constexpr int KROW = D * 2 + 16;             // bytes per LDS K row
  constexpr int VROWW = kBK / 2 + 2;           // dwords per LDS V^T row (18)
  constexpr int KBUF = kBK * KROW;             // bytes per K buffer
  constexpr int VBUF = D * VROWW * 4;          // bytes per V^T buffer
  constexpr int64_t kPageBytes = 16 * D * 2;
  static_assert(kPW * 64 == 16 * CH, "staging map: one thread per (row-of-page, chunk)");
  __shared__ __attribute__((aligned(16))) uint8_t s_k[2][KBUF];
  __shared__ __attribute__((aligned(16))) uint32_t s_v[2][VBUF / 4];

  const int g = p.group;
  const int tq = kRows / g;                    // query tokens per workgroup
  // Workgroup -> (sequence, kv-head, token tile).  Workgroups go to the 8
  // XCDs round-robin; (sequence, kv-head) pair u runs on XCD u % 8 with all
  // its tiles (they share K/V in that XCD's L2), so every XCD sees every
  // sequence and the XCDs get even work.  Later tiles attend to more keys and
  // are dispatched first.
  const int ntiles = p.num_tiles;
  const int b = blockIdx.x;
  const int xcd = b % 8, k = b / 8;
  const int u = (k / ntiles) * 8 + xcd;
  if (u >= p.num_seqs * p.num_kv_heads) return;
  const int tile = ntiles - 1 - (k % ntiles);
  const int s = u / p.num_kv_heads;
  const int hk = u - s * p.num_kv_heads;

  // (clamped to the rows of q, so that no value of query_start_loc leads
  // outside q / out)
  const int q_begin = min(max(p.query_start_loc[s], 0), p.num_tokens);
  const int Qs = min(max(p.query_start_loc[s + 1], q_begin), p.num_tokens) - q_begin;
  const int q0 = tile * tq;
  if (q0 >= Qs) return;
  const int nt = min(tq, Qs - q0);             // tokens of this tile
  const int n = min(p.context_lens[s], p.bt_stride * 16);
  const int pos0 = n - Qs + q0;                // position of the tile's first token
  const int p_last = pos0 + nt - 1;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 31, hf = lane >> 5;
  const int row = wave * 32 + col;             // row of this lane's query (0..127)
  const bool row_ok = row < nt * g;
  const int tok = min(row, nt * g - 1) / g;
  const int head = min(row, nt * g - 1) - tok * g;
  const int ppos = pos0 + tok;                 // query position of the row

  // Q operand: lane (row, hf) holds d = 64 hf + 8 t + i for k-step t.
  uint4 qr[8];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(p.q) +
                         ((int64_t)(q_begin + q0 + tok) * p.num_q_heads + hk * g + head) * D + 64 * hf;
#pragma unroll
    for (int t = 0; t < 8; ++t) qr[t] = *reinterpret_cast<const uint4*>(qp + 8 * t);
  }

  // Key blocks [kb0, kb_end) in steps of 32.
  int lo = 0;
  if (p.window > 0) lo = max(0, pos0 - p.window + 1);
  const int kb0 = (lo / kBK) * kBK;
  const int nblk = p_last >= 0 ? (p_last / kBK - kb0 / kBK + 1) : 0;

  const int32_t* bt = p.block_tables + (int64_t)s * p.bt_stride;
  const uint8_t* kpool = static_cast<const uint8_t*>(p.k_cache) + (int64_t)hk * kPageBytes;
  const uint8_t* vpool = static_cast<const uint8_t*>(p.v_cache) + (int64_t)hk * kPageBytes;
  const int64_t blk_stride = (int64_t)p.num_kv_heads * kPageBytes;

  // Staging maps (256 threads, one block = pages A and B of 16 rows):
  //  K: thread i loads row i / 16, 16-byte chunk i % 16 of both pages;
  //  V: thread i loads rows 2 kp and 2 kp + 1 (kp = i % 16: key pair of the
  //     block, page kp / 8) at chunk i / 16, and writes the 8 dwords
  //     (V[2kp][d], V[2kp+1][d]) of V^T: 64 lanes hit 64 distinct banks.
  const int k_r = threadIdx.x / CH, k_c = threadIdx.x % CH;
  const int v_kp = threadIdx.x % 16, v_c = threadIdx.x / 16;
  const int k_off = k_r * (D * 2) + k_c * 16;
  const int v_off = 2 * (v_kp & 7) * (D * 2) + v_c * 16;
  const bool v_pgB = v_kp >= 8;
  auto page_blk = [&](int j) __attribute__((always_inline)) {
    int blk = 0;
    if (j * 16 < n) blk = bt[j];
    return (unsigned)blk < (unsigned)p.num_blocks ? blk : 0;
  };
  // Loads are unconditional (rows at or past n are replaced by zeros when
  // written to LDS) so that nothing waits on them before the LDS write.
  auto fetch = [&](uint4 (&kr)[2], uint4 (&vr)[2], int kb) __attribute__((always_inline)) {
    const int j0 = kb >> 4;
    const int64_t pa = (int64_t)page_blk(j0) * blk_stride, pb = (int64_t)page_blk(j0 + 1) * blk_stride;
    kr[0] = *reinterpret_cast<const uint4*>(kpool + pa + k_off);
    kr[1] = *reinterpret_cast<const uint4*>(kpool + pb + k_off);
    const uint8_t* vp = vpool + (v_pgB ? pb : pa) + v_off;
    vr[0] = *reinterpret_cast<const uint4*>(vp);
    vr[1] = *reinterpret_cast<const uint4*>(vp + D * 2);
  };
  auto masked = [](uint4 x, bool keep) __attribute__((always_inline)) {
    const uint32_t m = keep ? 0xFFFFFFFFu : 0u;    // value-level select (no pointer select)
    return make_uint4(x.x & m, x.y & m, x.z & m, x.w & m);
  };
  auto stage = [&](int buf, const uint4 (&kr)[2], const uint4 (&vr)[2], int kb)
      __attribute__((always_inline)) {
    uint4 k0 = kr[0], k1 = kr[1], va = vr[0], vc = vr[1];
    if (kb + kBK > n) {                            // block crossing n: zero the rows past it
      k0 = masked(k0, kb + k_r < n);
      k1 = masked(k1, kb + 16 + k_r < n);
      va = masked(va, kb + 2 * v_kp < n);
      vc = masked(vc, kb + 2 * v_kp + 1 < n);
    }
    *reinterpret_cast<uint4*>(&s_k[buf][k_r * KROW + k_c * 16]) = k0;
    *reinterpret_cast<uint4*>(&s_k[buf][(16 + k_r) * KROW + k_c * 16]) = k1;
    const uint32_t a[4] = {va.x, va.y, va.z, va.w};
    const uint32_t b[4] = {vc.x, vc.y, vc.z, vc.w};
    uint32_t* vt = &s_v[buf][(v_c * 8) * VROWW + v_kp];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      vt[(2 * i) * VROWW] = __builtin_amdgcn_perm(b[i], a[i], 0x05040100u);
      vt[(2 * i + 1) * VROWW] = __builtin_amdgcn_perm(b[i], a[i], 0x07060302u);
    }
  };

  constexpr uint32_t kOnes = QF == kBF16 ? 0x3F803F80u : 0x3C003C00u;   // (1, 1)
  f32x16_t o[D / 32];
#pragma unroll
  for (int m = 0; m < D / 32; ++m) o[m] = f32x16_t{};
  float mrow = -INFINITY, lsum = 0.0f;
  const float c = p.score_scale;

  // One block: S^T, online softmax, O^T update.  buf holds the block's K and
  // V^T.  Lane reads: K rows col (16 bytes at d = 64 hf + 8 t), V^T rows
  // d = 32 m + col (8 bytes at key pairs 8 kap + 2 hf and + 4).
  const uint8_t* k_rd = &s_k[0][col * KROW + 128 * hf];
  const uint32_t* v_rd = &s_v[0][col * VROWW + 2 * hf];
  auto block = [&](int buf, int kb) __attribute__((always_inline)) {
    // ---- S^T = K Q^T ----
    uint4 ka[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) ka[t] = *reinterpret_cast<const uint4*>(k_rd + buf * KBUF + 16 * t);
    f32x16_t sacc = f32x16_t{};
#pragma unroll
    for (int t = 0; t < 8; ++t) sacc = mfma32<QF>(ka[t], qr[t], sacc);

    // ---- online softmax (row = col; this lane holds keys 8j + 4hf + i) ----
    // Scores stay unscaled up to the exponent (scale > 0: max(c s) = c max(s)),
    // which is then one fma per score: exp2(c s - m).
    float sc[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) sc[k] = sacc[k];
    const bool edge = (kb + kBK - 1 > pos0) || (p.window > 0 && kb <= p_last - p.window);
    if (edge) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = kb + 8 * j + 4 * hf + i;
          bool keep = t <= ppos;
          if (p.window > 0) keep = keep && (t > ppos - p.window);
          if (!keep) sc[4 * j + i] = -INFINITY;
        }
    }
    float mx = sc[0];
#pragma unroll
    for (int k = 1; k < 16; ++k) mx = fmaxf(mx, sc[k]);
    mx = half_max(mx) * c;
    const bool need = mx > mrow + kTauP;
    if (__any(need)) {
      const float mn = need ? fmaxf(mrow, mx) : mrow;
      const float alpha = (mrow == -INFINITY) ? 0.0f : fast_exp2(mrow - mn);
      mrow = mn;
      lsum *= alpha;
#pragma unroll
      for (int m = 0; m < D / 32; ++m)
#pragma unroll
        for (int k = 0; k < 16; ++k) o[m][k] *= alpha;
    }
    const float nmu = (mrow == -INFINITY) ? 0.0f : -mrow;
    uint32_t pw[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      pw[k] = pack2<QF>(fast_exp2(fmaf(sc[2 * k], c, nmu)), fast_exp2(fmaf(sc[2 * k + 1], c, nmu)));
      lsum = dot2<QF>(pw[k], kOnes, lsum);       // row sum of the rounded weights
    }

    // ---- O^T += V^T P^T ----
    const uint32_t* vb = v_rd + buf * (VBUF / 4);
#pragma unroll
    for (int kap = 0; kap < 2; ++kap) {
      const uint4 pb = make_uint4(pw[4 * kap], pw[4 * kap + 1], pw[4 * kap + 2], pw[4 * kap + 3]);
#pragma unroll
      for (int m = 0; m < D / 32; ++m) {
        const uint32_t* vr = vb + 32 * m * VROWW + 8 * kap;
        const uint2 a0 = *reinterpret_cast<const uint2*>(vr);
        const uint2 a1 = *reinterpret_cast<const uint2*>(vr + 4);
        o[m] = mfma32<QF>(make_uint4(a0.x, a0.y, a1.x, a1.y), pb, o[m]);
      }
    }
  };

  // Two register sets of staged loads: block bi + 2 is fetched while block bi
  // is computed and block bi + 1 is written to LDS.
  uint4 kr0[2], vr0[2], kr1[2], vr1[2];
  auto kb_of = [&](int bi) __attribute__((always_inline)) { return kb0 + min(bi, nblk - 1) * kBK; };
  if (nblk > 0) {
    fetch(kr0, vr0, kb_of(0));
    fetch(kr1, vr1, kb_of(1));
    stage(0, kr0, vr0, kb_of(0));
  }
  __syncthreads();
  for (int bi = 0; bi < nblk; bi += 2) {
    fetch(kr0, vr0, kb_of(bi + 2));            // (past the end: re-reads the last block)
    __builtin_amdgcn_sched_barrier(0);
    block(0, kb0 + bi * kBK);
    __builtin_amdgcn_sched_barrier(0);
    stage(1, kr1, vr1, kb_of(bi + 1));
    __syncthreads();
    if (bi + 1 >= nblk) break;
    fetch(kr1, vr1, kb_of(bi + 3));
    __builtin_amdgcn_sched_barrier(0);
    block(1, kb0 + (bi + 1) * kBK);
    __builtin_amdgcn_sched_barrier(0);
    stage(0, kr0, vr0, kb_of(bi + 2));
    __syncthreads();
  }

  // ---- finalize: out[row][d], d = 32 m + 8 j + 4 hf + i ----
  const float lt = lsum + __shfl_xor(lsum, 32);
  const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
  if (row_ok) {
    uint16_t* op = static_cast<uint16_t*>(p.out) +
                   ((int64_t)(q_begin + q0 + tok) * p.num_q_heads + hk * g + head) * D + 4 * hf;
#pragma unroll
    for (int m = 0; m < D / 32; ++m)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int k = 4 * j;
        const uint32_t w0 = (uint32_t)f32_to_16<QF>(o[m][k] * inv) |
                            ((uint32_t)f32_to_16<QF>(o[m][k + 1] * inv) << 16);
        const uint32_t w1 = (uint32_t)f32_to_16<QF>(o[m][k + 2] * inv) |
                            ((uint32_t)f32_to_16<QF>(o[m][k + 3] * inv) << 16);
        *reinterpret_cast<uint2*>(op + 32 * m + 8 * j) = make_uint2(w0, w1);
      }
  }
}

hipError_t launch_prefill(const PrefillParams& p, int head_dim, int q_fmt, hipStream_t stream) {
  if (head_dim != 128) return hipErrorNotSupported;
  const int tq = kRows / p.group;
  if (tq < 1) return hipErrorNotSupported;
  PrefillParams x = p;
  x.num_tiles = (p.max_query_len + tq - 1) / tq;
  const int64_t pairs = (int64_t)p.num_seqs * p.num_kv_heads;
  const int64_t grid = (pairs + 7) / 8 * 8 * x.num_tiles;
  if (grid == 0) return hipSuccess;
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  if (q_fmt == kBF16)
    hipLaunchKernelGGL((prefill_kernel<128, kBF16>), dim3((unsigned)grid), dim3(kPW * 64), 0, stream, x);
  else
    hipLaunchKernelGGL((prefill_kernel<128, kF16>), dim3((unsigned)grid), dim3(kPW * 64), 0, stream, x);
  return hipGetLastError();
}

}  // namespace vp

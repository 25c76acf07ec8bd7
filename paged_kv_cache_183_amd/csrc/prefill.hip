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
//  * V block transposed ([D][key], key pairs XOR-swizzled per 16 rows of D),
//    so that the P.V operand of a lane is two 8-byte reads.
// Per block and wave, on v_mfma_f32_32x32x16 (bf16 or f16, fp32 accumulate):
//  * S^T = K Q^T: the output column of a lane is its query row, so each lane
//    holds 16 scores of one row (keys 8j + 4h + i, h = lane / 32);
//  * online softmax per row in fp32 (log2 domain), the two half-waves of a
//    row combined with one lane exchange; the running max only moves when a
//    score exceeds it by more than 2^8;
//  * P is rounded to q's 16-bit format (the row sums use the rounded values)
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

template <int QF>
__device__ __forceinline__ float lo_f(uint32_t w) {
  if constexpr (QF == kBF16) return bitcast<float>(w << 16);
  else return (float)bitcast<half2_t>(w).x;
}
template <int QF>
__device__ __forceinline__ float hi_f(uint32_t w) {
  if constexpr (QF == kBF16) return bitcast<float>(w & 0xFFFF0000u);
  else return (float)bitcast<half2_t>(w).y;
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
  // Workgroup -> (sequence, kv-head, token tile), tiles of one (sequence,
  // kv-head) placed on the same XCD (workgroups go to XCDs round-robin).
  const int total = gridDim.x;
  const int b = blockIdx.x;
  const int xq = total / 8, xr = total % 8, xcd = b % 8;
  const int L = xcd * xq + min(xcd, xr) + b / 8;
  const int ntiles = p.num_tiles;
  const int tile = L % ntiles;
  const int sh = L / ntiles;
  const int s = sh / p.num_kv_heads;
  const int hk = sh - s * p.num_kv_heads;

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

  // Staging map: thread i -> row i / CH of a page, 16-byte chunk i % CH.
  const int st_r = threadIdx.x / CH, st_c = threadIdx.x % CH;
  const int32_t* bt = p.block_tables + (int64_t)s * p.bt_stride;
  const uint8_t* kpool = static_cast<const uint8_t*>(p.k_cache) + (int64_t)hk * kPageBytes;
  const uint8_t* vpool = static_cast<const uint8_t*>(p.v_cache) + (int64_t)hk * kPageBytes;
  const int64_t blk_stride = (int64_t)p.num_kv_heads * kPageBytes;

  // K: rows st_r of pages 0 and 1 of the block; V: key pair (2 st_r, 2 st_r + 1)
  // spans page st_r / 8, rows 2 (st_r % 8) and 2 (st_r % 8) + 1.
  uint4 kreg[2], vreg[2];
  auto page_blk = [&](int j) __attribute__((always_inline)) {
    int blk = 0;
    if (j * 16 < n) blk = bt[j];
    return (unsigned)blk < (unsigned)p.num_blocks ? blk : 0;
  };
  // Loads are unconditional (rows at or past n are replaced by zeros when
  // written to LDS) so that nothing waits on them before the LDS write.
  auto fetch = [&](int kb) __attribute__((always_inline)) {
    const int j0 = kb >> 4;
    const int b0 = page_blk(j0), b1 = page_blk(j0 + 1);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int bb = u ? b1 : b0;
      kreg[u] = *reinterpret_cast<const uint4*>(kpool + bb * blk_stride + st_r * (D * 2) + st_c * 16);
    }
    const int vb = (st_r >> 3) ? b1 : b0;
    const int vrow = 2 * (st_r & 7);
#pragma unroll
    for (int u = 0; u < 2; ++u)
      vreg[u] = *reinterpret_cast<const uint4*>(vpool + vb * blk_stride + (vrow + u) * (D * 2) + st_c * 16);
  };
  auto masked = [](uint4 x, bool keep) __attribute__((always_inline)) {
    const uint32_t m = keep ? 0xFFFFFFFFu : 0u;    // value-level select (no pointer select)
    return make_uint4(x.x & m, x.y & m, x.z & m, x.w & m);
  };
  auto stage = [&](int buf, int kb) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
      *reinterpret_cast<uint4*>(&s_k[buf][(16 * u + st_r) * KROW + st_c * 16]) =
          masked(kreg[u], kb + 16 * u + st_r < n);
    // V^T: dword (d, key pair kp) at d * VROWW + (kp ^ swz(d)).
    const int t0 = kb + 2 * st_r;                  // keys t0, t0 + 1 of this thread's pair
    const uint4 va = masked(vreg[0], t0 < n);
    const uint4 vc = masked(vreg[1], t0 + 1 < n);
    const uint32_t a[4] = {va.x, va.y, va.z, va.w};
    const uint32_t c[4] = {vc.x, vc.y, vc.z, vc.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d0 = st_c * 8 + 2 * i;
      const int swz = 2 * ((d0 >> 4) & 7);
      s_v[buf][d0 * VROWW + (st_r ^ swz)] = __builtin_amdgcn_perm(c[i], a[i], 0x05040100u);
      s_v[buf][(d0 + 1) * VROWW + (st_r ^ swz)] = __builtin_amdgcn_perm(c[i], a[i], 0x07060302u);
    }
  };

  f32x16_t o[D / 32];
#pragma unroll
  for (int m = 0; m < D / 32; ++m) o[m] = f32x16_t{};
  float mrow = -INFINITY, lsum = 0.0f;

  if (nblk > 0) {
    fetch(kb0);
    stage(0, kb0);
  }
  __syncthreads();
  for (int bi = 0; bi < nblk; ++bi) {
    const int kb = kb0 + bi * kBK;
    const int buf = bi & 1;
    const int kb_next = kb0 + min(bi + 1, nblk - 1) * kBK;   // (re-reads the last block at the end)
    fetch(kb_next);
    __builtin_amdgcn_sched_barrier(0);

    // ---- S^T = K Q^T ----
    f32x16_t sacc = f32x16_t{};
    const uint8_t* krow = &s_k[buf][col * KROW + 128 * hf];
#pragma unroll
    for (int t = 0; t < 8; ++t)
      sacc = mfma32<QF>(*reinterpret_cast<const uint4*>(krow + 16 * t), qr[t], sacc);

    // ---- online softmax (row = col; this lane holds keys 8j + 4hf + i) ----
    float sc[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) sc[k] = sacc[k] * p.score_scale;
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
    mx = fmaxf(mx, __shfl_xor(mx, 32));
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
    const float mu = (mrow == -INFINITY) ? 0.0f : mrow;
    uint32_t pw[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      pw[k] = pack2<QF>(fast_exp2(sc[2 * k] - mu), fast_exp2(sc[2 * k + 1] - mu));
      lsum += lo_f<QF>(pw[k]) + hi_f<QF>(pw[k]);
    }

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int kap = 0; kap < 2; ++kap) {
      const uint4 pb = make_uint4(pw[4 * kap], pw[4 * kap + 1], pw[4 * kap + 2], pw[4 * kap + 3]);
#pragma unroll
      for (int m = 0; m < D / 32; ++m) {
        const int d = 32 * m + col;
        const int swz = 2 * ((d >> 4) & 7);
        const uint32_t* vr = &s_v[buf][d * VROWW];
        const uint2 a0 = *reinterpret_cast<const uint2*>(vr + ((8 * kap + 2 * hf) ^ swz));
        const uint2 a1 = *reinterpret_cast<const uint2*>(vr + ((8 * kap + 4 + 2 * hf) ^ swz));
        o[m] = mfma32<QF>(make_uint4(a0.x, a0.y, a1.x, a1.y), pb, o[m]);
      }
    }

    __builtin_amdgcn_sched_barrier(0);
    stage(buf ^ 1, kb_next);
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
  const int64_t grid = (int64_t)p.num_seqs * p.num_kv_heads * x.num_tiles;
  if (grid == 0) return hipSuccess;
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  if (q_fmt == kBF16)
    hipLaunchKernelGGL((prefill_kernel<128, kBF16>), dim3((unsigned)grid), dim3(kPW * 64), 0, stream, x);
  else
    hipLaunchKernelGGL((prefill_kernel<128, kF16>), dim3((unsigned)grid), dim3(kPW * 64), 0, stream, x);
  return hipGetLastError();
}

}  // namespace vp

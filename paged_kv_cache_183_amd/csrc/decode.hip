// Paged attention decode for gfx950: one query token per sequence attends to
// its K/V, read page by page through the sequence's block table (paged
// attention over the block-paged KV cache of the vllm.cpp model forward,
// repository listing "What's implemented"; 16-token FP16/FP8 pages and block
// tables bound to shared physical pages, "Building and Deploying vllm.cpp",
// Step 3).  The pages give no kernel design; this one is built for CDNA4:
//
//  * Work unit = (sequence, kv-head, up to 8 query heads of its group,
//    partition of at most 64 pages).  NW = 4 waves split the partition's
//    pages round-robin; each page is one 16-token slice of one kv-head, 16*D
//    contiguous elements.
//  * Every lane issues 8-element (16 B for 16-bit, 8 B for FP8) loads; a wave
//    load instruction covers 64*8 contiguous elements (TPI token rows), fully
//    coalesced.  Lane (r, c) holds elements [8c, 8c+8) of token rows
//    r, r+TPI, ... of the page.  The next page's K and V are in flight while
//    the current one is computed (register double buffering).
//  * Q.K: the lane's 8-element slices go through packed dot2 (fp16 or bf16
//    pairs; FP8 codes are first converted exactly to q's 16-bit format), then
//    a DPP butterfly over the D/8 lanes of a token row gives every lane the
//    full dot products of its row for all query heads of the group.
//  * Online softmax in fp32, log2 domain.  The running max is only moved when
//    a new score exceeds it by more than 2^8 headroom (or on the first page),
//    so the accumulator is rarely rescaled; exact up to rounding.  Keys
//    outside [max(0, n - window), n) are skipped, never multiplied by zero:
//    their score is -inf and their V slice is replaced by zeros, so NaN
//    garbage in unused page rows cannot leak.
//  * P.V: fp32 FMAs of each probability with the lane's 8 V elements.
//  * End: token-row states are merged across lanes (xor shuffles), then
//    across waves through LDS, and the result is either the final output
//    (one partition) or a (max, sum, normalized output) triple per
//    partition, merged by decode_reduce_kernel with the log-sum-exp rule.
#include "common.h"
#include "kernels.h"

namespace vp {

constexpr int kNW = 4;         // waves per workgroup
constexpr float kTau = 8.0f;   // rescale headroom, log2 units

template <int KF> struct KvChunk { using T = uint4; };      // 8 x 16-bit
template <> struct KvChunk<kE4M3> { using T = uint2; };     // 8 x fp8

// 8 K elements -> 4 packed pairs in q's format.
template <int KF, int QF>
__device__ __forceinline__ void k_pairs(const typename KvChunk<KF>::T& x, uint32_t (&w)[4]) {
  if constexpr (KF != kE4M3) {
    w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
  } else if constexpr (QF == kF16) {
    w[0] = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x.x, 1.0f, false));
    w[1] = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x.x, 1.0f, true));
    w[2] = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x.y, 1.0f, false));
    w[3] = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x.y, 1.0f, true));
  } else {
    w[0] = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.x, 1.0f, false));
    w[1] = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.x, 1.0f, true));
    w[2] = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.y, 1.0f, false));
    w[3] = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.y, 1.0f, true));
  }
}

template <int QF>
__device__ __forceinline__ float dot8(const uint4& q, const uint32_t (&k)[4]) {
  float a = 0.0f;
  if constexpr (QF == kF16) {
    a = __builtin_amdgcn_fdot2(bitcast<half2_t>(q.x), bitcast<half2_t>(k[0]), a, false);
    a = __builtin_amdgcn_fdot2(bitcast<half2_t>(q.y), bitcast<half2_t>(k[1]), a, false);
    a = __builtin_amdgcn_fdot2(bitcast<half2_t>(q.z), bitcast<half2_t>(k[2]), a, false);
    a = __builtin_amdgcn_fdot2(bitcast<half2_t>(q.w), bitcast<half2_t>(k[3]), a, false);
  } else {
    a = __builtin_amdgcn_fdot2_f32_bf16(bitcast<bf16x2_t>(q.x), bitcast<bf16x2_t>(k[0]), a, false);
    a = __builtin_amdgcn_fdot2_f32_bf16(bitcast<bf16x2_t>(q.y), bitcast<bf16x2_t>(k[1]), a, false);
    a = __builtin_amdgcn_fdot2_f32_bf16(bitcast<bf16x2_t>(q.z), bitcast<bf16x2_t>(k[2]), a, false);
    a = __builtin_amdgcn_fdot2_f32_bf16(bitcast<bf16x2_t>(q.w), bitcast<bf16x2_t>(k[3]), a, false);
  }
  return a;
}

// 8 V elements -> fp32 (exact; FP8 codes stay in code units, v_scale is
// applied once at the end).
template <int KF>
__device__ __forceinline__ void v_f32(const typename KvChunk<KF>::T& x, float (&f)[8]) {
  if constexpr (KF == kE4M3) {
    float2_t a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(x.x, 1.0f, false);
    float2_t b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(x.x, 1.0f, true);
    float2_t c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(x.y, 1.0f, false);
    float2_t d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(x.y, 1.0f, true);
    f[0] = a.x; f[1] = a.y; f[2] = b.x; f[3] = b.y;
    f[4] = c.x; f[5] = c.y; f[6] = d.x; f[7] = d.y;
  } else {
    x2_to_f32<KF>(x.x, f[0], f[1]);
    x2_to_f32<KF>(x.y, f[2], f[3]);
    x2_to_f32<KF>(x.z, f[4], f[5]);
    x2_to_f32<KF>(x.w, f[6], f[7]);
  }
}

template <int D, int G, int KF, int QF>
__global__ __launch_bounds__(kNW * 64) void decode_kernel(DecodeParams p) {
  constexpr int CH = D / 8;            // lanes per token row
  constexpr int TPI = 64 / CH;         // token rows per wave load instruction
  constexpr int NK = 16 / TPI;         // load instructions per page (K or V)
  using LT = typename KvChunk<KF>::T;
  constexpr int EB = (KF == kE4M3) ? 1 : 2;
  constexpr int kInstrBytes = 64 * 8 * EB;
  constexpr int64_t kPageBytes = 16 * D * EB;

  __shared__ float s_acc[kNW][G][D];
  __shared__ float s_m[kNW][G];
  __shared__ float s_l[kNW][G];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int r = lane / CH;
  const int c = lane % CH;
  const int part = blockIdx.x;
  const int ngc = p.group / G;
  const int hk = blockIdx.y / ngc;
  const int h0 = hk * p.group + (blockIdx.y - hk * ngc) * G;
  const int s = blockIdx.z;

  const int n = min(p.context_lens[s], p.bt_stride * 16);
  if (n <= 0) {
    if (p.num_parts == 1) {   // single pass: nobody else writes this row
      uint16_t* o = static_cast<uint16_t*>(p.out) + ((int64_t)s * p.num_q_heads + h0) * D;
      for (int i = threadIdx.x; i < G * D; i += kNW * 64) o[i] = 0;
    }
    return;
  }
  const int lo = p.window > 0 ? max(0, n - p.window) : 0;
  const int lo_page = lo >> 4;
  const int hi_page = (n + 15) >> 4;
  const int first = max(lo_page, part * p.part_pages);
  const int last = min(hi_page, (part + 1) * p.part_pages);
  if (first >= last) return;
  const int p_lo = lo_page / p.part_pages;
  const int p_hi = (hi_page + p.part_pages - 1) / p.part_pages;
  const bool direct = (p_hi - p_lo) == 1;
  const int npages = last - first;

  // Query slices of the G heads: elements [8c, 8c+8) of each.
  uint4 qv[G];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(p.q) +
                         ((int64_t)s * p.num_q_heads + h0) * D + c * 8;
#pragma unroll
    for (int h = 0; h < G; ++h) qv[h] = *reinterpret_cast<const uint4*>(qp + h * D);
  }
  // Physical page ids of this partition, one per lane.
  int bt_lane = 0;
  if (lane < npages) {
    bt_lane = p.block_tables[(int64_t)s * p.bt_stride + first + lane];
    if ((unsigned)bt_lane >= (unsigned)p.num_blocks) bt_lane = 0;
  }

  const uint8_t* kbase = static_cast<const uint8_t*>(p.k_cache) + (int64_t)hk * kPageBytes + lane * (int)sizeof(LT);
  const uint8_t* vbase = static_cast<const uint8_t*>(p.v_cache) + (int64_t)hk * kPageBytes + lane * (int)sizeof(LT);
  const int64_t blk_stride = (int64_t)p.num_kv_heads * kPageBytes;

  auto load_page = [&](int j, LT (&kd)[NK], LT (&vd)[NK]) {
    const int blk = __builtin_amdgcn_readlane(bt_lane, j);
    const uint8_t* kp = kbase + blk * blk_stride;
    const uint8_t* vq = vbase + blk * blk_stride;
#pragma unroll
    for (int k = 0; k < NK; ++k) kd[k] = *reinterpret_cast<const LT*>(kp + k * kInstrBytes);
#pragma unroll
    for (int k = 0; k < NK; ++k) vd[k] = *reinterpret_cast<const LT*>(vq + k * kInstrBytes);
  };

  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.0f;
  }

  auto process = [&](const LT (&kd)[NK], const LT (&vd)[NK], int pg) {
    float sc[NK][G];
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      uint32_t kw[4];
      k_pairs<KF, QF>(kd[k], kw);
#pragma unroll
      for (int h = 0; h < G; ++h) sc[k][h] = dot8<QF>(qv[h], kw);
    }
#pragma unroll
    for (int k = 0; k < NK; ++k)
#pragma unroll
      for (int h = 0; h < G; ++h) sc[k][h] = group_sum<CH>(sc[k][h]);

    const int t0 = pg * 16;
    const bool full = (t0 >= lo) && (t0 + 16 <= n);
    float pm[G];
#pragma unroll
    for (int h = 0; h < G; ++h) pm[h] = -INFINITY;
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      const int t = t0 + k * TPI + r;
      const bool ok = full || (t >= lo && t < n);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float x = ok ? sc[k][h] * p.score_scale : -INFINITY;
        sc[k][h] = x;
        pm[h] = fmaxf(pm[h], x);
      }
    }
    bool need = false;
#pragma unroll
    for (int h = 0; h < G; ++h) need |= pm[h] > m[h] + kTau;
    if (need) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float mn = fmaxf(m[h], pm[h]);
        const float alpha = (m[h] == -INFINITY) ? 0.0f : fast_exp2(m[h] - mn);
        l[h] *= alpha;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] *= alpha;
        m[h] = mn;
      }
    }
    float ms[G];
#pragma unroll
    for (int h = 0; h < G; ++h) ms[h] = (m[h] == -INFINITY) ? 0.0f : m[h];
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      float pk[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        pk[h] = fast_exp2(sc[k][h] - ms[h]);
        l[h] += pk[h];
      }
      float vf[8];
      v_f32<KF>(vd[k], vf);
      if (!full) {
        const int t = t0 + k * TPI + r;
        if (!(t >= lo && t < n)) {
#pragma unroll
          for (int e = 0; e < 8; ++e) vf[e] = 0.0f;
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(pk[h], vf[e], acc[h][e]);
    }
  };

  {
    LT ka[NK], va[NK], kb[NK], vb[NK];
    int j = wave;
    if (j < npages) load_page(j, ka, va);
    while (j < npages) {
      int jn = j + kNW;
      if (jn < npages) load_page(jn, kb, vb);
      process(ka, va, first + j);
      j = jn;
      if (j >= npages) break;
      jn = j + kNW;
      if (jn < npages) load_page(jn, ka, va);
      process(kb, vb, first + j);
      j = jn;
    }
  }

  // Merge the TPI token-row states of the wave (lanes c, c+CH, c+2CH, ...).
#pragma unroll
  for (int off = CH; off < 64; off <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float m2 = __shfl_xor(m[h], off);
      const float l2 = __shfl_xor(l[h], off);
      const float mn = fmaxf(m[h], m2);
      const float f1 = (m[h] == -INFINITY) ? 0.0f : fast_exp2(m[h] - mn);
      const float f2 = (m2 == -INFINITY) ? 0.0f : fast_exp2(m2 - mn);
      l[h] = l[h] * f1 + l2 * f2;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] = acc[h][e] * f1 + __shfl_xor(acc[h][e], off) * f2;
      m[h] = mn;
    }
  }
  if (r == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) s_acc[wave][h][c * 8 + e] = acc[h][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      s_m[wave][h] = m[h];
      s_l[wave][h] = l[h];
    }
  }
  __syncthreads();

  // Merge the waves; one thread per output element.
  for (int i = threadIdx.x; i < G * D; i += kNW * 64) {
    const int h = i / D;
    const int d = i - h * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kNW; ++w) M = fmaxf(M, s_m[w][h]);
    float den = 0.0f, num = 0.0f;
#pragma unroll
    for (int w = 0; w < kNW; ++w) {
      const float f = (s_m[w][h] == -INFINITY) ? 0.0f : fast_exp2(s_m[w][h] - M);
      den = fmaf(s_l[w][h], f, den);
      num = fmaf(s_acc[w][h][d], f, num);
    }
    const int64_t row = (int64_t)s * p.num_q_heads + h0 + h;
    if (direct) {
      static_cast<uint16_t*>(p.out)[row * D + d] = f32_to_16<QF>(num / den * p.out_scale);
    } else {
      p.ws_o[(row * p.num_parts + part) * D + d] = num / den;
      if (d == 0) {
        p.ws_m[row * p.num_parts + part] = M;
        p.ws_l[row * p.num_parts + part] = den;
      }
    }
  }
}

// Log-sum-exp merge of the partition triples of one (sequence, query head).
template <int D, int QF>
__global__ __launch_bounds__(D) void decode_reduce_kernel(DecodeParams p) {
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  const int d = threadIdx.x;
  const int64_t row = (int64_t)s * p.num_q_heads + h;
  uint16_t* o = static_cast<uint16_t*>(p.out) + row * D + d;
  const int n = min(p.context_lens[s], p.bt_stride * 16);
  if (n <= 0) {
    *o = 0;
    return;
  }
  const int lo = p.window > 0 ? max(0, n - p.window) : 0;
  const int p_lo = (lo >> 4) / p.part_pages;
  const int p_hi = (((n + 15) >> 4) + p.part_pages - 1) / p.part_pages;
  if (p_hi - p_lo == 1) return;   // written directly by decode_kernel
  const float* mr = p.ws_m + row * p.num_parts;
  const float* lr = p.ws_l + row * p.num_parts;
  const float* orow = p.ws_o + row * p.num_parts * D + d;
  float M = -INFINITY;
  for (int q = p_lo; q < p_hi; ++q) M = fmaxf(M, mr[q]);
  float den = 0.0f, num = 0.0f;
  for (int q = p_lo; q < p_hi; ++q) {
    const float w = lr[q] * fast_exp2(mr[q] - M);
    den += w;
    num = fmaf(w, orow[(int64_t)q * D], num);
  }
  *o = f32_to_16<QF>(num / den * p.out_scale);
}

template <int D, int KF, int QF>
static hipError_t launch_dg(const DecodeParams& p, int gc, hipStream_t stream) {
  dim3 grid(p.num_parts, p.num_kv_heads * (p.group / gc), p.num_seqs);
  dim3 block(kNW * 64);
  switch (gc) {
#define VP_G(GG) case GG: hipLaunchKernelGGL((decode_kernel<D, GG, KF, QF>), grid, block, 0, stream, p); break;
    VP_G(1) VP_G(2) VP_G(3) VP_G(4) VP_G(5) VP_G(6) VP_G(7) VP_G(8)
#undef VP_G
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.num_parts == 1) return e;
  hipLaunchKernelGGL((decode_reduce_kernel<D, QF>), dim3(p.num_q_heads, p.num_seqs), dim3(D), 0, stream, p);
  return hipGetLastError();
}

// Query heads handled per workgroup: the whole group when g <= 8, else the
// largest divisor of g that is at most 8.
static int head_chunk(int g) {
  if (g <= 8) return g;
  for (int c = 8; c > 1; --c)
    if (g % c == 0) return c;
  return 1;
}

template <int D>
static hipError_t launch_d(const DecodeParams& p, int kv_fmt, int q_fmt, hipStream_t stream) {
  const int gc = head_chunk(p.group);
  if (kv_fmt == kF16 && q_fmt == kF16) return launch_dg<D, kF16, kF16>(p, gc, stream);
  if (kv_fmt == kBF16 && q_fmt == kBF16) return launch_dg<D, kBF16, kBF16>(p, gc, stream);
  if (kv_fmt == kE4M3 && q_fmt == kF16) return launch_dg<D, kE4M3, kF16>(p, gc, stream);
  if (kv_fmt == kE4M3 && q_fmt == kBF16) return launch_dg<D, kE4M3, kBF16>(p, gc, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeParams& p, int head_dim, int kv_fmt, int q_fmt, hipStream_t stream) {
  if (p.num_seqs == 0) return hipSuccess;
  if (head_dim == 128) return launch_d<128>(p, kv_fmt, q_fmt, stream);
  if (head_dim == 64) return launch_d<64>(p, kv_fmt, q_fmt, stream);
  return hipErrorInvalidValue;
}

}  // namespace vp

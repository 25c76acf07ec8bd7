// Cache-write scatter: new tokens' K/V rows go to their 16-token physical
// pages through a slot mapping (slot = page * 16 + row), one launch for the
// whole batch.  The pages store KV in block-paged FP16/FP8 pages ("Building
// and Deploying vllm.cpp", Step 3, --kv-cache-dtype and --block-size 16); the
// repository listing's device-resident cache work replaces per-row copies by
// one indexed launch ("Status & caveats", W1 indexed gather/scatter), which is
// the shape of this kernel.
//
// Work item = 8 consecutive elements of one (token, kv-head) row: one 16-byte
// load from k and from v, one 16-byte (16-bit pool) or 8-byte (FP8 pool)
// store into each pool.  Consecutive items of a row are consecutive lanes, so
// both the loads and the stores of a row coalesce.  FP8 pools (E4M3 or E5M2)
// take one scale per tensor or one per kv-head.
#include "common.h"
#include "kernels.h"

namespace vp {

// DST: SRC (bit copy), kE4M3 or kE5M2.
template <int SRC, int DST>
__global__ __launch_bounds__(256) void cache_write_kernel(CacheWriteParams p) {
  constexpr bool TO_FP8 = is_fp8(DST);
  const uint32_t total = p.num_items;
  const uint32_t per_tok = p.items_per_token;       // Hkv * D / 8
  const uint32_t per_head = p.items_per_head;       // D / 8
  for (uint32_t it = blockIdx.x * 256u + threadIdx.x; it < total; it += gridDim.x * 256u) {
    const uint32_t tok = it / per_tok;
    const uint32_t r = it - tok * per_tok;
    const uint32_t h = r / per_head;
    const uint32_t c = r - h * per_head;
    const int64_t slot = p.slot_mapping[tok];
    if (slot < 0 || slot >= p.num_slots) continue;   // padding token / out of range
    const int64_t blk = slot >> 4;
    const int64_t off = slot & 15;
    const int64_t src = (int64_t)tok * p.src_tok_stride + (int64_t)h * p.head_dim + c * 8;
    const int64_t dst = ((blk * p.num_kv_heads + h) * 16 + off) * p.head_dim + c * 8;
    const uint4 kx = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.k) + src);
    const uint4 vx = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.v) + src);
    if constexpr (!TO_FP8) {
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.k_cache) + dst) = kx;
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.v_cache) + dst) = vx;
    } else {
      const uint32_t kw[4] = {kx.x, kx.y, kx.z, kx.w};
      const uint32_t vw[4] = {vx.x, vx.y, vx.z, vx.w};
      const float ks = p.k_scales ? p.k_scales[h] : p.k_scale;
      const float vs = p.v_scales ? p.v_scales[h] : p.v_scale;
      uint32_t ko[2] = {0, 0}, vo[2] = {0, 0};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float a, b;
        x2_to_f32<SRC>(kw[i], a, b);
        // one correctly rounded fp32 division per element
        uint32_t ca = fp8_from_f32<DST>(a / ks), cb = fp8_from_f32<DST>(b / ks);
        ko[i >> 1] |= (ca | (cb << 8)) << ((i & 1) * 16);
        x2_to_f32<SRC>(vw[i], a, b);
        ca = fp8_from_f32<DST>(a / vs);
        cb = fp8_from_f32<DST>(b / vs);
        vo[i >> 1] |= (ca | (cb << 8)) << ((i & 1) * 16);
      }
      *reinterpret_cast<uint2*>(static_cast<uint8_t*>(p.k_cache) + dst) = make_uint2(ko[0], ko[1]);
      *reinterpret_cast<uint2*>(static_cast<uint8_t*>(p.v_cache) + dst) = make_uint2(vo[0], vo[1]);
    }
  }
}

template <int SRC>
static hipError_t launch_cw(const CacheWriteParams& p, int dst_fmt, uint32_t blocks, hipStream_t stream) {
  if (dst_fmt == kE4M3)
    hipLaunchKernelGGL((cache_write_kernel<SRC, kE4M3>), dim3(blocks), dim3(256), 0, stream, p);
  else if (dst_fmt == kE5M2)
    hipLaunchKernelGGL((cache_write_kernel<SRC, kE5M2>), dim3(blocks), dim3(256), 0, stream, p);
  else if (dst_fmt == SRC)
    hipLaunchKernelGGL((cache_write_kernel<SRC, SRC>), dim3(blocks), dim3(256), 0, stream, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_cache_write(const CacheWriteParams& p, int src_fmt, int dst_fmt, hipStream_t stream) {
  if (p.num_items == 0) return hipSuccess;
  uint32_t blocks = (p.num_items + 255u) / 256u;
  if (blocks > 65536u) blocks = 65536u;
  return src_fmt == kBF16 ? launch_cw<kBF16>(p, dst_fmt, blocks, stream)
                          : launch_cw<kF16>(p, dst_fmt, blocks, stream);
}

}  // namespace vp

// Plain random-page read: the practical ceiling of the decode's access pattern
// on this GPU, measured in the same session as the decode.  The decode streams
// every kept K and V page once, 4 KiB (16-bit, D = 128) or 2 KiB (FP8, or
// D = 64) pages in the random order of the block tables; this kernel reads a
// list of such pages exactly once with the decode's load shape (16-byte
// non-temporal loads, 64 lanes per page, the pages cut into one equal
// contiguous chunk of the list per wave) and 16 KiB in flight per wave (4, 8
// or 16 pages, the depth of the decode's 4 KiB K and V pages) and does no
// arithmetic but an XOR that keeps the loads alive.
#include "common.h"
#include "kernels.h"

namespace vp {

typedef uint32_t rp_u32x4 __attribute__((ext_vector_type(4)));

// CPL: 16-byte chunks per lane per page (page bytes / 1024); PIF: pages in
// flight per wave.
template <int CPL, int PIF>
__global__ __launch_bounds__(256) void read_pages_kernel(ReadPagesParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t per = (p.num_pages + p.num_waves - 1) / p.num_waves;
  const int64_t j0 = min(wave * per, p.num_pages);
  const int64_t j1 = min(j0 + per, p.num_pages);
  const int64_t count = j1 - j0;
  constexpr int kPageBytes = CPL * 1024;
  auto page_ptr = [&](int64_t j) __attribute__((always_inline)) {
    // past the end of the chunk: page 0 of the buffer, which every wave reads
    // there, so it stays in L2 (its values are not used)
    int id = 0;
    if (j < count) {
      id = __builtin_amdgcn_readfirstlane(p.page_ids[j0 + j]);
      id = (id >= 0 && id < p.num_base_pages) ? id : 0;
    }
    return p.base + (int64_t)id * kPageBytes + lane * 16;
  };
  uint32_t acc = 0;
  if (count > 0) {
    rp_u32x4 buf[PIF][CPL];
#pragma unroll
    for (int u = 0; u < PIF; ++u) {
      const uint8_t* a = page_ptr(u);
#pragma unroll
      for (int c = 0; c < CPL; ++c)
        buf[u][c] = __builtin_nontemporal_load(reinterpret_cast<const rp_u32x4*>(a + c * 1024));
    }
    for (int64_t jb = 0; jb < count; jb += PIF) {
#pragma unroll
      for (int u = 0; u < PIF; ++u) {
        if (jb + u < count) {
#pragma unroll
          for (int c = 0; c < CPL; ++c) acc ^= buf[u][c].x ^ buf[u][c].y ^ buf[u][c].z ^ buf[u][c].w;
        }
        const uint8_t* a = page_ptr(jb + u + PIF);
#pragma unroll
        for (int c = 0; c < CPL; ++c)
          buf[u][c] = __builtin_nontemporal_load(reinterpret_cast<const rp_u32x4*>(a + c * 1024));
      }
    }
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off);
  if (lane == 0) p.sink[wave] = acc;
}

hipError_t launch_read_pages(const ReadPagesParams& p, hipStream_t stream) {
  if (p.num_waves <= 0 || p.num_waves % 4 != 0) return hipErrorInvalidValue;
  const dim3 grid(p.num_waves / 4), block(256);
  switch (p.page_bytes) {
    case 1024: hipLaunchKernelGGL((read_pages_kernel<1, 16>), grid, block, 0, stream, p); break;
    case 2048: hipLaunchKernelGGL((read_pages_kernel<2, 8>), grid, block, 0, stream, p); break;
    case 4096: hipLaunchKernelGGL((read_pages_kernel<4, 4>), grid, block, 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace vp

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

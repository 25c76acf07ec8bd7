// Host-side layout of the block manager's state buffer and of its schedule
// workspace (the device code is in block_manager.hip).  Plain C++: it is also
// built into the host sanitizer test of the C ABI.
#include "kernels.h"

namespace vp {

namespace {
constexpr int kBlk = 16;          // tokens per block
}  // namespace

BmLayout bm_layout(int32_t num_blocks) {
  BmLayout L{};
  const int64_t N = num_blocks;
  int64_t cap = 64;
  while (cap < 2 * N) cap <<= 1;
  L.cap = (int32_t)cap;
  const int64_t sizes[kBmRegions] = {4 * N, 4 * N, 4 * N, 4 * N, 4 * N, 4 * N, 8 * N, 4 * kBlk * N,
                                     4 * cap, 4 * N, 4 * N};
  int64_t off = 256;                         // header
  for (int i = 0; i < kBmRegions; ++i) {
    L.off[i] = off;
    off += (sizes[i] + 255) / 256 * 256;
  }
  L.bytes = off;
  return L;
}

BmState bm_state(void* base, int32_t num_blocks) {
  const BmLayout L = bm_layout(num_blocks);
  uint8_t* p = static_cast<uint8_t*>(base);
  BmState S;
  S.hdr = reinterpret_cast<int32_t*>(p);
  S.free_stack = reinterpret_cast<int32_t*>(p + L.off[kBmFree]);
  S.ref = reinterpret_cast<int32_t*>(p + L.off[kBmRef]);
  S.ts = reinterpret_cast<uint32_t*>(p + L.off[kBmTs]);
  S.depth = reinterpret_cast<int32_t*>(p + L.off[kBmDepth]);
  S.parent = reinterpret_cast<int32_t*>(p + L.off[kBmParent]);
  S.flags = reinterpret_cast<int32_t*>(p + L.off[kBmFlags]);
  S.chash = reinterpret_cast<uint64_t*>(p + L.off[kBmHash]);
  S.tokens = reinterpret_cast<int32_t*>(p + L.off[kBmTokens]);
  S.table = reinterpret_cast<int32_t*>(p + L.off[kBmTable]);
  S.mark = reinterpret_cast<int32_t*>(p + L.off[kBmMark]);
  S.owner = reinterpret_cast<int32_t*>(p + L.off[kBmOwner]);
  S.num_blocks = num_blocks;
  S.cap = L.cap;
  return S;
}

size_t bm_workspace_bytes(int32_t num_seqs, int32_t mb) {
  const int64_t items = (int64_t)num_seqs * mb;
  return (size_t)((8 * items + 255) / 256 * 256 + (4 * items + 255) / 256 * 256);
}

}  // namespace vp

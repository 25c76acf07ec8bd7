// Test infrastructure: a host-only stand-in for the HIP runtime calls and the
// kernel launchers of libvllm_paged, so that the C-ABI layer (abi.cpp) can be
// built with g++ under AddressSanitizer and UndefinedBehaviorSanitizer and
// driven on a machine without a GPU.
//
// "Device memory" is host memory registered here (stub_register, or
// hipMallocAsync); hipPointerGetAttributes reports only registered ranges as
// device memory.  Each launcher checks the parameter block it receives and
// then writes (or reads) every byte the real kernel may write (or read)
// according to that block, so a workspace carved wrongly or an extent computed
// wrongly on the host shows up as a sanitizer error.
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>

#include "kernels.h"
#include "vllm_paged.h"

namespace {

std::map<uintptr_t, size_t>& ranges() {
  static std::map<uintptr_t, size_t> r;
  return r;
}

int g_fail = 0;

void check(bool ok, const char* what) {
  if (!ok) {
    std::fprintf(stderr, "stub check failed: %s\n", what);
    ++g_fail;
  }
}

// The registered range holding [p, p + n), or false.
bool inside(const void* p, size_t n) {
  if (n == 0) return true;
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  auto it = ranges().upper_bound(a);
  if (it == ranges().begin()) return false;
  --it;
  return a >= it->first && a + n <= it->first + it->second;
}

// Write (or read) n bytes at p: the sanitizers see every access.
void touch_w(const void* p, size_t n, const char* what) {
  check(inside(p, n), what);
  if (n) std::memset(const_cast<void*>(p), 0x5A, n);
}
// (a move onto itself: the sanitizer's interceptor checks the whole range)
void touch_r(const void* p, size_t n, const char* what) {
  check(inside(p, n), what);
  if (n) std::memmove(const_cast<void*>(p), p, n);
}

size_t esize(int fmt) { return vp::is_fp8(fmt) ? 1 : 2; }

}  // namespace

extern "C" {

// ---- test driver hooks ----
void stub_register(void* p, size_t n) { ranges()[reinterpret_cast<uintptr_t>(p)] = n; }
void stub_unregister(void* p) { ranges().erase(reinterpret_cast<uintptr_t>(p)); }
int stub_failures(void) { return g_fail; }
int stub_launches = 0;

// ---- HIP runtime calls used by abi.cpp ----
hipError_t hipPointerGetAttributes(hipPointerAttribute_t* attr, const void* ptr) {
  std::memset(attr, 0, sizeof(*attr));
  if (!inside(ptr, 1)) return hipErrorInvalidValue;
  attr->type = hipMemoryTypeDevice;
  attr->devicePointer = const_cast<void*>(ptr);
  return hipSuccess;
}
hipError_t hipGetLastError(void) { return hipSuccess; }
const char* hipGetErrorString(hipError_t e) { return e == hipSuccess ? "no error" : "stub error"; }
hipError_t hipGetDevice(int* d) {
  *d = 0;
  return hipSuccess;
}
hipError_t hipMallocAsync(void** p, size_t n, hipStream_t) {
  *p = std::aligned_alloc(256, (n + 255) / 256 * 256);
  stub_register(*p, n);
  return hipSuccess;
}
hipError_t hipFreeAsync(void* p, hipStream_t) {
  stub_unregister(p);
  std::free(p);
  return hipSuccess;
}
// The library's scratch array is a host array of this size in the host-only test.
hipError_t hipGetSymbolAddress(void** p, const void* sym) {
  *p = const_cast<void*>(sym);
  stub_register(*p, VLLM_PAGED_NOALLOC_SCRATCH_BYTES);
  return hipSuccess;
}

}  // extern "C"

namespace vp {

// A GPU of 256 CUs holding two decode workgroups each.
int decode_workers(int64_t pages_bound, int, int, int, int, bool) {
  const int64_t w = 256 * 2 * kDecodeWaves;
  const int64_t b = decode_workers_bound(pages_bound);
  return (int)(w < b ? w : b);
}

hipError_t launch_cache_write(const CacheWriteParams& p, int src_fmt, int dst_fmt, hipStream_t) {
  ++stub_launches;
  check(p.items_per_token == p.items_per_head * (uint32_t)p.num_kv_heads, "cache_write items");
  const int64_t T = p.num_items / p.items_per_token;
  const int64_t row = (int64_t)p.num_kv_heads * p.head_dim;
  touch_r(p.k, T * row * esize(src_fmt), "cache_write k");
  touch_r(p.v, T * row * esize(src_fmt), "cache_write v");
  touch_r(p.slot_mapping, T * 8, "cache_write slots");
  touch_w(p.k_cache, p.num_slots * row * esize(dst_fmt), "cache_write k_cache");
  touch_w(p.v_cache, p.num_slots * row * esize(dst_fmt), "cache_write v_cache");
  if (p.k_scales) touch_r(p.k_scales, p.num_kv_heads * 4, "cache_write k_scales");
  if (p.v_scales) touch_r(p.v_scales, p.num_kv_heads * 4, "cache_write v_scales");
  return hipSuccess;
}

// The bytes the decode kernel reads and writes.
static void decode_touch(const DecodeParams& p, int D, int kv_fmt, int q_fmt) {
  const int64_t B = p.num_seqs, G = p.head_chunk;
  const int64_t units = B * p.num_kv_heads * (p.group / G);
  check(p.group % G == 0 && G >= 1 && G <= 8, "decode head chunk");
  check(p.num_workers >= kDecodeWaves && p.num_workers % kDecodeWaves == 0, "decode waves");
  check(p.chunk_pages > 0 || p.num_workers <= p.max_chunks, "decode waves <= workspace chunks");
  // the chunks the kernel makes: one per wave (automatic) or ceil(pages / C); each writes 2 pieces
  const int64_t chunks = p.chunk_pages > 0 ? p.max_chunks : p.num_workers;
  touch_r(p.q, B * p.num_q_heads * D * esize(q_fmt), "decode q");
  touch_w(p.out, B * p.num_q_heads * D * esize(q_fmt), "decode out");
  touch_r(p.block_tables, B * p.bt_stride * 4, "decode block_tables");
  touch_r(p.context_lens, B * 4, "decode context_lens");
  const int64_t pool = (int64_t)p.num_blocks * p.num_kv_heads * 16 * D * esize(kv_fmt);
  touch_r(p.k_cache, pool, "decode k_cache");
  touch_r(p.v_cache, pool, "decode v_cache");
  // the workspace regions the kernel writes
  touch_w(p.ws_unit, units * 8, "decode ws_unit");
  touch_w(p.ws_prefix, (B + 3) * 4, "decode ws_prefix");
  const int64_t pieces = chunks * 2 * G;
  touch_w(p.ws_o, pieces * D * 4, "decode ws_o");
  touch_w(p.ws_m, pieces * 4, "decode ws_m");
  touch_w(p.ws_l, pieces * 4, "decode ws_l");
  touch_r(p.ws_spare, 16 * D * 2, "decode ws_spare");
  if (p.skip_tokens > 0) {
    touch_w(p.ws_uo, units * G * D * 4, "decode ws_uo");
    touch_w(p.ws_um, units * G * 4, "decode ws_um");
    touch_w(p.ws_ul, units * G * 4, "decode ws_ul");
  }
  if (p.k_scales) touch_r(p.k_scales, p.num_kv_heads * 4, "decode k_scales");
  if (p.v_scales) touch_r(p.v_scales, p.num_kv_heads * 4, "decode v_scales");
  if (p.new_slots) {
    touch_r(p.k_new, B * p.num_kv_heads * D * esize(q_fmt), "decode k_new");
    touch_r(p.v_new, B * p.num_kv_heads * D * esize(q_fmt), "decode v_new");
    touch_r(p.new_slots, B * 8, "decode new_slots");
    check(p.num_slots == (int64_t)p.num_blocks * 16, "decode num_slots");
  }
}

hipError_t launch_decode(const DecodeParams& p, int D, int kv_fmt, int q_fmt, hipStream_t s) {
  ++stub_launches;
  decode_touch(p, D, kv_fmt, q_fmt);
  return launch_decode_merge(p, D, q_fmt, s);
}

hipError_t launch_decode_merge(const DecodeParams& p, int D, int q_fmt, hipStream_t) {
  ++stub_launches;
  const int64_t B = p.num_seqs;
  if (p.num_splits > 0) {
    const int64_t rows = (int64_t)p.num_splits * B * p.num_q_heads;
    touch_r(p.pfx_o, rows * D * 4, "merge pfx_o");
    touch_r(p.pfx_m, rows * 4, "merge pfx_m");
    touch_r(p.pfx_l, rows * 4, "merge pfx_l");
  }
  touch_w(p.out, B * p.num_q_heads * D * esize(q_fmt), "merge out");
  return hipSuccess;
}

static void prefill_common(const PrefillParams& p, int D, int kv_fmt, int q_fmt, const char* w) {
  touch_r(p.q, (int64_t)p.num_tokens * p.num_q_heads * D * esize(q_fmt), w);
  touch_r(p.block_tables, (int64_t)p.num_seqs * p.bt_stride * 4, w);
  touch_r(p.context_lens, (int64_t)p.num_seqs * 4, w);
  const int64_t pool = (int64_t)p.num_blocks * p.num_kv_heads * 16 * D * esize(kv_fmt);
  touch_r(p.k_cache, pool, w);
  touch_r(p.v_cache, pool, w);
  if (p.k_scales) touch_r(p.k_scales, p.num_kv_heads * 4, w);
}

hipError_t launch_prefill(const PrefillParams& p, int D, int kv_fmt, int q_fmt, hipStream_t) {
  ++stub_launches;
  prefill_common(p, D, kv_fmt, q_fmt, "prefill inputs");
  touch_r(p.query_start_loc, ((int64_t)p.num_seqs + 1) * 4, "prefill query_start_loc");
  touch_w(p.out, (int64_t)p.num_tokens * p.num_q_heads * D * esize(q_fmt), "prefill out");
  if (p.v_scales) touch_r(p.v_scales, p.num_kv_heads * 4, "prefill v_scales");
  const size_t plan = prefill_plan_bytes(p.num_seqs, p.num_kv_heads, p.group, p.max_query_len);
  if (p.plan) {
    check(plan > 0, "prefill plan only where the order is built");
    touch_w(p.plan, (int64_t)plan, "prefill plan");
  } else {
    check(plan == 0, "prefill plan given where the order is built");
  }
  return hipSuccess;
}

hipError_t launch_decode_shared(const DecodeParams& dp, const PrefillParams& p, int D, int kv_fmt,
                                int q_fmt, hipStream_t s) {
  ++stub_launches;
  decode_touch(dp, D, kv_fmt, q_fmt);
  check(dp.skip_tokens == 16 * p.shared_pages && dp.num_splits == p.num_splits,
        "shared prefix: decode and prefix parts agree");
  // prefix mode: q holds one row per sequence
  PrefillParams c = p;
  c.num_tokens = p.num_seqs;
  prefill_common(c, D, kv_fmt, q_fmt, "shared prefix inputs");
  check(p.num_splits * p.split_pages >= p.shared_pages, "shared prefix splits");
  const int64_t rows = (int64_t)p.num_splits * p.num_seqs * p.num_q_heads;
  touch_w(p.pfx_o, rows * D * 4, "shared prefix pfx_o");
  touch_w(p.pfx_m, rows * 4, "shared prefix pfx_m");
  touch_w(p.pfx_l, rows * 4, "shared prefix pfx_l");
  return launch_decode_merge(dp, D, q_fmt, s);
}

hipError_t launch_chunked_local_plan(const LocalPlanParams& p, hipStream_t) {
  ++stub_launches;
  touch_r(p.query_start_loc, ((int64_t)p.num_seqs + 1) * 4, "plan query_start_loc");
  touch_r(p.context_lens, (int64_t)p.num_seqs * 4, "plan context_lens");
  touch_r(p.block_tables, (int64_t)p.num_seqs * p.bt_stride * 4, "plan block_tables");
  touch_w(p.v_query_start_loc, (p.num_virtual + 1) * 4, "plan v_query_start_loc");
  touch_w(p.v_context_lens, p.num_virtual * 4, "plan v_context_lens");
  touch_w(p.v_block_tables, p.num_virtual * (p.chunk / 16) * 4, "plan v_block_tables");
  return hipSuccess;
}

hipError_t launch_recycle_pages(const RecycleParams& p, hipStream_t) {
  ++stub_launches;
  touch_r(p.context_lens, (int64_t)p.num_seqs * 4, "recycle context_lens");
  touch_w(p.block_tables, (int64_t)p.num_seqs * p.bt_stride * 4, "recycle block_tables");
  touch_w(p.freed_offsets, ((int64_t)p.num_seqs + 1) * 4, "recycle freed_offsets");
  touch_w(p.freed_pages, (int64_t)p.num_seqs * p.bt_stride * 4, "recycle freed_pages");
  return hipSuccess;
}

hipError_t launch_read_pages(const ReadPagesParams& p, hipStream_t) {
  ++stub_launches;
  touch_r(p.base, p.num_base_pages * p.page_bytes, "read_pages buffer");
  touch_r(p.page_ids, p.num_pages * 4, "read_pages ids");
  touch_w(p.sink, (int64_t)p.num_waves * 4, "read_pages sink");
  return hipSuccess;
}

static void bm_touch(const BmState& st) {
  const BmLayout L = bm_layout(st.num_blocks);
  touch_w(st.hdr, L.bytes, "block manager state");
}

hipError_t launch_bm_init(const BmState& st, hipStream_t) {
  ++stub_launches;
  bm_touch(st);
  return hipSuccess;
}

hipError_t launch_bm_schedule(const BmScheduleParams& p, hipStream_t) {
  ++stub_launches;
  bm_touch(p.st);
  const int64_t B = p.num_seqs;
  touch_r(p.token_ids, p.num_token_ids * 4, "schedule token_ids");
  touch_r(p.token_start, (B + 1) * 4, "schedule token_start");
  touch_r(p.num_computed, B * 4, "schedule num_computed");
  touch_r(p.query_start_loc, (B + 1) * 4, "schedule query_start_loc");
  touch_w(p.block_tables, B * p.mb * 4, "schedule block_tables");
  touch_w(p.slot_mapping, (int64_t)p.sum_q * 8, "schedule slot_mapping");
  touch_w(p.num_cached, B * 4, "schedule num_cached");
  touch_w(p.status, 4, "schedule status");
  touch_w(p.ws_hash, B * p.mb * 8, "schedule ws_hash");
  touch_w(p.ws_cand, B * p.mb * 4, "schedule ws_cand");
  return hipSuccess;
}

hipError_t launch_bm_release(const BmReleaseParams& p, hipStream_t) {
  ++stub_launches;
  bm_touch(p.st);
  touch_r(p.block_tables, (int64_t)p.num_seqs * p.mb * 4, "release block_tables");
  touch_r(p.num_tokens, (int64_t)p.num_seqs * 4, "release num_tokens");
  return hipSuccess;
}

}  // namespace vp

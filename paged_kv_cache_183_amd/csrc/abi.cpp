// C ABI of the paged KV-cache library: host-side validation of every argument,
// then one or two asynchronous kernel launches on the caller's stream.  The
// conventions (flat, exception-free, status codes with a thread-local last
// error, runtime-checkable version, zero-valued option fields keeping the
// default behaviour) follow the engine's C ABI as its README describes it
// ("Use it as a library (C API)" and the note on the C ABI under the title).
#include "vllm_paged.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <string>

#include "kernels.h"

namespace {

thread_local std::string g_last_error;

vllm_status fail(vllm_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

vllm_status ok() {
  g_last_error.clear();
  return VLLM_OK;
}

#define VP_TRY(expr)                        \
  do {                                      \
    vllm_status st_ = (expr);               \
    if (st_ != VLLM_OK) return st_;         \
  } while (0)

const char* dtype_name(int32_t d) {
  switch (d) {
    case VLLM_DTYPE_F16: return "F16";
    case VLLM_DTYPE_BF16: return "BF16";
    case VLLM_DTYPE_FP8_E4M3: return "FP8_E4M3";
    case VLLM_DTYPE_FP8_E5M2: return "FP8_E5M2";
    case VLLM_DTYPE_I32: return "I32";
    case VLLM_DTYPE_I64: return "I64";
    case VLLM_DTYPE_F32: return "F32";
    default: return "unknown";
  }
}

int64_t numel(const vllm_tensor* t) {
  int64_t n = 1;
  for (int i = 0; i < t->ndim; ++i) n *= t->shape[i];
  return n;
}

int elem_bytes(int32_t d) {
  switch (d) {
    case VLLM_DTYPE_F16: case VLLM_DTYPE_BF16: return 2;
    case VLLM_DTYPE_FP8_E4M3: case VLLM_DTYPE_FP8_E5M2: return 1;
    case VLLM_DTYPE_I32: case VLLM_DTYPE_F32: return 4;
    case VLLM_DTYPE_I64: return 8;
    default: return 0;
  }
}

// Rank, non-negative extents, contiguous strides, non-null data when non-empty.
vllm_status check_tensor(const vllm_tensor* t, const char* name, int ndim) {
  if (!t) return fail(VLLM_ERR_INVALID_ARG, "%s: null tensor descriptor", name);
  if (t->ndim != ndim)
    return fail(VLLM_ERR_INVALID_ARG, "%s: expected rank %d, got %d", name, ndim, (int)t->ndim);
  bool empty = false;
  for (int i = 0; i < ndim; ++i) {
    if (t->shape[i] < 0) return fail(VLLM_ERR_INVALID_ARG, "%s: negative extent in dim %d", name, i);
    empty = empty || t->shape[i] == 0;
  }
  int64_t expect = 1;
  for (int i = ndim - 1; i >= 0 && !empty; --i) {      // an empty tensor has no layout
    if (t->shape[i] != 1 && t->stride[i] != expect)
      return fail(VLLM_ERR_INVALID_ARG, "%s: not contiguous (dim %d stride %lld, expected %lld)", name,
                  i, (long long)t->stride[i], (long long)expect);
    expect *= t->shape[i];
  }
  if (elem_bytes(t->dtype) == 0)
    return fail(VLLM_ERR_INVALID_ARG, "%s: unknown dtype %d", name, (int)t->dtype);
  if (numel(t) > 0 && t->data == nullptr)
    return fail(VLLM_ERR_INVALID_ARG, "%s: null data pointer", name);
  return VLLM_OK;
}

vllm_status check_dtype(const vllm_tensor* t, const char* name, int32_t want) {
  if (t->dtype != want)
    return fail(VLLM_ERR_UNSUPPORTED, "%s: dtype %s, expected %s", name, dtype_name(t->dtype),
                dtype_name(want));
  return VLLM_OK;
}

vllm_status check_align(const void* p, const char* name, uintptr_t a) {
  if ((reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0)
    return fail(VLLM_ERR_INVALID_ARG, "%s: data pointer not %u-byte aligned", name, (unsigned)a);
  return VLLM_OK;
}

// Device memory only: the cache and everything the kernels touch must live
// on the GPU (the listing's device-resident cache work asserts that every
// cache pointer is device memory).
vllm_status check_device_ptr(const void* p, const char* name) {
  hipPointerAttribute_t attr;
  hipError_t e = hipPointerGetAttributes(&attr, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(VLLM_ERR_DEVICE_PTR, "%s: not device memory (%s)", name, hipGetErrorString(e));
  }
  if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged)
    return fail(VLLM_ERR_DEVICE_PTR, "%s: not device memory (memory type %d)", name, (int)attr.type);
  return VLLM_OK;
}

vllm_status check_data(const vllm_tensor* t, const char* name, uintptr_t align) {
  if (numel(t) == 0) return VLLM_OK;
  VP_TRY(check_align(t->data, name, align));
  return check_device_ptr(t->data, name);
}

vllm_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return VLLM_OK;
  return fail(VLLM_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int fmt_of(int32_t d) {
  switch (d) {
    case VLLM_DTYPE_F16: return vp::kF16;
    case VLLM_DTYPE_BF16: return vp::kBF16;
    case VLLM_DTYPE_FP8_E4M3: return vp::kE4M3;
    case VLLM_DTYPE_FP8_E5M2: return vp::kE5M2;
    default: return -1;
  }
}

bool is_fp8_dtype(int32_t d) { return d == VLLM_DTYPE_FP8_E4M3 || d == VLLM_DTYPE_FP8_E5M2; }

// Per-kv-head scale arrays: device memory, 4-byte aligned (their Hkv values
// are read on the device).
vllm_status check_scales(const vllm_attn_opts* opts) {
  if (!opts) return VLLM_OK;
  if (opts->k_scales) {
    VP_TRY(check_align(opts->k_scales, "k_scales", 4));
    VP_TRY(check_device_ptr(opts->k_scales, "k_scales"));
  }
  if (opts->v_scales) {
    VP_TRY(check_align(opts->v_scales, "v_scales", 4));
    VP_TRY(check_device_ptr(opts->v_scales, "v_scales"));
  }
  return VLLM_OK;
}

vllm_status scale_of(float s, const char* name, float* out) {
  const float v = (s == 0.0f) ? 1.0f : s;
  if (!std::isfinite(v) || v <= 0.0f)
    return fail(VLLM_ERR_INVALID_ARG, "%s must be finite and > 0 (got %g)", name, (double)s);
  *out = v;
  return VLLM_OK;
}

int env_int(const char* name, int dflt) {
  const char* s = std::getenv(name);
  if (!s || !*s) return dflt;
  return std::atoi(s);
}

// Decode work split: tokens per chunk (a multiple of 16), or 0 for the
// automatic equal split over the waves the GPU holds at once.
vllm_status pick_chunk_tokens(int32_t requested, int32_t* tokens) {
  int32_t p = requested;
  if (p == 0) p = env_int("VLLM_PAGED_PARTITION", 0);
  if (p != 0 && (p < 16 || p % 16 != 0))
    return fail(VLLM_ERR_INVALID_ARG, "partition_size %d: must be 0 or a positive multiple of 16", (int)p);
  *tokens = p;
  return VLLM_OK;
}

struct DecodePlan {
  int32_t head_chunk, units_per_seq, chunk_pages;
  int64_t pages_bound, max_chunks;
  int32_t num_splits;
  size_t cnt_off, pre_off, o_off, m_off, l_off, spare_off, po_off, pm_off, pl_off, uo_off, um_off,
      ul_off, bytes;
};

// Workspace layout of a decode: per-unit piece records (2 ints per unit),
// page prefix (B + 3 ints), the partial outputs, maxima and sums of up to 2
// pieces per chunk, one spare page that the prefetch past the end of a
// stretch of pages reads (its values are never used), then (shared prefix
// only) the partial outputs, maxima and sums of the prefix splits and of the
// units decoded whole inside one chunk.  The kernels rewrite
// every part whose values they use, so the workspace needs no initialisation.
vllm_status plan_decode(int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t max_blocks,
                        int32_t chunk_tokens, int32_t shared_pages, DecodePlan* dp) {
  DecodePlan x{};
  x.head_chunk = vp::decode_head_chunk((int)(Hq / Hkv));
  x.units_per_seq = (int32_t)(Hkv * (Hq / Hkv / x.head_chunk));
  x.pages_bound = B * x.units_per_seq * max_blocks;
  if (x.pages_bound >= ((int64_t)1 << 31))
    return fail(VLLM_ERR_UNSUPPORTED, "batch too large: %lld pages of work", (long long)x.pages_bound);
  x.chunk_pages = chunk_tokens / 16;
  if (x.chunk_pages > 0) {
    // fixed chunks: ceil(T / C) <= ceil(pages_bound / C) whatever the grid
    x.max_chunks = (x.pages_bound + x.chunk_pages - 1) / x.chunk_pages;
  } else {
    // automatic split: one chunk per wave, ceil(T / ceil(T / W)) <= W chunks,
    // so the slots cover the largest wave count the launch can pick
    x.max_chunks = vp::decode_workers_bound(x.pages_bound);
  }
  if (x.max_chunks < 1) x.max_chunks = 1;
  auto up = [](size_t v) { return (v + 255) & ~size_t(255); };
  const size_t pieces = (size_t)x.max_chunks * 2 * (size_t)x.head_chunk;
  if (B * x.units_per_seq > (int64_t)(vp::kUnitBytes / 8))
    return fail(VLLM_ERR_UNSUPPORTED, "batch too large: %lld work units (at most %zu)",
                (long long)(B * x.units_per_seq), vp::kUnitBytes / 8);
  x.cnt_off = 0;
  x.pre_off = up((size_t)B * (size_t)x.units_per_seq * 8);
  x.o_off = x.pre_off + up((size_t)(B + 3) * 4);
  x.m_off = x.o_off + up(pieces * (size_t)D * 4);
  x.l_off = x.m_off + up(pieces * 4);
  x.spare_off = x.l_off + up(pieces * 4);
  // shared-prefix partials: [splits, B, Hq] rows of D outputs, max and sum
  x.num_splits = (shared_pages + vp::kPrefixSplitPages - 1) / vp::kPrefixSplitPages;
  const size_t prow = (size_t)x.num_splits * (size_t)B * (size_t)Hq;
  x.po_off = x.spare_off + up((size_t)16 * (size_t)D * 2);
  x.pm_off = x.po_off + up(prow * (size_t)D * 4);
  x.pl_off = x.pm_off + up(prow * 4);
  // whole-unit partials (shared prefix only): [units, G] rows
  const size_t urow = shared_pages > 0 ? (size_t)B * (size_t)x.units_per_seq * x.head_chunk : 0;
  x.uo_off = x.pl_off + up(prow * 4);
  x.um_off = x.uo_off + up(urow * (size_t)D * 4);
  x.ul_off = x.um_off + up(urow * 4);
  x.bytes = x.ul_off + up(urow * 4);
  *dp = x;
  return VLLM_OK;
}

}  // namespace

extern "C" {

int32_t vllm_abi_version(void) { return VLLM_PAGED_ABI_VERSION; }

const char* vllm_last_error(void) { return g_last_error.c_str(); }

vllm_status vllm_paged_cache_write(const vllm_tensor* k, const vllm_tensor* v,
                                   const vllm_tensor* slot_mapping, vllm_tensor* k_cache,
                                   vllm_tensor* v_cache, const vllm_attn_opts* opts,
                                   void* hip_stream) {
  VP_TRY(check_tensor(k, "k", 3));
  VP_TRY(check_tensor(v, "v", 3));
  VP_TRY(check_tensor(slot_mapping, "slot_mapping", 1));
  VP_TRY(check_tensor(k_cache, "k_cache", 4));
  VP_TRY(check_tensor(v_cache, "v_cache", 4));
  if (opts && opts->flags != 0) return fail(VLLM_ERR_INVALID_ARG, "opts.flags must be 0");
  const int64_t T = k->shape[0], Hkv = k->shape[1], D = k->shape[2];
  for (int i = 0; i < 3; ++i)
    if (v->shape[i] != k->shape[i]) return fail(VLLM_ERR_INVALID_ARG, "v shape differs from k");
  if (slot_mapping->shape[0] != T)
    return fail(VLLM_ERR_INVALID_ARG, "slot_mapping has %lld entries for %lld tokens",
                (long long)slot_mapping->shape[0], (long long)T);
  const int64_t NB = k_cache->shape[0];
  for (int i = 0; i < 4; ++i)
    if (v_cache->shape[i] != k_cache->shape[i])
      return fail(VLLM_ERR_INVALID_ARG, "v_cache shape differs from k_cache");
  if (k_cache->shape[2] != VLLM_PAGED_BLOCK_SIZE)
    return fail(VLLM_ERR_UNSUPPORTED, "block size %lld: only 16 is supported", (long long)k_cache->shape[2]);
  if (k_cache->shape[1] != Hkv || k_cache->shape[3] != D)
    return fail(VLLM_ERR_INVALID_ARG, "k_cache [%lld, %lld, 16, %lld] does not match k [T, %lld, %lld]",
                (long long)NB, (long long)k_cache->shape[1], (long long)k_cache->shape[3],
                (long long)Hkv, (long long)D);
  if (k->dtype != VLLM_DTYPE_F16 && k->dtype != VLLM_DTYPE_BF16)
    return fail(VLLM_ERR_UNSUPPORTED, "k: dtype %s, expected F16 or BF16", dtype_name(k->dtype));
  VP_TRY(check_dtype(v, "v", k->dtype));
  VP_TRY(check_dtype(slot_mapping, "slot_mapping", VLLM_DTYPE_I64));
  if (k_cache->dtype != k->dtype && !is_fp8_dtype(k_cache->dtype))
    return fail(VLLM_ERR_UNSUPPORTED, "k_cache: dtype %s with %s input", dtype_name(k_cache->dtype),
                dtype_name(k->dtype));
  VP_TRY(check_dtype(v_cache, "v_cache", k_cache->dtype));
  if (D % 8 != 0 || D > 512 || D == 0)
    return fail(VLLM_ERR_UNSUPPORTED, "head_dim %lld: must be a positive multiple of 8, <= 512", (long long)D);
  // (items of 8 elements below 2^31: the kernel's 32-bit item indices,
  // its unrolled strides included, never wrap)
  if ((double)T * (double)Hkv * (double)(D / 8) >= 2147483648.0)
    return fail(VLLM_ERR_UNSUPPORTED, "too many tokens for one call");
  const bool to_fp8 = is_fp8_dtype(k_cache->dtype);
  float ks = 1.0f, vs = 1.0f;
  if (to_fp8) {
    VP_TRY(scale_of(opts ? opts->k_scale : 0.0f, "k_scale", &ks));
    VP_TRY(scale_of(opts ? opts->v_scale : 0.0f, "v_scale", &vs));
  }
  if (T == 0 || Hkv == 0) return ok();
  if (to_fp8) VP_TRY(check_scales(opts));
  VP_TRY(check_data(k, "k", 16));
  VP_TRY(check_data(v, "v", 16));
  VP_TRY(check_data(slot_mapping, "slot_mapping", 8));
  VP_TRY(check_data(k_cache, "k_cache", to_fp8 ? 8 : 16));
  VP_TRY(check_data(v_cache, "v_cache", to_fp8 ? 8 : 16));

  vp::CacheWriteParams p{};
  p.k = k->data;
  p.v = v->data;
  p.slot_mapping = static_cast<const int64_t*>(slot_mapping->data);
  p.k_cache = k_cache->data;
  p.v_cache = v_cache->data;
  p.num_slots = NB * VLLM_PAGED_BLOCK_SIZE;
  p.src_tok_stride = Hkv * D;
  p.num_items = (uint32_t)(T * Hkv * (D / 8));
  p.items_per_token = (uint32_t)(Hkv * (D / 8));
  p.items_per_head = (uint32_t)(D / 8);
  p.num_kv_heads = (int32_t)Hkv;
  p.head_dim = (int32_t)D;
  p.k_scale = ks;
  p.v_scale = vs;
  p.k_scales = (to_fp8 && opts) ? opts->k_scales : nullptr;
  p.v_scales = (to_fp8 && opts) ? opts->v_scales : nullptr;
  VP_TRY(hip_status(vp::launch_cache_write(p, fmt_of(k->dtype), fmt_of(k_cache->dtype),
                                           (hipStream_t)hip_stream),
                    "cache_write launch"));
  return ok();
}

size_t vllm_paged_attn_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t max_blocks_per_seq,
                                      int32_t partition_size) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0 ||
      (head_dim != 64 && head_dim != 128) || max_blocks_per_seq < 0)
    return 0;
  int32_t chunk_tokens = 0;
  DecodePlan dp;
  if (pick_chunk_tokens(partition_size, &chunk_tokens) != VLLM_OK ||
      plan_decode(num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq, chunk_tokens,
                  0, &dp) != VLLM_OK)
    return 0;
  return dp.bytes;
}

size_t vllm_paged_attn_shared_prefix_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                                    int32_t num_kv_heads, int32_t head_dim,
                                                    int32_t max_blocks_per_seq, int32_t shared_pages,
                                                    int32_t partition_size) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0 ||
      (head_dim != 64 && head_dim != 128) || max_blocks_per_seq < 0 || shared_pages < 0 ||
      shared_pages > max_blocks_per_seq)
    return 0;
  int32_t chunk_tokens = 0;
  DecodePlan dp;
  if (pick_chunk_tokens(partition_size, &chunk_tokens) != VLLM_OK ||
      plan_decode(num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq, chunk_tokens,
                  shared_pages, &dp) != VLLM_OK)
    return 0;
  return dp.bytes;
}

}  // extern "C"

namespace {

// Scratch of the allocation-free decode (vllm_paged_attn_decode_noalloc): a
// file-scope device array in the library's code object, so each GPU the
// library runs on holds its own copy for the life of the process and no call
// allocates.  In host code `scratch` only names the symbol; its device
// address comes from hipGetSymbolAddress, looked up once per device (with the
// device current) on the entry point's first call there, and only that
// address is ever passed to a kernel.  The decode kernels rewrite every part
// of their workspace they read, so the array needs no clearing between calls;
// calls that overlap on one GPU share it and race.
constexpr size_t kScratchBytes = VLLM_PAGED_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

vllm_status scratch_address(void** out) {
  int dev = 0;
  VP_TRY(hip_status(hipGetDevice(&dev), "hipGetDevice"));
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(VLLM_ERR_UNSUPPORTED, "device %d: the allocation-free decode supports devices "
                "0..%d", dev, kMaxScratchDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return fail(VLLM_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return VLLM_OK;
}

// Decode, optionally with the first shared_pages pages of every sequence
// handled by the shared-prefix pass (read once per kv-head for the batch),
// and optionally with the cache write of each sequence's newest token fused
// into the decode kernel (k_new, v_new, slot_mapping).

vllm_status run_decode(vllm_tensor* out, const vllm_tensor* q, const vllm_tensor* k_cache,
                       const vllm_tensor* v_cache, const vllm_tensor* block_tables,
                       const vllm_tensor* context_lens, int32_t shared_pages, float scale,
                       int32_t window, const vllm_attn_opts* opts, void* hip_stream,
                       const vllm_tensor* k_new = nullptr, const vllm_tensor* v_new = nullptr,
                       const vllm_tensor* slot_mapping = nullptr, bool noalloc = false) {
  VP_TRY(check_tensor(out, "out", 3));
  VP_TRY(check_tensor(q, "q", 3));
  VP_TRY(check_tensor(k_cache, "k_cache", 4));
  VP_TRY(check_tensor(v_cache, "v_cache", 4));
  VP_TRY(check_tensor(block_tables, "block_tables", 2));
  VP_TRY(check_tensor(context_lens, "context_lens", 1));
  if (opts && opts->flags != 0) return fail(VLLM_ERR_INVALID_ARG, "opts.flags must be 0");
  const int64_t B = q->shape[0], Hq = q->shape[1], D = q->shape[2];
  for (int i = 0; i < 3; ++i)
    if (out->shape[i] != q->shape[i]) return fail(VLLM_ERR_INVALID_ARG, "out shape differs from q");
  for (int i = 0; i < 4; ++i)
    if (v_cache->shape[i] != k_cache->shape[i])
      return fail(VLLM_ERR_INVALID_ARG, "v_cache shape differs from k_cache");
  const int64_t NB = k_cache->shape[0], Hkv = k_cache->shape[1];
  if (k_cache->shape[2] != VLLM_PAGED_BLOCK_SIZE)
    return fail(VLLM_ERR_UNSUPPORTED, "block size %lld: only 16 is supported", (long long)k_cache->shape[2]);
  if (k_cache->shape[3] != D)
    return fail(VLLM_ERR_INVALID_ARG, "k_cache head_dim %lld != q head_dim %lld",
                (long long)k_cache->shape[3], (long long)D);
  if (block_tables->shape[0] != B || context_lens->shape[0] != B)
    return fail(VLLM_ERR_INVALID_ARG, "block_tables / context_lens must have %lld rows", (long long)B);
  if (Hkv <= 0 || Hq <= 0 || Hq % Hkv != 0)
    return fail(VLLM_ERR_INVALID_ARG, "num_q_heads %lld is not a positive multiple of num_kv_heads %lld",
                (long long)Hq, (long long)Hkv);
  if (window < 0) return fail(VLLM_ERR_INVALID_ARG, "window must be >= 0 (got %d)", (int)window);
  if (!std::isfinite(scale)) return fail(VLLM_ERR_INVALID_ARG, "scale must be finite");
  const bool append = k_new != nullptr;
  if (append) {                            // the newest token of each sequence, fused
    VP_TRY(check_tensor(k_new, "k_new", 3));
    VP_TRY(check_tensor(v_new, "v_new", 3));
    VP_TRY(check_tensor(slot_mapping, "slot_mapping", 1));
    for (const vllm_tensor* x : {k_new, v_new})
      if (x->shape[0] != B || x->shape[1] != Hkv || x->shape[2] != D)
        return fail(VLLM_ERR_INVALID_ARG, "k_new / v_new must be [%lld, %lld, %lld]", (long long)B,
                    (long long)Hkv, (long long)D);
    if (slot_mapping->shape[0] != B)
      return fail(VLLM_ERR_INVALID_ARG, "slot_mapping must have %lld entries", (long long)B);
    VP_TRY(check_dtype(k_new, "k_new", q->dtype));
    VP_TRY(check_dtype(v_new, "v_new", q->dtype));
    VP_TRY(check_dtype(slot_mapping, "slot_mapping", VLLM_DTYPE_I64));
  }
  if (q->dtype != VLLM_DTYPE_F16 && q->dtype != VLLM_DTYPE_BF16)
    return fail(VLLM_ERR_UNSUPPORTED, "q: dtype %s, expected F16 or BF16", dtype_name(q->dtype));
  VP_TRY(check_dtype(out, "out", q->dtype));
  if (k_cache->dtype != q->dtype && !is_fp8_dtype(k_cache->dtype))
    return fail(VLLM_ERR_UNSUPPORTED, "k_cache: dtype %s with %s queries", dtype_name(k_cache->dtype),
                dtype_name(q->dtype));
  VP_TRY(check_dtype(v_cache, "v_cache", k_cache->dtype));
  VP_TRY(check_dtype(block_tables, "block_tables", VLLM_DTYPE_I32));
  VP_TRY(check_dtype(context_lens, "context_lens", VLLM_DTYPE_I32));
  if (D != 64 && D != 128)
    return fail(VLLM_ERR_UNSUPPORTED, "head_dim %lld: supported 64, 128", (long long)D);
  if (NB > INT32_MAX || block_tables->shape[1] > INT32_MAX / 16 || B > 65535 || Hq > 65535)
    return fail(VLLM_ERR_UNSUPPORTED, "sizes beyond the supported range");
  const bool fp8 = is_fp8_dtype(k_cache->dtype);
  float ks = 1.0f, vs = 1.0f;
  if (fp8) {
    VP_TRY(scale_of(opts ? opts->k_scale : 0.0f, "k_scale", &ks));
    VP_TRY(scale_of(opts ? opts->v_scale : 0.0f, "v_scale", &vs));
  }
  int32_t chunk_tokens = 0;
  VP_TRY(pick_chunk_tokens(opts ? opts->partition_size : 0, &chunk_tokens));
  const int64_t max_blocks = block_tables->shape[1];
  DecodePlan dp;
  if (shared_pages < 0 || shared_pages > max_blocks)
    return fail(VLLM_ERR_INVALID_ARG, "shared_pages %d outside [0, max_blocks_per_seq = %lld]",
                (int)shared_pages, (long long)max_blocks);
  if (shared_pages > 0 && !(scale > 0.0f))
    return fail(VLLM_ERR_INVALID_ARG, "shared prefix: scale must be positive");
  VP_TRY(plan_decode(B, Hq, Hkv, D, max_blocks, chunk_tokens, shared_pages, &dp));
  if (noalloc) {
    if (opts && opts->workspace)
      return fail(VLLM_ERR_INVALID_ARG,
                  "the allocation-free decode uses the library's scratch: opts.workspace must be NULL");
    if (dp.bytes > kScratchBytes)
      return fail(VLLM_ERR_WORKSPACE,
                  "decode needs %zu bytes of scratch; the allocation-free decode has %zu "
                  "(a smaller batch, a larger partition_size, or vllm_paged_attn_decode with a "
                  "workspace)", dp.bytes, kScratchBytes);
  }
  if (B == 0) return ok();
  if (opts && opts->workspace && opts->workspace_bytes < dp.bytes)
    return fail(VLLM_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", opts->workspace_bytes, dp.bytes);
  VP_TRY(check_data(q, "q", 16));
  VP_TRY(check_data(out, "out", 16));
  VP_TRY(check_data(k_cache, "k_cache", fp8 ? 8 : 16));
  VP_TRY(check_data(v_cache, "v_cache", fp8 ? 8 : 16));
  VP_TRY(check_data(block_tables, "block_tables", 4));
  VP_TRY(check_data(context_lens, "context_lens", 4));
  if (fp8) VP_TRY(check_scales(opts));
  if (append) {
    VP_TRY(check_data(k_new, "k_new", 16));
    VP_TRY(check_data(v_new, "v_new", 16));
    VP_TRY(check_data(slot_mapping, "slot_mapping", 8));
  }

  hipStream_t stream = (hipStream_t)hip_stream;
  const int kv_fmt = fmt_of(k_cache->dtype), q_fmt = fmt_of(q->dtype);
  vp::DecodeParams p{};
  p.q = q->data;
  p.out = out->data;
  p.k_cache = k_cache->data;
  p.v_cache = v_cache->data;
  p.block_tables = static_cast<const int32_t*>(block_tables->data);
  p.context_lens = static_cast<const int32_t*>(context_lens->data);
  p.num_seqs = (int32_t)B;
  p.num_q_heads = (int32_t)Hq;
  p.num_kv_heads = (int32_t)Hkv;
  p.group = (int32_t)(Hq / Hkv);
  p.head_chunk = dp.head_chunk;
  p.bt_stride = (int32_t)max_blocks;
  p.num_blocks = (int32_t)NB;
  p.window = window;
  p.chunk_pages = dp.chunk_pages;
  p.max_chunks = (int32_t)dp.max_chunks;
  const bool fused = append;
  p.num_workers = dp.chunk_pages > 0
                      ? (int32_t)std::min<int64_t>(dp.max_chunks,
                                                   vp::decode_workers(dp.pages_bound, (int)D, kv_fmt,
                                                                      q_fmt, dp.head_chunk, fused))
                      : vp::decode_workers(dp.pages_bound, (int)D, kv_fmt, q_fmt, dp.head_chunk,
                                           fused);
  p.num_workers = std::max<int32_t>(vp::kDecodeWaves,
                                    (p.num_workers + vp::kDecodeWaves - 1) / vp::kDecodeWaves *
                                        vp::kDecodeWaves);
  // The automatic split makes one chunk per wave: the workspace holds the
  // pieces of at most max_chunks of them.
  if (dp.chunk_pages == 0 && p.num_workers > dp.max_chunks)
    return fail(VLLM_ERR_HIP, "internal: %d decode waves for %lld workspace chunks",
                (int)p.num_workers, (long long)dp.max_chunks);
  p.score_base = scale * 1.4426950408889634f;
  p.score_scale = p.score_base * ks;
  p.out_scale = vs;
  p.k_scales = (fp8 && opts) ? opts->k_scales : nullptr;
  p.v_scales = (fp8 && opts) ? opts->v_scales : nullptr;
  if (fused) {
    p.k_new = k_new->data;
    p.v_new = v_new->data;
    p.new_slots = static_cast<const int64_t*>(slot_mapping->data);
    p.num_slots = NB * VLLM_PAGED_BLOCK_SIZE;
    p.k_scale = ks;
    p.v_scale = vs;
  }

  void* ws = nullptr;
  bool owned = false;
  if (noalloc) {
    VP_TRY(scratch_address(&ws));        // after every argument check
  } else if (opts && opts->workspace) {
    ws = opts->workspace;
    VP_TRY(check_align(ws, "workspace", 256));
    VP_TRY(check_device_ptr(ws, "workspace"));
  } else {
    VP_TRY(hip_status(hipMallocAsync(&ws, dp.bytes, stream), "workspace hipMallocAsync"));
    owned = true;
  }
  char* base = static_cast<char*>(ws);
  p.ws_unit = reinterpret_cast<int32_t*>(base + dp.cnt_off);
  p.ws_prefix = reinterpret_cast<int32_t*>(base + dp.pre_off);
  p.ws_o = reinterpret_cast<float*>(base + dp.o_off);
  p.ws_m = reinterpret_cast<float*>(base + dp.m_off);
  p.ws_l = reinterpret_cast<float*>(base + dp.l_off);
  p.ws_spare = base + dp.spare_off;
  hipError_t e = hipSuccess;
  vp::PrefillParams sp{};
  if (shared_pages > 0) {
    sp.q = q->data;
    sp.k_cache = k_cache->data;
    sp.v_cache = v_cache->data;
    sp.block_tables = p.block_tables;
    sp.context_lens = p.context_lens;
    sp.num_seqs = (int32_t)B;
    sp.num_q_heads = (int32_t)Hq;
    sp.num_kv_heads = (int32_t)Hkv;
    sp.group = (int32_t)(Hq / Hkv);
    sp.bt_stride = (int32_t)max_blocks;
    sp.num_blocks = (int32_t)NB;
    sp.window = window;
    sp.score_scale = p.score_scale;
    sp.score_base = p.score_base;
    sp.k_scales = p.k_scales;
    sp.shared_pages = shared_pages;
    sp.split_pages = vp::kPrefixSplitPages;
    sp.num_splits = dp.num_splits;
    sp.pfx_o = reinterpret_cast<float*>(base + dp.po_off);
    sp.pfx_m = reinterpret_cast<float*>(base + dp.pm_off);
    sp.pfx_l = reinterpret_cast<float*>(base + dp.pl_off);
    p.skip_tokens = shared_pages * 16;
    p.num_splits = dp.num_splits;
    p.pfx_o = sp.pfx_o;
    p.pfx_m = sp.pfx_m;
    p.pfx_l = sp.pfx_l;
    p.ws_uo = reinterpret_cast<float*>(base + dp.uo_off);
    p.ws_um = reinterpret_cast<float*>(base + dp.um_off);
    p.ws_ul = reinterpret_cast<float*>(base + dp.ul_off);
  }
  if (e != hipSuccess) {
    // (nothing more is launched)
  } else if (shared_pages == 0) {
    e = vp::launch_decode(p, (int)D, kv_fmt, q_fmt, stream);
  } else {
    // the prefix tiles and the decode of every sequence's own pages in one
    // grid, then the merge, on the caller's stream
    e = vp::launch_decode_shared(p, sp, (int)D, kv_fmt, q_fmt, stream);
  }
  if (owned) {
    hipError_t e2 = hipFreeAsync(ws, stream);
    if (e == hipSuccess) e = e2;
  }
  VP_TRY(hip_status(e, "decode launch"));
  return ok();
}

}  // namespace

extern "C" {

vllm_status vllm_paged_attn_decode(vllm_tensor* out, const vllm_tensor* q,
                                   const vllm_tensor* k_cache, const vllm_tensor* v_cache,
                                   const vllm_tensor* block_tables,
                                   const vllm_tensor* context_lens, float scale, int32_t window,
                                   const vllm_attn_opts* opts, void* hip_stream) {
  return run_decode(out, q, k_cache, v_cache, block_tables, context_lens, 0, scale, window, opts,
                    hip_stream);
}

vllm_status vllm_paged_attn_decode_append(vllm_tensor* out, const vllm_tensor* q,
                                          const vllm_tensor* k_new, const vllm_tensor* v_new,
                                          const vllm_tensor* slot_mapping,
                                          vllm_tensor* k_cache, vllm_tensor* v_cache,
                                          const vllm_tensor* block_tables,
                                          const vllm_tensor* context_lens, float scale,
                                          int32_t window, const vllm_attn_opts* opts,
                                          void* hip_stream) {
  if (!k_new || !v_new || !slot_mapping)
    return fail(VLLM_ERR_INVALID_ARG, "k_new, v_new and slot_mapping are required");
  return run_decode(out, q, k_cache, v_cache, block_tables, context_lens, 0, scale, window, opts,
                    hip_stream, k_new, v_new, slot_mapping);
}

vllm_status vllm_paged_attn_decode_noalloc(vllm_tensor* out, const vllm_tensor* q,
                                           const vllm_tensor* k_cache, const vllm_tensor* v_cache,
                                           const vllm_tensor* block_tables,
                                           const vllm_tensor* context_lens, float scale,
                                           int32_t window, const vllm_attn_opts* opts,
                                           void* hip_stream) {
  return run_decode(out, q, k_cache, v_cache, block_tables, context_lens, 0, scale, window, opts,
                    hip_stream, nullptr, nullptr, nullptr, /*noalloc=*/true);
}

vllm_status vllm_paged_attn_decode_shared_prefix(vllm_tensor* out, const vllm_tensor* q,
                                                 const vllm_tensor* k_cache,
                                                 const vllm_tensor* v_cache,
                                                 const vllm_tensor* block_tables,
                                                 const vllm_tensor* context_lens,
                                                 int32_t shared_pages, float scale, int32_t window,
                                                 const vllm_attn_opts* opts, void* hip_stream) {
  return run_decode(out, q, k_cache, v_cache, block_tables, context_lens, shared_pages, scale,
                    window, opts, hip_stream);
}

vllm_status vllm_paged_attn_prefill(vllm_tensor* out, const vllm_tensor* q,
                                    const vllm_tensor* k_cache, const vllm_tensor* v_cache,
                                    const vllm_tensor* block_tables,
                                    const vllm_tensor* query_start_loc,
                                    const vllm_tensor* context_lens, int32_t max_query_len,
                                    float scale, int32_t window, const vllm_attn_opts* opts,
                                    void* hip_stream) {
  VP_TRY(check_tensor(out, "out", 3));
  VP_TRY(check_tensor(q, "q", 3));
  VP_TRY(check_tensor(k_cache, "k_cache", 4));
  VP_TRY(check_tensor(v_cache, "v_cache", 4));
  VP_TRY(check_tensor(block_tables, "block_tables", 2));
  VP_TRY(check_tensor(query_start_loc, "query_start_loc", 1));
  VP_TRY(check_tensor(context_lens, "context_lens", 1));
  if (opts && opts->flags != 0) return fail(VLLM_ERR_INVALID_ARG, "opts.flags must be 0");
  const int64_t sumQ = q->shape[0], Hq = q->shape[1], D = q->shape[2];
  for (int i = 0; i < 3; ++i)
    if (out->shape[i] != q->shape[i]) return fail(VLLM_ERR_INVALID_ARG, "out shape differs from q");
  for (int i = 0; i < 4; ++i)
    if (v_cache->shape[i] != k_cache->shape[i])
      return fail(VLLM_ERR_INVALID_ARG, "v_cache shape differs from k_cache");
  const int64_t NB = k_cache->shape[0], Hkv = k_cache->shape[1];
  const int64_t B = context_lens->shape[0];
  if (k_cache->shape[2] != VLLM_PAGED_BLOCK_SIZE)
    return fail(VLLM_ERR_UNSUPPORTED, "block size %lld: only 16 is supported", (long long)k_cache->shape[2]);
  if (k_cache->shape[3] != D)
    return fail(VLLM_ERR_INVALID_ARG, "k_cache head_dim %lld != q head_dim %lld",
                (long long)k_cache->shape[3], (long long)D);
  if (block_tables->shape[0] != B || query_start_loc->shape[0] != B + 1)
    return fail(VLLM_ERR_INVALID_ARG, "block_tables must have %lld rows and query_start_loc %lld entries",
                (long long)B, (long long)(B + 1));
  if (Hkv <= 0 || Hq <= 0 || Hq % Hkv != 0)
    return fail(VLLM_ERR_INVALID_ARG, "num_q_heads %lld is not a positive multiple of num_kv_heads %lld",
                (long long)Hq, (long long)Hkv);
  if (window < 0) return fail(VLLM_ERR_INVALID_ARG, "window must be >= 0 (got %d)", (int)window);
  if (max_query_len < 0) return fail(VLLM_ERR_INVALID_ARG, "max_query_len must be >= 0");
  if (!std::isfinite(scale) || !(scale > 0.0f))
    return fail(VLLM_ERR_INVALID_ARG, "prefill scale must be finite and positive");
  if (q->dtype != VLLM_DTYPE_F16 && q->dtype != VLLM_DTYPE_BF16)
    return fail(VLLM_ERR_UNSUPPORTED, "q: dtype %s, expected F16 or BF16", dtype_name(q->dtype));
  VP_TRY(check_dtype(out, "out", q->dtype));
  if (k_cache->dtype != q->dtype && !is_fp8_dtype(k_cache->dtype))
    return fail(VLLM_ERR_UNSUPPORTED, "prefill: k_cache dtype %s with %s queries",
                dtype_name(k_cache->dtype), dtype_name(q->dtype));
  VP_TRY(check_dtype(v_cache, "v_cache", k_cache->dtype));
  VP_TRY(check_dtype(block_tables, "block_tables", VLLM_DTYPE_I32));
  VP_TRY(check_dtype(query_start_loc, "query_start_loc", VLLM_DTYPE_I32));
  const bool fp8 = is_fp8_dtype(k_cache->dtype);
  float ks = 1.0f, vs = 1.0f;
  if (fp8) {
    VP_TRY(scale_of(opts ? opts->k_scale : 0.0f, "k_scale", &ks));
    VP_TRY(scale_of(opts ? opts->v_scale : 0.0f, "v_scale", &vs));
  }
  VP_TRY(check_dtype(context_lens, "context_lens", VLLM_DTYPE_I32));
  if (D != 64 && D != 128)
    return fail(VLLM_ERR_UNSUPPORTED, "prefill head_dim %lld: supported 64, 128", (long long)D);
  if (Hq / Hkv > 128) return fail(VLLM_ERR_UNSUPPORTED, "prefill: group size above 128");
  if (NB > INT32_MAX || block_tables->shape[1] > INT32_MAX / 16 || B > 65535 || Hq > 65535 ||
      sumQ > INT32_MAX)
    return fail(VLLM_ERR_UNSUPPORTED, "sizes beyond the supported range");
  if (sumQ == 0 || B == 0 || max_query_len == 0) return ok();
  VP_TRY(check_data(q, "q", 16));
  VP_TRY(check_data(out, "out", 16));
  VP_TRY(check_data(k_cache, "k_cache", 16));
  VP_TRY(check_data(v_cache, "v_cache", 16));
  VP_TRY(check_data(block_tables, "block_tables", 4));
  VP_TRY(check_data(query_start_loc, "query_start_loc", 4));
  VP_TRY(check_data(context_lens, "context_lens", 4));
  if (fp8) VP_TRY(check_scales(opts));

  vp::PrefillParams p{};
  p.q = q->data;
  p.out = out->data;
  p.k_cache = k_cache->data;
  p.v_cache = v_cache->data;
  p.block_tables = static_cast<const int32_t*>(block_tables->data);
  p.query_start_loc = static_cast<const int32_t*>(query_start_loc->data);
  p.context_lens = static_cast<const int32_t*>(context_lens->data);
  p.num_tokens = (int32_t)sumQ;
  p.num_seqs = (int32_t)B;
  p.num_q_heads = (int32_t)Hq;
  p.num_kv_heads = (int32_t)Hkv;
  p.group = (int32_t)(Hq / Hkv);
  p.bt_stride = (int32_t)block_tables->shape[1];
  p.num_blocks = (int32_t)NB;
  p.max_query_len = max_query_len;
  p.window = window;
  p.score_base = scale * 1.4426950408889634f;
  p.score_scale = p.score_base * ks;
  p.out_scale = vs;
  p.k_scales = (fp8 && opts) ? opts->k_scales : nullptr;
  p.v_scales = (fp8 && opts) ? opts->v_scales : nullptr;
  // the tile order's memory: the caller's workspace, else stream-ordered
  const size_t plan_bytes = vp::prefill_plan_bytes(B, Hkv, Hq / Hkv, max_query_len);
  const hipStream_t stream = (hipStream_t)hip_stream;
  void* ws = nullptr;
  bool owned = false;
  if (plan_bytes > 0) {
    if (opts && opts->workspace) {
      if (opts->workspace_bytes < plan_bytes)
        return fail(VLLM_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", opts->workspace_bytes,
                    plan_bytes);
      ws = opts->workspace;
      VP_TRY(check_align(ws, "workspace", 256));
      VP_TRY(check_device_ptr(ws, "workspace"));
    } else {
      VP_TRY(hip_status(hipMallocAsync(&ws, plan_bytes, stream), "workspace hipMallocAsync"));
      owned = true;
    }
    p.plan = static_cast<int2*>(ws);
  }
  hipError_t e = vp::launch_prefill(p, (int)D, fmt_of(k_cache->dtype), fmt_of(q->dtype), stream);
  if (owned) {
    const hipError_t e2 = hipFreeAsync(ws, stream);
    if (e == hipSuccess) e = e2;
  }
  VP_TRY(hip_status(e, "prefill launch"));
  return ok();
}

size_t vllm_paged_attn_prefill_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                              int32_t num_kv_heads, int32_t max_query_len) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0 ||
      num_q_heads / num_kv_heads > 128 || max_query_len < 0)
    return 0;
  return vp::prefill_plan_bytes(num_seqs, num_kv_heads, num_q_heads / num_kv_heads, max_query_len);
}

int64_t vllm_paged_chunked_local_virtual_count(int32_t num_seqs, int32_t num_tokens,
                                               int32_t chunk_size) {
  if (num_seqs < 0 || num_tokens < 0 || chunk_size <= 0 || chunk_size % 16 != 0) return 0;
  return (int64_t)(num_tokens / chunk_size) + 2 * (int64_t)num_seqs;
}

vllm_status vllm_paged_chunked_local_plan(const vllm_tensor* query_start_loc,
                                          const vllm_tensor* context_lens,
                                          const vllm_tensor* block_tables, int32_t chunk_size,
                                          vllm_tensor* v_query_start_loc,
                                          vllm_tensor* v_context_lens,
                                          vllm_tensor* v_block_tables, void* hip_stream) {
  VP_TRY(check_tensor(query_start_loc, "query_start_loc", 1));
  VP_TRY(check_tensor(context_lens, "context_lens", 1));
  VP_TRY(check_tensor(block_tables, "block_tables", 2));
  VP_TRY(check_tensor(v_query_start_loc, "v_query_start_loc", 1));
  VP_TRY(check_tensor(v_context_lens, "v_context_lens", 1));
  VP_TRY(check_tensor(v_block_tables, "v_block_tables", 2));
  for (const vllm_tensor* t : {query_start_loc, context_lens, block_tables, (const vllm_tensor*)v_query_start_loc,
                               (const vllm_tensor*)v_context_lens, (const vllm_tensor*)v_block_tables})
    if (t->dtype != VLLM_DTYPE_I32) return fail(VLLM_ERR_UNSUPPORTED, "plan tensors must be I32");
  if (chunk_size <= 0 || chunk_size % 16 != 0)
    return fail(VLLM_ERR_INVALID_ARG, "chunk_size %d: a positive multiple of 16", (int)chunk_size);
  const int64_t B = context_lens->shape[0];
  if (query_start_loc->shape[0] != B + 1 || block_tables->shape[0] != B)
    return fail(VLLM_ERR_INVALID_ARG, "query_start_loc needs %lld entries and block_tables %lld rows",
                (long long)(B + 1), (long long)B);
  const int64_t V = v_context_lens->shape[0];
  if (v_query_start_loc->shape[0] != V + 1 || v_block_tables->shape[0] != V ||
      v_block_tables->shape[1] != chunk_size / 16)
    return fail(VLLM_ERR_INVALID_ARG, "virtual tensors must be [V + 1], [V], [V, chunk_size / 16]");
  if (B > 65535 || block_tables->shape[1] > INT32_MAX / 16)
    return fail(VLLM_ERR_UNSUPPORTED, "sizes beyond the supported range");
  VP_TRY(check_data(query_start_loc, "query_start_loc", 4));
  VP_TRY(check_data(context_lens, "context_lens", 4));
  if (B > 0) VP_TRY(check_data(block_tables, "block_tables", 4));
  VP_TRY(check_data(v_query_start_loc, "v_query_start_loc", 4));
  if (V > 0) {
    VP_TRY(check_data(v_context_lens, "v_context_lens", 4));
    VP_TRY(check_data(v_block_tables, "v_block_tables", 4));
  }
  vp::LocalPlanParams p{};
  p.query_start_loc = static_cast<const int32_t*>(query_start_loc->data);
  p.context_lens = static_cast<const int32_t*>(context_lens->data);
  p.block_tables = static_cast<const int32_t*>(block_tables->data);
  p.v_query_start_loc = static_cast<int32_t*>(v_query_start_loc->data);
  p.v_context_lens = static_cast<int32_t*>(v_context_lens->data);
  p.v_block_tables = static_cast<int32_t*>(v_block_tables->data);
  p.num_seqs = (int32_t)B;
  p.num_tokens = -1;                 // sumQ = query_start_loc[B], read on the device
  p.bt_stride = (int32_t)block_tables->shape[1];
  p.chunk = chunk_size;
  p.num_virtual = V;
  VP_TRY(hip_status(vp::launch_chunked_local_plan(p, (hipStream_t)hip_stream), "plan launch"));
  return ok();
}

vllm_status vllm_paged_recycle_pages(const vllm_tensor* context_lens, vllm_tensor* block_tables,
                                     int32_t window, int32_t chunk_size,
                                     vllm_tensor* freed_offsets, vllm_tensor* freed_pages,
                                     void* hip_stream) {
  VP_TRY(check_tensor(context_lens, "context_lens", 1));
  VP_TRY(check_tensor(block_tables, "block_tables", 2));
  VP_TRY(check_tensor(freed_offsets, "freed_offsets", 1));
  VP_TRY(check_tensor(freed_pages, "freed_pages", 1));
  for (const vllm_tensor* t : {context_lens, (const vllm_tensor*)block_tables,
                               (const vllm_tensor*)freed_offsets, (const vllm_tensor*)freed_pages})
    if (t->dtype != VLLM_DTYPE_I32) return fail(VLLM_ERR_UNSUPPORTED, "recycle tensors must be I32");
  if (window < 0) return fail(VLLM_ERR_INVALID_ARG, "window must be >= 0");
  if (chunk_size < 0 || chunk_size % 16 != 0)
    return fail(VLLM_ERR_INVALID_ARG, "chunk_size %d: 0 or a positive multiple of 16", (int)chunk_size);
  const int64_t B = context_lens->shape[0], mb = block_tables->shape[1];
  if (block_tables->shape[0] != B || freed_offsets->shape[0] != B + 1 || freed_pages->shape[0] < B * mb)
    return fail(VLLM_ERR_INVALID_ARG, "freed_offsets needs %lld entries and freed_pages %lld",
                (long long)(B + 1), (long long)(B * mb));
  if (B > 65535 || mb > INT32_MAX / 16 || B * mb > INT32_MAX)
    return fail(VLLM_ERR_UNSUPPORTED, "sizes beyond the supported range");
  VP_TRY(check_data(freed_offsets, "freed_offsets", 4));
  if (B > 0) {
    VP_TRY(check_data(context_lens, "context_lens", 4));
    if (mb > 0) {
      VP_TRY(check_data(block_tables, "block_tables", 4));
      VP_TRY(check_data(freed_pages, "freed_pages", 4));
    }
  }
  vp::RecycleParams p{};
  p.context_lens = static_cast<const int32_t*>(context_lens->data);
  p.block_tables = static_cast<int32_t*>(block_tables->data);
  p.freed_offsets = static_cast<int32_t*>(freed_offsets->data);
  p.freed_pages = static_cast<int32_t*>(freed_pages->data);
  p.num_seqs = (int32_t)B;
  p.bt_stride = (int32_t)mb;
  p.window = window;
  p.chunk = chunk_size;
  VP_TRY(hip_status(vp::launch_recycle_pages(p, (hipStream_t)hip_stream), "recycle launch"));
  return ok();
}

vllm_status vllm_paged_read_pages(const vllm_tensor* buffer, const vllm_tensor* page_ids,
                                  int32_t page_bytes, vllm_tensor* sink, void* hip_stream) {
  if (!buffer) return fail(VLLM_ERR_INVALID_ARG, "buffer: null tensor descriptor");
  if (buffer->ndim < 1 || buffer->ndim > 4)
    return fail(VLLM_ERR_INVALID_ARG, "buffer: rank 1 to 4");
  VP_TRY(check_tensor(buffer, "buffer", buffer->ndim));
  VP_TRY(check_tensor(page_ids, "page_ids", 1));
  VP_TRY(check_tensor(sink, "sink", 1));
  VP_TRY(check_dtype(page_ids, "page_ids", VLLM_DTYPE_I32));
  VP_TRY(check_dtype(sink, "sink", VLLM_DTYPE_I32));
  if (page_bytes != 1024 && page_bytes != 2048 && page_bytes != 4096)
    return fail(VLLM_ERR_UNSUPPORTED, "page_bytes %d: supported 1024, 2048, 4096", (int)page_bytes);
  const int64_t W = sink->shape[0];
  if (W < 4 || W % 4 != 0 || W > (1 << 20))
    return fail(VLLM_ERR_INVALID_ARG, "sink: a multiple of 4 entries (one per wave), 4 .. 2^20");
  const int64_t nbytes = numel(buffer) * elem_bytes(buffer->dtype);
  if (nbytes < page_bytes) return fail(VLLM_ERR_INVALID_ARG, "buffer smaller than one page");
  if (page_ids->shape[0] == 0) return ok();
  VP_TRY(check_data(buffer, "buffer", 16));
  VP_TRY(check_data(page_ids, "page_ids", 4));
  VP_TRY(check_data(sink, "sink", 4));
  vp::ReadPagesParams p{};
  p.base = static_cast<const uint8_t*>(buffer->data);
  p.page_ids = static_cast<const int32_t*>(page_ids->data);
  p.sink = static_cast<uint32_t*>(sink->data);
  p.num_pages = page_ids->shape[0];
  p.num_base_pages = nbytes / page_bytes;
  p.page_bytes = page_bytes;
  p.num_waves = (int32_t)W;
  VP_TRY(hip_status(vp::launch_read_pages(p, (hipStream_t)hip_stream), "read_pages launch"));
  return ok();
}

size_t vllm_block_manager_state_size(int32_t num_blocks) {
  if (num_blocks < 1 || num_blocks > (1 << 24)) return 0;
  return (size_t)vp::bm_layout(num_blocks).bytes;
}

int32_t vllm_block_manager_state_layout(int32_t num_blocks, int64_t* offsets, int32_t n) {
  if (num_blocks < 1 || num_blocks > (1 << 24) || !offsets || n <= 0) return 0;
  const vp::BmLayout L = vp::bm_layout(num_blocks);
  int64_t all[vp::kBmRegions + 2];
  all[0] = 0;
  for (int i = 0; i < vp::kBmRegions; ++i) all[i + 1] = L.off[i];
  all[vp::kBmRegions + 1] = L.bytes;
  const int32_t m = std::min<int32_t>(n, vp::kBmRegions + 2);
  for (int i = 0; i < m; ++i) offsets[i] = all[i];
  return m;
}

namespace {
vllm_status check_bm_state(void* state, size_t state_bytes, int32_t num_blocks) {
  if (num_blocks < 1 || num_blocks > (1 << 24))
    return fail(VLLM_ERR_INVALID_ARG, "num_blocks %d outside [1, 2^24]", (int)num_blocks);
  if (!state) return fail(VLLM_ERR_INVALID_ARG, "state: null pointer");
  if (state_bytes < (size_t)vp::bm_layout(num_blocks).bytes)
    return fail(VLLM_ERR_INVALID_ARG, "state of %zu bytes, %lld needed", state_bytes,
                (long long)vp::bm_layout(num_blocks).bytes);
  VP_TRY(check_align(state, "state", 256));
  return check_device_ptr(state, "state");
}
}  // namespace

vllm_status vllm_block_manager_init(void* state, size_t state_bytes, int32_t num_blocks,
                                    void* hip_stream) {
  VP_TRY(check_bm_state(state, state_bytes, num_blocks));
  VP_TRY(hip_status(vp::launch_bm_init(vp::bm_state(state, num_blocks), (hipStream_t)hip_stream),
                    "block manager init launch"));
  return ok();
}

size_t vllm_block_manager_workspace_size(int32_t num_seqs, int32_t max_blocks_per_seq) {
  if (num_seqs < 0 || num_seqs > vp::kBmMaxSeqs || max_blocks_per_seq < 0) return 0;
  return vp::bm_workspace_bytes(num_seqs, max_blocks_per_seq);
}

vllm_status vllm_block_manager_schedule(void* state, int32_t num_blocks,
                                        const vllm_tensor* token_ids,
                                        const vllm_tensor* token_start,
                                        const vllm_tensor* num_computed,
                                        const vllm_tensor* query_start_loc,
                                        vllm_tensor* block_tables, vllm_tensor* slot_mapping,
                                        vllm_tensor* num_cached_tokens, vllm_tensor* status,
                                        uint32_t now, void* workspace, size_t workspace_bytes,
                                        void* hip_stream) {
  VP_TRY(check_tensor(token_ids, "token_ids", 1));
  VP_TRY(check_tensor(token_start, "token_start", 1));
  VP_TRY(check_tensor(num_computed, "num_computed", 1));
  VP_TRY(check_tensor(query_start_loc, "query_start_loc", 1));
  VP_TRY(check_tensor(block_tables, "block_tables", 2));
  VP_TRY(check_tensor(slot_mapping, "slot_mapping", 1));
  VP_TRY(check_tensor(num_cached_tokens, "num_cached_tokens", 1));
  VP_TRY(check_tensor(status, "status", 1));
  for (const vllm_tensor* x : {token_ids, token_start, num_computed, query_start_loc,
                               (const vllm_tensor*)block_tables, (const vllm_tensor*)num_cached_tokens,
                               (const vllm_tensor*)status})
    if (x->dtype != VLLM_DTYPE_I32) return fail(VLLM_ERR_UNSUPPORTED, "block manager metadata must be I32");
  VP_TRY(check_dtype(slot_mapping, "slot_mapping", VLLM_DTYPE_I64));
  const int64_t B = num_computed->shape[0], mb = block_tables->shape[1];
  if (token_start->shape[0] != B + 1 || query_start_loc->shape[0] != B + 1 ||
      block_tables->shape[0] != B || num_cached_tokens->shape[0] != B || status->shape[0] != 1)
    return fail(VLLM_ERR_INVALID_ARG,
                "token_start and query_start_loc need %lld entries, block_tables and "
                "num_cached_tokens %lld rows, status 1 entry", (long long)(B + 1), (long long)B);
  if (B > vp::kBmMaxSeqs || mb > 65535 || token_ids->shape[0] > INT32_MAX ||
      slot_mapping->shape[0] > INT32_MAX)
    return fail(VLLM_ERR_UNSUPPORTED, "batch above %d requests or rows above 65535 blocks",
                vp::kBmMaxSeqs);
  VP_TRY(check_bm_state(state, ~(size_t)0, num_blocks));
  const size_t need = vp::bm_workspace_bytes((int32_t)B, (int32_t)mb);
  if (workspace && workspace_bytes < need)
    return fail(VLLM_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  if (workspace) VP_TRY(check_align(workspace, "workspace", 256));
  VP_TRY(check_data(token_ids, "token_ids", 4));
  VP_TRY(check_data(token_start, "token_start", 4));
  VP_TRY(check_data(num_computed, "num_computed", 4));
  VP_TRY(check_data(query_start_loc, "query_start_loc", 4));
  VP_TRY(check_data(block_tables, "block_tables", 4));
  VP_TRY(check_data(slot_mapping, "slot_mapping", 8));
  VP_TRY(check_data(num_cached_tokens, "num_cached_tokens", 4));
  VP_TRY(check_data(status, "status", 4));
  hipStream_t stream = (hipStream_t)hip_stream;
  void* ws = workspace;
  if (!ws && need > 0) VP_TRY(hip_status(hipMallocAsync(&ws, need, stream), "workspace hipMallocAsync"));
  vp::BmScheduleParams p{};
  p.st = vp::bm_state(state, num_blocks);
  p.token_ids = static_cast<const int32_t*>(token_ids->data);
  p.token_start = static_cast<const int32_t*>(token_start->data);
  p.num_computed = static_cast<const int32_t*>(num_computed->data);
  p.query_start_loc = static_cast<const int32_t*>(query_start_loc->data);
  p.block_tables = static_cast<int32_t*>(block_tables->data);
  p.slot_mapping = static_cast<int64_t*>(slot_mapping->data);
  p.num_cached = static_cast<int32_t*>(num_cached_tokens->data);
  p.status = static_cast<int32_t*>(status->data);
  const int64_t items = B * mb;
  p.ws_hash = static_cast<uint64_t*>(ws);
  p.ws_cand = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(ws) + (8 * items + 255) / 256 * 256);
  p.num_token_ids = token_ids->shape[0];
  p.num_seqs = (int32_t)B;
  p.mb = (int32_t)mb;
  p.sum_q = (int32_t)slot_mapping->shape[0];
  p.now = now;
  hipError_t e = vp::launch_bm_schedule(p, stream);
  if (!workspace && ws) {
    const hipError_t e2 = hipFreeAsync(ws, stream);
    if (e == hipSuccess) e = e2;
  }
  VP_TRY(hip_status(e, "block manager schedule launch"));
  return ok();
}

vllm_status vllm_block_manager_release(void* state, int32_t num_blocks,
                                       const vllm_tensor* block_tables,
                                       const vllm_tensor* num_tokens, uint32_t now,
                                       void* hip_stream) {
  VP_TRY(check_tensor(block_tables, "block_tables", 2));
  VP_TRY(check_tensor(num_tokens, "num_tokens", 1));
  if (block_tables->dtype != VLLM_DTYPE_I32 || num_tokens->dtype != VLLM_DTYPE_I32)
    return fail(VLLM_ERR_UNSUPPORTED, "block manager metadata must be I32");
  const int64_t B = num_tokens->shape[0];
  if (block_tables->shape[0] != B)
    return fail(VLLM_ERR_INVALID_ARG, "block_tables must have %lld rows", (long long)B);
  if (B > vp::kBmMaxSeqs || block_tables->shape[1] > 65535)
    return fail(VLLM_ERR_UNSUPPORTED, "batch above %d requests or rows above 65535 blocks",
                vp::kBmMaxSeqs);
  VP_TRY(check_bm_state(state, ~(size_t)0, num_blocks));
  if (B == 0) return ok();
  VP_TRY(check_data(block_tables, "block_tables", 4));
  VP_TRY(check_data(num_tokens, "num_tokens", 4));
  vp::BmReleaseParams p{};
  p.st = vp::bm_state(state, num_blocks);
  p.block_tables = static_cast<const int32_t*>(block_tables->data);
  p.num_tokens = static_cast<const int32_t*>(num_tokens->data);
  p.num_seqs = (int32_t)B;
  p.mb = (int32_t)block_tables->shape[1];
  p.now = now;
  VP_TRY(hip_status(vp::launch_bm_release(p, (hipStream_t)hip_stream), "block manager release launch"));
  return ok();
}

}  // extern "C"

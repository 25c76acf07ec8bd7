// Test infrastructure: drives the C ABI of libvllm_paged, built on the host
// with g++ under AddressSanitizer and UndefinedBehaviorSanitizer against the
// stub HIP runtime and launchers of hip_host_stub.cpp.  Every entry point is
// called with valid arguments over a sweep of shapes (each launch then touches
// every byte its kernel may access) and with invalid ones (each must return
// its error status without launching).  Exit status 0 = every check passed and
// the sanitizers saw nothing.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <initializer_list>
#include <vector>

#include "vllm_paged.h"

extern "C" {
void stub_register(void* p, size_t n);
void stub_unregister(void* p);
int stub_failures(void);
extern int stub_launches;
}

namespace {

int g_bad = 0;

#define EXPECT(cond, ...)                                      \
  do {                                                         \
    if (!(cond)) {                                             \
      std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
      std::fprintf(stderr, __VA_ARGS__);                       \
      std::fprintf(stderr, " (%s)\n", vllm_last_error());      \
      ++g_bad;                                                 \
    }                                                          \
  } while (0)

// A "device" buffer: host memory registered with the stub, exactly `bytes`
// long (so the sanitizer sees one byte past it).
struct Buf {
  void* p = nullptr;
  size_t n = 0;
  explicit Buf(size_t bytes, bool device = true) : n(bytes) {
    p = std::aligned_alloc(256, (bytes + 255) / 256 * 256 + 256);
    std::memset(p, 0, bytes);
    if (device) stub_register(p, bytes);
  }
  ~Buf() {
    stub_unregister(p);
    std::free(p);
  }
  Buf(const Buf&) = delete;
  Buf& operator=(const Buf&) = delete;
};

int esize(int32_t dt) {
  switch (dt) {
    case VLLM_DTYPE_F16: case VLLM_DTYPE_BF16: return 2;
    case VLLM_DTYPE_FP8_E4M3: case VLLM_DTYPE_FP8_E5M2: return 1;
    case VLLM_DTYPE_I64: return 8;
    default: return 4;
  }
}

vllm_tensor T(const Buf* b, int32_t dt, std::initializer_list<int64_t> shape) {
  vllm_tensor t{};
  t.data = b ? b->p : nullptr;
  t.dtype = dt;
  t.ndim = (int32_t)shape.size();
  int i = 0;
  for (int64_t s : shape) t.shape[i++] = s;
  int64_t st = 1;
  for (int k = t.ndim - 1; k >= 0; --k) {
    t.stride[k] = st;
    st *= t.shape[k];
  }
  return t;
}

size_t bytes_of(int32_t dt, std::initializer_list<int64_t> shape) {
  size_t n = esize(dt);
  for (int64_t s : shape) n *= (size_t)s;
  return n;
}

// Decode (plain, append, noalloc or shared prefix) on one shape.
void decode_case(int B, int Hq, int Hkv, int D, int mb, int part, int window, int32_t qdt,
                 int32_t kvdt, int mode, int shared_pages = 0) {
  const int NB = B * mb < 64 ? B * mb + 1 : 65;     // block ids are clamped on the device
  Buf q(bytes_of(qdt, {B, Hq, D})), out(bytes_of(qdt, {B, Hq, D}));
  Buf kc(bytes_of(kvdt, {NB, Hkv, 16, D})), vc(bytes_of(kvdt, {NB, Hkv, 16, D}));
  Buf bt(bytes_of(VLLM_DTYPE_I32, {B, mb})), ctx(bytes_of(VLLM_DTYPE_I32, {B}));
  Buf kn(bytes_of(qdt, {B, Hkv, D})), vn(bytes_of(qdt, {B, Hkv, D})), sl(bytes_of(VLLM_DTYPE_I64, {B}));
  vllm_tensor tq = T(&q, qdt, {B, Hq, D}), to = T(&out, qdt, {B, Hq, D});
  vllm_tensor tk = T(&kc, kvdt, {NB, Hkv, 16, D}), tv = T(&vc, kvdt, {NB, Hkv, 16, D});
  vllm_tensor tb = T(&bt, VLLM_DTYPE_I32, {B, mb}), tc = T(&ctx, VLLM_DTYPE_I32, {B});
  vllm_tensor tkn = T(&kn, qdt, {B, Hkv, D}), tvn = T(&vn, qdt, {B, Hkv, D});
  vllm_tensor ts = T(&sl, VLLM_DTYPE_I64, {B});
  vllm_attn_opts o{};
  o.partition_size = part;
  o.k_scale = o.v_scale = 0.5f;
  const size_t ws_n = shared_pages ? vllm_paged_attn_shared_prefix_workspace_size(B, Hq, Hkv, D, mb,
                                                                                   shared_pages, part)
                                   : vllm_paged_attn_workspace_size(B, Hq, Hkv, D, mb, part);
  EXPECT(ws_n > 0, "workspace size B=%d Hq=%d Hkv=%d D=%d mb=%d part=%d", B, Hq, Hkv, D, mb, part);
  for (int own = 0; own < 2; ++own) {             // caller workspace of exactly ws_n, then internal
    Buf ws(ws_n);
    o.workspace = own ? nullptr : ws.p;
    o.workspace_bytes = own ? 0 : ws_n;
    vllm_status st;
    if (mode == 1)
      st = vllm_paged_attn_decode_append(&to, &tq, &tkn, &tvn, &ts, &tk, &tv, &tb, &tc, 0.1f, window,
                                         &o, nullptr);
    else if (mode == 2 && own == 0)
      continue;                                   // noalloc takes no workspace
    else if (mode == 2) {
      o.workspace = nullptr;
      st = vllm_paged_attn_decode_noalloc(&to, &tq, &tk, &tv, &tb, &tc, 0.1f, window, &o, nullptr);
    } else if (mode == 3)
      st = vllm_paged_attn_decode_shared_prefix(&to, &tq, &tk, &tv, &tb, &tc, shared_pages, 0.1f,
                                                window, &o, nullptr);
    else
      st = vllm_paged_attn_decode(&to, &tq, &tk, &tv, &tb, &tc, 0.1f, window, &o, nullptr);
    EXPECT(st == VLLM_OK, "decode mode %d B=%d Hq=%d Hkv=%d D=%d mb=%d part=%d", mode, B, Hq, Hkv,
           D, mb, part);
  }
}

void decode_sweep() {
  const int32_t dts[][2] = {{VLLM_DTYPE_F16, VLLM_DTYPE_F16}, {VLLM_DTYPE_BF16, VLLM_DTYPE_BF16},
                            {VLLM_DTYPE_F16, VLLM_DTYPE_FP8_E4M3}, {VLLM_DTYPE_BF16, VLLM_DTYPE_FP8_E5M2}};
  const int heads[][2] = {{1, 1}, {4, 2}, {8, 1}, {40, 8}, {12, 1}, {32, 8}};
  for (auto& dt : dts)
    for (auto& h : heads)
      for (int D : {64, 128})
        for (int B : {1, 3})
          for (int mb : {1, 3, 10, 37})
            for (int part : {0, 16, 512})
              for (int mode = 0; mode < 3; ++mode) decode_case(B, h[0], h[1], D, mb, part, 0, dt[0], dt[1], mode);
  // shared prefix (head_dim 128)
  for (int sp : {1, 16, 33})
    for (auto& h : heads) decode_case(4, h[0], h[1], 128, 40, 0, 0, VLLM_DTYPE_F16, VLLM_DTYPE_FP8_E4M3, 3, sp);
  // a large batch (page prefix from its own kernel) and the benchmark shapes
  decode_case(2100, 4, 2, 128, 4, 0, 0, VLLM_DTYPE_BF16, VLLM_DTYPE_BF16, 0);
  decode_case(32, 32, 8, 128, 256, 0, 0, VLLM_DTYPE_BF16, VLLM_DTYPE_BF16, 1);
  decode_case(16, 40, 8, 128, 2048, 512, 0, VLLM_DTYPE_F16, VLLM_DTYPE_F16, 1);
  decode_case(128, 32, 8, 128, 512, 0, 0, VLLM_DTYPE_F16, VLLM_DTYPE_FP8_E4M3, 3, 256);
}

void decode_errors() {
  const int B = 2, Hq = 4, Hkv = 2, D = 64, mb = 3, NB = 8;
  Buf q(bytes_of(VLLM_DTYPE_F16, {B, Hq, D})), out(bytes_of(VLLM_DTYPE_F16, {B, Hq, D}));
  Buf kc(bytes_of(VLLM_DTYPE_F16, {NB, Hkv, 16, D})), vc(bytes_of(VLLM_DTYPE_F16, {NB, Hkv, 16, D}));
  Buf bt(bytes_of(VLLM_DTYPE_I32, {B, mb})), ctx(bytes_of(VLLM_DTYPE_I32, {B}));
  Buf host(bytes_of(VLLM_DTYPE_F16, {B, Hq, D}), /*device=*/false);
  vllm_tensor tq = T(&q, VLLM_DTYPE_F16, {B, Hq, D}), to = T(&out, VLLM_DTYPE_F16, {B, Hq, D});
  vllm_tensor tk = T(&kc, VLLM_DTYPE_F16, {NB, Hkv, 16, D}), tv = T(&vc, VLLM_DTYPE_F16, {NB, Hkv, 16, D});
  vllm_tensor tb = T(&bt, VLLM_DTYPE_I32, {B, mb}), tc = T(&ctx, VLLM_DTYPE_I32, {B});
  const int before = stub_launches;
  auto dec = [&](vllm_tensor* o_, const vllm_tensor* q_, const vllm_tensor* k_, const vllm_tensor* b_,
                 const vllm_tensor* c_, int window, const vllm_attn_opts* opts) {
    return vllm_paged_attn_decode(o_, q_, k_, &tv, b_, c_, 0.1f, window, opts, nullptr);
  };
  EXPECT(dec(nullptr, &tq, &tk, &tb, &tc, 0, nullptr) == VLLM_ERR_INVALID_ARG, "null out");
  vllm_tensor bad = tq;
  bad.ndim = 7;                                    // rank beyond the descriptor
  EXPECT(dec(&to, &bad, &tk, &tb, &tc, 0, nullptr) == VLLM_ERR_INVALID_ARG, "rank 7");
  bad = tq;
  bad.shape[1] = -4;
  EXPECT(dec(&to, &bad, &tk, &tb, &tc, 0, nullptr) == VLLM_ERR_INVALID_ARG, "negative extent");
  bad = tq;
  bad.stride[0] = 3;
  EXPECT(dec(&to, &bad, &tk, &tb, &tc, 0, nullptr) == VLLM_ERR_INVALID_ARG, "strides");
  bad = tq;
  bad.dtype = 99;
  EXPECT(dec(&to, &bad, &tk, &tb, &tc, 0, nullptr) == VLLM_ERR_INVALID_ARG, "dtype 99");
  EXPECT(dec(&to, &tq, &tk, &tb, &tc, -1, nullptr) == VLLM_ERR_INVALID_ARG, "window");
  vllm_tensor hq = T(&host, VLLM_DTYPE_F16, {B, Hq, D});
  EXPECT(dec(&to, &hq, &tk, &tb, &tc, 0, nullptr) == VLLM_ERR_DEVICE_PTR, "host q");
  vllm_tensor k96 = T(&kc, VLLM_DTYPE_F16, {NB, Hkv, 16, 96});
  vllm_tensor q96 = T(&q, VLLM_DTYPE_F16, {1, Hq, 96});
  vllm_tensor o96 = T(&out, VLLM_DTYPE_F16, {1, Hq, 96});
  vllm_tensor b1 = T(&bt, VLLM_DTYPE_I32, {1, mb}), c1 = T(&ctx, VLLM_DTYPE_I32, {1});
  vllm_tensor v96 = T(&vc, VLLM_DTYPE_F16, {NB, Hkv, 16, 96});
  EXPECT(vllm_paged_attn_decode(&o96, &q96, &k96, &v96, &b1, &c1, 0.1f, 0, nullptr, nullptr) ==
             VLLM_ERR_UNSUPPORTED, "head_dim 96");
  vllm_attn_opts o{};
  o.partition_size = 24;
  EXPECT(dec(&to, &tq, &tk, &tb, &tc, 0, &o) == VLLM_ERR_INVALID_ARG, "partition 24");
  o = {};
  Buf small(64);
  o.workspace = small.p;
  o.workspace_bytes = small.n;
  EXPECT(dec(&to, &tq, &tk, &tb, &tc, 0, &o) == VLLM_ERR_WORKSPACE, "small workspace");
  o = {};
  o.flags = 1;
  EXPECT(dec(&to, &tq, &tk, &tb, &tc, 0, &o) == VLLM_ERR_INVALID_ARG, "flags");
  o = {};
  o.workspace = small.p;
  o.workspace_bytes = 1 << 20;
  EXPECT(vllm_paged_attn_decode_noalloc(&to, &tq, &tk, &tv, &tb, &tc, 0.1f, 0, &o, nullptr) ==
             VLLM_ERR_INVALID_ARG, "noalloc with a workspace");
  EXPECT(vllm_paged_attn_decode_shared_prefix(&to, &tq, &tk, &tv, &tb, &tc, mb + 1, 0.1f, 0, nullptr,
                                              nullptr) == VLLM_ERR_INVALID_ARG, "shared pages");
  EXPECT(stub_launches == before, "an invalid call launched");
}

void cache_write_cases() {
  for (int32_t src : {VLLM_DTYPE_F16, VLLM_DTYPE_BF16})
    for (int32_t dst : {src, (int32_t)VLLM_DTYPE_FP8_E4M3, (int32_t)VLLM_DTYPE_FP8_E5M2})
      for (int D : {8, 64, 128, 512})
        for (int Tk : {0, 1, 33}) {
          const int Hkv = 3, NB = 5;
          Buf k(bytes_of(src, {Tk, Hkv, D}) + 1), v(bytes_of(src, {Tk, Hkv, D}) + 1);
          Buf s(bytes_of(VLLM_DTYPE_I64, {Tk}) + 1);
          Buf kc(bytes_of(dst, {NB, Hkv, 16, D})), vc(bytes_of(dst, {NB, Hkv, 16, D}));
          vllm_tensor tk = T(&k, src, {Tk, Hkv, D}), tv = T(&v, src, {Tk, Hkv, D});
          vllm_tensor ts = T(&s, VLLM_DTYPE_I64, {Tk});
          vllm_tensor tkc = T(&kc, dst, {NB, Hkv, 16, D}), tvc = T(&vc, dst, {NB, Hkv, 16, D});
          vllm_attn_opts o{};
          EXPECT(vllm_paged_cache_write(&tk, &tv, &ts, &tkc, &tvc, &o, nullptr) == VLLM_OK,
                 "cache write D=%d T=%d", D, Tk);
          o.k_scale = -1.0f;
          const vllm_status bad = vllm_paged_cache_write(&tk, &tv, &ts, &tkc, &tvc, &o, nullptr);
          EXPECT(dst == src ? bad == VLLM_OK : bad == VLLM_ERR_INVALID_ARG, "negative fp8 scale");
        }
}

void prefill_cases() {
  for (int D : {128})
    for (int Hq : {8, 32, 64})
      for (int B : {1, 4}) {
        const int Hkv = 8, mb = 9, NB = B * mb, sumQ = 7 * B;
        Buf q(bytes_of(VLLM_DTYPE_BF16, {sumQ, Hq, D})), out(bytes_of(VLLM_DTYPE_BF16, {sumQ, Hq, D}));
        Buf kc(bytes_of(VLLM_DTYPE_BF16, {NB, Hkv, 16, D})), vc(bytes_of(VLLM_DTYPE_BF16, {NB, Hkv, 16, D}));
        Buf bt(bytes_of(VLLM_DTYPE_I32, {B, mb})), qsl(bytes_of(VLLM_DTYPE_I32, {B + 1}));
        Buf ctx(bytes_of(VLLM_DTYPE_I32, {B}));
        vllm_tensor tq = T(&q, VLLM_DTYPE_BF16, {sumQ, Hq, D}), to = T(&out, VLLM_DTYPE_BF16, {sumQ, Hq, D});
        vllm_tensor tk = T(&kc, VLLM_DTYPE_BF16, {NB, Hkv, 16, D}), tv = T(&vc, VLLM_DTYPE_BF16, {NB, Hkv, 16, D});
        vllm_tensor tb = T(&bt, VLLM_DTYPE_I32, {B, mb}), tqs = T(&qsl, VLLM_DTYPE_I32, {B + 1});
        vllm_tensor tc = T(&ctx, VLLM_DTYPE_I32, {B});
        EXPECT(vllm_paged_attn_prefill(&to, &tq, &tk, &tv, &tb, &tqs, &tc, 7, 0.1f, 0, nullptr, nullptr) ==
                   VLLM_OK, "prefill Hq=%d B=%d", Hq, B);
        EXPECT(vllm_paged_attn_prefill(&to, &tq, &tk, &tv, &tb, &tqs, &tc, 7, 0.0f, 0, nullptr, nullptr) ==
                   VLLM_ERR_INVALID_ARG, "prefill scale 0");
        EXPECT(vllm_paged_attn_prefill_workspace_size(B, Hq, Hkv, 7) == 0, "small grid: no order");
        // max_query_len is an upper bound: 8192 makes grids of 2048 and more
        // workgroups (the order is built) except at B = 1, Hq = 8 (512)
        const int tqk = 128 / (Hq / Hkv);
        const int64_t grid = (int64_t)(B * Hkv + 7) / 8 * 8 * ((8192 + tqk - 1) / tqk);
        const size_t pw = vllm_paged_attn_prefill_workspace_size(B, Hq, Hkv, 8192);
        EXPECT((pw > 0) == (grid >= 2048) && (pw == 0 || pw == (size_t)grid * 8),
               "prefill workspace size Hq=%d B=%d", Hq, B);
        if (pw == 0) continue;
        Buf pws(pw);
        vllm_attn_opts o{};
        o.workspace = pws.p;
        o.workspace_bytes = pw;
        EXPECT(vllm_paged_attn_prefill(&to, &tq, &tk, &tv, &tb, &tqs, &tc, 8192, 0.1f, 0, &o, nullptr) ==
                   VLLM_OK, "prefill, caller workspace");
        EXPECT(vllm_paged_attn_prefill(&to, &tq, &tk, &tv, &tb, &tqs, &tc, 8192, 0.1f, 0, nullptr, nullptr) ==
                   VLLM_OK, "prefill, own workspace");
        o.workspace_bytes = pw - 1;
        EXPECT(vllm_paged_attn_prefill(&to, &tq, &tk, &tv, &tb, &tqs, &tc, 8192, 0.1f, 0, &o, nullptr) ==
                   VLLM_ERR_WORKSPACE, "prefill, small workspace");
      }
  EXPECT(vllm_paged_attn_prefill_workspace_size(4097, 8, 8, 8192) == 0, "no order beyond 4096 sequences");
  EXPECT(vllm_paged_attn_prefill_workspace_size(4096, 8, 8, 8192) > 0, "order up to 4096 sequences");
  EXPECT(vllm_paged_attn_prefill_workspace_size(4, 8, 3, 7) == 0, "prefill workspace, Hq % Hkv");
  EXPECT(vllm_paged_attn_prefill_workspace_size(4, 8, 8, 0) == 0, "prefill workspace, no rows");
}

void local_and_manager_cases() {
  const int B = 3, mb = 20, L = 64;
  const int64_t V = vllm_paged_chunked_local_virtual_count(B, 50, L);
  Buf qsl(4 * (B + 1)), ctx(4 * B), bt(4 * B * mb);
  Buf vq(4 * (V + 1)), vctx(4 * V), vbt(4 * V * (L / 16));
  vllm_tensor tqs = T(&qsl, VLLM_DTYPE_I32, {B + 1}), tc = T(&ctx, VLLM_DTYPE_I32, {B});
  vllm_tensor tb = T(&bt, VLLM_DTYPE_I32, {B, mb});
  vllm_tensor tvq = T(&vq, VLLM_DTYPE_I32, {V + 1}), tvc = T(&vctx, VLLM_DTYPE_I32, {V});
  vllm_tensor tvb = T(&vbt, VLLM_DTYPE_I32, {V, L / 16});
  EXPECT(vllm_paged_chunked_local_plan(&tqs, &tc, &tb, L, &tvq, &tvc, &tvb, nullptr) == VLLM_OK, "plan");
  EXPECT(vllm_paged_chunked_local_plan(&tqs, &tc, &tb, 40, &tvq, &tvc, &tvb, nullptr) ==
             VLLM_ERR_INVALID_ARG, "plan chunk 40");
  Buf off(4 * (B + 1)), freed(4 * B * mb);
  vllm_tensor toff = T(&off, VLLM_DTYPE_I32, {B + 1}), tfr = T(&freed, VLLM_DTYPE_I32, {B * mb});
  EXPECT(vllm_paged_recycle_pages(&tc, &tb, 100, 64, &toff, &tfr, nullptr) == VLLM_OK, "recycle");
  const int NBk = 300;
  const size_t sb = vllm_block_manager_state_size(NBk);
  int64_t offs[16];
  EXPECT(vllm_block_manager_state_layout(NBk, offs, 16) == 13 && offs[12] == (int64_t)sb, "layout");
  Buf state(sb);
  EXPECT(vllm_block_manager_init(state.p, sb, NBk, nullptr) == VLLM_OK, "bm init");
  EXPECT(vllm_block_manager_init(state.p, sb - 1, NBk, nullptr) == VLLM_ERR_INVALID_ARG, "bm small");
  const int Tn = 100;
  Buf tok(4 * Tn), tst(4 * (B + 1)), nc(4 * B), slots(8 * Tn), ncached(4 * B), status(4);
  vllm_tensor ttok = T(&tok, VLLM_DTYPE_I32, {Tn}), ttst = T(&tst, VLLM_DTYPE_I32, {B + 1});
  vllm_tensor tnc = T(&nc, VLLM_DTYPE_I32, {B}), tsl = T(&slots, VLLM_DTYPE_I64, {Tn});
  vllm_tensor tnca = T(&ncached, VLLM_DTYPE_I32, {B}), tstat = T(&status, VLLM_DTYPE_I32, {1});
  const size_t wsn = vllm_block_manager_workspace_size(B, mb);
  Buf ws(wsn);
  EXPECT(vllm_block_manager_schedule(state.p, NBk, &ttok, &ttst, &tnc, &tqs, &tb, &tsl, &tnca, &tstat, 1,
                                     ws.p, wsn, nullptr) == VLLM_OK, "bm schedule");
  EXPECT(vllm_block_manager_schedule(state.p, NBk, &ttok, &ttst, &tnc, &tqs, &tb, &tsl, &tnca, &tstat, 1,
                                     nullptr, 0, nullptr) == VLLM_OK, "bm schedule, own workspace");
  EXPECT(vllm_block_manager_release(state.p, NBk, &tb, &tnc, 2, nullptr) == VLLM_OK, "bm release");
  Buf buf(8192), ids(4 * 9), sink(4 * 8);
  vllm_tensor tbuf = T(&buf, VLLM_DTYPE_FP8_E4M3, {8192}), tids = T(&ids, VLLM_DTYPE_I32, {9});
  vllm_tensor tsink = T(&sink, VLLM_DTYPE_I32, {8});
  EXPECT(vllm_paged_read_pages(&tbuf, &tids, 2048, &tsink, nullptr) == VLLM_OK, "read pages");
  EXPECT(vllm_paged_read_pages(&tbuf, &tids, 3000, &tsink, nullptr) == VLLM_ERR_UNSUPPORTED, "page size");
}

}  // namespace

int main() {
  EXPECT(vllm_abi_version() == VLLM_PAGED_ABI_VERSION, "version");
  decode_sweep();
  decode_errors();
  cache_write_cases();
  prefill_cases();
  local_and_manager_cases();
  const int stub_bad = stub_failures();
  std::printf("%d launches checked, %d ABI check failures, %d launch check failures\n", stub_launches,
              g_bad, stub_bad);
  return (g_bad || stub_bad) ? 1 : 0;
}

// Host-only check of libkvarn's C-ABI layer (kvarn_api.hip), built for the
// host alone with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_sanitize_host.py. The launchers are replaced by stubs that
// record the arguments they would launch with, so every validation path and
// the launch arguments derived from valid calls are checked without a GPU.
// Exit status 0 = every check held (the sanitizers abort on their first
// finding).
#include <stdio.h>
#include <string.h>

#include "kvarn_diag.h"
#include "kvarn_internal.h"

namespace kvarn {

static QuantArgs g_quant[4];
static int g_nquant = 0;
static AppendArgs g_append;
static DecodeArgs g_decode;
static DiagArgs g_diag;
static int g_calls = 0;
static hipError_t g_result = hipSuccess;

hipError_t launch_quantize(const QuantArgs &a, hipStream_t) {
  if (g_nquant < 4) g_quant[g_nquant] = a;
  ++g_nquant;
  ++g_calls;
  return g_result;
}
hipError_t launch_append(const AppendArgs &a, hipStream_t) {
  g_append = a;
  ++g_calls;
  return g_result;
}
static AppendArgs g_append_kv[2];
hipError_t launch_append_kv(const AppendArgs &k, const AppendArgs &v, hipStream_t) {
  g_append_kv[0] = k;
  g_append_kv[1] = v;
  ++g_calls;
  return g_result;
}
hipError_t launch_decode(const DecodeArgs &a, hipStream_t) {
  g_decode = a;
  ++g_calls;
  return g_result;
}
hipError_t launch_token_error(const DiagArgs &a, hipStream_t) {
  g_diag = a;
  ++g_calls;
  return g_result;
}
int decode_auto_wgs(int, int, int, int capacity, int) { return decode_max_wgs(capacity); }
static int g_scratch_queries = 0;
void *noalloc_scratch(hipError_t *) {
  ++g_scratch_queries;
  return reinterpret_cast<void *>(0xC0000);
}

}  // namespace kvarn

using namespace kvarn;

static int failures = 0;
#define CHECK(cond)                                                         \
  do {                                                                      \
    if (!(cond)) {                                                          \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond);    \
      ++failures;                                                           \
    }                                                                       \
  } while (0)

// fake, 16-byte aligned device addresses: never dereferenced, the stubs only
// record them
static void *P(uintptr_t a) { return reinterpret_cast<void *>(a); }

static kvarn_cache cache(int batch = 2, int heads = 4, int cap = 512, int kind = KVARN_K) {
  kvarn_cache c{};
  c.codes = static_cast<uint8_t *>(P(0x10000));
  c.row_scale = static_cast<float *>(P(0x20000));
  c.col_scale = static_cast<float *>(P(0x30000));
  c.batch = batch;
  c.kv_heads = heads;
  c.capacity = cap;
  c.kind = kind;
  return c;
}

static void check_fastdiv() {
  const uint32_t ds[] = {1, 2, 3, 5, 7, 8, 255, 256, 257, 1000, 65535, 65536, 1u << 20, 2147483647u};
  const uint32_t ns[] = {0, 1, 2, 3, 127, 128, 65535, 65536, 999999, 2147483647u, 2147483646u};
  for (uint32_t d : ds) {
    const FastDiv f = make_fastdiv(d);
    for (uint32_t n : ns) CHECK((uint32_t)(((uint64_t)n * f.m) >> f.s) == n / d);
    for (uint32_t k = 0; k < 1000; ++k) {
      const uint32_t n = (uint32_t)(((uint64_t)k * 2654435761u) % 2147483648u);
      CHECK((uint32_t)(((uint64_t)n * f.m) >> f.s) == n / d);
    }
  }
}

static void check_quantize() {
  kvarn_cache c = cache();
  const int64_t sb = 4 * 512 * 128, sh = 512 * 128, st = 128;
  g_calls = 0;
  CHECK(kvarn_quantize(nullptr, KVARN_DT_BF16, sb, sh, st, 256, 0, 4, &c, nullptr) == KVARN_ERR_NULL);
  CHECK(kvarn_quantize(nullptr, KVARN_DT_BF16, sb, sh, st, 0, 0, 4, &c, nullptr) == KVARN_OK);
  CHECK(kvarn_quantize(P(0x40000), KVARN_DT_BF16, sb, sh, st, 256, 0, 4, nullptr, nullptr) == KVARN_ERR_NULL);
  CHECK(kvarn_quantize(P(0x40000), 7, sb, sh, st, 256, 0, 4, &c, nullptr) == KVARN_ERR_DTYPE);
  CHECK(kvarn_quantize(P(0x40000), KVARN_DT_BF16, sb, sh, st, 100, 0, 4, &c, nullptr) == KVARN_ERR_SHAPE);
  CHECK(kvarn_quantize(P(0x40000), KVARN_DT_BF16, sb, sh, st, 256, 64, 4, &c, nullptr) == KVARN_ERR_SHAPE);
  CHECK(kvarn_quantize(P(0x40000), KVARN_DT_BF16, sb, sh, st, 256, 0, 65, &c, nullptr) == KVARN_ERR_SHAPE);
  CHECK(kvarn_quantize(P(0x40000), KVARN_DT_BF16, sb, sh, 64, 256, 0, 4, &c, nullptr) == KVARN_ERR_SHAPE);
  CHECK(kvarn_quantize(P(0x40000), KVARN_DT_BF16, sb, sh, st, 512, 128, 4, &c, nullptr) == KVARN_ERR_CAPACITY);
  CHECK(kvarn_quantize(P(0x40002), KVARN_DT_BF16, sb, sh, st, 256, 0, 4, &c, nullptr) == KVARN_ERR_ALIGN);
  CHECK(kvarn_quantize(P(0x40000), KVARN_DT_BF16, sb, sh, 132, 256, 0, 4, &c, nullptr) == KVARN_ERR_ALIGN);
  CHECK(kvarn_quantize_ex(P(0x40000), KVARN_DT_BF16, sb, sh, st, 256, 0, 4, 2u, &c, nullptr) == KVARN_ERR_FLAGS);
  kvarn_cache bad = cache();
  bad.capacity = 500;
  CHECK(kvarn_quantize(P(0x40000), KVARN_DT_BF16, sb, sh, st, 256, 0, 4, &bad, nullptr) == KVARN_ERR_SHAPE);
  bad = cache();
  bad.kind = 3;
  CHECK(kvarn_quantize(P(0x40000), KVARN_DT_BF16, sb, sh, st, 256, 0, 4, &bad, nullptr) == KVARN_ERR_DTYPE);
  bad = cache();
  bad.row_scale = static_cast<float *>(P(0x20004));
  CHECK(kvarn_quantize(P(0x40000), KVARN_DT_BF16, sb, sh, st, 256, 0, 4, &bad, nullptr) == KVARN_ERR_ALIGN);
  CHECK(g_calls == 0);  // nothing launched on a rejected call

  g_nquant = 0;
  CHECK(kvarn_quantize_ex(P(0x40000), KVARN_DT_F32, sb, sh, st, 256, 128, 3, KVARN_FLAG_NO_ROTATE, &c,
                          nullptr) == KVARN_OK);
  CHECK(g_nquant == 1);
  const QuantArgs &a = g_quant[0];
  CHECK(a.nblocks == 2u * 4u * 2u);
  CHECK(a.chunks == 2 && a.chunk0 == 1 && a.iters == 3 && a.capacity == 512);
  CHECK(a.batch == 2 && a.heads == 4 && a.kind == KVARN_K && a.dtype == KVARN_DT_F32);
  CHECK(a.flags == KVARN_FLAG_NO_ROTATE && a.pos == nullptr);
  CHECK(a.sb == sb && a.sh == sh && a.st == st);
  CHECK(a.div_chunks.d == 2u && a.div_heads.d == 4u);
  g_result = hipErrorInvalidValue;
  CHECK(kvarn_quantize(P(0x40000), KVARN_DT_BF16, sb, sh, st, 256, 0, 4, &c, nullptr) == KVARN_ERR_HIP);
  g_result = hipSuccess;
}

static void check_append() {
  kvarn_cache c = cache(3, 2, 256, KVARN_V);
  g_calls = 0;
  CHECK(kvarn_append(nullptr, KVARN_DT_BF16, static_cast<int32_t *>(P(0x50000)), &c, nullptr) == KVARN_ERR_NULL);
  CHECK(kvarn_append(P(0x40000), KVARN_DT_BF16, nullptr, &c, nullptr) == KVARN_ERR_NULL);
  CHECK(kvarn_append(P(0x40000), 9, static_cast<int32_t *>(P(0x50000)), &c, nullptr) == KVARN_ERR_DTYPE);
  CHECK(kvarn_append(P(0x40008), KVARN_DT_BF16, static_cast<int32_t *>(P(0x50000)), &c, nullptr) == KVARN_ERR_ALIGN);
  CHECK(kvarn_append_ex(P(0x40000), KVARN_DT_BF16, static_cast<int32_t *>(P(0x50000)), 4u, &c, nullptr) ==
        KVARN_ERR_FLAGS);
  CHECK(kvarn_append_rebalance(P(0x40000), KVARN_DT_BF16, static_cast<int32_t *>(P(0x50000)), nullptr, 4, 0u,
                               &c, nullptr) == KVARN_ERR_NULL);
  CHECK(kvarn_append_rebalance(P(0x40000), KVARN_DT_BF16, static_cast<int32_t *>(P(0x50000)), P(0x60000), 70,
                               0u, &c, nullptr) == KVARN_ERR_SHAPE);
  CHECK(g_calls == 0);
  CHECK(kvarn_append(P(0x40000), KVARN_DT_BF16, static_cast<int32_t *>(P(0x50000)), &c, nullptr) == KVARN_OK);
  CHECK(g_append.batch == 3 && g_append.heads == 2 && g_append.capacity == 256);
  CHECK(g_append.kind == KVARN_V && g_append.window == nullptr);
  g_nquant = 0;
  CHECK(kvarn_append_rebalance(P(0x40000), KVARN_DT_F32, static_cast<int32_t *>(P(0x50000)), P(0x60000), 2,
                               KVARN_FLAG_NO_ROTATE, &c, nullptr) == KVARN_OK);
  CHECK(g_append.window == P(0x60000));
  CHECK(g_nquant == 1);
  const QuantArgs &a = g_quant[0];
  CHECK(a.pos == P(0x50000) && a.x == P(0x60000) && a.chunks == 1 && a.nblocks == 6u);
  CHECK(a.st == 128 && a.sh == 128 * 128 && a.sb == 2 * 128 * 128 && a.iters == 2);

  // K and V in one launch
  kvarn_cache k = cache(3, 2, 256, KVARN_K), v = c;
  v.codes = static_cast<uint8_t *>(P(0x70000));
  v.row_scale = static_cast<float *>(P(0x74000));
  int32_t *pos = static_cast<int32_t *>(P(0x50000));
  g_calls = 0;
  CHECK(kvarn_append_kv(P(0x40000), nullptr, KVARN_DT_BF16, pos, 0u, &k, &v, nullptr) == KVARN_ERR_NULL);
  CHECK(kvarn_append_kv(P(0x40000), P(0x48000), KVARN_DT_BF16, pos, 0u, &v, &k, nullptr) == KVARN_ERR_DTYPE);
  kvarn_cache v2 = cache(3, 2, 512, KVARN_V);
  CHECK(kvarn_append_kv(P(0x40000), P(0x48000), KVARN_DT_BF16, pos, 0u, &k, &v2, nullptr) == KVARN_ERR_SHAPE);
  CHECK(kvarn_append_kv(P(0x40000), P(0x48000), KVARN_DT_BF16, pos, 2u, &k, &v, nullptr) == KVARN_ERR_FLAGS);
  CHECK(g_calls == 0);
  CHECK(kvarn_append_kv(P(0x40000), P(0x48000), KVARN_DT_F32, pos, KVARN_FLAG_NO_ROTATE, &k, &v, nullptr) ==
        KVARN_OK);
  CHECK(g_calls == 1);
  CHECK(g_append_kv[0].x == P(0x40000) && g_append_kv[1].x == P(0x48000));
  CHECK(g_append_kv[0].kind == KVARN_K && g_append_kv[1].kind == KVARN_V);
  CHECK(g_append_kv[0].codes == k.codes && g_append_kv[1].codes == v.codes);
  CHECK(g_append_kv[0].pos == pos && g_append_kv[1].pos == pos);
  CHECK(g_append_kv[0].dtype == KVARN_DT_F32 && g_append_kv[1].flags == KVARN_FLAG_NO_ROTATE);
  CHECK(g_append_kv[0].batch == 3 && g_append_kv[0].heads == 2 && g_append_kv[1].capacity == 256);
  CHECK(g_append_kv[0].window == nullptr && g_append_kv[1].window == nullptr);
}

static void check_decode() {
  kvarn_cache k = cache(2, 4, 1024, KVARN_K), v = cache(2, 4, 1024, KVARN_V);
  v.codes = static_cast<uint8_t *>(P(0x70000));
  const int32_t *lens = static_cast<int32_t *>(P(0x50000));
  float *out = static_cast<float *>(P(0x80000));
  const size_t need = kvarn_decode_workspace_bytes(2, 16, 1024);
  // 2 x 16 counters (256 bytes), then 2 workgroups of partials per row
  CHECK(need == 256 + (size_t)2 * 16 * 2 * 130 * 4);
  CHECK(kvarn_decode_workspace_bytes(2, 16, 1000) == 0);
  CHECK(kvarn_decode_workspace_bytes(-1, 16, 1024) == 0);
  void *ws = P(0x90000);
  g_calls = 0;
  CHECK(kvarn_decode_attn(nullptr, KVARN_DT_BF16, 16, &k, &v, lens, 0.1f, out, 0, ws, need, nullptr) ==
        KVARN_ERR_NULL);
  CHECK(kvarn_decode_attn(P(0x40000), KVARN_DT_BF16, 16, &v, &k, lens, 0.1f, out, 0, ws, need, nullptr) ==
        KVARN_ERR_DTYPE);
  CHECK(kvarn_decode_attn(P(0x40000), KVARN_DT_BF16, 14, &k, &v, lens, 0.1f, out, 0, ws, need, nullptr) ==
        KVARN_ERR_SHAPE);
  CHECK(kvarn_decode_attn(P(0x40000), KVARN_DT_BF16, 40, &k, &v, lens, 0.1f, out, 0, ws, need, nullptr) ==
        KVARN_ERR_SHAPE);  // 10 query heads per kv-head
  CHECK(kvarn_decode_attn(P(0x40000), KVARN_DT_BF16, 16, &k, &v, lens, 0.1f, out, 0, ws, need - 1, nullptr) ==
        KVARN_ERR_WORKSPACE);
  CHECK(kvarn_decode_attn(P(0x40000), KVARN_DT_BF16, 16, &k, &v, lens, 0.1f, out, -1, ws, need, nullptr) ==
        KVARN_ERR_SHAPE);
  CHECK(kvarn_decode_attn(P(0x40000), KVARN_DT_BF16, 16, &k, &v, lens, __builtin_nanf(""), out, 0, ws, need,
                          nullptr) == KVARN_ERR_SHAPE);
  CHECK(kvarn_decode_attn_ex(P(0x40000), KVARN_DT_BF16, 16, &k, &v, lens, 0.1f, 8u, out, 0, ws, need,
                             nullptr) == KVARN_ERR_FLAGS);
  kvarn_cache v2 = v;
  v2.capacity = 512;
  CHECK(kvarn_decode_attn(P(0x40000), KVARN_DT_BF16, 16, &k, &v2, lens, 0.1f, out, 0, ws, need, nullptr) ==
        KVARN_ERR_SHAPE);
  CHECK(g_calls == 0);
  CHECK(kvarn_decode_attn(P(0x40000), KVARN_DT_F32, 16, &k, &v, lens, 0.25f, out, 100, ws, need, nullptr) ==
        KVARN_OK);
  CHECK(g_decode.n_wg == 2);  // 100 splits: 25 workgroups, clamped to 8 chunks / 4
  CHECK(g_decode.q_heads == 16 && g_decode.kv_heads == 4 && g_decode.batch == 2);
  CHECK(g_decode.k_codes == k.codes && g_decode.v_codes == v.codes && g_decode.scale == 0.25f);
  CHECK(g_decode.counters == ws && g_decode.out == out && g_decode.q_dtype == KVARN_DT_F32);
  CHECK((char *)g_decode.partial == (char *)ws + 256);
  CHECK(kvarn_decode_attn(P(0x40000), KVARN_DT_BF16, 16, &k, &v, lens, 0.25f, out, 3, ws, need, nullptr) ==
        KVARN_OK);
  CHECK(g_decode.n_wg == 1);
}

static void check_decode_noalloc() {
  kvarn_cache k = cache(2, 4, 1024, KVARN_K), v = cache(2, 4, 1024, KVARN_V);
  const int32_t *lens = static_cast<int32_t *>(P(0x50000));
  float *out = static_cast<float *>(P(0x80000));
  g_calls = 0;
  g_scratch_queries = 0;
  CHECK(kvarn_decode_attn_noalloc(nullptr, KVARN_DT_BF16, 16, &k, &v, lens, 0.1f, 0u, out, 0,
                                  nullptr) == KVARN_ERR_NULL);
  CHECK(kvarn_decode_attn_noalloc(P(0x40000), KVARN_DT_BF16, 14, &k, &v, lens, 0.1f, 0u, out, 0,
                                  nullptr) == KVARN_ERR_SHAPE);
  // partials beyond the fixed array: 64 sequences x 64 query heads x 16 workgroups x 520 B
  kvarn_cache kb = cache(64, 8, 128 * 1024, KVARN_K), vb = cache(64, 8, 128 * 1024, KVARN_V);
  CHECK(kvarn_decode_attn_noalloc(P(0x40000), KVARN_DT_BF16, 64, &kb, &vb, lens, 0.1f, 0u, out,
                                  64, nullptr) == KVARN_ERR_WORKSPACE);
  CHECK(g_calls == 0 && g_scratch_queries == 0);
  CHECK(kvarn_decode_attn_noalloc(P(0x40000), KVARN_DT_BF16, 16, &k, &v, lens, 0.5f,
                                  KVARN_FLAG_ONE_SCALE, out, 0, nullptr) == KVARN_OK);
  CHECK(g_calls == 1 && g_scratch_queries == 1);
  CHECK((void *)g_decode.counters == P(0xC0000) && g_decode.n_wg == 2 && g_decode.scale == 0.5f);
  CHECK((char *)g_decode.partial == (char *)P(0xC0000) + 256);
  CHECK(g_decode.flags == KVARN_FLAG_ONE_SCALE);
}

static void check_token_error() {
  kvarn_cache c = cache(2, 2, 256, KVARN_K);
  float *r = static_cast<float *>(P(0xA0000)), *q = static_cast<float *>(P(0xB0000));
  g_calls = 0;
  CHECK(kvarn_token_error(P(0x40000), KVARN_DT_BF16, 2 * 256 * 128, 256 * 128, 128, 300, 0, 0u, &c, r, q,
                          nullptr) == KVARN_ERR_CAPACITY);
  CHECK(kvarn_token_error(P(0x40000), KVARN_DT_BF16, 2 * 256 * 128, 256 * 128, 128, 10, 0, 0u, &c, nullptr,
                          q, nullptr) == KVARN_ERR_NULL);
  CHECK(kvarn_token_error(P(0x40000), KVARN_DT_BF16, 2 * 256 * 128, 256 * 128, 128, 10, 0, 0u, &c,
                          static_cast<float *>(P(0xA0002)), q, nullptr) == KVARN_ERR_ALIGN);
  CHECK(kvarn_token_error(P(0x40000), KVARN_DT_BF16, 2 * 256 * 128, 256 * 128, 128, 0, 0, 0u, &c, nullptr,
                          nullptr, nullptr) == KVARN_OK);
  CHECK(g_calls == 0);
  CHECK(kvarn_token_error(P(0x40000), KVARN_DT_BF16, 2 * 256 * 128, 256 * 128, 128, 10, 3, 1u, &c, r, q,
                          nullptr) == KVARN_OK);
  CHECK(g_diag.tokens == 10 && g_diag.token_offset == 3 && g_diag.flags == 1u);
}

static void check_head_dim() {
  g_calls = 0;
  kvarn_cache c = cache(2, 2, 256, KVARN_K);
  c.head_dim = 96;
  CHECK(kvarn_quantize(P(0x40000), KVARN_DT_BF16, 0, 0, 128, 256, 0, 4, &c, nullptr) == KVARN_ERR_SHAPE);
  c.head_dim = 256;
  // a token row narrower than the head
  CHECK(kvarn_quantize(P(0x40000), KVARN_DT_BF16, 2 * 256 * 256, 256 * 256, 128, 256, 0, 4, &c, nullptr) ==
        KVARN_ERR_SHAPE);
  CHECK(g_calls == 0);
  g_nquant = 0;
  CHECK(kvarn_quantize(P(0x40000), KVARN_DT_BF16, 2 * 256 * 256, 256 * 256, 256, 256, 0, 4, &c, nullptr) ==
        KVARN_OK);
  CHECK(g_quant[0].head_dim == 256);
  CHECK(kvarn_append(P(0x40000), KVARN_DT_BF16, static_cast<int32_t *>(P(0x50000)), &c, nullptr) == KVARN_OK);
  CHECK(g_append.head_dim == 256);
  float *r = static_cast<float *>(P(0xA0000)), *q = static_cast<float *>(P(0xB0000));
  CHECK(kvarn_token_error(P(0x40000), KVARN_DT_BF16, 2 * 256 * 256, 256 * 256, 256, 10, 0, 0u, &c, r, q,
                          nullptr) == KVARN_OK);
  CHECK(g_diag.head_dim == 256);
  // decode: K and V must share the head size, and partials are sized by it
  kvarn_cache k = cache(2, 4, 1024, KVARN_K), v = cache(2, 4, 1024, KVARN_V);
  k.head_dim = v.head_dim = 64;
  const size_t need = kvarn_decode_workspace_bytes_ex(2, 16, 1024, 64);
  CHECK(need == 256 + (size_t)2 * 16 * 2 * (64 + 2) * 4);
  CHECK(kvarn_decode_workspace_bytes_ex(2, 16, 1024, 96) == 0);
  CHECK(kvarn_decode_workspace_bytes_ex(2, 16, 1024, 128) == kvarn_decode_workspace_bytes(2, 16, 1024));
  const int32_t *lens = static_cast<int32_t *>(P(0x50000));
  float *out = static_cast<float *>(P(0x80000));
  v.head_dim = 256;
  CHECK(kvarn_decode_attn(P(0x40000), KVARN_DT_BF16, 16, &k, &v, lens, 0.1f, out, 0, P(0x90000), need,
                          nullptr) == KVARN_ERR_SHAPE);
  v.head_dim = 64;
  CHECK(kvarn_decode_attn(P(0x40000), KVARN_DT_BF16, 16, &k, &v, lens, 0.1f, out, 0, P(0x90000), need - 1,
                          nullptr) == KVARN_ERR_WORKSPACE);
  CHECK(kvarn_decode_attn(P(0x40000), KVARN_DT_BF16, 16, &k, &v, lens, 0.1f, out, 0, P(0x90000), need,
                          nullptr) == KVARN_OK);
  CHECK(g_decode.head_dim == 64 && g_decode.n_wg == 2);
}

static void check_status_strings() {
  for (int s = -9; s <= 1; ++s) {
    const char *t = kvarn_status_string(s);
    CHECK(t != nullptr && strlen(t) > 0);
  }
}

int main() {
  check_fastdiv();
  check_quantize();
  check_append();
  check_decode();
  check_decode_noalloc();
  check_token_error();
  check_head_dim();
  check_status_strings();
  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("kvarn_api host check ok\n");
  return 0;
}
